// Fused dequantizing product for a few activation rows (bf16 x, up to 16 rows; w4_gemv
// sends most shapes with 2 <= M <= 16 here) on the matrix cores.
//
// y[m, n] = sum_g scale16[n, g] * sum_{k in g} (q[n, k] - zero[n, g]) x[m, k] (page
// "Weight quantization", section "How it works": the dequantized weight is
// (code - zero) * scale and the scale multiplies once per group), with the M dot
// products per weight done by v_mfma_f32_16x16x32_bf16 instead of the vector ALU.  The
// weight stream stays the bound for every M up to 16: with VALU dot products the work
// per weight grows with M, and the pages note that batched decode moves towards compute
// (page "Weight quantization" › "Implementation notes": past a batch of about 16-32,
// dequantization inside the product turns compute-heavy).
//
// Exact operands: the matrix instruction aligns the 32 products of a step and the
// accumulator to the largest before it rounds, so an operand with a bias (128 + q, the
// bias removed later through sum x) would lose bits in proportion to the bias, not to the
// result.  The B operand is the exact bf16 value q - zero of every code: v_and_or_b32
// builds binary16 1024 + q (or 1024 + 16 q for the codes at bits 4..7 of a half word),
// v_pk_add_f16 subtracts 1024 + zero (1024 + 16 zero) exactly, and two scaled conversions
// (binary16 -> E4M3 -> bf16, exact for these small integers; the second one scales the
// 16 (q - zero) values back by 2^-4) give bf16.  x enters unchanged as bf16, every product
// is exact, and a code equal to its zero contributes exactly 0.  (The resident-x kernel
// further down takes binary16 x and the binary16 codes themselves where that pays.)
//
// Mapping (gfx950, wave64):
//   * the waves of a workgroup split K: wave w takes groups [w*gpw, (w+1)*gpw);
//     a workgroup owns 16*T consecutive rows (T tiles of 16), and partial sums
//     of its waves are added through LDS in wave order (deterministic);
//   * a wave works through its groups a pair at a time.  The codes of a pair
//     reach the wave's LDS with loads of 8 rows x 128 contiguous bytes (eight
//     full lines; a load in the MFMA lane order, 16 rows x 64 bytes, touches
//     sixteen half lines), x of each group (16 rows x 128 inputs) with loads
//     of 4 rows x 256 contiguous bytes, and the scale/zero words go straight
//     to registers.  XOR swizzles of the 16-byte chunks let each lane read
//     its MFMA operands back with no bank conflicts.  The loads of the next
//     pair are issued as soon as the current pair is read out of LDS, so they
//     are in flight while the current pair is computed;
//   * MFMA step s (s = 0..3) of a group: A = x rows (lane l supplies row l % 16,
//     k = 32*(l/16) + 8s .. +7), B = the exact codes of the tile's 16 rows (lane l
//     supplies column l % 16, same k).  Four steps give P[m][n] = sum (q - zero) x for
//     the group in a fresh accumulator, and acc += scale16 * P (one FMA per output);
//   * the 16x16 result sits in lane l as column n = l % 16, rows
//     m = 4*(l/16) + v (v = 0..3): one scale/zero word per lane and tile.
#include <atomic>
#include <type_traits>

#include "w4_internal.h"

namespace w4 {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kRedStride = 17;  // floats per row of the LDS partial sums (16 + pad)

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }

typedef __attribute__((ext_vector_type(2))) _Float16 f16x2_t;
typedef __attribute__((ext_vector_type(2))) short s16x2_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;

__device__ __forceinline__ uint32_t add2h(uint32_t a, uint32_t b) {
    return __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2_t, a) + __builtin_bit_cast(f16x2_t, b));
}

// Constants of the code unpack, kept in registers so that v_and_or_b32 is selected.
struct CodeConsts {
    uint32_t m_lo, m_hi, magic, e4;
    __device__ __forceinline__ CodeConsts() {
        asm volatile("s_mov_b32 %0, 0x000F000F" : "=s"(m_lo));
        asm volatile("s_mov_b32 %0, 0x00F000F0" : "=s"(m_hi));
        asm volatile("v_mov_b32 %0, 0x64006400" : "=v"(magic));
        asm volatile("s_mov_b32 %0, 0xE4E4E4E4" : "=s"(e4));
    }
    // binary16 pairs -(1024 + zero) and -(1024 + 16 zero) from bytes 2 and 3 of a
    // scale/zero word
    __device__ __forceinline__ uint32_t z1(uint32_t szw) const { return __builtin_amdgcn_perm(e4, szw, 0x04020402u); }
    __device__ __forceinline__ uint32_t z16(uint32_t szw) const { return __builtin_amdgcn_perm(e4, szw, 0x04030403u); }
};

// Scale of the bf16 conversion of the values 16 (q - zero): back to q - zero.
constexpr float kSixteenthBack = 0.0625f;

// The eight codes of a prepared word (inputs 0..7: pairs at bits 4j / 16 + 4j) as the
// exact bf16 values q - zero, in input order.
__device__ __forceinline__ u32x4_t exact_codes(uint32_t w, uint32_t z1, uint32_t z16, const CodeConsts& c) {
    const uint32_t u = w >> 8;
    const f16x2_t h0 = __builtin_bit_cast(f16x2_t, add2h((w & c.m_lo) | c.magic, z1));   // inputs 0, 1
    const f16x2_t h1 = __builtin_bit_cast(f16x2_t, add2h((w & c.m_hi) | c.magic, z16));  // 2, 3 (x16)
    const f16x2_t h2 = __builtin_bit_cast(f16x2_t, add2h((u & c.m_lo) | c.magic, z1));   // 4, 5
    const f16x2_t h3 = __builtin_bit_cast(f16x2_t, add2h((u & c.m_hi) | c.magic, z16));  // 6, 7 (x16)
    // the first conversion of each pair writes the low half of a register whose high half
    // the second one writes: start from h0 / h2 themselves, so no zeroed register is needed
    s16x2_t e01 = __builtin_bit_cast(s16x2_t, h0), e23 = __builtin_bit_cast(s16x2_t, h2);
    e01 = __builtin_amdgcn_cvt_scalef32_pk_fp8_f16(e01, h0, 1.0f, false);
    e01 = __builtin_amdgcn_cvt_scalef32_pk_fp8_f16(e01, h1, 1.0f, true);
    e23 = __builtin_amdgcn_cvt_scalef32_pk_fp8_f16(e23, h2, 1.0f, false);
    e23 = __builtin_amdgcn_cvt_scalef32_pk_fp8_f16(e23, h3, 1.0f, true);
    const uint32_t f01 = __builtin_bit_cast(uint32_t, e01), f23 = __builtin_bit_cast(uint32_t, e23);
    const u32x4_t r = {
        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(f01, 1.0f, false)),
        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(f01, kSixteenthBack, true)),
        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(f23, 1.0f, false)),
        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(f23, kSixteenthBack, true))};
    return r;
}

typedef __attribute__((ext_vector_type(8))) _Float16 f16x8_t;
typedef __attribute__((ext_vector_type(2))) unsigned short u16x2_t;

__device__ __forceinline__ f16x8_t as_f16x8(u32x4_t v) { return __builtin_bit_cast(f16x8_t, v); }

// The eight codes of a prepared word as the exact binary16 values q - zero (inputs 0, 1, 4,
// 5) and 16 (q - zero) (inputs 2, 3, 6, 7), in input order.
__device__ __forceinline__ u32x4_t exact_codes_f16(uint32_t w, uint32_t z1, uint32_t z16, const CodeConsts& c) {
    const uint32_t u = w >> 8;
    const u32x4_t r = {add2h((w & c.m_lo) | c.magic, z1), add2h((w & c.m_hi) | c.magic, z16),
                       add2h((u & c.m_lo) | c.magic, z1), add2h((u & c.m_hi) | c.magic, z16)};
    return r;
}

__device__ __forceinline__ u16x2_t as_u16x2(uint32_t v) { return __builtin_bit_cast(u16x2_t, v); }

// bf16 pair -> binary16 pair of x * 2^-E by integer steps (c2 = (F_max - 30) << 7 in both
// halves, or (F_max - 26) << 7 for a further 2^-4): exact whenever the result is a normal
// binary16 value, which the caller's range check guarantees; a zero stays zero.
__device__ __forceinline__ uint32_t to_f16_pair(uint32_t xb, uint32_t c2) {
    const u16x2_t mag = as_u16x2(xb & 0x7FFF7FFFu);
    const u16x2_t r = __builtin_elementwise_sub_sat(mag, as_u16x2(c2)) << (unsigned short)3;
    return __builtin_bit_cast(uint32_t, r) | (xb & 0x80008000u);
}

__device__ __forceinline__ uint32_t max_across_rows(uint32_t v) {
    // maximum over the four lanes l % 16 + 16 j (j = 0..3)
    const auto h = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    const uint32_t a = max((uint32_t)h[0], (uint32_t)h[1]);
    const auto q = __builtin_amdgcn_permlane16_swap(a, a, false, false);
    return max((uint32_t)q[0], (uint32_t)q[1]);
}

__device__ __forceinline__ uint32_t bf16_bits_rne(float f) {
    const uint32_t u = __float_as_uint(f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ void lds_dma16(const void* g, uint32_t lds_addr);
// the same load with a uniform base address in SGPRs and a per-lane 32-bit byte offset
__device__ __forceinline__ void lds_dma16_sv(const void* sbase, uint32_t voff, uint32_t lds_addr) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(voff), "s"(sbase), "s"(lds_addr)
                 : "memory");
}
__device__ __forceinline__ void lds_dma4_sv(const void* sbase, uint32_t voff, uint32_t lds_addr) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1"
                 :
                 : "v"(voff), "s"(sbase), "s"(lds_addr)
                 : "memory");
}
constexpr int kXStageBytes = 16 * 256;   // x of one group: 16 rows x 128 inputs (bf16)

// T: tiles of 16 rows per workgroup; CH: groups whose loads are issued together (a pair)
template <int T, int CH>
__global__ __launch_bounds__(512) void gemv_mfma_kernel(const uint8_t* __restrict__ wq,
                                                         const uint32_t* __restrict__ sz,
                                                         const uint16_t* __restrict__ x,
                                                         void* __restrict__ yv, int y_bf16, int N,
                                                         int K, int M, int gpw) {
    static_assert(CH == 2, "codes are staged a group pair at a time");
    constexpr int RW = 16 * T;
    constexpr int kWaveBytes = CH * kXStageBytes + 2 * T * 1024;
    // per wave CH x stages and 2T code blocks during the group loop; afterwards the same
    // bytes hold the partial sums [waves][RW][kRedStride]
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    float* red = reinterpret_cast<float*>(smem);

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: SGPR addresses
    const int n_waves = blockDim.x >> 6;
    const int Kg = K >> 7;
    const int r0 = blockIdx.x * RW;
    const int col = lane & 15;
    const int kb = lane >> 4;
    const int g0 = wave * gpw;
    const int g1 = min(Kg, g0 + gpw);
    const int64_t row_bytes = K >> 1;

    const uint32_t xstage = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)smem + wave * kWaveBytes);
    const uint32_t cstage = xstage + CH * kXStageBytes;
    const uint8_t* xstage_p = smem + wave * kWaveBytes;
    const uint8_t* cstage_p = xstage_p + CH * kXStageBytes;

    // Codes of a group pair reach LDS as 2T loads of 8 rows x 128 contiguous bytes (eight
    // full lines).  In the load for rows 8d .. 8d+7 of tile t, lane l takes row 8d + (l >> 3),
    // group h = ((l >> 2) & 1) ^ d of the pair and 16-byte piece p = (l & 3) ^ (l >> 4), so
    // that the reads in MFMA lane order below hit 16 distinct bank quads per 16 lanes.
    // Rows past N repeat row N-1 (never stored).
    // Each lane's byte offset from group 0 of the workgroup's first row is fixed; the group
    // pair moves a uniform base.  (In the last pair of a wave with an odd number of groups the
    // lanes of group g + 1 read the next group: the next wave's, the next row's, or for the
    // last row the first bytes of the scale/zero words; scale 0 drops it.)
    const uint8_t* wrow0 = wq + (int64_t)r0 * row_bytes;
    uint32_t coff[T][2];
#pragma unroll
    for (int d = 0; d < 2; ++d) {
        const int chalf = ((lane >> 2) & 1) ^ d;
#pragma unroll
        for (int t = 0; t < T; ++t) {
            const int n = min(r0 + 16 * t + 8 * d + (lane >> 3), N - 1);
            coff[t][d] = (uint32_t)((int64_t)(n - r0) * row_bytes) + 16 * ((lane & 3) ^ (lane >> 4)) + 64 * chalf;
        }
    }
    // scale/zero word of this lane's row (column col of the MFMA tile) in each tile
    const uint32_t* szrow[T];
#pragma unroll
    for (int t = 0; t < T; ++t) {
        const int n = min(r0 + 16 * t + col, N - 1);
        szrow[t] = sz + (int64_t)(n >> 2) * Kg * 4 + (n & 3);
    }
    // x of a group reaches the x stage with loads of 4 rows x 256 contiguous bytes (chunk c
    // of row r at slot c ^ (r & 15)); rows m >= M repeat row M-1.  Only the first ceil(M/4)
    // quads of rows are loaded: MFMA rows past them read stale stage bytes and give only
    // outputs m >= M, which are dropped.
    const int xquads = (M + 3) >> 2;
    uint32_t xoff[4];   // bytes from x
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = 4 * i + (lane >> 4);
        xoff[i] = 2u * (uint32_t)(min(r, M - 1) * K + 8 * ((lane & 15) ^ (r & 15)));
    }

    const CodeConsts cc;
    const f32x4_t zero4 = {0.0f, 0.0f, 0.0f, 0.0f};

    f32x4_t acc[T];
#pragma unroll
    for (int t = 0; t < T; ++t) acc[t] = zero4;

    // binary16 x for up to four rows of x: x * 2^-E per row of x, E putting the row's
    // largest value over this wave's groups just under 2^16 (a pass over those groups of x,
    // lane l reading row l >> 4, chunk l & 15), exact when every non-zero value lands on a
    // normal binary16 (within 2^25 of the largest, also after the further 2^-4 at the inputs
    // of the 16 (q - zero) codes).  Each group pair's staged x is then converted where it
    // landed, all 64 lanes holding rows of x, and the codes need no bf16 conversion (9
    // instead of 17 vector instructions per eight codes).  A wave whose rows do not all pass
    // keeps bf16 x.  Measured on MI355X (70B down 8192 x 28672 at M = 4: 32.3 -> 29.9 us);
    // with eight rows the pass and the conversion cost more than the codes save (33.6 -> 37.6).
    bool f16 = false;
    int fq = 0;   // largest bf16 exponent field of row lane >> 4
    if (xquads == 1 && g0 < g1) {
        const uint16_t* xr = x + (int64_t)min(lane >> 4, M - 1) * K + 8 * (lane & 15);
        u16x2_t vmax = {0, 0}, vmin = {0xFFFF, 0xFFFF};
        // batches of 16 groups: every load of a batch is in flight before any is used
        for (int gb = g0; gb < g1; gb += 16) {
            u32x4_t v[16];
#pragma unroll
            for (int u = 0; u < 16; ++u)
                v[u] = *reinterpret_cast<const u32x4_t*>(xr + (int64_t)min(gb + u, g1 - 1) * 128);
#pragma unroll
            for (int u = 0; u < 16; ++u)
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    const u16x2_t mag = as_u16x2(v[u][d] & 0x7FFF7FFFu);
                    vmax = __builtin_elementwise_max(vmax, mag);
                    vmin = __builtin_elementwise_min(vmin, mag - (unsigned short)1);  // 0 -> 0xFFFF
                }
        }
        // over the 16 lanes of the row (one 16-lane row of the wave)
        uint32_t mx = max(vmax.x, vmax.y), mn = min(vmin.x, vmin.y);
        mx = max(mx, (uint32_t)__builtin_amdgcn_mov_dpp((int)mx, 0x128, 0xF, 0xF, false));
        mn = min(mn, (uint32_t)__builtin_amdgcn_mov_dpp((int)mn, 0x128, 0xF, 0xF, false));
        mx = max(mx, (uint32_t)__builtin_amdgcn_mov_dpp((int)mx, 0x124, 0xF, 0xF, false));
        mn = min(mn, (uint32_t)__builtin_amdgcn_mov_dpp((int)mn, 0x124, 0xF, 0xF, false));
        mx = max(mx, (uint32_t)__builtin_amdgcn_mov_dpp((int)mx, 0x122, 0xF, 0xF, false));
        mn = min(mn, (uint32_t)__builtin_amdgcn_mov_dpp((int)mn, 0x122, 0xF, 0xF, false));
        mx = max(mx, (uint32_t)__builtin_amdgcn_mov_dpp((int)mx, 0x121, 0xF, 0xF, false));
        mn = min(mn, (uint32_t)__builtin_amdgcn_mov_dpp((int)mn, 0x121, 0xF, 0xF, false));
        fq = (int)(mx >> 7);
        const int mnz = (int)mn + 1;
        const bool bad = mnz != 0x10000 && (fq < 30 || fq == 255 || mnz < ((fq - 25) << 7));
        f16 = __builtin_amdgcn_ballot_w64(bad) == 0;
    }
    const uint32_t xce = (uint32_t)((fq - 30) << 7) * 0x00010001u;   // conversion constants
    const uint32_t xco = (uint32_t)((fq - 26) << 7) * 0x00010001u;
    uint8_t* xstage_w = smem + wave * kWaveBytes;

    uint32_t sb[2][CH][T];
    // loads of the pair g, g+1 (a group past the wave's range repeats its last group: a cache
    // hit that contributes nothing): codes, scale/zero words, x
    auto issue = [&](auto bc, int g) {
        constexpr int b = decltype(bc)::value;
        const uint8_t* cbase = wrow0 + (int64_t)g * 64;
#pragma unroll
        for (int t = 0; t < T; ++t)
#pragma unroll
            for (int d = 0; d < 2; ++d) lds_dma16_sv(cbase, coff[t][d], cstage + (2 * t + d) * 1024);
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const int gc = min(g + c, g1 - 1);
#pragma unroll
            for (int t = 0; t < T; ++t) sb[b][c][t] = szrow[t][gc * 4];
            const uint8_t* xbase = reinterpret_cast<const uint8_t*>(x) + (int64_t)gc * 256;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (i < xquads) lds_dma16_sv(xbase, xoff[i], xstage + c * kXStageBytes + i * 1024);
        }
        __builtin_amdgcn_sched_barrier(0);  // keep the loads ahead of the compute
    };
    auto step = [&](auto fc, auto bc, int g) {
        constexpr bool F = decltype(fc)::value;
        constexpr int b = decltype(bc)::value;
        // every load of this pair has landed (the next pair's are not issued yet)
        __builtin_amdgcn_s_waitcnt(0x0F70);
        asm volatile("" ::: "memory");
        if constexpr (F) {
            // binary16 x: each lane converts the 16 bytes it staged (row lane >> 4), in place
#pragma unroll
            for (int c = 0; c < CH; ++c) {
                u32x4_t* slot = reinterpret_cast<u32x4_t*>(xstage_w + c * kXStageBytes + 16 * lane);
                u32x4_t v = *slot;
#pragma unroll
                for (int d = 0; d < 4; ++d) v[d] = to_f16_pair(v[d], (d & 1) ? xco : xce);
                *slot = v;
            }
            __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
            asm volatile("" ::: "memory");
        }
        u32x4_t xb[CH][4];
        u32x4_t wb[CH][T];
#pragma unroll
        for (int c = 0; c < CH; ++c)
#pragma unroll
            for (int s = 0; s < 4; ++s)
                xb[c][s] = *reinterpret_cast<const u32x4_t*>(
                    xstage_p + c * kXStageBytes + col * 256 + (((4 * kb + s) ^ col) * 16));
        const int cd = col >> 3, cr = col & 7;
#pragma unroll
        for (int c = 0; c < CH; ++c)
#pragma unroll
            for (int t = 0; t < T; ++t)
                wb[c][t] = *reinterpret_cast<const u32x4_t*>(
                    cstage_p + (2 * t + cd) * 1024 + 16 * (8 * cr + 4 * (c ^ cd) + (kb ^ (cr >> 1))));
        // the stages are read out before the next pair lands in them
        __builtin_amdgcn_s_waitcnt(0xC07F);
        asm volatile("" ::: "memory");
        if (g + CH < g1) issue(std::integral_constant<int, b ^ 1>{}, g + CH);
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            // a group past the wave's range is computed with scale 0 (no branch)
            const float keep = g + c < g1 ? 1.0f : 0.0f;
#pragma unroll
            for (int t = 0; t < T; ++t) {
                const uint32_t szw = sb[b][c][t];
                const uint32_t z1 = cc.z1(szw), z16 = cc.z16(szw);
                f32x4_t p = zero4;
                if constexpr (F) {
#pragma unroll
                    for (int s = 0; s < 4; ++s)
                        p = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                            as_f16x8(xb[c][s]), as_f16x8(exact_codes_f16(wb[c][t][s], z1, z16, cc)), p, 0, 0, 0);
                } else {
#pragma unroll
                    for (int s = 0; s < 4; ++s)
                        p = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            as_bf16x8(xb[c][s]), as_bf16x8(exact_codes(wb[c][t][s], z1, z16, cc)), p, 0, 0, 0);
                }
                const float sc =
                    keep * (float)__builtin_bit_cast(_Float16, (uint16_t)(szw & 0xFFFFu));
#pragma unroll
                for (int v = 0; v < 4; ++v) acc[t][v] = fmaf(sc, p[v], acc[t][v]);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    };

    // (a wave without groups skips the loop; the host sizes the grid so that none is)
    auto run = [&](auto fc) {
        issue(std::integral_constant<int, 0>{}, g0);
        for (int g = g0; g < g1; g += 2 * CH) {
            step(fc, std::integral_constant<int, 0>{}, g);
            if (g + CH >= g1) break;
            step(fc, std::integral_constant<int, 1>{}, g + CH);
        }
    };
    if (g0 < g1) {
        if (f16)
            run(std::integral_constant<bool, true>{});
        else
            run(std::integral_constant<bool, false>{});
    }

    // 2^E of the rows m = 4 kb + v this lane accumulates (binary16 x has at most four rows:
    // row m's exponent sits in lanes 16 m .. 16 m + 15)
    int ev[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        const int a0 = __shfl(fq, 16 * v);   // rows past the fourth are never stored here
        ev[v] = f16 ? a0 - 127 - 15 : 0;
    }
    __syncthreads();   // every wave is done with its stages: the LDS now takes the sums
    // partial sums of this wave: lane holds column n = col, rows m = 4*kb + v
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int m = 4 * kb + v;
            if (m < M) red[(wave * RW + 16 * t + col) * kRedStride + m] = ldexpf(acc[t][v], ev[v]);
        }
    __syncthreads();

    const int rows_here = min(RW, N - r0);
    for (int i = threadIdx.x; i < rows_here * M; i += blockDim.x) {
        const int m = i / rows_here;
        const int r = i - m * rows_here;
        float v = 0.0f;
        for (int w = 0; w < n_waves; ++w) v += red[(w * RW + r) * kRedStride + m];
        const int64_t o = (int64_t)m * N + r0 + r;
        if (y_bf16)
            static_cast<uint16_t*>(yv)[o] = (uint16_t)bf16_bits_rne(v);
        else
            static_cast<float*>(yv)[o] = v;
    }
}

// Variant for K <= 8192 (at most eight groups per wave, at most eight waves): x resident in
// registers, codes straight into registers.
//   * Each wave keeps the A operands of its groups (x, four MFMA steps per group) in
//     registers, then walks all rows of the workgroup in steps of 16.  The A operands
//     arrive through the wave's LDS area in two rounds of four groups, with loads of
//     4 rows x 256 contiguous bytes.
//   * Codes load straight into registers.  Load d = 2p + h of a row step covers rows
//     8h .. 8h + 7 x the 128 contiguous bytes of groups 2p, 2p + 1 (eight full cache lines):
//     lane l takes row 8h + (l & 7), group 2p + ((l >> 3) & 1), 16-byte piece l >> 4.  The
//     MFMA wants lane l to hold row l & 15 of one group, so the two loads of a pair are
//     exchanged between lanes l and l ^ 8 (one DPP row rotation by 8 and one select per
//     register, four instructions per 32 codes).  A load in the MFMA lane order itself
//     (16 rows x 64 bytes) touches sixteen half lines and streams 5-20 % slower; staging
//     the codes through an LDS ring (direct-to-LDS loads) streamed about 16 % slower than
//     these register loads on the 70B gate_up shape.
//   * The loads are buffer loads from a uniform base with fixed 32-bit lane offsets, so a
//     load costs no address arithmetic; the next row step's loads of a group pair go out
//     as soon as that pair of the current step has been used, so one set of registers
//     holds the codes (x takes 128 of the 256).  With more than eight rows of x the first
//     row step instead goes through LDS with direct-to-LDS loads while x is converted, when
//     the registers are busy.
//   * A row step starts at row min(r0 + 16 t, N - 16): the last step of the last
//     workgroup moves back into the matrix and stores only its new rows, so no load needs
//     a per-lane bound.
//   * Scale/zero: lane (col, kb) loads the word of group g + kb of its row; three permlane
//     swaps give every lane of the column the words of all four groups.
//   * Partial sums of the waves meet in LDS after every row step (double-buffered, one
//     barrier per step), scaled there by each wave's 2^E.
//   * A row step is compiled per activation format and per whether it issues the next
//     step's loads, so its eight groups are straight-line code.
//   * A wave whose x converts exactly to binary16 with one power-of-two exponent (over
//     its groups and all rows of x) keeps binary16 x in its A operands and uses the exact
//     binary16 codes with v_mfma_f32_16x16x32_f16: 9 instead of 17 vector instructions per
//     eight codes, for about 1000 once per workgroup at 16 rows of x.  With up to eight rows
//     each lane converts the bytes it staged (all 64 lanes hold rows of x) before the reads
//     in MFMA order, a quarter (M <= 4) or half (M <= 8) of that work.
constexpr int kXrGroups = 8;                        // groups per wave
constexpr int kXrWaveLds = 17 * 1024;               // per wave: x staging (16 KB), then the
                                                    // first row step (8.5 KB) and E (64 B)
constexpr int kXrRedBytes = 2 * 16 * kRedStride * 4;   // per wave: two row steps

__device__ __forceinline__ void lds_dma16(const void* g, uint32_t lds_addr) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(g), "s"(lds_addr)
                 : "memory", "m0");
}
__device__ __forceinline__ void lds_dma4(const void* g, uint32_t lds_addr) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
                 :
                 : "v"(g), "s"(lds_addr)
                 : "memory", "m0");
}

// s_waitcnt immediate waiting for vmcnt <= n only (gfx9 encoding)
constexpr int vm_imm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x70 | 0xF00; }

// barrier for LDS data only: no fence, so no wait for the code loads in flight
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// v: one word per lane; returns b[j] = v of lane (l % 16) + 16 j, for every lane l
__device__ __forceinline__ void bcast_rows(uint32_t v, uint32_t (&b)[4]) {
    const auto h = __builtin_amdgcn_permlane32_swap(v, v, false, false);   // (r0 r1 r0 r1), (r2 r3 r2 r3)
    const auto lo = __builtin_amdgcn_permlane16_swap((uint32_t)h[0], (uint32_t)h[0], false, false);
    const auto hi = __builtin_amdgcn_permlane16_swap((uint32_t)h[1], (uint32_t)h[1], false, false);
    b[0] = (uint32_t)lo[0];
    b[1] = (uint32_t)lo[1];
    b[2] = (uint32_t)hi[0];
    b[3] = (uint32_t)hi[1];
}

// lane i of each 16-lane row takes the value of lane i ^ 8
__device__ __forceinline__ uint32_t ror8(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x128, 0xF, 0xF, false);
}

__global__ __launch_bounds__(512) void gemv_mfma_xr_kernel(const uint8_t* __restrict__ wq,
                                                         const uint32_t* __restrict__ sz,
                                                         const uint16_t* __restrict__ x,
                                                         void* __restrict__ yv, int y_bf16, int N,
                                                         int K, int M, int gpw, int R) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];  // per-wave areas, then partial sums

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: SGPR addresses
    const int n_waves = blockDim.x >> 6;
    const int Kg = K >> 7;
    const int r0 = blockIdx.x * R;
    const int col = lane & 15;
    const int kb = lane >> 4;
    const int g0 = wave * gpw;
    const int ng = min(Kg - g0, gpw);   // >= 1: the host sizes the block so every wave has groups
    const int64_t row_bytes = K >> 1;
    const int steps = min(R, N - r0 + 15) >> 4;   // the last workgroup may have fewer rows
    const bool upper = (lane & 8) != 0;           // lanes 8..15 of each 16-lane row

    const uint32_t smem_lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)smem;
    const uint32_t area = __builtin_amdgcn_readfirstlane(smem_lds + wave * kXrWaveLds);
    const uint8_t* area_p = smem + wave * kXrWaveLds;
    float* red = reinterpret_cast<float*>(smem + n_waves * kXrWaveLds);   // [2][waves][16][stride]

    const CodeConsts cc;
    const f32x4_t zero4 = {0.0f, 0.0f, 0.0f, 0.0f};

    // lane byte offsets of code loads 2p and 2p + 1 from a row step's first row and the
    // wave's first group (plus 128 p).  Groups past the wave's range read the next bytes of
    // the prepared buffer (at most 448 past a row; the scale/zero words follow the codes),
    // which scale 0 drops.
    uint32_t coff[2];
#pragma unroll
    for (int h = 0; h < 2; ++h)
        coff[h] = (uint32_t)((8 * h + (lane & 7)) * row_bytes) + 64 * ((lane >> 3) & 1) + 16 * kb;
    const int sg0 = g0 + min(kb, ng - 1);
    auto step_row = [&](int t) __attribute__((always_inline)) { return min(r0 + 16 * t, N - 16); };
    auto code_base = [&](int t) __attribute__((always_inline)) {
        return wq + (int64_t)step_row(t) * row_bytes + (int64_t)g0 * 64;
    };
    // scale/zero words: lane (col, kb) takes row col's word of groups g0 + kb and g0 + 4 + kb
    // (four groups = 64 bytes further).  Past the wave's groups the lane reads whatever word
    // follows (scale 0 drops it); the resource ends with the words, so a read past them
    // returns 0 and touches no memory.
    const uint32_t sgo0 = 16u * (uint32_t)sg0;
    auto load_sz = [&](int t, uint32_t (&s)[2]) __attribute__((always_inline)) {
        const int rb = step_row(t);
        const uint32_t* sq = sz + (int64_t)(rb >> 2) * Kg * 4;
        const int nrec = (((N + 3) >> 2) - (rb >> 2)) * Kg * 16;
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t*>(sq), 0, nrec, 0x00020000);
        const int rr = (rb & 3) + col;
        const uint32_t o = 4u * (uint32_t)((rr >> 2) * Kg * 4 + (rr & 3)) + sgo0;
        s[0] = __builtin_amdgcn_raw_buffer_load_b32(rs, (int)o, 0, 0);
        s[1] = __builtin_amdgcn_raw_buffer_load_b32(rs, (int)o, 64, 0);
    };
    // buffer loads: uniform base in the resource, the lane's 32-bit offset, the pair's
    // 128 bytes as the scalar offset; non-temporal (every byte is read once)
    auto load_pair = [&](const uint8_t* cb, int p, u32x4_t (&c)[8]) __attribute__((always_inline)) {
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(cb), 0, 0x7FFFFFFF, 0x00020000);
        c[2 * p] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, (int)coff[0], 128 * p, 2));
        c[2 * p + 1] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, (int)coff[1], 128 * p, 2));
    };
    // ---- x of this wave's groups (A operands), once per workgroup, and the first row step.
    // x goes through the wave's LDS area in two rounds of four groups, with loads of 4 rows x
    // 256 contiguous bytes (chunk c of row r at slot c ^ (r & 15)); loading it straight into
    // the MFMA lane order made each load touch 32 lines.  Only ceil(M/4) quads of rows are
    // loaded; the lanes of rows past them hold zeros.
    //
    // binary16 x: x * 2^-E, one E per wave putting the largest value of its x (all rows, its
    // groups) just under 2^16; exact when every non-zero value lands on a normal binary16
    // (within 2^25 of the largest, also after the further 2^-4 at the inputs of the 16 (q -
    // zero) codes).  The codes then need no bf16 conversion.  A wave whose x does not pass
    // keeps bf16 x.  Each wave scales its partial sums by 2^E (a scalar) before they are
    // combined, so the combine is a plain sum (with an exponent per row of x, reading the
    // exponents there cost qkv 0.5-0.7 us at M = 4 and 8).  Scaling by a power of two
    // commutes with the roundings, so the results are those of one exponent per row.
    const int xquads = (M + 3) >> 2;
    const u32x4_t zero_x = {0u, 0u, 0u, 0u};
    u32x4_t xa[kXrGroups][4];
    u32x4_t c[8];      // codes of the current row step
    uint32_t s[2];     // its scale/zero words
    bool f16 = false;
    int fw = 0;        // the wave's largest bf16 exponent field over its x (uniform)
    if (xquads <= 2) {
        // up to eight rows of x: each lane converts the 16 bytes it loaded (row 4i + (lane >> 4)
        // of quad i), where all 64 lanes hold rows of x, and writes them back for the reads
        // in MFMA lane order (at M = 4 a quarter of the work of converting the MFMA operands;
        // qkv 16.7 -> 14.3 us, gate_up 47.3 -> 45.3).  The first row step's loads go straight
        // into registers, in flight while x is converted.
        u32x4_t raw[kXrGroups][2];
#pragma unroll
        for (int half = 0; half < 2; ++half) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int gc = g0 + min(4 * half + q, ng - 1);
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    if (i < xquads) {
                        const int r = 4 * i + (lane >> 4);
                        const uint16_t* src = x + (int64_t)min(r, M - 1) * K + gc * 128 + 8 * ((lane & 15) ^ (r & 15));
                        lds_dma16(src, area + q * 4096 + i * 1024);
                    }
                }
            }
            __builtin_amdgcn_s_waitcnt(vm_imm(0));
            asm volatile("" ::: "memory");
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int i = 0; i < 2; ++i)
                    if (i < xquads)
                        raw[4 * half + q][i] = *reinterpret_cast<const u32x4_t*>(area_p + q * 4096 + i * 1024 + 16 * lane);
            // the reads have returned before the next loads overwrite the area
            __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
            asm volatile("" ::: "memory");
        }
        {
            load_sz(0, s);
            const uint8_t* cb = code_base(0);
#pragma unroll
            for (int p = 0; p < 4; ++p) load_pair(cb, p, c);
        }

        {
            uint32_t mxq[2] = {0, 0}, mnq[2] = {0xFFFFu, 0xFFFFu};   // per row, over its 16 lanes
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                if (i < xquads) {
                    u16x2_t vmax = {0, 0}, vmin = {0xFFFF, 0xFFFF};
#pragma unroll
                    for (int j = 0; j < kXrGroups; ++j)
#pragma unroll
                        for (int d = 0; d < 4; ++d) {
                            const u16x2_t mag = as_u16x2(raw[j][i][d] & 0x7FFF7FFFu);
                            vmax = __builtin_elementwise_max(vmax, mag);
                            vmin = __builtin_elementwise_min(vmin, mag - (unsigned short)1);  // 0 -> 0xFFFF
                        }
                    uint32_t mx = max(vmax.x, vmax.y), mn = min(vmin.x, vmin.y);
                    mx = max(mx, ror8(mx));
                    mn = min(mn, ror8(mn));
                    mx = max(mx, (uint32_t)__builtin_amdgcn_mov_dpp((int)mx, 0x124, 0xF, 0xF, false));
                    mn = min(mn, (uint32_t)__builtin_amdgcn_mov_dpp((int)mn, 0x124, 0xF, 0xF, false));
                    mx = max(mx, (uint32_t)__builtin_amdgcn_mov_dpp((int)mx, 0x122, 0xF, 0xF, false));
                    mn = min(mn, (uint32_t)__builtin_amdgcn_mov_dpp((int)mn, 0x122, 0xF, 0xF, false));
                    mx = max(mx, (uint32_t)__builtin_amdgcn_mov_dpp((int)mx, 0x121, 0xF, 0xF, false));
                    mn = min(mn, (uint32_t)__builtin_amdgcn_mov_dpp((int)mn, 0x121, 0xF, 0xF, false));
                    mxq[i] = mx;
                    mnq[i] = mn;
                }
            }
            // one exponent for the wave: its largest value over all rows of x
            fw = __builtin_amdgcn_readfirstlane((int)(max_across_rows(max(mxq[0], mxq[1])) >> 7));
            bool bad = false;
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int mnz = (int)mnq[i] + 1;
                bad |= mnz != 0x10000 && (fw < 30 || fw == 255 || mnz < ((fw - 25) << 7));
            }
            f16 = __builtin_amdgcn_ballot_w64(bad) == 0;
        }
        // back to LDS (converted or not), then the A operands in MFMA lane order
#pragma unroll
        for (int half = 1; half >= 0; --half) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    if (i < xquads) {
                        if (f16) {
                            const uint32_t ce = (uint32_t)((fw - 30) << 7) * 0x00010001u;
                            const uint32_t co = (uint32_t)((fw - 26) << 7) * 0x00010001u;
#pragma unroll
                            for (int d = 0; d < 4; ++d)
                                raw[4 * half + q][i][d] = to_f16_pair(raw[4 * half + q][i][d], (d & 1) ? co : ce);
                        }
                        *reinterpret_cast<u32x4_t*>(smem + wave * kXrWaveLds + q * 4096 + i * 1024 + 16 * lane) =
                            raw[4 * half + q][i];
                    }
                }
            }
            __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): the writes have landed
            asm volatile("" ::: "memory");
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int sq = 0; sq < 4; ++sq)
                    xa[4 * half + q][sq] = col < 4 * xquads ? *reinterpret_cast<const u32x4_t*>(
                        area_p + q * 4096 + col * 256 + (((4 * kb + sq) ^ col) * 16)) : zero_x;
            __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): read before the next writes
            asm volatile("" ::: "memory");
        }
    } else {
        // more rows of x: the MFMA operands are converted in place; the first row step goes
        // through the LDS area by direct-to-LDS loads (lane l's bytes at 16 l) while x is
        // converted, when the registers are busy
#pragma unroll
        for (int half = 0; half < 2; ++half) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int gc = g0 + min(4 * half + q, ng - 1);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if (i < xquads) {
                        const int r = 4 * i + (lane >> 4);
                        const uint16_t* src = x + (int64_t)min(r, M - 1) * K + gc * 128 + 8 * ((lane & 15) ^ (r & 15));
                        lds_dma16(src, area + q * 4096 + i * 1024);
                    }
                }
            }
            __builtin_amdgcn_s_waitcnt(vm_imm(0));
            asm volatile("" ::: "memory");
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int s = 0; s < 4; ++s)
                    xa[4 * half + q][s] = col < M ? *reinterpret_cast<const u32x4_t*>(
                        area_p + q * 4096 + col * 256 + (((4 * kb + s) ^ col) * 16)) : zero_x;
            // the reads have returned before the next loads overwrite the area
            __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
            asm volatile("" ::: "memory");
        }
        // the first row step goes through the (now free) LDS area by direct-to-LDS loads (lane
        // l's bytes at 16 l), so that no registers are held for it during the x conversion
        {
            const int rb = step_row(0);
            const uint32_t* sq = sz + (int64_t)(rb >> 2) * Kg * 4;
            const int rr = (rb & 3) + col;
            const uint32_t o = (uint32_t)((rr >> 2) * Kg * 4 + (rr & 3));
            lds_dma4(sq + o + 4 * sg0, area + 8 * 1024);
            lds_dma4(sq + o + 4 * g0 + 4 * min(4 + kb, ng - 1), area + 8 * 1024 + 256);
            const uint8_t* cb = code_base(0);
#pragma unroll
            for (int d = 0; d < 8; ++d) lds_dma16(cb + 128 * (d >> 1) + coff[d & 1], area + d * 1024);
        }

        {
            u16x2_t vmax = {0, 0}, vmin = {0xFFFF, 0xFFFF};
            // (scheduling barriers per group keep the compiler from spreading the work over many
            // temporaries beside the 128 registers of x)
#pragma unroll
            for (int j = 0; j < kXrGroups; ++j) {
#pragma unroll
                for (int q = 0; q < 4; ++q)
#pragma unroll
                    for (int d = 0; d < 4; ++d) {
                        const u16x2_t mag = as_u16x2(xa[j][q][d] & 0x7FFF7FFFu);
                        vmax = __builtin_elementwise_max(vmax, mag);
                        vmin = __builtin_elementwise_min(vmin, mag - (unsigned short)1);
                    }
                __builtin_amdgcn_sched_barrier(0);
            }
            // one exponent for the wave: its largest value over all rows of x (the lanes of a
            // 16-lane row hold the 16 rows of x, the four 16-lane rows the same rows)
            uint32_t mx = max_across_rows(max(vmax.x, vmax.y));
            uint32_t mn = 0xFFFFu - max_across_rows(0xFFFFu - min(vmin.x, vmin.y));
            mx = max(mx, ror8(mx));
            mn = min(mn, ror8(mn));
            mx = max(mx, (uint32_t)__builtin_amdgcn_mov_dpp((int)mx, 0x124, 0xF, 0xF, false));
            mn = min(mn, (uint32_t)__builtin_amdgcn_mov_dpp((int)mn, 0x124, 0xF, 0xF, false));
            mx = max(mx, (uint32_t)__builtin_amdgcn_mov_dpp((int)mx, 0x122, 0xF, 0xF, false));
            mn = min(mn, (uint32_t)__builtin_amdgcn_mov_dpp((int)mn, 0x122, 0xF, 0xF, false));
            mx = max(mx, (uint32_t)__builtin_amdgcn_mov_dpp((int)mx, 0x121, 0xF, 0xF, false));
            mn = min(mn, (uint32_t)__builtin_amdgcn_mov_dpp((int)mn, 0x121, 0xF, 0xF, false));
            fw = __builtin_amdgcn_readfirstlane((int)(mx >> 7));
            const int mnz = __builtin_amdgcn_readfirstlane((int)mn) + 1;
            f16 = !(mnz != 0x10000 && (fw < 30 || fw == 255 || mnz < ((fw - 25) << 7)));
            if (f16) {
                // x passes through an empty asm statement so that the conversion recomputes the
                // magnitudes instead of keeping the 128 from the range check alive
#pragma unroll
                for (int j = 0; j < kXrGroups; ++j)
#pragma unroll
                    for (int q = 0; q < 4; ++q)
#pragma unroll
                        for (int d = 0; d < 4; ++d) {
                            uint32_t v = xa[j][q][d];
                            asm volatile("" : "+v"(v));
                            xa[j][q][d] = v;
                        }
                const uint32_t ce = (uint32_t)((fw - 30) << 7) * 0x00010001u;
                const uint32_t co = (uint32_t)((fw - 26) << 7) * 0x00010001u;
#pragma unroll
                for (int j = 0; j < kXrGroups; ++j) {
#pragma unroll
                    for (int q = 0; q < 4; ++q)
#pragma unroll
                        for (int d = 0; d < 4; ++d) xa[j][q][d] = to_f16_pair(xa[j][q][d], (d & 1) ? co : ce);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        }

        __builtin_amdgcn_s_waitcnt(vm_imm(0));
        asm volatile("" ::: "memory");
#pragma unroll
        for (int d = 0; d < 8; ++d) c[d] = *reinterpret_cast<const u32x4_t*>(area_p + d * 1024 + 16 * lane);
        s[0] = *reinterpret_cast<const uint32_t*>(area_p + 8 * 1024 + 4 * lane);
        s[1] = *reinterpret_cast<const uint32_t*>(area_p + 8 * 1024 + 256 + 4 * lane);
    }

    const int ew = f16 ? fw - 127 - 15 : 0;   // the wave's partial sums are scaled by 2^ew

    // one row step; F: binary16 x and codes (else bf16), MORE: the next row step's loads are
    // issued here, group pair by group pair as the registers of a pair are used.  Both are
    // compile-time, so the eight groups are straight-line code.
    auto row_step = [&](auto fc, auto mc, int t) __attribute__((always_inline)) {
        constexpr bool F = decltype(fc)::value;
        constexpr bool MORE = decltype(mc)::value;
        uint32_t szw[4];
        const uint32_t s_hi = s[1];
        bcast_rows(s[0], szw);
        if constexpr (MORE) load_sz(t + 1, s);
        const uint8_t* cbn = code_base(t + 1);
        f32x4_t acc = zero4;
#pragma unroll
        for (int pp = 0; pp < 4; ++pp) {
            // exchange lanes l and l ^ 8: c[2pp] then holds group 2pp of rows 0..15 in MFMA
            // lane order (row l & 15, piece l >> 4), c[2pp + 1] group 2pp + 1
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const uint32_t a = c[2 * pp][v], b = c[2 * pp + 1][v];
                const uint32_t ra = ror8(a), rb = ror8(b);
                c[2 * pp][v] = upper ? rb : a;
                c[2 * pp + 1][v] = upper ? b : ra;
            }
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const int j = 2 * pp + hh;
                if (j == 4) bcast_rows(s_hi, szw);
                const uint32_t word = szw[j % 4];
                const uint32_t z1 = cc.z1(word), z16 = cc.z16(word);
                f32x4_t p = zero4;
                if constexpr (F) {
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        p = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                            as_f16x8(xa[j][q]), as_f16x8(exact_codes_f16(c[j][q], z1, z16, cc)), p, 0, 0, 0);
                } else {
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        p = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            as_bf16x8(xa[j][q]), as_bf16x8(exact_codes(c[j][q], z1, z16, cc)), p, 0, 0, 0);
                }
                // a group past the wave's range is computed with scale 0 (no branch)
                const float keep = j < ng ? 1.0f : 0.0f;
                const float sc = keep * (float)__builtin_bit_cast(_Float16, (uint16_t)(word & 0xFFFFu));
#pragma unroll
                for (int v = 0; v < 4; ++v) acc[v] = fmaf(sc, p[v], acc[v]);
                __builtin_amdgcn_sched_barrier(0);
            }
            if constexpr (MORE) load_pair(cbn, pp, c);
            __builtin_amdgcn_sched_barrier(0);
        }
        // partial sums of this row step: lane holds column (row) col, rows m = 4 kb + v of x
        float* rbuf = red + ((t & 1) * n_waves + wave) * 16 * kRedStride;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int m = 4 * kb + v;
            if (m < M) rbuf[col * kRedStride + m] = ldexpf(acc[v], ew);
        }
        lds_barrier();
        const int rb = step_row(t);
        const int rfirst = r0 + 16 * t;   // rows below were written by the previous step
        for (int i = tid; i < 16 * M; i += blockDim.x) {
            const int r = i & 15;
            const int m = i >> 4;
            const int row = rb + r;
            if (row >= rfirst) {
                const float* rs = red + (t & 1) * n_waves * 16 * kRedStride;
                float v = 0.0f;
                for (int w = 0; w < n_waves; ++w) v += rs[(w * 16 + r) * kRedStride + m];
                const int64_t o = (int64_t)m * N + row;
                if (y_bf16)
                    static_cast<uint16_t*>(yv)[o] = (uint16_t)bf16_bits_rne(v);
                else
                    static_cast<float*>(yv)[o] = v;
            }
        }
    };
    using True = std::integral_constant<bool, true>;
    using False = std::integral_constant<bool, false>;
    auto all_steps = [&](auto fc) __attribute__((always_inline)) {
        for (int t = 0; t + 1 < steps; ++t) row_step(fc, True{}, t);
        row_step(fc, False{}, steps - 1);
    };
    if (f16)
        all_steps(True{});
    else
        all_steps(False{});
}

template <int T>
hipError_t launch_t(const uint8_t* wq, const uint32_t* sz, const uint16_t* x, void* y, int y_bf16,
                    int n, int k, int m, int gpw, int waves, hipStream_t s) {
    const dim3 grid((unsigned)((n + 16 * T - 1) / (16 * T)));
    const dim3 block((unsigned)(64 * waves));
    const size_t red_bytes = (size_t)waves * 16 * T * kRedStride * sizeof(float);
    const size_t stage_bytes = (size_t)waves * (2 * kXStageBytes + 2 * T * 1024);
    const size_t shmem = red_bytes > stage_bytes ? red_bytes : stage_bytes;
    if (shmem > 65536) {
        static std::atomic<int> raised{0};
        if (!raised.load(std::memory_order_relaxed)) {
            hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(gemv_mfma_kernel<T, 2>),
                                               hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
            if (e != hipSuccess) return e;
            raised.store(1, std::memory_order_relaxed);
        }
    }
    hipLaunchKernelGGL((gemv_mfma_kernel<T, 2>), grid, block, shmem, s, wq, sz, x, y, y_bf16,
                       n, k, m, gpw);
    return hipGetLastError();
}

}  // namespace

// Streaming kernel: waves per workgroup about eight groups of K each, at most eight
// (12 KB of LDS stages per wave; on the 70B down shape eight waves of 28 groups ran faster
// than sixteen of 14), two tiles (32 rows) per workgroup: the fastest of the settings
// measured on MI355X at the 70B shapes.
// Rows per workgroup of the resident-x kernel: one round of workgroups (one per CU), a
// multiple of 16.  Holding x pays off from three row steps on; below that the streaming
// kernel is used (measured on MI355X at the 70B shapes: o 8192x8192 streams faster, qkv and
// gate_up run faster with x resident).
static int xr_rows(int n) {
    static std::atomic<int> cus{0};
    int cu = cus.load(std::memory_order_relaxed);
    if (cu == 0) {
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            cu <= 0)
            cu = 256;
        cus.store(cu, std::memory_order_relaxed);
    }
    const long wgs = (long)cu;
    const int r = (int)((n + wgs - 1) / wgs);
    return (r + 15) / 16 * 16;
}

// K <= 8192 and at least three row steps per workgroup: the resident-x kernel.
static hipError_t launch_xr(const uint8_t* wq, const uint32_t* sz, const uint16_t* x, void* y, int yb,
                     int n, int k, int m, int R, hipStream_t s) {
    const int kg = k / kGroup;
    const int waves = (kg + kXrGroups - 1) / kXrGroups;
    const int gpw = (kg + waves - 1) / waves;
    const size_t shmem = (size_t)waves * (kXrWaveLds + kXrRedBytes);
    if (shmem > 65536) {
        static std::atomic<int> raised{0};
        if (!raised.load(std::memory_order_relaxed)) {
            hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(gemv_mfma_xr_kernel),
                                               hipFuncAttributeMaxDynamicSharedMemorySize,
                                               (int)(8 * (kXrWaveLds + kXrRedBytes)));
            if (e != hipSuccess) return e;
            raised.store(1, std::memory_order_relaxed);
        }
    }
    const dim3 grid((unsigned)((n + R - 1) / R));
    const dim3 block((unsigned)(64 * waves));
    // binary16 x costs about 1000 vector instructions per lane and workgroup and saves 256 per
    // row step; measured on MI355X it pays from the minimum of three row steps on (qkv
    // 10240 x 8192 at M = 4, 8, 16: 15.9-16.5 us against 17.2-18.0 with bf16 x)
    hipLaunchKernelGGL(gemv_mfma_xr_kernel, grid, block, shmem, s, wq, sz, x, y, yb, n, k, m, gpw, R);
    return hipGetLastError();
}

bool gemv_resident_x_takes(int64_t n, int64_t k) {
    if (k / kGroup > kXrGroups * 8) return false;
    return xr_rows((int)n) >= 48;
}

hipError_t launch_gemv_mfma(const uint8_t* prepared, int64_t n, int64_t k, const uint16_t* x,
                            int64_t m, void* y, bool y_bf16, hipStream_t s) {
    const int kg = (int)(k / kGroup);
    if (gemv_resident_x_takes(n, k))
        return launch_xr(prepared, reinterpret_cast<const uint32_t*>(prepared + sz_offset(n, k)),
                         x, y, y_bf16 ? 1 : 0, (int)n, (int)k, (int)m, xr_rows((int)n), s);
    constexpr int per_wave = 8;
    int waves = (kg + per_wave - 1) / per_wave;
    if (waves > 8) waves = 8;
    if (waves < 1) waves = 1;
    const int gpw = (kg + waves - 1) / waves;
    waves = (kg + gpw - 1) / gpw;
    const uint8_t* wq = prepared;
    const uint32_t* sz = reinterpret_cast<const uint32_t*>(prepared + sz_offset(n, k));
    const int yb = y_bf16 ? 1 : 0;
    const int N = (int)n, K = (int)k, M = (int)m;
    return launch_t<2>(wq, sz, x, y, yb, N, K, M, gpw, waves, s);
}

}  // namespace w4
