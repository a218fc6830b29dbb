// Fused dequantizing matrix-vector product for decode (1 <= M <= 16).
//
// Computes y[m, n] = sum_g scale16[n, g] * sum_{k in g} (q[n, k] - zero[n, g]) x[m, k]
// (page "Weight quantization", section "How it works": the dequantized weight is
// (code - zero) * scale, and the group's scale multiplies once per group; section "Code":
// the group loop of the dot routine) without writing any dequantized weight to memory.
// Decode reads every weight once, so the kernel is a stream over HBM (page "LLM
// Quantization Architecture in Depth" › "Why fewer bits make decoding faster").
//
// Exact operands.  The matrix instructions and the dot2 instructions of gfx950 align all
// addends of one instruction to the largest before rounding, so an operand carrying a
// bias (for example 128 + q, with the bias removed later through sum x) loses bits in
// proportion to the bias times |x|, not to the size of the result: a group whose codes
// mostly equal its zero, with large x there, would come out far outside the tolerance.
// Every product here multiplies the exact difference q - zero:
//   * v_and_or_b32((word >> s), 0x000F000F, 0x64006400) gives the binary16 pair
//     (1024 + q_a, 1024 + q_b) and one v_pk_add_f16 with (-(1024 + zero)) x 2 gives the
//     exact pair (q_a - zero, q_b - zero).  The codes at bits 4..7 / 20..23 of a word are
//     taken where they are, as (1024 + 16 q) - (1024 + 16 zero) = 16 (q - zero), and
//     their activations carry a factor 2^-4 instead, so a word of eight codes needs one
//     shift;
//   * x (bf16) enters as binary16 x * 2^-E, with E chosen per wave and row of x (the
//     wave's 2048 inputs, 4096 with two slices per lane) so that the largest value lands
//     just under 2^16.  bf16 has 8 significant bits
//     and binary16 11, so the conversion (integer steps on the bits) is exact for every
//     value that lands on a normal binary16, i.e. within 2^25 of the wave's largest;
//     v_dot2_f32_f16 then multiplies exactly and accumulates in f32, the group term is
//     scale16 * D (one v_fma_mix_f32 takes the binary16 scale as it is), and the wave's row
//     sums are scaled by 2^E before the waves are combined;
//   * binary32 x, and a wave with a bf16 value outside that window, take the exact path
//     instead: the same exact codes, converted to binary32, times x
//     in binary32 with one FMA per input (for bf16 x, one row at a time in a loop of its
//     own that reads x again, so that the rare path adds no registers to the fast one).
// Either way a code equal to its zero contributes exactly 0, and the rounding error is
// a few binary32 ulps of the sums of |(q - zero) x|, far inside 1e-3 * sum |w_hat x|.
//
// Mapping (gfx950, wave64):
//   * lane u of the workgroup owns the 16-byte slice u of every row (32 inputs, a
//     quarter of a group); its x values stay in registers for the whole workgroup, so
//     each row costs one 16-byte load per lane and a wave load covers 1 KiB of
//     contiguous weights;
//   * a workgroup holds ceil(K/2048) waves and walks rows_per_wg rows in steps of four
//     rows through two register buffers: the loads of the next step are issued before a
//     step is computed (scheduling barriers keep them in order, so the compiler's in-order
//     wait counts stay exact and a step waits only for its own loads).  The first step's
//     loads follow x's directly, so they are in flight while x is converted.  With bf16 x
//     (and binary32 x two rows at a time) the waves meet at a barrier before each step's
//     loads, so the workgroup reads the step's rows whole;
//   * groups of up to eight waves end the launch with a round of workgroups that take
//     half the rows of the others, which shortens the tail of the weight stream; at M = 1 a
//     matrix too small to fill one round of eight-row workgroups runs workgroups of a
//     single step (four rows), which doubles the waves per CU;
//   * the scale/zero words of the four rows of a step are one 16-byte load; two
//     v_perm_b32 build the binary16 pairs -(1024 + zero) and -(1024 + 16 zero) from the
//     zero bytes of the word;
//   * reduction of the four rows across the wave: v_permlane32_swap and
//     v_permlane16_swap transpose-and-add (each lane ends with one row), DPP row
//     rotations finish the 16-lane sums; waves are combined through LDS.  No atomics, so
//     results are deterministic.
#include <atomic>
#include <type_traits>

#include "w4_internal.h"

namespace w4 {
namespace {

typedef __attribute__((ext_vector_type(2))) _Float16 f16x2_t;
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kRowsPerStep = 4;
constexpr int kChunk = 2;  // steps of four rows in registers at a time (two buffers)

// one 16-byte weight slice, marked non-temporal: every byte is read exactly once
__device__ __forceinline__ u32x4_t load_stream(const u32x4_t* p) { return __builtin_nontemporal_load(p); }

__device__ __forceinline__ float dot2h(uint32_t a, uint32_t b, float acc) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, a), __builtin_bit_cast(f16x2_t, b), acc,
                                  false);
}

__device__ __forceinline__ uint32_t add2h(uint32_t a, uint32_t b) {
    return __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2_t, a) + __builtin_bit_cast(f16x2_t, b));
}

__device__ __forceinline__ uint32_t bf16_bits_rne(float f) {
    const uint32_t u = __float_as_uint(f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

typedef __attribute__((ext_vector_type(2))) unsigned short u16x2_t;

__device__ __forceinline__ u16x2_t as_u16x2(uint32_t v) { return __builtin_bit_cast(u16x2_t, v); }
__device__ __forceinline__ uint32_t as_u32(u16x2_t v) { return __builtin_bit_cast(uint32_t, v); }

// bf16 pair -> binary16 pair of x * 2^-E by integer steps: with c = (F_max - 30) << 7 (or
// (F_max - 26) << 7 for a further 2^-4), ((|bits| - c) << 3) re-biases the exponent field
// from bf16 to binary16 and widens the 7 mantissa bits to 10; the sign is put back.  The
// subtraction saturates at 0, so a zero stays zero.  Exact whenever the result is a normal
// binary16 value, which the slice's range check guarantees.
__device__ __forceinline__ uint32_t to_f16_pair(uint32_t xb, uint32_t c2) {
    const u16x2_t mag = as_u16x2(xb & 0x7FFF7FFFu);
    const u16x2_t r = __builtin_elementwise_sub_sat(mag, as_u16x2(c2)) << (unsigned short)3;
    return as_u32(r) | (xb & 0x80008000u);
}

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                                 0xF, 0xF, false));
}

// exchange the upper 32 lanes of a with the lower 32 lanes of b
__device__ __forceinline__ void swap32(float& a, float& b) {
    const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, a),
                                                    __builtin_bit_cast(uint32_t, b), false, false);
    a = __builtin_bit_cast(float, (uint32_t)r[0]);
    b = __builtin_bit_cast(float, (uint32_t)r[1]);
}

// exchange the odd 16-lane rows of a with the even 16-lane rows of b
__device__ __forceinline__ void swap16(float& a, float& b) {
    const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, a),
                                                    __builtin_bit_cast(uint32_t, b), false, false);
    a = __builtin_bit_cast(float, (uint32_t)r[0]);
    b = __builtin_bit_cast(float, (uint32_t)r[1]);
}

template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
    return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}

// maximum over the 64 lanes of the wave, in every lane (permlane swaps, then DPP rotations)
__device__ __forceinline__ int wave_max(int v) {
    const auto h = __builtin_amdgcn_permlane32_swap((uint32_t)v, (uint32_t)v, false, false);
    v = max((int)h[0], (int)h[1]);
    const auto q = __builtin_amdgcn_permlane16_swap((uint32_t)v, (uint32_t)v, false, false);
    v = max((int)q[0], (int)q[1]);
    v = max(v, dpp_i<0x128>(v));  // row_ror:8
    v = max(v, dpp_i<0x124>(v));  // row_ror:4
    v = max(v, dpp_i<0x122>(v));  // row_ror:2
    v = max(v, dpp_i<0x121>(v));  // row_ror:1
    return v;
}

// four per-lane row values -> lane l holds the wave-wide sum of row (l >> 4) & 3
__device__ __forceinline__ float reduce4(float a0, float a1, float a2, float a3) {
    swap32(a0, a2);
    swap32(a1, a3);
    float k0 = a0 + a2;  // lanes 0-31: row 0, lanes 32-63: row 2
    float k1 = a1 + a3;  // lanes 0-31: row 1, lanes 32-63: row 3
    swap16(k0, k1);
    float k = k0 + k1;   // 16-lane row r of the wave holds output row r
    k += dpp<0x128>(k);  // row_ror:8
    k += dpp<0x124>(k);  // row_ror:4
    k += dpp<0x122>(k);  // row_ror:2
    k += dpp<0x121>(k);  // row_ror:1
    return k;
}

// scale bits of a scale/zero word (binary16, or bfloat16 for SBF16) as binary32
template <bool SBF16>
__device__ __forceinline__ float word_scale(uint32_t szw) {
    return SBF16 ? __uint_as_float(szw << 16) : (float)__builtin_bit_cast(_Float16, (uint16_t)(szw & 0xFFFFu));
}

// SBF16: the scale bits are bfloat16 (else binary16); gshift: log2(group / 32), the slices
// of one group (a group of 32, 64 or 128 inputs has its own scale/zero word)
template <int MT, bool XF32, int SPT, int MAXT, bool RAGGED, bool SBF16, bool ONE = false>
__global__ __launch_bounds__(MAXT, (MT == 1 && !XF32 && SPT == 1) ? 6 : 1) void gemv_kernel(const u32x4_t* __restrict__ wq,
                                                    const u32x4_t* __restrict__ sz4,
                                                    const void* __restrict__ xv,
                                                    void* __restrict__ yv, int y_bf16, int N,
                                                    int K, int M, int rows_per_wg, int gshift,
                                                    int tail_first, int tail_rows) {
    constexpr int R = kRowsPerStep;
    constexpr int CH = kChunk;
    extern __shared__ float red[];          // [waves][rows_per_wg][MT]

    const int S = K >> 5;
    const int Kg = K >> (5 + gshift);
    const int T = blockDim.x;
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int n_waves = T >> 6;
    // workgroups from tail_first on (the last ones dispatched) take tail_rows rows each, so
    // the launch ends on short workgroups; rows_per_wg is the LDS row stride of both kinds
    const int row_stride = rows_per_wg;
    const bool in_tail = (int)blockIdx.x >= tail_first;
    const int r0 = in_tail ? tail_first * rows_per_wg + ((int)blockIdx.x - tail_first) * tail_rows
                           : (int)blockIdx.x * rows_per_wg;
    if (in_tail) rows_per_wg = tail_rows;
    const int r_end = min(N, r0 + rows_per_wg);

    // slice j of this lane is threadIdx.x + j*T (16 bytes of every row).  With a ragged
    // K the lanes past the last slice read the last slice and their x is zero.
    int sl[SPT];
    bool act[SPT];
    uint32_t woff[SPT], soff[SPT];
#pragma unroll
    for (int j = 0; j < SPT; ++j) {
        sl[j] = threadIdx.x + j * T;
        act[j] = RAGGED ? sl[j] < S : true;
        const int slc = RAGGED ? min(sl[j], S - 1) : sl[j];
        woff[j] = (uint32_t)slc * 16u;
        soff[j] = (uint32_t)(slc >> gshift) * 16u;
    }

    const char* wbase = reinterpret_cast<const char*>(wq);
    const char* sbase = reinterpret_cast<const char*>(sz4);
    const int64_t row_bytes = (int64_t)S * 16;

    // rows_per_wg is a multiple of CH*4 (every chunk is whole), or four with ONE; rows past N
    // repeat row N-1 (their sums are never stored)
    u32x4_t wb[CH][R][SPT];
    u32x4_t sb[CH][SPT];
    // loads of the step (four rows) at local row rb into buffer c: the scale/zero words of
    // the four rows (one 16-byte load), then the rows' slices
    // buffer loads: a uniform base per step (the step's first row, or its row quad's
    // scale/zero words), the lane's fixed 32-bit offset, and the row within the step as the
    // scalar offset, so a load needs no per-lane address arithmetic
    auto issue_step = [&](auto cc, int rb) {
        constexpr int c = decltype(cc)::value;
        const int r = min(r0 + rb, N - 1);
        const char* srow = sbase + (int64_t)(r >> 2) * Kg * 16;
        const __amdgpu_buffer_rsrc_t srs =
            __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(srow), 0, 0x7FFFFFFF, 0x00020000);
#pragma unroll
        for (int j = 0; j < SPT; ++j)
            sb[c][j] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(srs, (int)soff[j], 0, 0));
        const char* rowp = wbase + (int64_t)r * row_bytes;
        const __amdgpu_buffer_rsrc_t wrs =
            __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(rowp), 0, 0x7FFFFFFF, 0x00020000);
#pragma unroll
        for (int rr = 0; rr < R; ++rr) {
            // rows past N repeat row N-1 (their sums are never stored)
            const int so = (min(r0 + rb + rr, N - 1) - r) * (int)row_bytes;
#pragma unroll
            for (int j = 0; j < SPT; ++j)
                wb[c][rr][j] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(wrs, (int)woff[j], so, 2));
        }
        // loads stay in step order, so a step only waits for its own loads
        __builtin_amdgcn_sched_barrier(0);
    };

    // ---- x slices first: their loads complete before the weight stream that follows
    uint32_t xb[SPT][MT][16];   // bf16 pairs (binary32 x is read by the exact path itself)
    if constexpr (!XF32) {
#pragma unroll
        for (int j = 0; j < SPT; ++j)
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                const bool ok = act[j] && (MT == 1 || m < M);  // zero x for idle lanes and absent rows
                const uint4* px = reinterpret_cast<const uint4*>(
                    static_cast<const uint16_t*>(xv) + (int64_t)m * K + (int64_t)sl[j] * 32);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const uint4 v = ok ? px[q] : make_uint4(0, 0, 0, 0);
                    xb[j][m][4 * q + 0] = v.x;
                    xb[j][m][4 * q + 1] = v.y;
                    xb[j][m][4 * q + 2] = v.z;
                    xb[j][m][4 * q + 3] = v.w;
                }
            }
    }
    using B0 = std::integral_constant<int, 0>;
    using B1 = std::integral_constant<int, 1>;
    __builtin_amdgcn_sched_barrier(0);  // x loads first: waiting for x never waits for weights
    // the first step's weight loads go out right behind x, so their latency overlaps the
    // conversion of x (they are not used if the exact path runs)
    issue_step(B0{}, 0);

    // binary32 x for the exact path, resident
    uint32_t xs[XF32 ? SPT : 1][XF32 ? MT : 1][32];
    if constexpr (XF32) {
#pragma unroll
        for (int j = 0; j < SPT; ++j)
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                const bool ok = act[j] && (MT == 1 || m < M);
                const uint4* px = reinterpret_cast<const uint4*>(
                    static_cast<const float*>(xv) + (int64_t)m * K + (int64_t)sl[j] * 32);
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    const uint4 v = ok ? px[q] : make_uint4(0, 0, 0, 0);
                    xs[j][m][4 * q + 0] = v.x;
                    xs[j][m][4 * q + 1] = v.y;
                    xs[j][m][4 * q + 2] = v.z;
                    xs[j][m][4 * q + 3] = v.w;
                }
            }
    }

    // ---- binary16 activations and the per-wave exponents (fast path): x * 2^-E puts the
    // wave's largest value in [2^15, 2^16); every non-zero value must land on a normal
    // binary16 (also after the further 2^-4 at pairs 1 and 3 of every word, which meet codes
    // scaled by 16): within 2^25 of the largest.  Waves with tiny (below 2^-97) or
    // non-finite values take the exact path; an all-zero wave converts to zeros.
    uint32_t xp[SPT][MT][16];
    int xw[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) xw[m] = 0;
    bool exact = XF32;
    if constexpr (!XF32) {
        bool bad = false;
        int fmx[SPT][MT], mz[SPT][MT];
#pragma unroll
        for (int j = 0; j < SPT; ++j)
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                u16x2_t vmax = {0, 0}, vmin = {0xFFFF, 0xFFFF};
#pragma unroll
                for (int p = 0; p < 16; ++p) {
                    const u16x2_t mag = as_u16x2(xb[j][m][p] & 0x7FFF7FFFu);
                    vmax = __builtin_elementwise_max(vmax, mag);
                    vmin = __builtin_elementwise_min(vmin, mag - (unsigned short)1);  // 0 -> 0xFFFF
                }
                fmx[j][m] = (int)(max(vmax.x, vmax.y) >> 7);
                mz[j][m] = (int)min(vmin.x, vmin.y) + 1;
            }
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            int fw = fmx[0][m];
#pragma unroll
            for (int j = 1; j < SPT; ++j) fw = max(fw, fmx[j][m]);
            fw = __builtin_amdgcn_readfirstlane(wave_max(fw));   // uniform: an SGPR
            xw[m] = fw - 127 - 15;
            const uint32_t ce = (uint32_t)((fw - 30) << 7) * 0x00010001u;
            const uint32_t co = (uint32_t)((fw - 26) << 7) * 0x00010001u;
#pragma unroll
            for (int j = 0; j < SPT; ++j) {
                bad |= mz[j][m] != 0x10000 && (fw < 30 || fw == 255 || mz[j][m] < ((fw - 25) << 7));
#pragma unroll
                for (int p = 0; p < 16; ++p) xp[j][m][p] = to_f16_pair(xb[j][m][p], (p & 1) ? co : ce);
            }
        }
        exact = __builtin_amdgcn_ballot_w64(bad) != 0;
    }

    uint32_t m_lo, m_hi, magic, e4;
    asm volatile("s_mov_b32 %0, 0x000F000F" : "=s"(m_lo));
    asm volatile("s_mov_b32 %0, 0x00F000F0" : "=s"(m_hi));
    asm volatile("v_mov_b32 %0, 0x64006400" : "=v"(magic));
    asm volatile("s_mov_b32 %0, 0xE4E4E4E4" : "=s"(e4));

    // the codes of one row slice as exact binary16 pairs (q - zero, or 16 (q - zero) for the
    // pairs that meet x * 2^-4)
    auto unpack_codes = [&](const u32x4_t& wv, uint32_t szw, uint32_t (&pr)[16]) {
        // -(1024 + zero) and -(1024 + 16 zero) as binary16 pairs (word bytes 2, 3)
        const uint32_t z1 = __builtin_amdgcn_perm(e4, szw, 0x04020402u);
        const uint32_t z16 = __builtin_amdgcn_perm(e4, szw, 0x04030403u);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const uint32_t w = wv[t];
            const uint32_t u = w >> 8;
            pr[4 * t + 0] = add2h((w & m_lo) | magic, z1);
            pr[4 * t + 1] = add2h((w & m_hi) | magic, z16);
            pr[4 * t + 2] = add2h((u & m_lo) | magic, z1);
            pr[4 * t + 3] = add2h((u & m_hi) | magic, z16);
        }
    };

    // one step (four rows) from buffer c; its sums go to the LDS rows rb .. rb + 3
    auto compute_step = [&](auto cc, int rb) {
        constexpr int c = decltype(cc)::value;
        float acc[R][MT];
#pragma unroll
        for (int rr = 0; rr < R; ++rr)
#pragma unroll
            for (int m = 0; m < MT; ++m) acc[rr][m] = 0.0f;
        if constexpr (!XF32) {
            // v_dot2_f32_f16: binary16 exact codes times binary16 activations
#pragma unroll
            for (int j = 0; j < SPT; ++j)
#pragma unroll
                for (int rr = 0; rr < R; ++rr) {
                    const uint32_t szw = sb[c][j][rr];
                    // lanes past the last slice read real (unrelated) scales: weight 0
                    const float s = act[j] ? word_scale<SBF16>(szw) : 0.0f;
                    uint32_t pr[16];
                    unpack_codes(wb[c][rr][j], szw, pr);
#pragma unroll
                    for (int m = 0; m < MT; ++m) {
                        // the chain starts with the three-operand form and a zero accumulator
                        float d;
                        asm("v_dot2_f32_f16 %0, %1, %2, 0" : "=v"(d) : "v"(pr[0]), "v"(xp[j][m][0]));
#pragma unroll
                        for (int i = 1; i < 16; ++i) d = dot2h(pr[i], xp[j][m][i], d);
                        acc[rr][m] = fmaf(s, d, acc[rr][m]);
                    }
                }
        } else {
            // binary32 x: exact codes times resident binary32 x, one FMA per input
#pragma unroll
            for (int j = 0; j < SPT; ++j)
#pragma unroll
                for (int rr = 0; rr < R; ++rr) {
                    const uint32_t szw = sb[c][j][rr];
                    const float s = act[j] ? word_scale<SBF16>(szw) : 0.0f;
                    uint32_t pr[16];
                    unpack_codes(wb[c][rr][j], szw, pr);
#pragma unroll
                    for (int m = 0; m < MT; ++m) {
                        float d = 0.0f;
#pragma unroll
                        for (int p = 0; p < 16; ++p) {
                            const f16x2_t h = __builtin_bit_cast(f16x2_t, pr[p]);
                            const float sc = (p & 1) ? 0.0625f : 1.0f;
                            d = fmaf((float)h[0] * sc, __uint_as_float(xs[j][m][2 * p]), d);
                            d = fmaf((float)h[1] * sc, __uint_as_float(xs[j][m][2 * p + 1]), d);
                        }
                        acc[rr][m] = fmaf(s, d, acc[rr][m]);
                    }
                }
        }
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            const float k = reduce4(acc[0][m], acc[1][m], acc[2][m], acc[3][m]);
            if ((lane & 15) == 0) red[(wave * row_stride + rb + (lane >> 4)) * MT + m] = ldexpf(k, xw[m]);
        }
    };

    // With bf16 x the waves of a workgroup meet at a barrier before each step's loads (no
    // memory wait: the previous step's loads stay in flight), so that together they read the
    // step's four whole rows at once instead of drifting over many rows.  Measured on MI355X:
    // 70B decode step 6.52-6.53 -> 6.42-6.44 ms at M = 1, 0.1-0.2 us per shape faster at
    // M = 2.  With binary32 x (several times the vector work per input) it ran the launches
    // of two rows 0.9-2.6 us faster per shape but cost up to 3 us at one row and 6 us with two
    // slices per lane, so only the former take it.  The pipelined loop below
    // passes rows_per_wg / 4 - 1 barriers (none in one-step workgroups); a wave on the exact
    // path passes as many, so that every barrier of the workgroup pairs up.
    constexpr bool kLockstep = SPT == 1 && !ONE && (XF32 ? MT == 2 : MT <= 2);

    // bf16 x outside the binary16 window (rare): the wave runs the exact path, one row at a
    // time with loads of its own -- a separate loop, so that it adds nothing to the
    // registers of the pipelined fast path
    auto run_exact_bf16 = [&]() {
        float a0[MT], a1[MT], a2[MT], a3[MT];
#pragma unroll 1
        for (int i = 0; i < rows_per_wg; ++i) {
            const int row = min(r0 + i, N - 1);
            const char* srow = sbase + (int64_t)(row >> 2) * Kg * 16;
            float v[MT];
#pragma unroll
            for (int m = 0; m < MT; ++m) v[m] = 0.0f;
#pragma unroll
            for (int j = 0; j < SPT; ++j) {
                const u32x4_t wv = *reinterpret_cast<const u32x4_t*>(wbase + (int64_t)row * row_bytes + woff[j]);
                const uint32_t szw = *reinterpret_cast<const uint32_t*>(srow + soff[j] + 4 * (row & 3));
                const float s = act[j] ? word_scale<SBF16>(szw) : 0.0f;
                uint32_t pr[16];
                unpack_codes(wv, szw, pr);
#pragma unroll
                for (int m = 0; m < MT; ++m) {
                    const bool ok = act[j] && (MT == 1 || m < M);
                    const uint4* px = reinterpret_cast<const uint4*>(
                        static_cast<const uint16_t*>(xv) + (int64_t)m * K + (int64_t)sl[j] * 32);
                    // read x again for every row (an opaque pointer keeps the loads, and the 32
                    // binary32 values made from them, from being hoisted out of the row loop)
                    asm volatile("" : "+v"(px));
                    float d = 0.0f;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const uint4 xv4 = ok ? px[q] : make_uint4(0, 0, 0, 0);
                        const uint32_t xq[4] = {xv4.x, xv4.y, xv4.z, xv4.w};
#pragma unroll
                        for (int t = 0; t < 4; ++t) {
                            // pair 4q + t of the slice; odd pairs carry codes x 16
                            const f16x2_t h = __builtin_bit_cast(f16x2_t, pr[4 * q + t]);
                            const float sc = (t & 1) ? 0.0625f : 1.0f;
                            d = fmaf((float)h[0] * sc, __uint_as_float(xq[t] << 16), d);
                            d = fmaf((float)h[1] * sc, __uint_as_float(xq[t] & 0xFFFF0000u), d);
                        }
                    }
                    v[m] = fmaf(s, d, v[m]);
                }
            }
            // four rows per reduction: rows i-3 .. i in a0 .. a3
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                a0[m] = a1[m];
                a1[m] = a2[m];
                a2[m] = a3[m];
                a3[m] = v[m];
            }
            if ((i & 3) == 3) {
#pragma unroll
                for (int m = 0; m < MT; ++m) {
                    const float k = reduce4(a0[m], a1[m], a2[m], a3[m]);
                    if ((lane & 15) == 0) red[(wave * row_stride + (i - 3) + (lane >> 4)) * MT + m] = k;
                }
                if constexpr (kLockstep)
                    if (i + 1 < rows_per_wg) __builtin_amdgcn_s_barrier();
            }
        }
    };

    if (!XF32 && exact) {
        run_exact_bf16();
    } else if constexpr (ONE) {
        compute_step(B0{}, 0);   // workgroups of one step (four rows)
    } else {
        // two buffers of one step: the next step's loads are in flight while a step is
        // computed (rows_per_wg is a multiple of 8); with kLockstep the waves meet before
        // each step's loads
        int rb = 0;
        for (; rb + 2 * R < rows_per_wg; rb += 2 * R) {
            if constexpr (kLockstep) __builtin_amdgcn_s_barrier();
            issue_step(B1{}, rb + R);
            compute_step(B0{}, rb);
            if constexpr (kLockstep) __builtin_amdgcn_s_barrier();
            issue_step(B0{}, rb + 2 * R);
            compute_step(B1{}, rb + R);
        }
        if constexpr (kLockstep) __builtin_amdgcn_s_barrier();
        issue_step(B1{}, rb + R);
        compute_step(B0{}, rb);
        compute_step(B1{}, rb + R);
    }
    __syncthreads();

    const int rows_here = r_end - r0;
    for (int t = threadIdx.x; t < rows_here * MT; t += T) {
        const int rloc = t / MT;
        const int m = t - rloc * MT;
        if (m >= M) continue;
        float v = 0.0f;
        for (int w = 0; w < n_waves; ++w) v += red[(w * row_stride + rloc) * MT + m];
        const int64_t o = (int64_t)m * N + r0 + rloc;
        if (y_bf16)
            static_cast<uint16_t*>(yv)[o] = (uint16_t)bf16_bits_rne(v);
        else
            static_cast<float*>(yv)[o] = v;
    }
}

struct GemvArgs {
    const u32x4_t* wq;
    const u32x4_t* sz4;
    const void* x;
    void* y;
    int y_bf16, n, k, m, rows;
    int gshift;       // log2(group / 32)
    bool scale_bf16;
};

constexpr int kMaxRowsPerWg = 64;

int compute_units() {
    static std::atomic<int> cached{0};
    int v = cached.load(std::memory_order_relaxed);
    if (v > 0) return v;
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
        cus = 256;
    cached.store(cus, std::memory_order_relaxed);
    return cus;
}

// Rows per workgroup chosen from the number of resident workgroups: measured on MI355X,
// groups of up to 8 waves stream best with about three rounds of resident groups (finer
// work, shorter tail), the 14-wave groups of K ~ 28K with one; rows a multiple of the chunk.
template <typename Kern>
int rows_for(Kern kernel, int block, int n, int mt, int chunk_rows, std::atomic<int>* cache) {
    const int waves = block / 64;
    int resident = cache[waves].load(std::memory_order_relaxed);
    if (resident == 0) {
        const size_t smem = (size_t)waves * kMaxRowsPerWg * mt * sizeof(float);
        int r = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&r, kernel, block, smem) != hipSuccess || r < 1)
            r = 1;
        cache[waves].store(r, std::memory_order_relaxed);
        resident = r;
    }
    const int rounds = waves <= 8 ? 3 : 1;
    const long wgs = (long)resident * compute_units() * rounds;
    int rows = (int)((n + wgs - 1) / wgs);
    rows = (rows + chunk_rows - 1) / chunk_rows * chunk_rows;
    if (rows < chunk_rows) rows = chunk_rows;
    if (rows > kMaxRowsPerWg) rows = kMaxRowsPerWg / chunk_rows * chunk_rows;
    return rows;
}

// Small matrices that fill less than one round of resident groups at the smallest chunk take
// workgroups of one step (four rows), twice the waves per CU, when those still fit in one
// round (measured on MI355X, 4096 x 4096 at M = 1: 4.4 against 4.9 us with bf16 x, 5.7
// against 6.3 us with binary32 x).  Only groups of up to four waves: the six-wave groups of
// 4096 x 11008 ran 9.4 against 8.9 us with them.
bool one_step_fits(int n, int rows, int chunk_rows, int resident) {
    const long slots = (long)resident * compute_units();
    return rows == chunk_rows && (n + rows - 1) / rows < slots && (n + kRowsPerStep - 1) / kRowsPerStep <= slots;
}

template <int MT, bool XF32, int SPT, int MAXT, bool RAGGED, bool SBF16>
hipError_t launch_var(GemvArgs a, dim3 block, hipStream_t s) {
    constexpr int CR = kChunk * kRowsPerStep;
    static std::atomic<int> cache[17];
    auto kern = gemv_kernel<MT, XF32, SPT, MAXT, RAGGED, SBF16>;
    a.rows = rows_for(kern, (int)block.x, a.n, MT, CR, cache);
    if constexpr (MT == 1 && SPT == 1) {
        if (block.x <= 256 &&
            one_step_fits(a.n, a.rows, CR, cache[block.x / 64].load(std::memory_order_relaxed))) {
            const dim3 grid((unsigned)((a.n + kRowsPerStep - 1) / kRowsPerStep));
            const size_t shmem = (size_t)(block.x / 64) * kRowsPerStep * MT * sizeof(float);
            hipLaunchKernelGGL((gemv_kernel<MT, XF32, SPT, MAXT, RAGGED, SBF16, true>), grid, block, shmem, s,
                               a.wq, a.sz4, a.x, a.y, a.y_bf16, a.n, a.k, a.m, kRowsPerStep, a.gshift,
                               (int)grid.x, kRowsPerStep);
            return hipGetLastError();
        }
    }
    unsigned wgs = (unsigned)((a.n + a.rows - 1) / a.rows);
    // A short last round: the last round of resident workgroups takes half the rows.
    // Workgroups start in index order as earlier ones finish, so the final ones otherwise
    // start late with a full share and stream alone at the end.  Measured on MI355X
    // (57344x8192 at M = 1): 38.3-38.4 us against 39.5-40.0 us; the one-round 14-wave
    // groups of K ~ 28K run slower with it, so they keep equal shares.
    int tail_first = (int)wgs, tail_rows = a.rows;
    const int half = block.x <= 512 ? a.rows / 2 : 0;
    if (half >= CR && half % CR == 0) {
        const long round = (long)cache[block.x / 64].load(std::memory_order_relaxed) * compute_units();
        const long main_wgs = ((long)a.n - round * half) / a.rows;
        if (main_wgs > 0) {
            tail_first = (int)main_wgs;
            tail_rows = half;
            const long rest = (long)a.n - main_wgs * a.rows;
            wgs = (unsigned)(main_wgs + (rest + half - 1) / half);
        }
    }
    const dim3 grid(wgs);
    const size_t shmem = (size_t)(block.x / 64) * a.rows * MT * sizeof(float);
    hipLaunchKernelGGL(kern, grid, block, shmem, s, a.wq, a.sz4, a.x, a.y, a.y_bf16, a.n, a.k, a.m,
                       a.rows, a.gshift, tail_first, tail_rows);
    return hipGetLastError();
}

template <int MT, bool XF32, int SPT, int MAXT, bool SBF16>
hipError_t launch_one(const GemvArgs& a, dim3 block, hipStream_t s) {
    const bool ragged = (int)block.x * SPT * 32 != a.k;
    return ragged ? launch_var<MT, XF32, SPT, MAXT, true, SBF16>(a, block, s)
                  : launch_var<MT, XF32, SPT, MAXT, false, SBF16>(a, block, s);
}

// Instantiated variants (MT = rows of x per launch, SPT = 16-byte slices per lane):
//   M=1 bf16:   SPT 1, up to 1024 threads (K <= 32768)
//   otherwise:  up to 512 threads; SPT 1 for K <= 16384, SPT 2 up to 32768; MT up to 3
//               (bf16, SPT 1), 2 (binary32, SPT 1), 1 (SPT 2) so that the registers fit
//               the 256-VGPR budget of a 512-thread group without spilling
int max_mt(bool x_f32, int spt) {
    if (spt != 1) return 1;
    return x_f32 ? 2 : 3;
}

template <bool SB>
hipError_t dispatch_t(bool x_f32, int spt, int mt, const GemvArgs& a, dim3 block, hipStream_t s) {
    if (!x_f32 && mt == 1 && spt == 1)
        return block.x > 512 ? launch_one<1, false, 1, 1024, SB>(a, block, s)
                             : launch_one<1, false, 1, 512, SB>(a, block, s);
#define W4_CASE(MTV, XF, SP) \
    if (mt == MTV && x_f32 == XF && spt == SP) return launch_one<MTV, XF, SP, 512, SB>(a, block, s);
    W4_CASE(2, false, 1) W4_CASE(3, false, 1)
    W4_CASE(1, false, 2)
    W4_CASE(1, true, 1) W4_CASE(2, true, 1)
    W4_CASE(1, true, 2)
#undef W4_CASE
    return hipErrorInvalidValue;
}

hipError_t dispatch(bool x_f32, int spt, int mt, const GemvArgs& a, dim3 block, hipStream_t s) {
    return a.scale_bf16 ? dispatch_t<true>(x_f32, spt, mt, a, block, s)
                        : dispatch_t<false>(x_f32, spt, mt, a, block, s);
}

}  // namespace

hipError_t launch_gemv(const uint8_t* prepared, int64_t n, int64_t k, const void* x, bool x_f32,
                       int64_t m, void* y, bool y_bf16, hipStream_t s) {
    // bf16 rows: the matrix-core kernels read the weights once for all rows.  The dot2
    // kernel below does M times the vector work per weight; it stays faster (measured on
    // MI355X at the 70B shapes) at one row, and at two rows while it needs a single pass over
    // the weights (K <= 16384) unless the resident-x kernel has more than 16384 rows to
    // spread its x conversion over (gate_up 57344 x 8192 at M = 2: 46.8 us against 49.4;
    // qkv 10240 x 8192: 16.2 against 14.7).
    const bool one_pass = k <= 16384;
    const bool dot2_wins = m == 1 || (m == 2 && one_pass && !(n > 16384 && gemv_resident_x_takes(n, k)));
    if (!x_f32 && !dot2_wins)
        return launch_gemv_mfma(prepared, n, k, static_cast<const uint16_t*>(x), m, y, y_bf16, s);
    return launch_gemv_dot2(prepared, n, k, kGroup, false, x, x_f32, m, y, y_bf16, s);
}

hipError_t launch_gemv_dot2(const uint8_t* prepared, int64_t n, int64_t k, int group,
                            bool scale_bf16, const void* x, bool x_f32, int64_t m, void* y,
                            bool y_bf16, hipStream_t s) {
    const int S = (int)(k / 32);
    GemvArgs a;
    a.wq = reinterpret_cast<const u32x4_t*>(prepared);
    a.sz4 = reinterpret_cast<const u32x4_t*>(prepared + sz_offset(n, k));
    a.y_bf16 = y_bf16 ? 1 : 0;
    a.n = (int)n;
    a.k = (int)k;
    a.rows = 0;
    a.gshift = group == 32 ? 0 : group == 64 ? 1 : 2;
    a.scale_bf16 = scale_bf16;
    const bool wide = !x_f32 && m == 1;      // one slice per lane, up to 1024 threads
    const int spt = wide ? 1 : (S <= 512 ? 1 : 2);
    const int waves = (S + 64 * spt - 1) / (64 * spt);
    const dim3 block(64 * waves);
    const int mt_max = max_mt(x_f32, spt);
    for (int64_t m0 = 0; m0 < m; m0 += mt_max) {
        const int mc = (int)((m - m0) < mt_max ? (m - m0) : mt_max);
        a.x = x_f32 ? (const void*)(static_cast<const float*>(x) + m0 * k)
                    : (const void*)(static_cast<const uint16_t*>(x) + m0 * k);
        a.y = y_bf16 ? (void*)(static_cast<uint16_t*>(y) + m0 * n)
                     : (void*)(static_cast<float*>(y) + m0 * n);
        a.m = mc;
        hipError_t err = dispatch(x_f32, spt, mc, a, block, s);
        if (err != hipSuccess) return err;
    }
    return hipSuccess;
}

}  // namespace w4
