// Prefill-sized W4A16 product Y = X * w_hat^T on the matrix cores.
//
// Prefill multiplies large matrices, so it is bound by the matrix units, and a
// weight-only format has to turn the 4-bit codes back into 16-bit values before they
// reach them (page "LLM Quantization Architecture in Depth" › "Why fewer bits make
// decoding faster"; page "Quantization" › "The idea in one minute").  Per group the
// product is scale16 * sum_k (q - zero) x (page "Weight quantization", section "How it
// works": the dequantized weight (code - zero) * scale, one multiply per group):
//
//   * exact operands.  The matrix instruction aligns its products and the accumulator
//     to the largest before it rounds, so the B operand must be the exact q - zero, not a
//     biased code.  v_and_or_b32 builds binary16 1024 + q (1024 + 16 q for the codes at
//     bits 4..7 of a half word) and v_pk_add_f16 subtracts 1024 + zero (1024 + 16 zero)
//     exactly, so B is binary16 q - zero (or 16 (q - zero)) and the product runs on
//     v_mfma_f32_32x32x16_f16;
//   * the A operand is X in binary16: a pre-pass writes X' = X * 2^-E[m] per row (and a
//     further 2^-4 at the inputs that meet the 16 (q - zero) codes), with E[m] putting
//     the row's largest value just under 2^16.  bf16 has 8 significant bits and binary16
//     11, so X' is exact for every value within 2^28 of the row's largest; a row with a
//     value outside that window is marked, and a fix-up pass recomputes its outputs with
//     one binary32 FMA per weight after the product;
//   * a K step is one group (128 inputs); eight MFMA steps give P = sum (q - zero) x' in a
//     fresh accumulator and acc += scale16 * P, one FMA per accumulator element; at the
//     end y = acc * 2^E[m].  No weight is rounded and a code equal to its zero adds 0.
//
// Tiling: 512 threads (8 waves) per 128 x 256 output tile; wave (wm, wn) owns rows
// 64wm..+64 and columns 64wn..+64 as 2 x 2 MFMA tiles of 32 x 32.  Operands reach LDS
// through a three-stage ring filled two groups ahead by global_load_lds_dwordx4.
//
// MFMA operand order: lane l supplies row (l % 32) of its operand and, in MFMA step s of
// a group, the eight k values 64*(l/32) + 8s .. +7 -- the same k for both operands, so
// each output is a dot product over matching k.  The 32 x 32 f32 result sits in lane l
// as column (l % 32) and rows 8*(v/4) + 4*(l/32) + (v%4) for element v = 0..15.
#include "w4_internal.h"

namespace w4 {
namespace {

typedef __attribute__((ext_vector_type(8))) _Float16 f16x8_t;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int BM = 128;
constexpr int BN = 256;
constexpr int BK = kGroup;
constexpr int GT = 512;                  // threads per workgroup
constexpr int kXcds = 8;                 // accelerator complex dies of MI355X, each with its own L2
constexpr int kGroupM = 8;               // M tiles per band of the XCD-aware tile order
constexpr int kPrepThreads = 256;
constexpr int kPrepKeep = 4;             // 16-byte chunks per thread kept between the passes

__device__ __forceinline__ uint32_t bf16_bits_rne(float f) {
    const uint32_t u = __float_as_uint(f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ uint32_t add2h(uint32_t a, uint32_t b) {
    return __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2_t, a) + __builtin_bit_cast(f16x2_t, b));
}

__device__ __forceinline__ f16x8_t as_f16x8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
    const u32x4_t v = {a, b, c, d};
    return __builtin_bit_cast(f16x8_t, v);
}

// Input k of a row meets a code scaled by 16 when k % 8 is 2, 3, 6 or 7 (the codes at bits
// 4..7 and 20..23 of the two half words of a prepared word).
__device__ __forceinline__ int extra_shift(int k) { return (k & 2) ? 4 : 0; }

// ---- pre-pass: X' = X * 2^-E[m] (and 2^-4 more at the inputs of scaled codes) in binary16,
// E[m] per row, bad[m] = 1 when some value of the row does not convert exactly.  One
// workgroup per row, 16 bytes (eight inputs) per thread and step.
__global__ __launch_bounds__(kPrepThreads) void xprep_kernel(const uint16_t* __restrict__ X, int K,
                                                             uint16_t* __restrict__ Xh,
                                                             int* __restrict__ E, int* __restrict__ bad) {
    __shared__ uint32_t red[kPrepThreads / 64];
    const int m = blockIdx.x;
    const uint4* row = reinterpret_cast<const uint4*>(X + (int64_t)m * K);
    uint4* out = reinterpret_cast<uint4*>(Xh + (int64_t)m * K);
    const int chunks = K / 8;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;

    // the first kPrepKeep chunks of each thread stay in registers between the two passes
    // (all of a row up to K = 8192); the rest is read again
    uint4 keep[kPrepKeep];
    uint32_t ef = 1;  // an all-zero or subnormal row uses the smallest normal exponent
#pragma unroll
    for (int j = 0; j < kPrepKeep; ++j) {
        const int c = threadIdx.x + j * kPrepThreads;
        keep[j] = c < chunks ? row[c] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < kPrepKeep; ++j) {
        const uint32_t w[4] = {keep[j].x, keep[j].y, keep[j].z, keep[j].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) ef = max(ef, max((w[i] >> 7) & 0xFFu, (w[i] >> 23) & 0xFFu));
    }
    for (int c = threadIdx.x + kPrepKeep * kPrepThreads; c < chunks; c += kPrepThreads) {
        const uint4 v = row[c];
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) ef = max(ef, max((w[i] >> 7) & 0xFFu, (w[i] >> 23) & 0xFFu));
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) ef = max(ef, (uint32_t)__shfl_xor((int)ef, o));
    if (lane == 0) red[wave] = ef;
    __syncthreads();
#pragma unroll
    for (int w = 0; w < kPrepThreads / 64; ++w) ef = max(ef, red[w]);
    const int e = (int)ef - 127 - 15;  // the row's largest value lands in [2^15, 2^16)

    bool b = false;
    for (int c = threadIdx.x, j = 0; c < chunks; c += kPrepThreads, ++j) {
        const uint4 v = j < kPrepKeep ? keep[min(j, kPrepKeep - 1)] : row[c];
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
        uint32_t h[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int es = e + extra_shift(2 * i);
            const float lo = __uint_as_float(w[i] << 16), hi = __uint_as_float(w[i] & 0xFFFF0000u);
            const _Float16 hl = (_Float16)ldexpf(lo, -es), hh = (_Float16)ldexpf(hi, -es);
            b |= ldexpf((float)hl, es) != lo || ldexpf((float)hh, es) != hi;
            const f16x2_t p = {hl, hh};
            h[i] = __builtin_bit_cast(uint32_t, p);
        }
        out[c] = make_uint4(h[0], h[1], h[2], h[3]);
    }
    const int any = __syncthreads_or(b ? 1 : 0);
    if (threadIdx.x == 0) {
        E[m] = e;
        bad[m] = any ? 1 : 0;
    }
}

// One stage of the LDS ring: the operands of one group (K step).
//   X:  128 rows x 16 chunks of 16 bytes (binary16); chunk c of row r sits at slot c ^ (r & 15)
//   W:  256 columns x 4 pieces of 16 bytes (the 64 code bytes of the group);
//       piece p of column n sits at slot p ^ ((n >> 2) & 3)
//   SZ: the scale/zero words of the 256 columns, in column order
// The swizzles keep the 16-byte reads of the MFMA operands free of bank conflicts.
constexpr int kStages = 3;
constexpr int kXBytes = BM * BK * 2;          // 32768
constexpr int kWBytes = BN * BK / 2;          // 16384
constexpr int kSzBytes = 1024;                // 256 words (64 lanes x 16 bytes)
constexpr int kStageBytes = kXBytes + kWBytes + kSzBytes;

// 16 bytes per lane from global memory straight into LDS: lane l of the wave writes
// bytes [16 l, 16 l + 16) after the wave-uniform LDS address.  Issued as inline
// assembly so that the compiler does not order the LDS reads of other stages
// behind these loads; the kernel waits for them itself (vmcnt) before the barrier
// that publishes a stage.
__device__ __forceinline__ void load_lds16(const void* g, uint32_t lds_addr) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(g), "s"(lds_addr)
                 : "memory", "m0");
}
// the same with a uniform base address in SGPRs and a 32-bit byte offset per lane
__device__ __forceinline__ void load_lds16_sv(const void* sbase, uint32_t voff, uint32_t lds_addr) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(voff), "s"(sbase), "s"(lds_addr)
                 : "memory", "m0");
}

__global__ __launch_bounds__(GT) void gemm_kernel(const uint8_t* __restrict__ wq,
                                                  const uint32_t* __restrict__ sz,
                                                  const uint16_t* __restrict__ Xh,
                                                  const int* __restrict__ E,
                                                  void* __restrict__ Y, int y_bf16, int M, int N,
                                                  int K, int tiles_m, int tiles_n, int group_m,
                                                  int per_xcd) {
    __shared__ __attribute__((aligned(16))) uint8_t ring[kStages * kStageBytes];

    // Tile order: workgroup b runs on XCD b % kXcds, and each XCD takes a contiguous
    // range of a grouped order (group_m tiles of M per band, N within the band), so the
    // workgroups resident on one XCD at a time cover a compact block of tiles and share
    // their X rows and weight columns in that XCD's L2.
    const int t = (int)(blockIdx.x % kXcds) * per_xcd + (int)(blockIdx.x / kXcds);
    if (t >= tiles_m * tiles_n) return;
    const int band = t / (group_m * tiles_n);
    const int first_m = band * group_m;
    const int gm = min(tiles_m - first_m, group_m);
    const int r = t - band * group_m * tiles_n;
    const int n0 = (r / gm) * BN;
    const int m0 = (first_m + r % gm) * BM;

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int wm = wave >> 2;        // 0..1: rows 64wm..
    const int wn = wave & 3;         // 0..3: columns 64wn..
    const int Kg = K / kGroup;
    const int64_t row_bytes = K / 2;
    const int h = lane >> 5;
    const int l32 = lane & 31;
    const int n_quads = (N + 3) >> 2;

    // ---- per-lane byte offsets of the stage loads from the tile's first row (X') or column
    // (W) at group 0; the group moves a uniform base held in SGPRs
    // X': wave w fills rows 16w .. 16w+15 with four 1 KiB loads of four rows each
    uint32_t xoff[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = 16 * wave + 4 * i + (lane >> 4);
        const int c = (lane & 15) ^ (row & 15);
        xoff[i] = 2u * (uint32_t)((min(m0 + row, M - 1) - m0) * K + 8 * c);
    }
    // W: wave w fills columns 32w .. 32w+31 with two loads of sixteen columns
    uint32_t woff[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int col = 32 * wave + 16 * i + (lane >> 2);
        const int piece = (lane & 3) ^ ((col >> 2) & 3);
        woff[i] = (uint32_t)((int64_t)(min(n0 + col, N - 1) - n0) * row_bytes) + 16 * piece;
    }
    const uint8_t* xtile = reinterpret_cast<const uint8_t*>(Xh) + (int64_t)m0 * K * 2;
    const uint8_t* wtile = wq + (int64_t)n0 * row_bytes;
    // SZ (wave 0): lane = column quad
    const uint32_t* szsrc = sz + (int64_t)min((n0 >> 2) + lane, n_quads - 1) * Kg * 4;

    // LDS address of the ring (wave-uniform)
    const uint32_t ring_lds = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)ring);
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    auto issue_stage = [&](int st, int kg) {
        const uint32_t base = ring_lds + st * kStageBytes;
        const uint8_t* xg = xtile + (int64_t)kg * BK * 2;
        const uint8_t* wg = wtile + (int64_t)kg * (BK / 2);
#pragma unroll
        for (int i = 0; i < 4; ++i) load_lds16_sv(xg, xoff[i], base + (4 * wave_u + i) * 1024);
#pragma unroll
        for (int i = 0; i < 2; ++i) load_lds16_sv(wg, woff[i], base + kXBytes + (2 * wave_u + i) * 1024);
        if (wave_u == 0) load_lds16(szsrc + kg * 4, base + kXBytes + kWBytes);
    };

    // constants of the code unpack, kept in registers so that v_and_or_b32 is selected
    uint32_t m_lo, m_hi, magic, e4;
    asm volatile("s_mov_b32 %0, 0x000F000F" : "=s"(m_lo));
    asm volatile("s_mov_b32 %0, 0x00F000F0" : "=s"(m_hi));
    asm volatile("v_mov_b32 %0, 0x64006400" : "=v"(magic));
    asm volatile("s_mov_b32 %0, 0xE4E4E4E4" : "=s"(e4));

    f32x16_t acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = (f32x16_t){};

    issue_stage(0, 0);
    if (Kg > 1) issue_stage(1, 1);

    for (int kg = 0; kg < Kg; ++kg) {
        // this wave's loads of group kg have landed (at most one later stage, six or seven
        // loads, may still be in flight); the barrier makes every wave's loads visible and
        // frees the stage that group kg+2 reuses
        if (kg + 1 < Kg) {
            if (wave_u == 0)
                __builtin_amdgcn_s_waitcnt(0xF77);  // vmcnt(7)
            else
                __builtin_amdgcn_s_waitcnt(0xF76);  // vmcnt(6)
        } else {
            __builtin_amdgcn_s_waitcnt(0xF70);  // vmcnt(0)
        }
        __syncthreads();
        if (kg + 2 < Kg) issue_stage((kg + 2) % kStages, kg + 2);

        const uint8_t* base = ring + (kg % kStages) * kStageBytes;
        const uint8_t* xs = base;
        const uint8_t* ws = base + kXBytes;
        const uint32_t* szs = reinterpret_cast<const uint32_t*>(base + kXBytes + kWBytes);

        // codes of this lane's two columns: pieces 2h and 2h+1 of each
        u32x4_t wc[2][2];
        uint32_t szc[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int col = 64 * wn + 32 * j + l32;
            const int sw = (col >> 2) & 3;
#pragma unroll
            for (int e = 0; e < 2; ++e)
                wc[j][e] = *reinterpret_cast<const u32x4_t*>(ws + col * 64 + (((2 * h + e) ^ sw) * 16));
            szc[j] = szs[col];
        }
        uint32_t z1[2], z16[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            // binary16 pairs -(1024 + zero) and -(1024 + 16 zero) from bytes 2 and 3
            z1[j] = __builtin_amdgcn_perm(e4, szc[j], 0x04020402u);
            z16[j] = __builtin_amdgcn_perm(e4, szc[j], 0x04030403u);
        }

        // ---- eight MFMA steps over the group into fresh accumulators P
        f32x16_t P[2][2];
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            f16x8_t a[2], b[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int row = 64 * wm + 32 * i + l32;
                const int c = 8 * h + s;
                a[i] = *reinterpret_cast<const f16x8_t*>(xs + row * 256 + ((c ^ (row & 15)) * 16));
            }
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const uint32_t w = wc[j][s >> 2][s & 3];  // codes of k = 64h + 8s .. +7
                const uint32_t u = w >> 8;
                b[j] = as_f16x8(add2h((w & m_lo) | magic, z1[j]), add2h((w & m_hi) | magic, z16[j]),
                                add2h((u & m_lo) | magic, z1[j]), add2h((u & m_hi) | magic, z16[j]));
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    if (s == 0) {
                        const f32x16_t zero = {};
                        P[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i], b[j], zero, 0, 0, 0);
                    } else {
                        P[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i], b[j], P[i][j], 0, 0, 0);
                    }
                }
        }

        // ---- group term: acc += scale16 * P
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const float sc = (float)__builtin_bit_cast(_Float16, (uint16_t)(szc[j] & 0xFFFFu));
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[i][j][v] = fmaf(sc, P[i][j][v], acc[i][j][v]);
        }
    }

#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int row = m0 + 64 * wm + 32 * i + 8 * (v >> 2) + 4 * h + (v & 3);
            if (row >= M) continue;
            const int e = E[row];
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int c = n0 + 64 * wn + 32 * j + l32;
                if (c < N) {
                    const float yv = ldexpf(acc[i][j][v], e);
                    const int64_t o = (int64_t)row * N + c;
                    if (y_bf16)
                        static_cast<uint16_t*>(Y)[o] = (uint16_t)bf16_bits_rne(yv);
                    else
                        static_cast<float*>(Y)[o] = yv;
                }
            }
        }
}

// ---- fix-up pass: rows of X marked by the pre-pass are recomputed with one binary32 FMA
// per weight, (q - zero) * x exactly converted.  Workgroup b owns weight rows
// [64 b, 64 b + 64) (16 per wave); it finds the marked rows of X itself (so a product with
// none costs one scan of M flags), in increasing order.
constexpr int kFixRowsPerWg = 64;

__global__ __launch_bounds__(256) void fixup_kernel(const uint8_t* __restrict__ wq,
                                                    const uint32_t* __restrict__ sz,
                                                    const uint16_t* __restrict__ X,
                                                    const int* __restrict__ bad,
                                                    void* __restrict__ Y, int y_bf16, int M, int N,
                                                    int K) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int Kg = K / kGroup;
    const int S = K / 32;                 // 16-byte slices per row
    const int64_t row_bytes = K / 2;
    // the common case, no marked row: all threads scan the flags at once and leave
    bool any = false;
    for (int i = threadIdx.x; i < M; i += blockDim.x) any |= bad[i] != 0;
    if (!__syncthreads_or(any ? 1 : 0)) return;
    for (int mb = 0; mb < M; mb += 64) {
        const int mi = mb + lane;
        uint64_t marked = __builtin_amdgcn_ballot_w64(mi < M && bad[mi] != 0);
        while (marked) {
            const int m = mb + __builtin_ctzll(marked);
            marked &= marked - 1;
            const uint16_t* xr = X + (int64_t)m * K;
            for (int rr = 0; rr < kFixRowsPerWg / 4; ++rr) {
                const int n = blockIdx.x * kFixRowsPerWg + wave * (kFixRowsPerWg / 4) + rr;
                if (n >= N) break;
                float acc = 0.0f;
                for (int sl = lane; sl < S; sl += 64) {
                    const u32x4_t wv = *reinterpret_cast<const u32x4_t*>(wq + n * row_bytes + 16 * sl);
                    const uint32_t szw = sz[sz_index(n, sl >> 2, Kg)];
                    const int zero = (int)((szw >> 16) & 0xFFu);
                    const float sc = (float)__builtin_bit_cast(_Float16, (uint16_t)(szw & 0xFFFFu));
                    const uint4* px = reinterpret_cast<const uint4*>(xr + 32 * sl);
                    float d = 0.0f;
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        const uint4 xv = px[t];
                        const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const int ce = (int)((wv[t] >> (4 * j)) & 0xFu);
                            const int co = (int)((wv[t] >> (16 + 4 * j)) & 0xFu);
                            d = fmaf((float)(ce - zero), __uint_as_float(xw[j] << 16), d);
                            d = fmaf((float)(co - zero), __uint_as_float(xw[j] & 0xFFFF0000u), d);
                        }
                    }
                    acc = fmaf(sc, d, acc);
                }
#pragma unroll
                for (int o = 32; o >= 1; o >>= 1) acc += __shfl_xor(acc, o);
                if (lane == 0) {
                    const int64_t o = (int64_t)m * N + n;
                    if (y_bf16)
                        static_cast<uint16_t*>(Y)[o] = (uint16_t)bf16_bits_rne(acc);
                    else
                        static_cast<float*>(Y)[o] = acc;
                }
            }
        }
    }
}

int64_t align256(int64_t b) { return (b + 255) / 256 * 256; }

}  // namespace

// workspace: X' [M, K] binary16 | E [M] int32 | bad [M] int32
size_t gemm_workspace(int64_t m, int64_t k) {
    return (size_t)(align256(m * k * 2) + align256(m * 4) + align256(m * 4));
}

hipError_t launch_gemm(const uint8_t* prepared, int64_t n, int64_t k, const void* X, int64_t m,
                       void* Y, bool y_bf16, void* workspace, hipStream_t s) {
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    uint16_t* Xh = reinterpret_cast<uint16_t*>(ws);
    int* E = reinterpret_cast<int*>(ws + align256(m * k * 2));
    int* bad = reinterpret_cast<int*>(ws + align256(m * k * 2) + align256(m * 4));
    const uint16_t* Xb = static_cast<const uint16_t*>(X);
    const uint32_t* sz = reinterpret_cast<const uint32_t*>(prepared + sz_offset(n, k));
    hipLaunchKernelGGL(xprep_kernel, dim3((unsigned)m), dim3(kPrepThreads), 0, s, Xb, (int)k, Xh, E, bad);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int tiles_n = (int)((n + BN - 1) / BN);
    const int tiles_m = (int)((m + BM - 1) / BM);
    const int group_m = tiles_m < kGroupM ? tiles_m : kGroupM;
    const int per_xcd = (tiles_m * tiles_n + kXcds - 1) / kXcds;
    hipLaunchKernelGGL(gemm_kernel, dim3((unsigned)(per_xcd * kXcds)), dim3(GT), 0, s, prepared, sz, Xh, E,
                       Y, y_bf16 ? 1 : 0, (int)m, (int)n, (int)k, tiles_m, tiles_n, group_m, per_xcd);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(fixup_kernel, dim3((unsigned)((n + kFixRowsPerWg - 1) / kFixRowsPerWg)), dim3(256), 0,
                       s, prepared, sz, Xb, bad, Y, y_bf16 ? 1 : 0, (int)m, (int)n, (int)k);
    return hipGetLastError();
}

}  // namespace w4
