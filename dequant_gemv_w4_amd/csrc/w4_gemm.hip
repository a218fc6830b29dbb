// Prefill-sized W4A16 product Y = X * w_hat^T on bf16 MFMA.
//
// Prefill multiplies large matrices, so it is bound by the matrix units, and a
// weight-only format has to turn the 4-bit codes back into 16-bit values
// before they reach them (page "LLM Quantization Architecture in Depth" ›
// "Why fewer bits make decoding faster"; page "Quantization" › "The idea in
// one minute").  The group term of page "Weight quantization" (section "How it
// works"), scale16 * (sum q*x - zero * sum x), is applied per group on the f32
// accumulator:
//
//   * a K step is one group (128 inputs).  The B operand of
//     v_mfma_f32_32x32x16_bf16 is built in registers straight from the packed
//     codes: v_and_or_b32 turns two codes into the bf16 pair (128+q0, 128+q1),
//     exactly, in natural k order (the kernel layout puts input pairs in the
//     two halves of a word).  Eight MFMA steps give P = sum (128+q) x for the
//     group in a fresh accumulator;
//   * S[m][g] = sum x over the group comes from a pre-pass that runs the very
//     same MFMA sequence with a B operand of ones, so a group whose codes are
//     all 0 gives P = 128*S exactly (scaling by 128 commutes with rounding);
//   * acc += scale16 * (P - (128 + zero) * S): two FMAs per accumulator element
//     per group; no weight is rounded to bf16.
//
// Tiling: 512 threads (8 waves) per 128 x 256 output tile; wave (wm, wn) owns
// rows 64wm..+64 and columns 64wn..+64 as 2 x 2 MFMA tiles of 32 x 32.  The X
// tile (128 x 128 bf16) is double-buffered in LDS (rows padded by 16 bytes);
// weights and the scale/zero words are loaded one group ahead into registers.
//
// MFMA operand order: lane l supplies row (l % 32) of its operand and, in MFMA
// step s of a group, the eight k values 64*(l/32) + 8s .. +7 -- the same k for
// both operands, so each output is a dot product over matching k.  The 32 x 32
// f32 result sits in lane l as column (l % 32) and rows 8*(v/4) + 4*(l/32) +
// (v%4) for element v = 0..15.
#include <cstdlib>

#include "w4_internal.h"

namespace w4 {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int BM = 128;
constexpr int BN = 256;
constexpr int BK = kGroup;
constexpr int GT = 512;                  // threads per workgroup
constexpr int kXcds = 8;                 // accelerator complex dies of MI355X, each with its own L2

__device__ __forceinline__ uint32_t bf16_bits_rne(float f) {
    const uint32_t u = __float_as_uint(f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ bf16x8_t as_bf16x8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
    const u32x4_t v = {a, b, c, d};
    return __builtin_bit_cast(bf16x8_t, v);
}

__device__ __forceinline__ void load_lds16(const void* g, uint32_t lds_addr);

// ---- pre-pass: S^T[g][m] = sum of x[m, 128g .. 128g+127] by the MFMA sequence of the GEMM
// (the same A operands in the same MFMA steps, B = ones).  Each wave stages its 32 rows x
// 128 inputs in LDS with loads of 4 rows x 256 contiguous bytes (chunk c of row r at slot
// c ^ (r & 15)), then reads the A operands from there: one load per lane straight into
// the MFMA lane order would touch 64 lines per instruction.  Rows past M repeat row M-1
// (their sums are never used).
__global__ __launch_bounds__(256) void xsum_kernel(const uint16_t* __restrict__ X, int M, int K,
                                                   float* __restrict__ St, int m_pad) {
    __shared__ __attribute__((aligned(16))) uint8_t stage[4][32 * 256];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int Kg = K / kGroup;
    const int tile = blockIdx.x * 4 + wave;      // (m tile, group) pairs, m fastest
    const int n_mt = (M + 31) / 32;
    if (tile >= n_mt * Kg) return;
    const int mt = tile % n_mt;
    const int g = tile / n_mt;
    const uint32_t base = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)stage[wave]);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int r = 4 * i + (lane >> 4);
        const int c = (lane & 15) ^ (r & 15);
        const int row = min(mt * 32 + r, M - 1);
        load_lds16(X + (int64_t)row * K + g * kGroup + 8 * c, base + i * 1024);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's rows have landed
    asm volatile("" ::: "memory");
    const int r = lane & 31;
    const int h = lane >> 5;
    const bf16x8_t ones = as_bf16x8(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u);
    f32x16_t acc;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
        const int c = 8 * h + s;
        const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(&stage[wave][r * 256 + ((c ^ (r & 15)) * 16)]);
        if (s == 0) {
            const f32x16_t zero = {};
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, ones, zero, 0, 0, 0);
        } else {
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, ones, acc, 0, 0, 0);
        }
    }
    // column (lane % 32) == 0 holds all 32 rows in lanes 0 and 32
    if ((lane & 31) == 0) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int rr = mt * 32 + 8 * (v >> 2) + 4 * h + (v & 3);
            St[(int64_t)g * m_pad + rr] = acc[v];
        }
    }
}

// One stage of the LDS ring: the operands of one group (K step).
//   X:  128 rows x 16 chunks of 16 bytes; chunk c of row r sits at slot c ^ (r & 15)
//   W:  256 columns x 4 pieces of 16 bytes (the 64 code bytes of the group);
//       piece p of column n sits at slot p ^ ((n >> 2) & 3)
//   SZ: the scale/zero words of the 256 columns, in column order
//   S:  the group sums of the 128 rows
// The swizzles keep the 16-byte reads of the MFMA operands free of bank conflicts.
constexpr int kStages = 3;
constexpr int kXBytes = BM * BK * 2;          // 32768
constexpr int kWBytes = BN * BK / 2;          // 16384
constexpr int kSzBytes = 1024;                // 256 words (64 lanes x 16 bytes)
constexpr int kSBytes = 1024;                 // 128 floats, the load covers 256
constexpr int kStageBytes = kXBytes + kWBytes + kSzBytes + kSBytes;

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

__global__ __launch_bounds__(GT) void gemm_kernel(const uint8_t* __restrict__ wq,
                                                  const uint32_t* __restrict__ sz,
                                                  const uint16_t* __restrict__ X,
                                                  const float* __restrict__ St, int m_pad,
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

    // ---- per-lane global addresses of the stage loads (group 0; a group adds a fixed step)
    // X: wave w fills rows 16w .. 16w+15 with four 1 KiB loads of four rows each
    const uint16_t* xsrc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = 16 * wave + 4 * i + (lane >> 4);
        const int c = (lane & 15) ^ (row & 15);
        xsrc[i] = X + (int64_t)min(m0 + row, M - 1) * K + 8 * c;
    }
    // W: wave w fills columns 32w .. 32w+31 with two loads of sixteen columns
    const uint8_t* wsrc[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int col = 32 * wave + 16 * i + (lane >> 2);
        const int piece = (lane & 3) ^ ((col >> 2) & 3);
        wsrc[i] = wq + (int64_t)min(n0 + col, N - 1) * row_bytes + 16 * piece;
    }
    // SZ (wave 0): lane = column quad; S (wave 1): lane = four rows
    const uint32_t* szsrc = sz + (int64_t)min((n0 >> 2) + lane, n_quads - 1) * Kg * 4;
    const float* ssrc = St + min(m0 + 4 * lane, m_pad - 4);

    // LDS address of the ring (wave-uniform)
    const uint32_t ring_lds = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)ring);
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    auto issue_stage = [&](int st, int kg) {
        const uint32_t base = ring_lds + st * kStageBytes;
#pragma unroll
        for (int i = 0; i < 4; ++i) load_lds16(xsrc[i] + kg * BK, base + (4 * wave_u + i) * 1024);
#pragma unroll
        for (int i = 0; i < 2; ++i)
            load_lds16(wsrc[i] + kg * (BK / 2), base + kXBytes + (2 * wave_u + i) * 1024);
        if (wave_u == 0) load_lds16(szsrc + kg * 4, base + kXBytes + kWBytes);
        if (wave_u == 1) load_lds16(ssrc + (int64_t)kg * m_pad, base + kXBytes + kWBytes + kSzBytes);
    };

    uint32_t nib_mask, bias_bits;
    asm volatile("s_mov_b32 %0, 0x000F000F" : "=s"(nib_mask));
    asm volatile("v_mov_b32 %0, 0x43004300" : "=v"(bias_bits));

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
        if (kg + 1 < Kg)
            __builtin_amdgcn_s_waitcnt(0xF76);  // vmcnt(6)
        else
            __builtin_amdgcn_s_waitcnt(0xF70);  // vmcnt(0)
        __syncthreads();
        if (kg + 2 < Kg) issue_stage((kg + 2) % kStages, kg + 2);

        const uint8_t* base = ring + (kg % kStages) * kStageBytes;
        const uint8_t* xs = base;
        const uint8_t* ws = base + kXBytes;
        const uint32_t* szs = reinterpret_cast<const uint32_t*>(base + kXBytes + kWBytes);
        const float* ss = reinterpret_cast<const float*>(base + kXBytes + kWBytes + kSzBytes);

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

        // ---- eight MFMA steps over the group into fresh accumulators P
        f32x16_t P[2][2];
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            bf16x8_t a[2], b[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int row = 64 * wm + 32 * i + l32;
                const int c = 8 * h + s;
                a[i] = *reinterpret_cast<const bf16x8_t*>(xs + row * 256 + ((c ^ (row & 15)) * 16));
            }
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const uint32_t w = wc[j][s >> 2][s & 3];  // codes of k = 64h + 8s .. +7
                b[j] = as_bf16x8((w & nib_mask) | bias_bits, ((w >> 4) & nib_mask) | bias_bits,
                                 ((w >> 8) & nib_mask) | bias_bits,
                                 ((w >> 12) & nib_mask) | bias_bits);
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    if (s == 0) {
                        const f32x16_t zero = {};
                        P[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], zero, 0, 0, 0);
                    } else {
                        P[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], P[i][j], 0, 0, 0);
                    }
                }
        }

        // ---- group term: acc += scale16 * (P - (128 + zero) * S)
        float sc[2], zb[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            sc[j] = (float)__builtin_bit_cast(_Float16, (uint16_t)(szc[j] & 0xFFFFu));
            zb[j] = (float)((szc[j] >> 16) & 0xFFu);
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float4 s4 = *reinterpret_cast<const float4*>(&ss[64 * wm + 32 * i + 8 * q + 4 * h]);
                const float sv[4] = {s4.x, s4.y, s4.z, s4.w};
#pragma unroll
                for (int rr = 0; rr < 4; ++rr)
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        const int v = 4 * q + rr;
                        acc[i][j][v] = fmaf(sc[j], fmaf(-zb[j], sv[rr], P[i][j][v]), acc[i][j][v]);
                    }
            }
        }
    }

#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int row = m0 + 64 * wm + 32 * i + 8 * (v >> 2) + 4 * h + (v & 3);
                const int c = n0 + 64 * wn + 32 * j + l32;
                if (row < M && c < N) {
                    const int64_t o = (int64_t)row * N + c;
                    if (y_bf16)
                        static_cast<uint16_t*>(Y)[o] = (uint16_t)bf16_bits_rne(acc[i][j][v]);
                    else
                        static_cast<float*>(Y)[o] = acc[i][j][v];
                }
            }
}

int64_t m_padded(int64_t m) { return (m + BM - 1) / BM * BM; }

}  // namespace

size_t gemm_workspace(int64_t m, int64_t k) {
    return (size_t)(k / kGroup) * (size_t)m_padded(m) * sizeof(float);
}

hipError_t launch_gemm(const uint8_t* prepared, int64_t n, int64_t k, const void* X, int64_t m,
                       void* Y, bool y_bf16, void* workspace, hipStream_t s) {
    const int64_t kg = k / kGroup;
    const int m_pad = (int)m_padded(m);
    float* St = static_cast<float*>(workspace);
    const int64_t tiles = ((m + 31) / 32) * kg;
    hipLaunchKernelGGL(xsum_kernel, dim3((unsigned)((tiles + 3) / 4)), dim3(256), 0, s,
                       static_cast<const uint16_t*>(X), (int)m, (int)k, St, m_pad);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    static const int group_env = [] {
        const char* e = getenv("W4A16_GEMM_GROUP_M");
        return e ? atoi(e) : 8;
    }();
    const int tiles_n = (int)((n + BN - 1) / BN);
    const int tiles_m = (int)((m + BM - 1) / BM);
    const int group_m = group_env < 1 ? 1 : (group_env > tiles_m ? tiles_m : group_env);
    const int per_xcd = (tiles_m * tiles_n + kXcds - 1) / kXcds;
    const dim3 grid((unsigned)(per_xcd * kXcds));
    hipLaunchKernelGGL(gemm_kernel, grid, dim3(GT), 0, s, prepared,
                       reinterpret_cast<const uint32_t*>(prepared + sz_offset(n, k)),
                       static_cast<const uint16_t*>(X), St, m_pad, Y, y_bf16 ? 1 : 0, (int)m,
                       (int)n, (int)k, tiles_m, tiles_n, group_m, per_xcd);
    return hipGetLastError();
}

}  // namespace w4
