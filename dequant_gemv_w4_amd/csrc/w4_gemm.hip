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
constexpr int XS = BK + 8;               // bf16 per LDS row of the X tile (16-byte pad)

__device__ __forceinline__ uint32_t bf16_bits_rne(float f) {
    const uint32_t u = __float_as_uint(f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ bf16x8_t as_bf16x8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
    const u32x4_t v = {a, b, c, d};
    return __builtin_bit_cast(bf16x8_t, v);
}

// ---- pre-pass: S^T[g][m] = sum of x[m, 128g .. 128g+127] by the MFMA sequence of the GEMM
__global__ __launch_bounds__(256) void xsum_kernel(const uint16_t* __restrict__ X, int M, int K,
                                                   float* __restrict__ St, int m_pad) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int Kg = K / kGroup;
    const int tile = blockIdx.x * 4 + wave;      // (m tile, group) pairs, m fastest
    const int n_mt = (M + 31) / 32;
    if (tile >= n_mt * Kg) return;
    const int mt = tile % n_mt;
    const int g = tile / n_mt;
    const int row = mt * 32 + (lane & 31);
    const int h = lane >> 5;
    const bf16x8_t ones = as_bf16x8(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u);
    f32x16_t acc;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
        uint4 v = make_uint4(0, 0, 0, 0);
        if (row < M)
            v = *reinterpret_cast<const uint4*>(X + (int64_t)row * K + g * kGroup + 64 * h + 8 * s);
        const bf16x8_t a = as_bf16x8(v.x, v.y, v.z, v.w);
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
            const int r = mt * 32 + 8 * (v >> 2) + 4 * h + (v & 3);
            St[(int64_t)g * m_pad + r] = acc[v];
        }
    }
}

__global__ __launch_bounds__(GT) void gemm_kernel(const uint8_t* __restrict__ wq,
                                                  const uint32_t* __restrict__ sz,
                                                  const uint16_t* __restrict__ X,
                                                  const float* __restrict__ St, int m_pad,
                                                  void* __restrict__ Y, int y_bf16, int M, int N,
                                                  int K) {
    __shared__ __attribute__((aligned(16))) uint16_t xs[2][BM * XS];
    __shared__ __attribute__((aligned(16))) float ss[2][BM];

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int wm = wave >> 2;        // 0..1: rows 64wm..
    const int wn = wave & 3;         // 0..3: columns 64wn..
    const int n0 = blockIdx.x * BN;
    const int m0 = blockIdx.y * BM;
    const int Kg = K / kGroup;
    const int64_t row_bytes = K / 2;
    const int h = lane >> 5;
    const int l32 = lane & 31;

    uint32_t nib_mask, bias_bits;
    asm volatile("s_mov_b32 %0, 0x000F000F" : "=s"(nib_mask));
    asm volatile("v_mov_b32 %0, 0x43004300" : "=v"(bias_bits));

    // weight rows of this lane (one per N tile), clamped inside the matrix
    int wrow[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) wrow[j] = min(n0 + 64 * wn + 32 * j + l32, N - 1);

    // ---- staging of one group: X tile (global -> registers -> LDS), S, weights, scale/zero
    uint4 xr[4];             // 512 threads x 4 x 16 B = the 32 KB X tile
    u32x4_t wr[2][2];        // [N tile][half of the 32 bytes] codes of the next group
    uint32_t szr[2];
    float sr = 0.0f;
    auto load_group = [&](int kg) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int idx = tid + i * GT;       // 0..2047: 128 rows x 16 pieces
            const int r = idx >> 4;
            const int c = (idx & 15) * 8;
            xr[i] = make_uint4(0, 0, 0, 0);
            if (m0 + r < M)
                xr[i] = *reinterpret_cast<const uint4*>(X + (int64_t)(m0 + r) * K + kg * BK + c);
        }
        if (tid < BM) sr = St[(int64_t)kg * m_pad + m0 + tid];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const uint8_t* p = wq + (int64_t)wrow[j] * row_bytes + kg * (BK / 2) + 32 * h;
            wr[j][0] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
            wr[j][1] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p + 16));
            szr[j] = sz[sz_index(wrow[j], kg, Kg)];
        }
    };
    auto store_group = [&](int buf) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int idx = tid + i * GT;
            const int r = idx >> 4;
            const int c = (idx & 15) * 8;
            *reinterpret_cast<uint4*>(&xs[buf][r * XS + c]) = xr[i];
        }
        if (tid < BM) ss[buf][tid] = sr;
    };

    f32x16_t acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = (f32x16_t){};

    load_group(0);
    store_group(0);
    u32x4_t wc[2][2];
    uint32_t szc[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        wc[j][0] = wr[j][0];
        wc[j][1] = wr[j][1];
        szc[j] = szr[j];
    }
    __syncthreads();

    for (int kg = 0; kg < Kg; ++kg) {
        const int buf = kg & 1;
        if (kg + 1 < Kg) load_group(kg + 1);

        // ---- eight MFMA steps over the group into fresh accumulators P
        f32x16_t P[2][2];
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            bf16x8_t a[2], b[2];
#pragma unroll
            for (int i = 0; i < 2; ++i)
                a[i] = *reinterpret_cast<const bf16x8_t*>(
                    &xs[buf][(64 * wm + 32 * i + l32) * XS + 64 * h + 8 * s]);
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
                const float4 s4 = *reinterpret_cast<const float4*>(
                    &ss[buf][64 * wm + 32 * i + 8 * q + 4 * h]);
                const float sv[4] = {s4.x, s4.y, s4.z, s4.w};
#pragma unroll
                for (int r = 0; r < 4; ++r)
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        const int v = 4 * q + r;
                        acc[i][j][v] = fmaf(sc[j], fmaf(-zb[j], sv[r], P[i][j][v]), acc[i][j][v]);
                    }
            }
        }

        if (kg + 1 < Kg) {
            store_group(buf ^ 1);
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                wc[j][0] = wr[j][0];
                wc[j][1] = wr[j][1];
                szc[j] = szr[j];
            }
        }
        __syncthreads();
    }

#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int r = m0 + 64 * wm + 32 * i + 8 * (v >> 2) + 4 * h + (v & 3);
                const int c = n0 + 64 * wn + 32 * j + l32;
                if (r < M && c < N) {
                    const int64_t o = (int64_t)r * N + c;
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
    const dim3 grid((unsigned)((n + BN - 1) / BN), (unsigned)((m + BM - 1) / BM));
    hipLaunchKernelGGL(gemm_kernel, grid, dim3(GT), 0, s, prepared,
                       reinterpret_cast<const uint32_t*>(prepared + sz_offset(n, k)),
                       static_cast<const uint16_t*>(X), St, m_pad, Y, y_bf16 ? 1 : 0, (int)m,
                       (int)n, (int)k);
    return hipGetLastError();
}

}  // namespace w4
