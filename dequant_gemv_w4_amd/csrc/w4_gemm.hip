// Prefill-sized W4A16 product Y = X * w_hat^T on bf16 MFMA.
//
// Prefill multiplies large matrices, so it is bound by the matrix units, and a
// weight-only format has to turn the 4-bit codes back into 16-bit values
// before they reach them (page "LLM Quantization Architecture in Depth" ›
// "Why fewer bits make decoding faster"; page "Quantization" › "The idea in
// one minute").  Each K step covers exactly one quantization group (128
// inputs), so one scale and one zero per weight row apply to the whole tile:
// w_hat = bf16((code - zero) * scale16) is written to LDS and fed to
// v_mfma_f32_32x32x16_bf16 with f32 accumulation.
//
// Tiling: 128 x 128 output tile per 256-thread workgroup, each wave a 64 x 64
// quadrant made of 2 x 2 MFMA tiles of 32 x 32; LDS rows are padded by 16
// bytes to spread the banks of the 16-byte operand reads.
//
// MFMA operand order: lane l supplies row (l % 32) of its operand and the
// eight k values (l / 32) * 8 .. +7 of the current 16-wide k step, the same k
// assignment for both operands, so each output element is a dot product over
// matching k.  The 32 x 32 f32 result sits in lane l as column (l % 32) and
// rows 8 * (v / 4) + 4 * (l / 32) + (v % 4) for element v = 0..15.
#include "w4_internal.h"

namespace w4 {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;

constexpr int BM = 128;
constexpr int BN = 128;
constexpr int BK = kGroup;
constexpr int LDS_STRIDE = BK + 8;  // bf16 elements per LDS row

__device__ __forceinline__ uint32_t bf16_bits_rne(float f) {
    const uint32_t u = __float_as_uint(f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__global__ __launch_bounds__(256) void gemm_kernel(const uint8_t* __restrict__ wq,
                                                   const uint32_t* __restrict__ sz,
                                                   const uint16_t* __restrict__ X,
                                                   void* __restrict__ Y, int y_bf16, int M, int N,
                                                   int K) {
    __shared__ __attribute__((aligned(16))) uint16_t xs[BM * LDS_STRIDE];
    __shared__ __attribute__((aligned(16))) uint16_t ws[BN * LDS_STRIDE];

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int n0 = blockIdx.x * BN;
    const int m0 = blockIdx.y * BM;
    const int wm = (wave >> 1) * 64;
    const int wn = (wave & 1) * 64;
    const int Kg = K / kGroup;
    const int64_t row_bytes = K / 2;

    f32x16_t acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

    for (int kg = 0; kg < Kg; ++kg) {
        // X tile: 128 rows x 128 bf16 (16 x 16-byte pieces per row)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int idx = tid + i * 256;
            const int r = idx >> 4;
            const int c = (idx & 15) * 8;
            uint4 v = make_uint4(0, 0, 0, 0);
            if (m0 + r < M)
                v = *reinterpret_cast<const uint4*>(X + (int64_t)(m0 + r) * K + kg * BK + c);
            *reinterpret_cast<uint4*>(xs + r * LDS_STRIDE + c) = v;
        }
        // W tile: row r = tid / 2, half h = tid % 2 holds 64 codes (32 bytes)
        {
            const int r = tid >> 1;
            const int h = tid & 1;
            const int row = n0 + r;
            uint4 a = make_uint4(0, 0, 0, 0), b = make_uint4(0, 0, 0, 0);
            uint32_t szv = 0;
            if (row < N) {
                const uint4* p = reinterpret_cast<const uint4*>(wq + (int64_t)row * row_bytes +
                                                                kg * (BK / 2) + h * 32);
                a = p[0];
                b = p[1];
                szv = sz[sz_index(row, kg, Kg)];
            }
            const float s = (float)__builtin_bit_cast(_Float16, (uint16_t)(szv & 0xFFFFu));
            const float z = (float)((szv >> 16) & 0xFFu) - 128.0f;
            const uint32_t words[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
            uint32_t out[32];
#pragma unroll
            for (int t = 0; t < 8; ++t) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float ce = (float)((words[t] >> (4 * j)) & 0xFu);
                    const float co = (float)((words[t] >> (16 + 4 * j)) & 0xFu);
                    out[4 * t + j] = bf16_bits_rne((ce - z) * s) | (bf16_bits_rne((co - z) * s) << 16);
                }
            }
            uint4* dst = reinterpret_cast<uint4*>(ws + r * LDS_STRIDE + h * 64);
#pragma unroll
            for (int q = 0; q < 8; ++q)
                dst[q] = make_uint4(out[4 * q], out[4 * q + 1], out[4 * q + 2], out[4 * q + 3]);
        }
        __syncthreads();

#pragma unroll
        for (int kk = 0; kk < BK; kk += 16) {
            bf16x8_t av[2], bv[2];
            const int koff = kk + (lane >> 5) * 8;
#pragma unroll
            for (int i = 0; i < 2; ++i)
                av[i] = *reinterpret_cast<const bf16x8_t*>(xs + (wm + i * 32 + (lane & 31)) * LDS_STRIDE + koff);
#pragma unroll
            for (int j = 0; j < 2; ++j)
                bv[j] = *reinterpret_cast<const bf16x8_t*>(ws + (wn + j * 32 + (lane & 31)) * LDS_STRIDE + koff);
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[i], bv[j], acc[i][j], 0, 0, 0);
        }
        __syncthreads();
    }

#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int r = m0 + wm + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
                const int c = n0 + wn + j * 32 + (lane & 31);
                if (r < M && c < N) {
                    const int64_t o = (int64_t)r * N + c;
                    if (y_bf16)
                        static_cast<uint16_t*>(Y)[o] = (uint16_t)bf16_bits_rne(acc[i][j][v]);
                    else
                        static_cast<float*>(Y)[o] = acc[i][j][v];
                }
            }
}

}  // namespace

hipError_t launch_gemm(const uint8_t* prepared, int64_t n, int64_t k, const void* X, int64_t m,
                       void* Y, bool y_bf16, hipStream_t s) {
    const dim3 grid((unsigned)((n + BN - 1) / BN), (unsigned)((m + BM - 1) / BM));
    hipLaunchKernelGGL(gemm_kernel, grid, dim3(256), 0, s, prepared,
                       reinterpret_cast<const uint32_t*>(prepared + sz_offset(n, k)),
                       static_cast<const uint16_t*>(X), Y, y_bf16 ? 1 : 0, (int)m, (int)n, (int)k);
    return hipGetLastError();
}

}  // namespace w4
