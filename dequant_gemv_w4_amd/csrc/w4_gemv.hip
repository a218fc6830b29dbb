// Fused dequantizing matrix-vector product for decode (1 <= M <= 16).
//
// Computes y[m, n] = sum_g scale16[n, g] * (sum_{k in g} q[n, k] x[m, k]
//                                          - zero[n, g] * sum_{k in g} x[m, k])
// (page "Weight quantization", section "How it works": one multiply per group;
// section "Code": the group loop of the dot routine) without writing any
// dequantized weight to memory.  Decode reads every weight once, so the kernel
// is a stream over HBM (page "LLM Quantization Architecture in Depth" › "Why
// fewer bits make decoding faster").
//
// Mapping (gfx950, wave64):
//   * lane u of the workgroup owns the 16-byte slice u of every row (32
//     inputs, a quarter of a group); its x values stay in registers as bf16
//     pairs for the whole workgroup, so each row costs one 16-byte load per
//     lane and a wave load covers 1 KiB of contiguous weights;
//   * a workgroup holds ceil(K/2048) waves and walks rows_per_wg rows, four at
//     a time, prefetching the next four rows while it computes the current;
//   * unpack: (word >> 4j) & 0x000F000F | 0x43004300 turns the two codes of an
//     input pair into the bf16 values 128+q, and v_dot2_f32_bf16 multiplies the
//     pair by the matching x pair and accumulates in f32: D = sum (128+q)*x.
//     The slice sum S = sum x is computed once per workgroup by the same
//     instruction sequence with the pair (1, 1), so the slice's share of the
//     group term is scale16 * (D - (128 + zero) * S) = scale16 * (sum q*x -
//     zero * sum x).  Because scaling by 128 commutes with rounding, a slice
//     whose codes are all 0 gives D = 128*S exactly and contributes exactly 0;
//     a one-hot x gives exactly (q - zero) * scale16;
//   * reduction: across lanes with a transposed butterfly over the four rows,
//     then across waves through LDS; no atomics, so results are deterministic.
// Binary32 activations are split into two bf16 parts (hi = bf16(x),
// lo = bf16(x - hi)) that are accumulated separately and added at the end.
#include "w4_internal.h"

namespace w4 {
namespace {

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// one 16-byte weight slice, marked non-temporal: every byte is read exactly once
__device__ __forceinline__ u32x4_t load_stream(const u32x4_t* p) { return __builtin_nontemporal_load(p); }

constexpr int kRowsPerStep = 4;
constexpr int kMaxThreads = 1024;

__device__ __forceinline__ float dot2(uint32_t w, uint32_t x, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w),
                                           __builtin_bit_cast(bf16x2_t, x), acc, false);
}

__device__ __forceinline__ uint32_t bf16_bits_rne(float f) {
    const uint32_t u = __float_as_uint(f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// sum of the 32 bf16 values held as 16 pairs, accumulated by the same dot2
// chain (same order, same instruction) that the weights use, with the pair (1, 1)
__device__ __forceinline__ float pair_sum(const uint32_t (&p)[16]) {
    float d = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) d = dot2(0x3F803F80u, p[i], d);
    return d;
}

template <int MT, bool XF32, int SPT, int MAXT>
__global__ __launch_bounds__(MAXT) void gemv_kernel(const u32x4_t* __restrict__ wq,
                                                    const uint32_t* __restrict__ sz,
                                                    const void* __restrict__ xv,
                                                    void* __restrict__ yv, int y_bf16, int N,
                                                    int K, int M, int rows_per_wg) {
    constexpr int XE = XF32 ? 2 * MT : MT;  // bf16 operand rows
    extern __shared__ float red[];          // [waves][rows_per_wg][XE]

    const int S = K >> 5;
    const int Kg = K >> 7;
    const int T = blockDim.x;
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int n_waves = T >> 6;

    // slice j of this lane is threadIdx.x + j*T (16 bytes of every row)
    int sl[SPT];
    bool act[SPT];
#pragma unroll
    for (int j = 0; j < SPT; ++j) {
        sl[j] = threadIdx.x + j * T;
        act[j] = sl[j] < S;
    }

    // ---- x slices in registers, plus sum(x) of each slice
    uint32_t xr[SPT][XE][16];
    float sx[SPT][XE];
#pragma unroll
    for (int j = 0; j < SPT; ++j) {
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            const bool ok = act[j] && m < M;
            if constexpr (XF32) {
                const float4* px = reinterpret_cast<const float4*>(
                    static_cast<const float*>(xv) + (int64_t)m * K + (int64_t)sl[j] * 32);
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    const float4 f = ok ? px[q] : make_float4(0.f, 0.f, 0.f, 0.f);
                    const float v[4] = {f.x, f.y, f.z, f.w};
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const uint32_t h0 = bf16_bits_rne(v[2 * h]);
                        const uint32_t h1 = bf16_bits_rne(v[2 * h + 1]);
                        const uint32_t l0 = bf16_bits_rne(v[2 * h] - __uint_as_float(h0 << 16));
                        const uint32_t l1 = bf16_bits_rne(v[2 * h + 1] - __uint_as_float(h1 << 16));
                        xr[j][2 * m][2 * q + h] = h0 | (h1 << 16);
                        xr[j][2 * m + 1][2 * q + h] = l0 | (l1 << 16);
                    }
                }
            } else {
                const uint4* px = reinterpret_cast<const uint4*>(
                    static_cast<const uint16_t*>(xv) + (int64_t)m * K + (int64_t)sl[j] * 32);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const uint4 v = ok ? px[q] : make_uint4(0, 0, 0, 0);
                    xr[j][m][4 * q + 0] = v.x;
                    xr[j][m][4 * q + 1] = v.y;
                    xr[j][m][4 * q + 2] = v.z;
                    xr[j][m][4 * q + 3] = v.w;
                }
            }
        }
#pragma unroll
        for (int e = 0; e < XE; ++e) sx[j][e] = pair_sum(xr[j][e]);
    }

    const int r0 = blockIdx.x * rows_per_wg;
    const int r_end = min(N, r0 + rows_per_wg);
    const bool up32 = (lane & 32) != 0;
    const bool up16 = (lane & 16) != 0;

    const u32x4_t zero4 = {0u, 0u, 0u, 0u};
    u32x4_t wcur[kRowsPerStep][SPT];
    uint32_t scur[kRowsPerStep][SPT];
#pragma unroll
    for (int rr = 0; rr < kRowsPerStep; ++rr) {
        const int row = r0 + rr;
#pragma unroll
        for (int j = 0; j < SPT; ++j) {
            const bool ok = act[j] && row < r_end;
            wcur[rr][j] = ok ? load_stream(wq + (int64_t)row * S + sl[j]) : zero4;
            scur[rr][j] = ok ? sz[(int64_t)row * Kg + (sl[j] >> 2)] : 0u;
        }
    }

    for (int rb = r0; rb < r_end; rb += kRowsPerStep) {
        // prefetch the next four rows
        u32x4_t wnext[kRowsPerStep][SPT];
        uint32_t snext[kRowsPerStep][SPT];
#pragma unroll
        for (int rr = 0; rr < kRowsPerStep; ++rr) {
            const int row = rb + kRowsPerStep + rr;
#pragma unroll
            for (int j = 0; j < SPT; ++j) {
                const bool ok = act[j] && row < r_end;
                wnext[rr][j] = ok ? load_stream(wq + (int64_t)row * S + sl[j]) : zero4;
                snext[rr][j] = ok ? sz[(int64_t)row * Kg + (sl[j] >> 2)] : 0u;
            }
        }

        float acc[kRowsPerStep][XE];
#pragma unroll
        for (int rr = 0; rr < kRowsPerStep; ++rr) {
#pragma unroll
            for (int e = 0; e < XE; ++e) acc[rr][e] = 0.0f;
#pragma unroll
            for (int j = 0; j < SPT; ++j) {
                uint32_t pr[16];
#pragma unroll
                for (int t = 0; t < 4; ++t)
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        pr[4 * t + q] = ((wcur[rr][j][t] >> (4 * q)) & 0x000F000Fu) | 0x43004300u;
                const float s = (float)__builtin_bit_cast(_Float16, (uint16_t)(scur[rr][j] & 0xFFFFu));
                const float zb = (float)(((scur[rr][j] >> 16) & 0xFFu) + 128u);
#pragma unroll
                for (int e = 0; e < XE; ++e) {
                    float d = 0.0f;
#pragma unroll
                    for (int i = 0; i < 16; ++i) d = dot2(pr[i], xr[j][e][i], d);
                    acc[rr][e] = fmaf(s, fmaf(-zb, sx[j][e], d), acc[rr][e]);
                }
            }
        }

        // transposed butterfly: lane keeps row 2*up32 + up16, summed over the wave
#pragma unroll
        for (int e = 0; e < XE; ++e) {
            float k0 = up32 ? acc[2][e] : acc[0][e];
            float s0 = up32 ? acc[0][e] : acc[2][e];
            float k1 = up32 ? acc[3][e] : acc[1][e];
            float s1 = up32 ? acc[1][e] : acc[3][e];
            k0 += __shfl_xor(s0, 32);
            k1 += __shfl_xor(s1, 32);
            float k = up16 ? k1 : k0;
            const float sd = up16 ? k0 : k1;
            k += __shfl_xor(sd, 16);
            k += __shfl_xor(k, 8);
            k += __shfl_xor(k, 4);
            k += __shfl_xor(k, 2);
            k += __shfl_xor(k, 1);
            if ((lane & 15) == 0) {
                const int rloc = rb - r0 + (up32 ? 2 : 0) + (up16 ? 1 : 0);
                red[(wave * rows_per_wg + rloc) * XE + e] = k;
            }
        }
#pragma unroll
        for (int rr = 0; rr < kRowsPerStep; ++rr)
#pragma unroll
            for (int j = 0; j < SPT; ++j) {
                wcur[rr][j] = wnext[rr][j];
                scur[rr][j] = snext[rr][j];
            }
    }
    __syncthreads();

    const int rows_here = r_end - r0;
    for (int t = threadIdx.x; t < rows_here * MT; t += T) {
        const int rloc = t / MT;
        const int m = t - rloc * MT;
        if (m >= M) continue;
        float v = 0.0f;
        for (int w = 0; w < n_waves; ++w) {
            const float* p = red + (w * rows_per_wg + rloc) * XE;
            if constexpr (XF32)
                v += p[2 * m] + p[2 * m + 1];
            else
                v += p[m];
        }
        const int64_t o = (int64_t)m * N + r0 + rloc;
        if (y_bf16)
            static_cast<uint16_t*>(yv)[o] = (uint16_t)bf16_bits_rne(v);
        else
            static_cast<float*>(yv)[o] = v;
    }
}

struct GemvArgs {
    const u32x4_t* wq;
    const uint32_t* sz;
    const void* x;
    void* y;
    int y_bf16, n, k, m, rows;
};

template <int MT, bool XF32, int SPT, int MAXT>
hipError_t launch_one(const GemvArgs& a, dim3 grid, dim3 block, size_t shmem, hipStream_t s) {
    hipLaunchKernelGGL((gemv_kernel<MT, XF32, SPT, MAXT>), grid, block, shmem, s, a.wq, a.sz, a.x,
                       a.y, a.y_bf16, a.n, a.k, a.m, a.rows);
    return hipGetLastError();
}

// Instantiated variants (MT = rows of x per launch, SPT = 16-byte slices per lane):
//   M=1 bf16:          SPT 1, up to 1024 threads (K <= 32768)
//   otherwise:         up to 512 threads; SPT 1 for K <= 16384, SPT 2 up to 32768;
//                      MT up to 8 (bf16, SPT 1), 2 (bf16, SPT 2), 3 (f32, SPT 1), 1 (f32, SPT 2)
//                      so that the x registers fit the 256-VGPR budget of a 512-thread group.
int max_mt(bool x_f32, int spt) {
    if (!x_f32) return spt == 1 ? 8 : 2;
    return spt == 1 ? 3 : 1;
}

hipError_t dispatch(bool x_f32, int spt, int mt, const GemvArgs& a, dim3 grid, dim3 block,
                    size_t shmem, hipStream_t s) {
#define W4_CASE(MTV, XF, SP, MX) \
    if (mt == MTV && x_f32 == XF && spt == SP) return launch_one<MTV, XF, SP, MX>(a, grid, block, shmem, s);
    if (!x_f32 && mt == 1 && block.x > 512) return launch_one<1, false, 1, 1024>(a, grid, block, shmem, s);
    W4_CASE(1, false, 1, 512) W4_CASE(2, false, 1, 512) W4_CASE(3, false, 1, 512)
    W4_CASE(4, false, 1, 512) W4_CASE(5, false, 1, 512) W4_CASE(6, false, 1, 512)
    W4_CASE(7, false, 1, 512) W4_CASE(8, false, 1, 512)
    W4_CASE(1, false, 2, 512) W4_CASE(2, false, 2, 512)
    W4_CASE(1, true, 1, 512) W4_CASE(2, true, 1, 512) W4_CASE(3, true, 1, 512)
    W4_CASE(1, true, 2, 512)
#undef W4_CASE
    return hipErrorInvalidValue;
}

int rows_per_workgroup(int64_t n) {
    static const int forced = [] {
        const char* e = getenv("W4A16_GEMV_ROWS");
        return e ? atoi(e) : 0;
    }();
    int r = forced > 0 ? forced : (int)(n / 512);
    r = r / kRowsPerStep * kRowsPerStep;
    if (r < kRowsPerStep) r = kRowsPerStep;
    if (r > 64) r = 64;
    return r;
}

}  // namespace

hipError_t launch_gemv(const uint8_t* prepared, int64_t n, int64_t k, const void* x, bool x_f32,
                       int64_t m, void* y, bool y_bf16, hipStream_t s) {
    const int S = (int)(k / 32);
    const int rows = rows_per_workgroup(n);
    const dim3 grid((unsigned)((n + rows - 1) / rows));
    GemvArgs a;
    a.wq = reinterpret_cast<const u32x4_t*>(prepared);
    a.sz = reinterpret_cast<const uint32_t*>(prepared + sz_offset(n, k));
    a.y_bf16 = y_bf16 ? 1 : 0;
    a.n = (int)n;
    a.k = (int)k;
    a.rows = rows;
    const bool wide = !x_f32 && m == 1;      // one slice per lane, up to 1024 threads
    const int spt = wide ? 1 : (S <= 512 ? 1 : 2);
    const int waves = (S + 64 * spt - 1) / (64 * spt);
    const dim3 block(64 * waves);
    const int mt_max = max_mt(x_f32, spt);
    for (int64_t m0 = 0; m0 < m; m0 += mt_max) {
        const int mc = (int)((m - m0) < mt_max ? (m - m0) : mt_max);
        const int xe = x_f32 ? 2 * mc : mc;
        const size_t shmem = (size_t)waves * rows * xe * sizeof(float);
        a.x = x_f32 ? (const void*)(static_cast<const float*>(x) + m0 * k)
                    : (const void*)(static_cast<const uint16_t*>(x) + m0 * k);
        a.y = y_bf16 ? (void*)(static_cast<uint16_t*>(y) + m0 * n)
                     : (void*)(static_cast<float*>(y) + m0 * n);
        a.m = mc;
        hipError_t err = dispatch(x_f32, spt, mc, a, grid, block, shmem, s);
        if (err != hipSuccess) return err;
    }
    return hipSuccess;
}

}  // namespace w4
