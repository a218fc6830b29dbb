// W8A8 for prefill, in FP8 E4M3 or INT8: per-row quantization and the product on the
// matrix cores.
//
// Prefill is bound by the matrix units, so a weight-only format barely speeds it up; the
// arithmetic itself has to be narrower, with activations quantized too: W8A8 in FP8 or
// INT8 (page "LLM Quantization Architecture in Depth" › "Why fewer bits make decoding
// faster" and "Number formats, scales and granularity": E4M3 for weights and activations,
// largest value 448; dynamic per-token activation scales).
//
// Quantization (w8_quantize_rows_kernel, one workgroup per row), in binary64 as in the
// page's program ("Quantization" › "Code": per-tensor / per-channel absmax scales):
//   * E4M3: the scale is the row's largest magnitude over 448 (1 for an all-zero row);
//     each value divided by it is capped at 448 and rounded, halves to even, on the grid of
//     3 mantissa bits of its binary exponent (exponents below -6 use the grid of -6).
//     Codes are OCP E4M3 bytes (sign, exponent with bias 7, mantissa), the byte the gfx950
//     matrix cores take as format 0; a value that rounds to zero keeps its sign;
//   * INT8: the step is the largest magnitude over 127; codes are the quotients rounded to
//     the nearest integer, halves to even, clamped to [-128, 127].
// The scale is stored as binary32.  The kernel gives the codes of that binary64 arithmetic
// while rounding most values in binary32 (e4m3_byte_recip, int8_byte_recip).
//
// Product: Y[m, n] = sx[m] * sw[n] * sum_k qx[m, k] * qw[n, k].  FP8 runs on
// v_mfma_scale_f32_32x32x64_f8f6f4 (block scales left at 2^0) with binary32 accumulation
// (every product of two E4M3 values is exact in binary32); INT8 on v_mfma_i32_32x32x32_i8
// with exact int32 sums.  w8_gemm_ring_kernel (the default for both): 512 threads per
// 128 x 256 output tile, wave (wm, wn) owns 64 x 64 as 2 x 2 MFMA tiles, a K step is 128
// inputs loaded straight into a three-stage LDS ring two steps ahead.
// In LDS, 16-byte chunk c of row r sits at slot
// c ^ ((r / 2) & 7) (w8_slot), so the operand reads of 16 consecutive rows, which share a
// cycle, touch 16 different 16-byte bank groups.  For FP8 a lane
// supplies row (lane % 32) and the 32 inputs 32 * (lane / 32) .. +31 of a 64-input MFMA
// step, the same inputs for both operands, so each output is a dot product over matching
// inputs whatever order the unit sums them in.
#include "w4_internal.h"

namespace w4 {
namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef int v8i_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kQT = 256;          // threads of a quantizer workgroup (one row)
constexpr double kFp8Max = 448.0;

// E4M3 rounding of a magnitude m <= 448: u = m in units of its grid step 2^(ex-3)
// (ex = its binary exponent, at least -6); scaling by a power of two is exact
__device__ __forceinline__ double e4m3_units(double m, int& ex) {
    int e = 0;
    (void)frexp(m, &e);                            // m = f * 2^e, f in [0.5, 1)
    ex = max(e - 1, -6);
    return ldexp(m, 3 - ex);
}

// byte of the rounded magnitude q * 2^(ex-3) with the given sign bit
__device__ __forceinline__ uint32_t e4m3_encode(uint32_t sign, double q, int ex) {
    const double r = fmin(ldexp(q, ex - 3), kFp8Max);
    if (r == 0.0) return sign;
    if (r < 0x1p-6) return sign | (uint32_t)(r * 512.0);   // subnormal: r = m * 2^-9
    int E = 0;
    const double f = frexp(r, &E);                 // r = (2f) * 2^(E-1)
    return sign | ((uint32_t)(E + 6) << 3) | (uint32_t)((2.0 * f - 1.0) * 8.0);
}

// E4M3 byte of a binary64 quotient t (the rounding described at the top of the file)
__device__ __forceinline__ uint32_t e4m3_byte(double t) {
    if (t == 0.0) return 0u;
    int ex = 0;
    const double u = e4m3_units(fmin(fabs(t), kFp8Max), ex);
    return e4m3_encode(t < 0.0 ? 0x80u : 0u, rint(u), ex);
}

// The codes without binary64 arithmetic per value.  r32 is 1 / s (correctly rounded in
// binary64, then to binary32), so t = v * r32 in binary32 is within 2^-23 relative of v / s
// and of its correctly rounded binary64 quotient.  In grid units (below 16 for E4M3, below
// 128 for INT8) the two differ by less than 2^-19 and 2^-16; where t lies more than 2^-17
// (E4M3) or 2^-13 (INT8) from a rounding boundary both give the same code.  The other
// values (windows of 2^-16 and 2^-12 per unit: about 1.5 in 10^5 and 2.4 in 10^4),
// non-finite ones and scales outside [2^-100, 2^100] take the binary64 quotient.  An E4M3
// quotient below 2^-12 rounds to a zero with the sign of v.
__device__ __forceinline__ bool clear_of_half(float u, float margin) {
    return fabsf(__builtin_amdgcn_fractf(u) - 0.5f) > margin;
}

__device__ __forceinline__ uint32_t e4m3_byte_recip(float v, double s, float r32, bool rcp_ok) {
    if (rcp_ok) {
        const float m = fabsf(v * r32);
        const uint32_t sign = v < 0.0f ? 0x80u : 0u;
        if (m < 0x1p-12f) return sign;
        const int ex = max(__builtin_amdgcn_frexp_expf(m) - 1, -6);   // binary exponent
        const float u = ldexpf(m, 3 - ex);                              // in units of 2^(ex-3)
        // below 448 * (1 + 2^-22), so u < 14.5 at ex = 8: no value rounds past 448
        if (clear_of_half(u, 0x1p-17f)) {
            // the byte of q * 2^(ex-3): exponent field ex + 7 and mantissa q - 8 for
            // 8 <= q <= 16 (q = 16 carries into the exponent), the subnormal q < 8 at ex = -6
            return sign | (uint32_t)(8 * ex + 48 + (int)rintf(u));
        }
    }
    return e4m3_byte((double)v / s);
}

template <bool IN_BF16>
__device__ __forceinline__ void load8(const void* a, int64_t i, float* v) {
    if constexpr (IN_BF16) {
        const u32x4_t w = *reinterpret_cast<const u32x4_t*>(static_cast<const uint16_t*>(a) + i);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            v[2 * q] = __uint_as_float(w[q] << 16);
            v[2 * q + 1] = __uint_as_float(w[q] & 0xFFFF0000u);
        }
    } else {
        const u32x4_t w0 = *reinterpret_cast<const u32x4_t*>(static_cast<const float*>(a) + i);
        const u32x4_t w1 = *reinterpret_cast<const u32x4_t*>(static_cast<const float*>(a) + i + 4);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            v[q] = __uint_as_float(w0[q]);
            v[4 + q] = __uint_as_float(w1[q]);
        }
    }
}

// INT8 (symmetric, page "Quantization" › "How it really works" and "Code"): the step is the
// row's largest magnitude over 127 (1 for an all-zero row), in binary64; code = the
// binary64 quotient rounded to the nearest integer, halves to even, clamped to [-128, 127].
__device__ __forceinline__ uint32_t int8_byte(double t) {
    const double q = fmin(fmax(rint(t), -128.0), 127.0);
    return (uint32_t)(uint8_t)(int8_t)(int)q;
}

__device__ __forceinline__ uint32_t int8_byte_recip(float v, double s, float r32, bool rcp_ok) {
    const float t = v * r32;
    if (rcp_ok && clear_of_half(t, 0x1p-13f))   // |t| <= 127 (1 + 2^-22): no clamp needed
        return (uint32_t)(uint8_t)(int8_t)(int)rintf(t);
    return int8_byte((double)v / s);
}

// values per thread kept in registers between the two steps when K <= kQT * kQVals
constexpr int kQVals = 32;

template <bool INT8>
__device__ __forceinline__ uint2 w8_codes8(const float* v, double s, float rs, bool rcp_ok) {
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        if constexpr (INT8) {
            lo |= int8_byte_recip(v[q], s, rs, rcp_ok) << (8 * q);
            hi |= int8_byte_recip(v[4 + q], s, rs, rcp_ok) << (8 * q);
        } else {
            lo |= e4m3_byte_recip(v[q], s, rs, rcp_ok) << (8 * q);
            hi |= e4m3_byte_recip(v[4 + q], s, rs, rcp_ok) << (8 * q);
        }
    }
    return make_uint2(lo, hi);
}

// One workgroup per row.  Rows of up to kQT * kQVals values are loaded once, all loads
// issued before the first is used, and kept in registers for the second step; longer rows
// are read twice in a loop.
template <bool IN_BF16, bool INT8>
__global__ __launch_bounds__(kQT) void w8_quantize_rows_kernel(const void* __restrict__ a,
                                                                int64_t K,
                                                                uint8_t* __restrict__ codes,
                                                                float* __restrict__ scales,
                                                                uint32_t* __restrict__ status) {
    __shared__ float wmax[kQT / 64];
    const int64_t row = blockIdx.x;
    const void* src = IN_BF16 ? (const void*)(static_cast<const uint16_t*>(a) + row * K)
                              : (const void*)(static_cast<const float*>(a) + row * K);
    uint8_t* dst = codes + row * K;
    const bool cached = K <= (int64_t)kQT * kQVals;
    float vc[kQVals];
    float amax = 0.0f;
    bool finite = true;
    if (cached) {
#pragma unroll
        for (int c = 0; c < kQVals / 8; ++c) {
            const int64_t i = (int64_t)threadIdx.x * 8 + (int64_t)c * kQT * 8;
            if (i < K) {
                load8<IN_BF16>(src, i, &vc[8 * c]);
            } else {
#pragma unroll
                for (int q = 0; q < 8; ++q) vc[8 * c + q] = 0.0f;
            }
        }
#pragma unroll
        for (int q = 0; q < kQVals; ++q) {
            finite &= isfinite(vc[q]);
            amax = fmaxf(amax, fabsf(vc[q]));
        }
    } else {
        for (int64_t i = (int64_t)threadIdx.x * 8; i < K; i += kQT * 8) {
            float v[8];
            load8<IN_BF16>(src, i, v);
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                finite &= isfinite(v[q]);
                amax = fmaxf(amax, fabsf(v[q]));
            }
        }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
    if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = amax;
    if (!finite && status) atomicOr(status, 1u);
    __syncthreads();
    amax = wmax[0];
#pragma unroll
    for (int w = 1; w < kQT / 64; ++w) amax = fmaxf(amax, wmax[w]);
    const double s = amax == 0.0f ? 1.0 : (double)amax / (INT8 ? 127.0 : kFp8Max);
    if (threadIdx.x == 0) scales[row] = (float)s;
    const float rs = (float)(1.0 / s);
    const bool rcp_ok = s >= 0x1p-100 && s <= 0x1p100;
    if (cached) {
#pragma unroll
        for (int c = 0; c < kQVals / 8; ++c) {
            const int64_t i = (int64_t)threadIdx.x * 8 + (int64_t)c * kQT * 8;
            if (i < K) *reinterpret_cast<uint2*>(dst + i) = w8_codes8<INT8>(&vc[8 * c], s, rs, rcp_ok);
        }
    } else {
        for (int64_t i = (int64_t)threadIdx.x * 8; i < K; i += kQT * 8) {
            float v[8];
            load8<IN_BF16>(src, i, v);
            *reinterpret_cast<uint2*>(dst + i) = w8_codes8<INT8>(v, s, rs, rcp_ok);
        }
    }
}

constexpr int kFK = 128;  // K step (bytes = inputs)

// LDS slot of 16-byte chunk c (0..7) of tile row r (rows of 128 bytes).  A 16-lane quarter
// of a 16-byte read takes one LDS cycle when its 16 rows hit 16 different 16-byte groups of
// the 256-byte bank row: row r covers groups 8 (r & 1) .. +7, and c ^ ((r >> 1) & 7) spreads
// the 8 row pairs over them (c ^ (r & 7) repeats every 8 rows: two lanes per bank group).
// The map is its own inverse: the loader fetches chunk w8_slot(r, s) into slot s.
__device__ __forceinline__ int w8_slot(int r, int c) { return c ^ ((r >> 1) & 7); }

// 16 bytes per lane from global memory straight into LDS: lane l of the wave writes bytes
// [16 l, 16 l + 16) after the wave-uniform LDS address.  Inline assembly, so the compiler
// does not order the LDS reads of other stages behind these loads; the kernel waits for
// them itself (vmcnt) before the barrier that publishes a stage.
__device__ __forceinline__ void w8_load_lds16(const void* g, uint32_t lds_addr) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(g), "s"(lds_addr)
                 : "memory", "m0");
}

// The product with a three-stage LDS ring filled by direct loads two steps ahead:
// 512 threads, 128 x 256 output tile, wave (wm, wn) owns 64 x 64 (2 x 2 MFMA tiles).  A
// stage is the X tile (128 rows x 128 inputs, 16 KiB) and the W tile (256 x 128, 32 KiB),
// chunk c of row r at slot w8_slot(r, c): each wave issues 2 X and 4 W loads of 8 rows x
// 128 bytes per stage, lane l loading chunk w8_slot(row, l % 8) of row l / 8 so that it
// lands in its swizzled slot.
constexpr int kRingStages = 3;
constexpr int kRingX = 128 * kFK;
constexpr int kRingW = 256 * kFK;
constexpr int kRingStage = kRingX + kRingW;

// INT8: v_mfma_i32_32x32x32_i8 (exact int32 sums); a lane supplies row (lane % 32) and the
// 16 inputs 32 s + 16 (lane / 32) .. +15 of MFMA step s, one 16-byte chunk.
typedef int v4i_t __attribute__((ext_vector_type(4)));
typedef int i32x16_t __attribute__((ext_vector_type(16)));

constexpr int kW8Xcds = 8;   // accelerator complex dies of MI355X, each with its own L2

template <bool INT8>
__global__ __launch_bounds__(512) void w8_gemm_ring_kernel(
    const uint8_t* __restrict__ X, const float* __restrict__ sx, const uint8_t* __restrict__ W,
    const float* __restrict__ sw, void* __restrict__ Y, int y_bf16, int M, int N, int K,
    int tiles_m, int tiles_n, int group_m, int per_xcd) {
    __shared__ __attribute__((aligned(16))) uint8_t ring[kRingStages * kRingStage];
    // Tile order: workgroup b runs on XCD b % 8 and each XCD takes a contiguous range of a
    // grouped order (group_m tiles of M per band, N within the band), so the workgroups
    // resident on one XCD cover a compact block of tiles and share X rows and W columns in
    // that XCD's L2.  Slots past the last tile exit.
    const int t = (int)(blockIdx.x % kW8Xcds) * per_xcd + (int)(blockIdx.x / kW8Xcds);
    if (t >= tiles_m * tiles_n) return;
    const int band = t / (group_m * tiles_n);
    const int first_m = band * group_m;
    const int gm = min(tiles_m - first_m, group_m);
    const int rb = t - band * group_m * tiles_n;
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int wm = wave >> 2;
    const int wn = wave & 3;
    const int m0 = (first_m + rb % gm) * 128;
    const int n0 = (rb / gm) * 256;

    // per-lane sources of this wave's loads (step 0; a step adds 128 bytes)
    const uint8_t* xsrc[2];
    const uint8_t* wsrc[4];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int r = 8 * (2 * wave + i) + (lane >> 3);
        xsrc[i] = X + (int64_t)min(m0 + r, M - 1) * K + 16 * w8_slot(r, lane & 7);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = 8 * (4 * wave + i) + (lane >> 3);
        wsrc[i] = W + (int64_t)min(n0 + r, N - 1) * K + 16 * w8_slot(r, lane & 7);
    }
    const uint32_t ring_lds = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)ring);
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    auto issue = [&](int st, int kt) {
        const uint32_t base = ring_lds + st * kRingStage;
#pragma unroll
        for (int i = 0; i < 2; ++i)
            w8_load_lds16(xsrc[i] + (int64_t)kt * kFK, base + (2 * wave_u + i) * 1024);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            w8_load_lds16(wsrc[i] + (int64_t)kt * kFK, base + kRingX + (4 * wave_u + i) * 1024);
    };
    auto operand = [&](const uint8_t* t, int r, int kh) {
        const int c0 = 4 * kh + 2 * (lane >> 5);
        const u32x4_t lo = *reinterpret_cast<const u32x4_t*>(&t[r * kFK + (w8_slot(r, c0) << 4)]);
        const u32x4_t hi = *reinterpret_cast<const u32x4_t*>(&t[r * kFK + (w8_slot(r, c0 + 1) << 4)]);
        const v8i_t v = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                         (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
        return v;
    };

    f32x16_t acc[2][2];
    i32x16_t iacc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            acc[i][j] = (f32x16_t){};
            iacc[i][j] = (i32x16_t){};
        }
    auto chunk = [&](const uint8_t* t, int r, int c) {
        return __builtin_bit_cast(v4i_t, *reinterpret_cast<const u32x4_t*>(&t[r * kFK + (w8_slot(r, c) << 4)]));
    };

    const int Kt = K / kFK;
    issue(0, 0);
    if (Kt > 1) issue(1, 1);
    for (int kt = 0; kt < Kt; ++kt) {
        // this wave's loads of step kt have landed (the six of step kt+1 may still be in
        // flight); the barrier makes every wave's loads visible and frees the stage that
        // step kt+2 reuses
        if (kt + 1 < Kt)
            __builtin_amdgcn_s_waitcnt(0xF76);  // vmcnt(6)
        else
            __builtin_amdgcn_s_waitcnt(0xF70);  // vmcnt(0)
        __syncthreads();
        if (kt + 2 < Kt) issue((kt + 2) % kRingStages, kt + 2);
        const uint8_t* xs = ring + (kt % kRingStages) * kRingStage;
        const uint8_t* ws = xs + kRingX;
        if constexpr (INT8) {
            v4i_t xa[4][2], wb[4][2];
#pragma unroll
            for (int st = 0; st < 4; ++st) {
#pragma unroll
                for (int i = 0; i < 2; ++i) xa[st][i] = chunk(xs, 64 * wm + 32 * i + (lane & 31), 2 * st + (lane >> 5));
#pragma unroll
                for (int j = 0; j < 2; ++j) wb[st][j] = chunk(ws, 64 * wn + 32 * j + (lane & 31), 2 * st + (lane >> 5));
            }
#pragma unroll
            for (int st = 0; st < 4; ++st)
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int j = 0; j < 2; ++j)
                        iacc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(xa[st][i], wb[st][j], iacc[i][j], 0, 0, 0);
            continue;
        }
        v8i_t xa[2][2], wb[2][2];
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) {
#pragma unroll
            for (int i = 0; i < 2; ++i) xa[kh][i] = operand(xs, 64 * wm + 32 * i + (lane & 31), kh);
#pragma unroll
            for (int j = 0; j < 2; ++j) wb[kh][j] = operand(ws, 64 * wn + 32 * j + (lane & 31), kh);
        }
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                        xa[kh][i], wb[kh][j], acc[i][j], 0, 0, 0, 127, 0, 127);
    }

#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int c = n0 + 64 * wn + 32 * j + (lane & 31);
            if (c >= N) continue;
            const float scw = sw[c];
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int r = m0 + 64 * wm + 32 * i + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
                if (r >= M) continue;
                const float y = (INT8 ? (float)iacc[i][j][v] : acc[i][j][v]) * sx[r] * scw;
                const int64_t o = (int64_t)r * N + c;
                if (y_bf16) {
                    const uint32_t u = __float_as_uint(y);
                    static_cast<uint16_t*>(Y)[o] = (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
                } else {
                    static_cast<float*>(Y)[o] = y;
                }
            }
        }
}

template <bool INT8>
hipError_t launch_ring(const uint8_t* xq, const float* sx, int64_t m, const uint8_t* wq,
                       const float* sw, int64_t n, int64_t k, void* y, bool y_bf16,
                       hipStream_t s) {
    // bands of 8 M tiles in the XCD-aware order (measured on MI355X at 4096 x 28672 x 8192:
    // bands of 4, 16 and 32 ran 1-4 % slower for FP8)
    const int tiles_n = (int)((n + 255) / 256);
    const int tiles_m = (int)((m + 127) / 128);
    const int group_m = tiles_m < 8 ? tiles_m : 8;
    const int per_xcd = (tiles_m * tiles_n + kW8Xcds - 1) / kW8Xcds;
    hipLaunchKernelGGL(w8_gemm_ring_kernel<INT8>, dim3((unsigned)(per_xcd * kW8Xcds)), dim3(512),
                       0, s, xq, sx, wq, sw, y, y_bf16 ? 1 : 0, (int)m, (int)n, (int)k, tiles_m,
                       tiles_n, group_m, per_xcd);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_w8_quantize_rows(const void* a, bool bf16, int64_t rows, int64_t k,
                                    uint8_t* codes, float* scales, uint32_t* status,
                                    hipStream_t s, bool int8) {
    const dim3 grid((unsigned)rows), block(kQT);
    if (int8) {
        if (bf16)
            hipLaunchKernelGGL((w8_quantize_rows_kernel<true, true>), grid, block, 0, s, a, k, codes, scales, status);
        else
            hipLaunchKernelGGL((w8_quantize_rows_kernel<false, true>), grid, block, 0, s, a, k, codes, scales, status);
    } else if (bf16) {
        hipLaunchKernelGGL((w8_quantize_rows_kernel<true, false>), grid, block, 0, s, a, k, codes, scales, status);
    } else {
        hipLaunchKernelGGL((w8_quantize_rows_kernel<false, false>), grid, block, 0, s, a, k, codes, scales, status);
    }
    return hipGetLastError();
}

hipError_t launch_int8_gemm(const uint8_t* xq, const float* sx, int64_t m, const uint8_t* wq,
                            const float* sw, int64_t n, int64_t k, void* y, bool y_bf16,
                            hipStream_t s) {
    return launch_ring<true>(xq, sx, m, wq, sw, n, k, y, y_bf16, s);
}

hipError_t launch_fp8_gemm(const uint8_t* xq, const float* sx, int64_t m, const uint8_t* wq,
                           const float* sw, int64_t n, int64_t k, void* y, bool y_bf16,
                           hipStream_t s) {
    // measured on MI355X at 4096 x 28672 x 8192: the three-stage ring 1.09-1.10 ms; register
    // staging two steps ahead 1.14-1.16 ms with 128 x 256 tiles, 1.16 ms with 256 x 128,
    // 1.58 ms with 128 x 128 tiles
    return launch_ring<false>(xq, sx, m, wq, sw, n, k, y, y_bf16, s);
}

}  // namespace w4
