// Round-to-nearest asymmetric 4-bit quantization (group 128) and the
// canonical <-> kernel layout permutations.
//
// Quantizer: page "Weight quantization", section "How it works" (scale, zero
// and code formulas) and section "Code" (range widened to contain 0, scale 1
// for an empty range, binary32 arithmetic, Rust-style rounding of halves away
// from zero, the even input index in the low nibble).
//
// Symmetric variant (page "Quantization" › "How it really works" › "The mechanics:
// scale, round, clamp"): step = max|w| / 7 (1 for an all-zero group), code =
// clamp(round(w / step), -8, 7) with halves to even (rintf), stored as code + 8 with
// zero 8, so the products' (stored - zero) * scale16 holds unchanged.
//
// Work split: 32 lanes own one group (4 consecutive weights each, one 16-byte
// load), a wave owns two groups, a 256-thread block eight.  The group's
// minimum and maximum are a 32-lane butterfly; every lane then derives the
// same scale and zero and writes its two packed bytes, so a wave stores 128
// contiguous bytes.
#include "w4_internal.h"

namespace w4 {
namespace {

__device__ __forceinline__ float clamp_code_keep_nan(float t) {
    // f32 clamp to [0, 15] that leaves NaN unchanged (the f32 zero feeds the codes)
    return (t != t) ? t : fminf(fmaxf(t, 0.0f), 15.0f);
}

__device__ __forceinline__ uint32_t to_code(float t) {
    // clamp, then convert to a byte; NaN becomes 0 (fmaxf returns the non-NaN operand)
    return (uint32_t)fminf(fmaxf(t, 0.0f), 15.0f);
}

template <bool BF16>
__device__ __forceinline__ void load4(const void* __restrict__ W, int64_t idx, float v[4]) {
    if constexpr (BF16) {
        const uint2 raw = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(W) + idx);
        v[0] = __uint_as_float(raw.x << 16);
        v[1] = __uint_as_float(raw.x & 0xFFFF0000u);
        v[2] = __uint_as_float(raw.y << 16);
        v[3] = __uint_as_float(raw.y & 0xFFFF0000u);
    } else {
        const float4 f = *reinterpret_cast<const float4*>(static_cast<const float*>(W) + idx);
        v[0] = f.x; v[1] = f.y; v[2] = f.z; v[3] = f.w;
    }
}

template <bool BF16, bool SYM>
__global__ __launch_bounds__(256) void quantize_kernel(const void* __restrict__ W, int64_t n_groups,
                                                       uint16_t* __restrict__ packed16,
                                                       uint16_t* __restrict__ scales,
                                                       uint8_t* __restrict__ zeros,
                                                       uint32_t* __restrict__ status) {
#pragma clang fp contract(off)
    const int lane = threadIdx.x & 31;
    const int64_t gi = (int64_t)blockIdx.x * 8 + (threadIdx.x >> 5);
    const bool valid = gi < n_groups;

    float v[4] = {0.f, 0.f, 0.f, 0.f};
    if (valid) load4<BF16>(W, gi * kGroup + lane * 4, v);

    bool bad = false;
    float lo = v[0], hi = v[0];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        bad |= !__builtin_isfinite(v[i]);
        lo = fminf(lo, v[i]);
        hi = fmaxf(hi, v[i]);
    }
#pragma unroll
    for (int d = 16; d >= 1; d >>= 1) {
        lo = fminf(lo, __shfl_xor(lo, d, 32));
        hi = fmaxf(hi, __shfl_xor(hi, d, 32));
    }
    float s, zc;
    uint32_t c[4];
    bool nonempty;
    if constexpr (SYM) {
        const float amax = fmaxf(fabsf(lo), fabsf(hi));
        nonempty = amax > 0.0f;
        s = nonempty ? amax / 7.0f : 1.0f;    // IEEE division
        zc = 8.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i)   // rintf: halves to even; a NaN quotient clamps to -8
            c[i] = (uint32_t)(fminf(fmaxf(rintf(v[i] / s), -8.0f), 7.0f) + 8.0f);
    } else {
        lo = fminf(lo, 0.0f);  // zero stays exactly representable
        hi = fmaxf(hi, 0.0f);
        nonempty = hi > lo;
        s = nonempty ? (hi - lo) / 15.0f : 1.0f;   // IEEE division
        zc = clamp_code_keep_nan(roundf(-lo / s));  // roundf: halves away from zero
#pragma unroll
        for (int i = 0; i < 4; ++i) c[i] = to_code(roundf(v[i] / s) + zc);
    }

    if (!valid) return;
    packed16[gi * (kGroup / 4) + lane] = (uint16_t)(c[0] | (c[1] << 4) | (c[2] << 8) | (c[3] << 12));
    if (bad && status) atomicOr(status, 1u);  // W4_STATUS_NONFINITE
    if (lane == 0) {
        const uint16_t s16 = __builtin_bit_cast(uint16_t, (_Float16)s);  // round to nearest even
        scales[gi] = s16;
        zeros[gi] = (uint8_t)to_code(zc);
        uint32_t flags = 0;
        if ((s16 & 0x7FFFu) == 0x7C00u) flags |= 2u;          // W4_STATUS_SCALE_OVERFLOW
        if ((s16 & 0x7FFFu) == 0 && nonempty) flags |= 4u;   // W4_STATUS_SCALE_ZERO
        if (flags && status) atomicOr(status, flags);
    }
}

__global__ __launch_bounds__(256) void prepare_kernel(const uint4* __restrict__ packed,
                                                      const uint16_t* __restrict__ scales,
                                                      const uint8_t* __restrict__ zeros,
                                                      int64_t n_vec, int64_t n_rows, int64_t kg,
                                                      uint4* __restrict__ out_words,
                                                      uint32_t* __restrict__ out_sz) {
    const int64_t n_words = (n_rows + 3) / 4 * 4 * kg;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_vec; i += stride) {
        uint4 w = packed[i];
        w.x = to_kernel_word(w.x);
        w.y = to_kernel_word(w.y);
        w.z = to_kernel_word(w.z);
        w.w = to_kernel_word(w.w);
        out_words[i] = w;
    }
    // one pass over the destination words: row-group q = i / (4 kg), group g, row 4q + r
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_words; i += stride) {
        const int64_t q = i / (4 * kg);
        const int64_t rem = i - q * 4 * kg;
        const int64_t g = rem >> 2;
        const int64_t row = 4 * q + (rem & 3);
        uint32_t v = 0;
        if (row < n_rows) {
            const int64_t src = row * kg + g;
            v = (uint32_t)scales[src] | ((((uint32_t)zeros[src] + 128u) & 0xFFu) << 16);
        }
        out_sz[i] = v;
    }
}

__global__ __launch_bounds__(256) void unprepare_kernel(const uint4* __restrict__ words,
                                                        const uint32_t* __restrict__ sz,
                                                        int64_t n_vec, int64_t n_rows, int64_t kg,
                                                        uint4* __restrict__ packed,
                                                        uint16_t* __restrict__ scales,
                                                        uint8_t* __restrict__ zeros) {
    const int64_t n_groups = n_rows * kg;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_vec; i += stride) {
        uint4 w = words[i];
        w.x = to_canonical_word(w.x);
        w.y = to_canonical_word(w.y);
        w.z = to_canonical_word(w.z);
        w.w = to_canonical_word(w.w);
        packed[i] = w;
    }
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_groups; i += stride) {
        const int64_t row = i / kg;
        const uint32_t v = sz[sz_index(row, i - row * kg, kg)];
        scales[i] = (uint16_t)(v & 0xFFFFu);
        zeros[i] = (uint8_t)(((v >> 16) - 128u) & 0xFFu);
    }
}

int64_t elementwise_blocks(int64_t work) {
    int64_t b = (work + 255) / 256;
    if (b > 65536) b = 65536;
    if (b < 1) b = 1;
    return b;
}

}  // namespace

hipError_t launch_quantize(const void* W, bool bf16, bool symmetric, int64_t n_groups,
                           uint8_t* packed, uint16_t* scales, uint8_t* zeros, uint32_t* status,
                           hipStream_t s) {
    const int64_t blocks = (n_groups + 7) / 8;
    uint16_t* p16 = reinterpret_cast<uint16_t*>(packed);
    auto kern = bf16 ? (symmetric ? quantize_kernel<true, true> : quantize_kernel<true, false>)
                     : (symmetric ? quantize_kernel<false, true> : quantize_kernel<false, false>);
    hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(256), 0, s, W, n_groups, p16, scales,
                       zeros, status);
    return hipGetLastError();
}

hipError_t launch_prepare(const uint8_t* packed, const uint16_t* scales, const uint8_t* zeros,
                          int64_t n, int64_t k, uint8_t* prepared, hipStream_t s) {
    const int64_t n_vec = packed_bytes(n, k) / 16;
    const int64_t n_words = sz_words(n, k);
    const int64_t blocks = elementwise_blocks(n_vec > n_words ? n_vec : n_words);
    hipLaunchKernelGGL(prepare_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                       reinterpret_cast<const uint4*>(packed), scales, zeros, n_vec, n, k / kGroup,
                       reinterpret_cast<uint4*>(prepared),
                       reinterpret_cast<uint32_t*>(prepared + sz_offset(n, k)));
    return hipGetLastError();
}

hipError_t launch_unprepare(const uint8_t* prepared, int64_t n, int64_t k, uint8_t* packed,
                            uint16_t* scales, uint8_t* zeros, hipStream_t s) {
    const int64_t n_vec = packed_bytes(n, k) / 16;
    const int64_t n_groups = n * (k / kGroup);
    const int64_t blocks = elementwise_blocks(n_vec > n_groups ? n_vec : n_groups);
    hipLaunchKernelGGL(unprepare_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                       reinterpret_cast<const uint4*>(prepared),
                       reinterpret_cast<const uint32_t*>(prepared + sz_offset(n, k)), n_vec,
                       n, k / kGroup, reinterpret_cast<uint4*>(packed), scales, zeros);
    return hipGetLastError();
}

}  // namespace w4
