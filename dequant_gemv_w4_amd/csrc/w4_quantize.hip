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
// Storage variants (page "Quantization" › "Code": int4 groups of 128 and of 32;
// page "Weight quantization" › "Implementation notes": scales kept in fp16 or bf16;
// "Code" and "Complexity and constants": a 4-bit zero per group): groups of 32, 64 or
// 128 inputs; the binary32 step stored as binary16 or bfloat16 (both round to nearest
// even); zeros one per byte or two per byte, packed over the flat [N, K/group] array with
// the even index in the low nibble.  The codes and the step do not depend on the storage.
//
// Work split: G/16 lanes own one group (16 weights each, four 16-byte loads of
// binary32 weights), a 256-thread block 4096/G groups.  The group's minimum and
// maximum are a butterfly over those lanes; every lane then derives the same scale
// and zero and writes its eight packed bytes, so the lanes of a group store its G/2
// bytes.  With 4-bit zeros the first lane of an even group also takes the odd
// group's zero (the next G/16 lanes of the same wave) and writes the shared byte.
#include <cstdlib>

#include "w4_internal.h"

namespace w4 {
namespace {

__device__ __forceinline__ float clamp_code_keep_nan(float t) {
    // f32 clamp to [0, 15] that leaves NaN unchanged (the f32 zero feeds the codes)
    return (t != t) ? t : fminf(fmaxf(t, 0.0f), 15.0f);
}

// Rounding of the binary32 quotient v / s without a division per weight.  t = v * rcp(s)
// (v_rcp_f32, within 1 ulp) is within 1.6 * 2^-23 relative of v / s, and the correctly
// rounded quotient within 2^-24 relative; for |v / s| < 16, the range of every in-group
// quotient, the two differ by less than 2^-18.  So where t lies more than 2^-17 from the
// nearest k + 1/2, the rounded quotient and rintf(t) are the same integer.  Only the
// other weights (a window of 2^-16 per unit: about 1.5 in 10^5), NaN and infinite values, and groups
// whose scale falls outside [2^-120, 2^120] take the IEEE division.
__device__ __forceinline__ bool clear_of_half(float t) {
    return fabsf(__builtin_amdgcn_fractf(t) - 0.5f) > 0x1p-17f;
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

__device__ __forceinline__ uint16_t bf16_bits_rne(float f) {
    const uint32_t u = __float_as_uint(f);
    return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// LPG: lanes per group, each lane quantizes 16 weights of its group (group = 16 LPG
// inputs).  Lane i of a group holds the 16-byte chunks i, i + LPG, i + 2 LPG, i + 3 LPG of
// the group's binary32 weights, so each of the four loads of a wave covers LPG*16
// contiguous bytes of each of its 64/LPG groups (eight full 128-byte lines at group 128).
template <bool BF16, bool SYM, int LPG>
__global__ __launch_bounds__(256) void quantize_kernel(const void* __restrict__ W, int64_t n_groups,
                                                       uint16_t* __restrict__ packed16,
                                                       uint16_t* __restrict__ scales,
                                                       uint8_t* __restrict__ zeros,
                                                       uint32_t* __restrict__ status,
                                                       int scale_bf16, int zero4) {
#pragma clang fp contract(off)
    constexpr int G = 16 * LPG;
    const int lane = threadIdx.x & (LPG - 1);
    const int64_t gi = (int64_t)blockIdx.x * (256 / LPG) + (threadIdx.x / LPG);
    const bool valid = gi < n_groups;
    float v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = 0.0f;
    if (valid) {
#pragma unroll
        for (int j = 0; j < 4; ++j) load4<BF16>(W, gi * G + (lane + LPG * j) * 4, &v[4 * j]);
    }
    bool bad = false;
    float lo = v[0], hi = v[0];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        bad |= !__builtin_isfinite(v[i]);
        lo = fminf(lo, v[i]);
        hi = fmaxf(hi, v[i]);
    }
#pragma unroll
    for (int d = LPG / 2; d >= 1; d >>= 1) {
        lo = fminf(lo, __shfl_xor(lo, d, LPG));
        hi = fmaxf(hi, __shfl_xor(hi, d, LPG));
    }
    float s, zc;
    uint32_t c[16];
    bool nonempty;
    if constexpr (SYM) {
        const float amax = fmaxf(fabsf(lo), fabsf(hi));
        nonempty = amax > 0.0f;
        s = nonempty ? amax / 7.0f : 1.0f;    // IEEE division
        zc = 8.0f;
        const float r = __builtin_amdgcn_rcpf(s);
        const bool rcp_ok = s >= 0x1p-120f && s <= 0x1p120f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {   // rintf: halves to even; a NaN quotient clamps to -8
            const float t = v[i] * r;
            const float q = (rcp_ok && clear_of_half(t)) ? rintf(t) : rintf(v[i] / s);
            c[i] = (uint32_t)(fminf(fmaxf(q, -8.0f), 7.0f) + 8.0f);
        }
    } else {
        lo = fminf(lo, 0.0f);  // zero stays exactly representable
        hi = fmaxf(hi, 0.0f);
        nonempty = hi > lo;
        s = nonempty ? (hi - lo) / 15.0f : 1.0f;   // IEEE division
        zc = clamp_code_keep_nan(roundf(-lo / s));  // roundf: halves away from zero
        const float r = __builtin_amdgcn_rcpf(s);
        const bool rcp_ok = s >= 0x1p-120f && s <= 0x1p120f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const float t = v[i] * r;
            const float q = (rcp_ok && clear_of_half(t)) ? rintf(t) : roundf(v[i] / s);
            c[i] = to_code(q + zc);
        }
    }
    const uint32_t zbyte = to_code(zc);
    // the odd neighbour's zero, LPG lanes up in the same wave (64 / LPG groups per wave, an
    // even number, so an even group's partner never crosses the wave)
    const uint32_t zodd = __shfl((int)zbyte, (int)(threadIdx.x & 63) + LPG, 64) & 0xFu;

    if (valid) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
            packed16[gi * (G / 4) + lane + LPG * j] =
                (uint16_t)(c[4 * j] | (c[4 * j + 1] << 4) | (c[4 * j + 2] << 8) | (c[4 * j + 3] << 12));
        if (bad && status) atomicOr(status, 1u);  // W4_STATUS_NONFINITE
        if (lane == 0) {
            const uint16_t s16 = scale_bf16 ? bf16_bits_rne(s)
                                            : __builtin_bit_cast(uint16_t, (_Float16)s);  // nearest even
            const uint32_t inf_bits = scale_bf16 ? 0x7F80u : 0x7C00u;
            scales[gi] = s16;
            if (!zero4) {
                zeros[gi] = (uint8_t)zbyte;
            } else if ((gi & 1) == 0) {
                const bool pair = gi + 1 < n_groups;
                zeros[gi >> 1] = (uint8_t)(zbyte | (pair ? zodd << 4 : 0u));
            }
            uint32_t flags = 0;
            if ((s16 & 0x7FFFu) == inf_bits) flags |= 2u;           // W4_STATUS_SCALE_OVERFLOW
            if ((s16 & 0x7FFFu) == 0 && nonempty) flags |= 4u;     // W4_STATUS_SCALE_ZERO
            if (flags && status) atomicOr(status, flags);
        }
    }
}

__global__ __launch_bounds__(256) void prepare_kernel(const uint4* __restrict__ packed,
                                                      const uint16_t* __restrict__ scales,
                                                      const uint8_t* __restrict__ zeros,
                                                      int64_t n_vec, int64_t n_rows, int64_t kg,
                                                      int zero4, uint4* __restrict__ out_words,
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
            const uint32_t z = zero4 ? ((uint32_t)zeros[src >> 1] >> (4 * (src & 1))) & 0xFu
                                     : (uint32_t)zeros[src];
            v = (uint32_t)scales[src] | ((z & 0xFFu) << 16) | (((z << 4) & 0xFFu) << 24);
        }
        out_sz[i] = v;
    }
}

__global__ __launch_bounds__(256) void unprepare_kernel(const uint4* __restrict__ words,
                                                        const uint32_t* __restrict__ sz,
                                                        int64_t n_vec, int64_t n_rows, int64_t kg,
                                                        int zero4, uint4* __restrict__ packed,
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
    auto zero_of = [&](int64_t i) {
        const int64_t row = i / kg;
        return (sz[sz_index(row, i - row * kg, kg)] >> 16) & 0xFFu;
    };
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_groups; i += stride) {
        const int64_t row = i / kg;
        const uint32_t v = sz[sz_index(row, i - row * kg, kg)];
        scales[i] = (uint16_t)(v & 0xFFFFu);
        if (!zero4) zeros[i] = (uint8_t)((v >> 16) & 0xFFu);
    }
    if (zero4) {
        // one thread per byte: groups 2i and 2i+1
        const int64_t n_bytes = (n_groups + 1) / 2;
        for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_bytes; i += stride) {
            uint32_t b = zero_of(2 * i) & 0xFu;
            if (2 * i + 1 < n_groups) b |= (zero_of(2 * i + 1) & 0xFu) << 4;
            zeros[i] = (uint8_t)b;
        }
    }
}

int64_t elementwise_blocks(int64_t work) {
    int64_t b = (work + 255) / 256;
    if (b > 65536) b = 65536;
    if (b < 1) b = 1;
    return b;
}

}  // namespace

hipError_t launch_quantize(const void* W, bool bf16, const Fmt& f, int64_t n_groups,
                           uint8_t* packed, uint16_t* scales, uint8_t* zeros, uint32_t* status,
                           hipStream_t s) {
    // 16 weights per lane: 0.198-0.209 ms against 0.224-0.31 ms with 4 weights per lane
    // (28672 x 8192 binary32 on MI355X; vector instructions 66 M against 119 M per call)
    const int lpg = f.group / 16;
    const int64_t blocks = (n_groups + (256 / lpg) - 1) / (256 / lpg);
    uint16_t* p16 = reinterpret_cast<uint16_t*>(packed);
#define W4_Q(LPG)                                                                              \
    if (lpg == LPG) {                                                                          \
        auto kern = bf16 ? (f.symmetric ? quantize_kernel<true, true, LPG>                     \
                                        : quantize_kernel<true, false, LPG>)                   \
                         : (f.symmetric ? quantize_kernel<false, true, LPG>                    \
                                        : quantize_kernel<false, false, LPG>);                 \
        hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(256), 0, s, W, n_groups, p16,    \
                           scales, zeros, status, f.scale_bf16 ? 1 : 0, f.zero4 ? 1 : 0);      \
        return hipGetLastError();                                                              \
    }
    W4_Q(8) W4_Q(4) W4_Q(2)
#undef W4_Q
    return hipErrorInvalidValue;
}

hipError_t launch_prepare(const uint8_t* packed, const uint16_t* scales, const uint8_t* zeros,
                          int64_t n, int64_t k, const Fmt& f, uint8_t* prepared, hipStream_t s) {
    const int64_t n_vec = packed_bytes(n, k) / 16;
    const int64_t n_words = sz_words_g(n, k, f.group);
    const int64_t blocks = elementwise_blocks(n_vec > n_words ? n_vec : n_words);
    hipLaunchKernelGGL(prepare_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                       reinterpret_cast<const uint4*>(packed), scales, zeros, n_vec, n, k / f.group,
                       f.zero4 ? 1 : 0, reinterpret_cast<uint4*>(prepared),
                       reinterpret_cast<uint32_t*>(prepared + sz_offset(n, k)));
    return hipGetLastError();
}

hipError_t launch_unprepare(const uint8_t* prepared, int64_t n, int64_t k, const Fmt& f,
                            uint8_t* packed, uint16_t* scales, uint8_t* zeros, hipStream_t s) {
    const int64_t n_vec = packed_bytes(n, k) / 16;
    const int64_t n_groups = n * (k / f.group);
    const int64_t blocks = elementwise_blocks(n_vec > n_groups ? n_vec : n_groups);
    hipLaunchKernelGGL(unprepare_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                       reinterpret_cast<const uint4*>(prepared),
                       reinterpret_cast<const uint32_t*>(prepared + sz_offset(n, k)), n_vec, n,
                       k / f.group, f.zero4 ? 1 : 0, reinterpret_cast<uint4*>(packed), scales,
                       zeros);
    return hipGetLastError();
}

}  // namespace w4
