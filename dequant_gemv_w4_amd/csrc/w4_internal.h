// Internal definitions shared by the libw4a16 kernels and host code.
//
// Prepared ("kernel") layout, format version 3.  The canonical arrays are
// rearranged so that one 16-byte load feeds 32 codes to a lane and the unpack
// needs no data movement between lanes (page "LLM Quantization Architecture in
// Depth" › "Kernels and memory layout: the format is a contract": packed
// weights are pre-shuffled and scales sit beside them; architecture page,
// stage "Memory Layout": scale interleaving).
//
//   region A, offset 0:   N rows x (K/2) bytes.  Each aligned 32-bit word holds
//                         the 8 codes c0..c7 of 8 consecutive inputs, stored as
//                         bits [4j, 4j+4)      = c(2j)    (j = 0..3)
//                         bits [16+4j, 20+4j)  = c(2j+1)
//                         so (word >> 4j) & 0x000F000F places the codes of the
//                         input pair (2j, 2j+1) in the low bits of two 16-bit
//                         halves, the same order as a bf16 pair of x in memory.
//   region B, offset A_bytes rounded up to 256:
//                         ceil(N/4) x (K/128) x 4 32-bit words; the word of row
//                         n and group g is at ((n/4) * (K/128) + g) * 4 + n%4, so
//                         the words of four consecutive rows of one group form
//                         one 16-byte load.  Word: bits 0..15 the binary16
//                         scale, bits 16..23 the zero, bits 24..31 the zero times
//                         16 (mod 256): with the byte 0xE4 these two bytes form
//                         the binary16 values -(1024 + zero) and -(1024 + 16 zero)
//                         that turn the unpacked codes into exact q - zero.  Rows
//                         past N are zero words.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4 {

constexpr int kGroup = 128;

inline __host__ __device__ int64_t packed_bytes(int64_t n, int64_t k) { return n * (k / 2); }
inline __host__ __device__ int64_t sz_offset(int64_t n, int64_t k) {
    return (packed_bytes(n, k) + 255) / 256 * 256;
}
inline __host__ __device__ int64_t sz_words(int64_t n, int64_t k) {
    return (n + 3) / 4 * 4 * (k / kGroup);
}
inline __host__ __device__ int64_t prepared_total(int64_t n, int64_t k) {
    return sz_offset(n, k) + sz_words(n, k) * 4;
}
// the same layout for a group of 32, 64 or 128 inputs: one scale/zero word per row and
// group, four rows of one group per 16 bytes
inline __host__ __device__ int64_t sz_words_g(int64_t n, int64_t k, int64_t group) {
    return (n + 3) / 4 * 4 * (k / group);
}
inline __host__ __device__ int64_t prepared_total_g(int64_t n, int64_t k, int64_t group) {
    return sz_offset(n, k) + sz_words_g(n, k, group) * 4;
}
// index of the scale/zero word of row n, group g
inline __host__ __device__ int64_t sz_index(int64_t n, int64_t g, int64_t kg) {
    return ((n >> 2) * kg + g) * 4 + (n & 3);
}

// canonical word (code i at bits 4i) -> prepared word
__device__ __forceinline__ uint32_t to_kernel_word(uint32_t w) {
    uint32_t e = w & 0x0F0F0F0Fu;          // c0 c2 c4 c6 at bits 0, 8, 16, 24
    uint32_t o = (w >> 4) & 0x0F0F0F0Fu;   // c1 c3 c5 c7
    e = (e | (e >> 4)) & 0x00FF00FFu;
    e = (e | (e >> 8)) & 0x0000FFFFu;      // c0 c2 c4 c6 at bits 0, 4, 8, 12
    o = (o | (o >> 4)) & 0x00FF00FFu;
    o = (o | (o >> 8)) & 0x0000FFFFu;
    return e | (o << 16);
}

// prepared word -> canonical word
__device__ __forceinline__ uint32_t to_canonical_word(uint32_t p) {
    uint32_t e = p & 0xFFFFu;
    uint32_t o = p >> 16;
    e = (e | (e << 8)) & 0x00FF00FFu;
    e = (e | (e << 4)) & 0x0F0F0F0Fu;
    o = (o | (o << 8)) & 0x00FF00FFu;
    o = (o | (o << 4)) & 0x0F0F0F0Fu;
    return e | (o << 4);
}

// Launch wrappers (defined in the .hip files); return hipSuccess or the launch error.
// Storage variant of the weight format: group of 32, 64 or 128 inputs, scale stored as
// binary16 or bfloat16 bits, zeros one per byte or two per byte (flat over [N, K/group],
// even index in the low nibble), asymmetric or symmetric codes.
struct Fmt {
    int group = 128;
    bool scale_bf16 = false;
    bool zero4 = false;
    bool symmetric = false;
};

hipError_t launch_quantize(const void* W, bool bf16, const Fmt& f, int64_t n_groups,
                           uint8_t* packed, uint16_t* scales, uint8_t* zeros, uint32_t* status,
                           hipStream_t s);
hipError_t launch_prepare(const uint8_t* packed, const uint16_t* scales, const uint8_t* zeros,
                          int64_t n, int64_t k, const Fmt& f, uint8_t* prepared, hipStream_t s);
hipError_t launch_unprepare(const uint8_t* prepared, int64_t n, int64_t k, const Fmt& f,
                            uint8_t* packed, uint16_t* scales, uint8_t* zeros, hipStream_t s);
hipError_t launch_gemv(const uint8_t* prepared, int64_t n, int64_t k, const void* x, bool x_f32,
                       int64_t m, void* y, bool y_bf16, hipStream_t s);
// the one-row (dot2) kernel on any group size and scale type (w4_gemv routes here and to
// the matrix-core kernels for the canonical format)
hipError_t launch_gemv_dot2(const uint8_t* prepared, int64_t n, int64_t k, int group,
                            bool scale_bf16, const void* x, bool x_f32, int64_t m, void* y,
                            bool y_bf16, hipStream_t s);
hipError_t launch_gemv_mfma(const uint8_t* prepared, int64_t n, int64_t k, const uint16_t* x,
                            int64_t m, void* y, bool y_bf16, hipStream_t s);
// Whether launch_gemv_mfma runs the shape on the resident-x kernel (x held in registers for
// all the workgroup's rows, codes loaded straight into registers): K of at most 64 groups and
// at least 48 rows per workgroup when one workgroup runs per compute unit.
bool gemv_resident_x_takes(int64_t n, int64_t k);
size_t gemm_workspace(int64_t m, int64_t k);
hipError_t launch_stream_read(const void* buf, int64_t bytes, uint32_t* sink, hipStream_t s);
// 8-bit rows: E4M3 codes, or symmetric INT8 codes when int8 is set
hipError_t launch_w8_quantize_rows(const void* a, bool bf16, int64_t rows, int64_t k,
                                    uint8_t* codes, float* scales, uint32_t* status,
                                    hipStream_t s, bool int8 = false);
hipError_t launch_int8_gemm(const uint8_t* xq, const float* sx, int64_t m, const uint8_t* wq,
                            const float* sw, int64_t n, int64_t k, void* y, bool y_bf16,
                            hipStream_t s);
hipError_t launch_fp8_gemm(const uint8_t* xq, const float* sx, int64_t m, const uint8_t* wq,
                           const float* sw, int64_t n, int64_t k, void* y, bool y_bf16,
                           hipStream_t s);
hipError_t launch_gemm(const uint8_t* prepared, int64_t n, int64_t k, const void* X, int64_t m,
                       void* Y, bool y_bf16, void* workspace, hipStream_t s);

}  // namespace w4
