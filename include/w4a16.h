/*
 * libw4a16 -- asymmetric group-wise 4-bit weights (group 128) and fused
 * dequantizing matrix-vector / matrix-matrix products for AMD gfx950.
 *
 * Plain C ABI: every buffer is a raw device pointer owned by the caller, every
 * size is an integer, every call is asynchronous on the given HIP stream.
 * The library never allocates, frees or synchronizes device memory.
 *
 * Format (page "Weight quantization", sections "How it works" and "Code";
 * the affine map is also given on "LLM Quantization Architecture in Depth"
 * › "Number formats, scales and granularity"):
 *   - W is [N, K] row-major (N outputs, K inputs); groups are 128 consecutive
 *     inputs of one row, so K must be a multiple of 128.
 *   - per group: lo = min(min(w), 0), hi = max(max(w), 0);
 *     scale = (hi - lo) / 15 in binary32, or 1 when hi == lo;
 *     zero  = clamp(round(-lo / scale), 0, 15);
 *     code  = clamp(round(w / scale) + zero, 0, 15);
 *     round = nearest, halves away from zero; every step one IEEE binary32
 *     operation (true division, no fused multiply-add, subnormals kept).
 *   - canonical storage: packed [N, K/2] bytes, code of the even input index in
 *     the low nibble; scales [N, K/128] binary16 bit patterns (the binary32
 *     scale rounded to nearest even); zeros [N, K/128] bytes.
 *   - w_hat = (code - zero) * scale16 and the products use, per group,
 *     scale16 * sum (code - zero) * x: one multiply per group, with the exact
 *     difference code - zero as the operand of every product.
 *
 * Readings of points the pages leave open are fixed above: halves away from
 * zero, codes from the binary32 scale, fp16 stored scale, byte zero.
 *
 * Errors: the return value reports argument validation and launch failures
 * synchronously; W4_ERR_HIP carries the runtime's message in
 * w4_last_hip_error().  Data conditions found on the device are OR-ed into the
 * optional status word (see w4_quantize).  Nothing falls back to another code
 * path: an unsupported request is refused.
 *
 * Threading: no mutable global state except a per-device architecture check
 * done once; calls from several host threads are safe.  Calls that share an
 * output buffer must be ordered by the caller.
 */
#ifndef W4A16_H
#define W4A16_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define W4_GROUP 128
#define W4_FORMAT_VERSION 3
#define W4_GEMV_MAX_M 16
#define W4_GEMV_MAX_K 32768
#define W4_FP8_MAX_K 65536
#define W4_GEMM_MAX_K (1 << 20)

typedef enum {
    W4_OK = 0,
    W4_ERR_NULL = 1,         /* a required pointer is NULL */
    W4_ERR_SHAPE = 2,        /* N < 1, K < 128, K % 128 != 0, M out of range, size limit */
    W4_ERR_ALIGN = 3,        /* a pointer breaks its stated alignment */
    W4_ERR_DTYPE = 4,        /* dtype value not accepted by this call */
    W4_ERR_UNSUPPORTED = 5,  /* request outside the fixed format */
    W4_ERR_ARCH = 6,         /* current device is not gfx950 */
    W4_ERR_WORKSPACE = 7,    /* workspace missing or too small */
    W4_ERR_HIP = 8,          /* HIP runtime error; see w4_last_hip_error() */
    W4_ERR_BUFFER = 9        /* destination buffer smaller than required */
} w4_status;

typedef enum { W4_F32 = 0, W4_BF16 = 1 } w4_dtype;

/* Device status word bits written by w4_quantize (OR-ed, never cleared). */
#define W4_STATUS_NONFINITE      1u  /* a weight was NaN or +-inf (outputs undefined) */
#define W4_STATUS_SCALE_OVERFLOW 2u  /* a binary32 scale rounded to binary16 infinity */
#define W4_STATUS_SCALE_ZERO     4u  /* a non-empty group's scale rounded to binary16 zero */

/*
 * w4_quantize -- round-to-nearest quantization of W (page "Weight quantization",
 * "How it works": scale, zero and code formulas; "Code": range widened to 0,
 * f32 arithmetic, nibble packing with the even index low).
 *   W          [N, K] row-major, binary32 (wt = W4_F32) or bfloat16 (W4_BF16); 16-B aligned.
 *   packed     out [N, K/2] bytes; 16-B aligned.
 *   scales_f16 out [N, K/128] binary16 bit patterns; 2-B aligned.
 *   zeros      out [N, K/128] bytes.
 *   d_status   optional device word (may be NULL); W4_STATUS_* bits are OR-ed in.
 * Requires N >= 1, K >= 128, K % 128 == 0.  Deterministic; bit-exact with the
 * formulas above for finite input.
 */
w4_status w4_quantize(const void* W, w4_dtype wt, int64_t N, int64_t K,
                      uint8_t* packed, uint16_t* scales_f16, uint8_t* zeros,
                      uint32_t* d_status, hipStream_t stream);

/*
 * w4_quantize_symmetric -- the symmetric variant (page "Quantization" › "How it
 * really works" › "The mechanics: scale, round, clamp"): per group of 128 the step
 * is max|w| / 7 (1 for an all-zero group), each code is round(w / step) with halves
 * to even, clamped to [-8, 7]; one binary32 operation per step.  Written in the same
 * canonical arrays as w4_quantize: stored code = code + 8, every zero = 8, scale =
 * the step rounded to binary16 -- so w4_prepare, w4_gemv and w4_gemm take the result
 * unchanged ((stored - zero) * scale16 is the dequantized weight).
 * Arguments, alignment, errors and d_status bits as w4_quantize.
 */
w4_status w4_quantize_symmetric(const void* W, w4_dtype wt, int64_t N, int64_t K,
                                uint8_t* packed, uint16_t* scales_f16, uint8_t* zeros,
                                uint32_t* d_status, hipStream_t stream);

/*
 * Kernel layout ("pre-shuffled" weights with interleaved scale and zero: page
 * "LLM Quantization Architecture in Depth" › "Kernels and memory layout: the
 * format is a contract"; the stage list's "Memory Layout" on the
 * architecture page).  The prepared buffer is opaque; its size is
 * w4_prepared_bytes(N, K).  w4_prepare is a bijection of the canonical arrays
 * and w4_unprepare is its exact inverse.
 *   packed/scales_f16/zeros  canonical arrays as produced by w4_quantize
 *                            (packed 16-B aligned, scales 2-B aligned).
 *   prepared                 [w4_prepared_bytes(N, K)] bytes, 256-B aligned.
 * The products read zeros 0..15 (what w4_quantize writes); the round trip holds for
 * any byte.
 */
size_t w4_prepared_bytes(int64_t N, int64_t K);
w4_status w4_prepare(const uint8_t* packed, const uint16_t* scales_f16, const uint8_t* zeros,
                     int64_t N, int64_t K, void* prepared, size_t prepared_bytes,
                     hipStream_t stream);
w4_status w4_unprepare(const void* prepared, int64_t N, int64_t K,
                       uint8_t* packed, uint16_t* scales_f16, uint8_t* zeros,
                       hipStream_t stream);

/*
 * w4_gemv -- decode-sized product y[m, n] = sum_k w_hat[n, k] * x[m, k] for
 * 1 <= M <= 16, never forming w_hat in memory (page "Weight quantization",
 * "How it works": the per-group factored dot; architecture page stage "Fused
 * Kernels": dequantization inside the product).  Every product multiplies the exact
 * value q - zero of a code (a code equal to its zero adds exactly 0); bf16 x enters
 * the one-row kernel as binary16 x * 2^-E, E per wave of 2048 inputs (exact within 2^25
 * of the wave's largest value; a wave with a value outside that window, and binary32 x,
 * use one binary32 FMA per input instead), and the matrix-core kernels (2 <= M <= 16;
 * M = 2 stays on the one-row kernel unless the matrix has more than 16384 rows and
 * K <= 8192) as binary16 x * 2^-E with binary16 codes where x converts exactly (on
 * matrices with K <= 8192 and at least 48 rows per compute unit, E per wave; on the
 * others with M <= 4, E per wave and row of x), else as bf16 with bf16 q - zero codes.
 *   prepared  from w4_prepare (256-B aligned).
 *   x         [M, K] row-major, bfloat16 (xt = W4_BF16) or binary32 (W4_F32); 16-B aligned.
 *   y         [M, N] row-major, binary32 (yt = W4_F32) or bfloat16 (W4_BF16); must
 *             not overlap the inputs; 4-B aligned.
 * Requires K <= W4_GEMV_MAX_K.  Accumulates in binary32; deterministic (no atomics).
 */
w4_status w4_gemv(const void* prepared, int64_t N, int64_t K,
                  const void* x, w4_dtype xt, int64_t M,
                  void* y, w4_dtype yt, hipStream_t stream);

/*
 * Storage variants of the format (page "Quantization" › "Code": int4 groups of 128
 * and of 32; page "Weight quantization" › "Implementation notes": scales kept in fp16
 * or bf16; "Code" and "Complexity and constants": a 4-bit zero per group).
 *   group       32, 64 or 128 consecutive inputs of one row share a scale and a zero.
 *   scale_bf16  0: scales are binary16 bit patterns; 1: bfloat16 bit patterns.  Either
 *               is the binary32 step rounded to nearest even.
 *   zero_bits   8: zeros [N, K/group] bytes; 4: two zeros per byte over the flat
 *               [N, K/group] array (index i at byte i/2, even index in the low nibble),
 *               ceil(N*K/group / 2) bytes.
 *   symmetric   0: the asymmetric method of w4_quantize; 1: that of
 *               w4_quantize_symmetric (zero 8).
 * The codes and the binary32 step do not depend on the storage; {128, 0, 8, 0} is the
 * canonical format of w4_quantize and {128, 0, 8, 1} that of w4_quantize_symmetric.
 * The prepared layout of a format with group 128 and binary16 scales is the canonical
 * one (zeros are widened to the kernel's byte), so w4_gemv and w4_gemm take it; other
 * formats are read by w4_gemv_fmt only.  A format outside these values is refused with
 * W4_ERR_UNSUPPORTED.
 */
typedef struct {
    int32_t group;
    int32_t scale_bf16;
    int32_t zero_bits;
    int32_t symmetric;
} w4_format;

/* bytes of the zeros array of a format (0 for an invalid format or shape) */
size_t w4_zeros_bytes(int64_t N, int64_t K, const w4_format* fmt);

/*
 * w4_quantize_fmt -- w4_quantize / w4_quantize_symmetric in format *fmt.
 *   scales  out [N, K/group] 16-bit patterns of the format's scale type; 2-B aligned.
 *   zeros   out, w4_zeros_bytes(N, K, fmt) bytes.
 * Requires K % 128 == 0 (as every product does).  Other arguments, errors and d_status
 * bits as w4_quantize; with bfloat16 scales W4_STATUS_SCALE_OVERFLOW / _ZERO refer to
 * bfloat16 infinity / zero.
 */
w4_status w4_quantize_fmt(const void* W, w4_dtype wt, int64_t N, int64_t K,
                          const w4_format* fmt, uint8_t* packed, uint16_t* scales,
                          uint8_t* zeros, uint32_t* d_status, hipStream_t stream);

/*
 * w4_prepare_fmt / w4_unprepare_fmt -- the kernel layout of a format: the code region
 * of w4_prepare followed by one scale/zero word per row and group (four rows of one
 * group per 16 bytes).  Size w4_prepared_bytes_fmt(N, K, fmt); 256-B aligned.
 * w4_unprepare_fmt is the exact inverse.
 */
size_t w4_prepared_bytes_fmt(int64_t N, int64_t K, const w4_format* fmt);
w4_status w4_prepare_fmt(const uint8_t* packed, const uint16_t* scales, const uint8_t* zeros,
                         int64_t N, int64_t K, const w4_format* fmt, void* prepared,
                         size_t prepared_bytes, hipStream_t stream);
w4_status w4_unprepare_fmt(const void* prepared, int64_t N, int64_t K, const w4_format* fmt,
                           uint8_t* packed, uint16_t* scales, uint8_t* zeros,
                           hipStream_t stream);

/*
 * w4_gemv_fmt -- w4_gemv on the prepared layout of format *fmt (page "Weight
 * quantization", "How it works": scale * sum (code - zero) * x per group).  The
 * canonical-layout formats (group 128, binary16 scales) take w4_gemv's kernels; the
 * others run on its one-row (VALU) kernel at every M, in steps of up to four rows of x.
 * Arguments, limits and errors as w4_gemv.
 */
w4_status w4_gemv_fmt(const void* prepared, int64_t N, int64_t K, const w4_format* fmt,
                      const void* x, w4_dtype xt, int64_t M,
                      void* y, w4_dtype yt, hipStream_t stream);

/*
 * w4_gemm -- prefill-sized product Y[M, N] = X[M, K] * w_hat^T for any M >= 1
 * (page "LLM Quantization Architecture in Depth" › "Why fewer bits make
 * decoding faster": prefill is compute bound and weight-only formats must turn
 * weights back into 16-bit values before the matrix units).  The codes enter the
 * binary16 MFMA as the exact values q - zero and X as binary16 X * 2^-E[m] (E per
 * row, exact for every value within 2^28 of the row's largest); per group the f32
 * accumulator receives scale16 * P (page "Weight quantization", "How it works": the
 * dequantized weight (code - zero) * scale, one multiply per group), so no weight
 * and no activation is rounded.  Rows of X with a value outside that window are
 * recomputed by a fix-up pass with one binary32 FMA per weight.
 *   prepared  from w4_prepare.
 *   X         [M, K] bfloat16 row-major; 16-B aligned.
 *   Y         [M, N] row-major, binary32 or bfloat16; 4-B aligned.
 *   workspace device scratch of w4_gemm_workspace_bytes(M, N, K) bytes (the binary16
 *             copy of X, then per row its exponent and a window flag, each part
 *             256-B aligned), 16-B aligned; contents need no initialisation.  Calls
 *             sharing a workspace must be ordered.
 * Limits: N, K as w4_prepare and K <= W4_GEMM_MAX_K (the kernels address the operands of
 * a 128 x 256 tile with 32-bit offsets); 1 <= M <= 65535*128; at most 2^31 - 9 output
 * tiles of 128 x 256 (else W4_ERR_SHAPE; w4_gemm_workspace_bytes returns 0).
 */
size_t w4_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K);
w4_status w4_gemm(const void* prepared, int64_t N, int64_t K,
                  const void* X, int64_t M, void* Y, w4_dtype yt,
                  void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * w4_gemm_noalloc -- w4_gemm for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).  Same
 * product, same kernels, bit-identical Y; the workspace is a fixed array of
 * W4_GEMM_NOALLOC_MAX_WORKSPACE bytes in the library's device data, one copy per GPU,
 * held until the process ends.  The call allocates nothing (no hipMalloc, no allocating
 * library routine); its first call on a device looks up that device's copy once.
 *   Arguments, alignment and limits as w4_gemm, and in addition
 *   w4_gemm_workspace_bytes(M, N, K) <= W4_GEMM_NOALLOC_MAX_WORKSPACE, else
 *   W4_ERR_WORKSPACE before any device work (about M * K <= 8.3e6: M = 256 at
 *   K = 28672, M = 1024 at K = 8192).
 * Every call on one GPU shares that GPU's array, which keeps the last call's contents
 * (each call writes all it reads, nothing needs clearing): calls that may overlap on one
 * GPU -- on different streams without ordering, or from several threads -- race and give
 * undefined Y.  Order them on one stream, or use w4_gemm with workspaces of their own.
 */
#define W4_GEMM_NOALLOC_MAX_WORKSPACE (16u << 20)
w4_status w4_gemm_noalloc(const void* prepared, int64_t N, int64_t K,
                          const void* X, int64_t M, void* Y, w4_dtype yt, hipStream_t stream);

/*
 * W8A8 in FP8 E4M3 for prefill (page "LLM Quantization Architecture in Depth" › "Why fewer
 * bits make decoding faster": prefill is compute bound, so its arithmetic must be narrower,
 * with activations quantized too; › "Number formats, scales and granularity": E4M3, largest
 * value 448, dynamic per-token activation scales; page "Quantization" › "Code": FP8 E4M3
 * per-channel scaling, rounding to 3 mantissa bits with subnormals).
 *
 * w4_fp8_quantize_rows -- per-row E4M3 quantization of A [rows, K] (weights: one row per
 * output channel; activations: one row per token, at run time).
 *   scale[r] = max_k |A[r, k]| / 448 in binary64 (1 for an all-zero row), stored rounded to
 *   binary32; code = E4M3 byte of A[r, k] / scale[r] (binary64 quotient, magnitude capped at
 *   448, rounded halves-to-even on the grid of 3 mantissa bits of its binary exponent,
 *   exponents below -6 on the grid of -6).  Bytes are OCP E4M3: sign bit 7, exponent bits
 *   6..3 with bias 7, mantissa bits 2..0; 0x7E = 448; a value that rounds to zero keeps its
 *   sign (0x80); 0x7F/0xFF (NaN) are never written.
 *   A       [rows, K] row-major, binary32 (at = W4_F32) or bfloat16 (W4_BF16); 16-B aligned.
 *   codes   [rows, K] bytes, 16-B aligned.   scales  [rows] binary32, 4-B aligned.
 *   d_status  optional device word: bit 0 is OR-ed in if a row holds a non-finite value
 *             (its codes are then undefined).
 * Requires K a multiple of 128, 128 <= K <= W4_FP8_MAX_K.
 *
 * w4_fp8_gemm -- Y[m, n] = sx[m] * sw[n] * sum_k value(xq[m, k]) * value(wq[n, k]) on the
 * FP8 matrix cores with binary32 accumulation (each product of two E4M3 values is exact).
 *   xq, sx   [M, K] codes and [M] scales of the activations (w4_fp8_quantize_rows).
 *   wq, sw   [N, K] codes and [N] scales of the weights.
 *   Y        [M, N] row-major, binary32 (yt = W4_F32) or bfloat16 (W4_BF16); must not
 *            overlap the inputs.  Codes 16-B aligned, scales 4-B, Y 4-B (2-B for bf16).
 * Requires K a multiple of 128, 128 <= K <= W4_FP8_MAX_K.  Deterministic (no atomics).
 */
w4_status w4_fp8_quantize_rows(const void* A, w4_dtype at, int64_t rows, int64_t K,
                               uint8_t* codes, float* scales, uint32_t* d_status,
                               hipStream_t stream);
w4_status w4_fp8_gemm(const uint8_t* xq, const float* sx, int64_t M, const uint8_t* wq,
                      const float* sw, int64_t N, int64_t K, void* Y, w4_dtype yt,
                      hipStream_t stream);

/*
 * W8A8 in INT8 (page "Quantization" › "How it really works" and "Code": symmetric 8-bit
 * codes with one absmax scale per block; the architecture page names INT8 beside FP8 for
 * W8A8 prefill).
 *
 * w4_int8_quantize_rows -- per-row symmetric INT8: step[r] = max_k |A[r, k]| / 127 in
 *   binary64 (1 for an all-zero row), stored rounded to binary32; code = A[r, k] / step[r]
 *   in binary64, rounded to the nearest integer with halves to even, clamped to
 *   [-128, 127].  Arguments, alignment, limits and status as w4_fp8_quantize_rows, with
 *   codes [rows, K] int8.
 * w4_int8_gemm -- Y[m, n] = sx[m] * sw[n] * sum_k xq[m, k] * wq[n, k] on the INT8 matrix
 *   cores; the sums are exact int32 (|sum| <= K * 128 * 128 < 2^31 for K <= W4_FP8_MAX_K),
 *   then converted to binary32 and scaled.  Arguments, alignment and limits as
 *   w4_fp8_gemm.  Deterministic.
 */
w4_status w4_int8_quantize_rows(const void* A, w4_dtype at, int64_t rows, int64_t K,
                                int8_t* codes, float* scales, uint32_t* d_status,
                                hipStream_t stream);
w4_status w4_int8_gemm(const int8_t* xq, const float* sx, int64_t M, const int8_t* wq,
                       const float* sw, int64_t N, int64_t K, void* Y, w4_dtype yt,
                       hipStream_t stream);

/*
 * w4_stream_read -- measurement probe, not part of the method: reads `bytes` bytes of
 * device memory at `buf` once with plain streaming loads (8192 workgroups, each a
 * contiguous share, non-temporal 16-byte loads) and discards them, so a product's rate
 * can be compared with a kernel that only reads the same bytes in the same launch
 * pattern (page "Weight quantization", "Complexity and constants": decode time is bytes
 * read / bandwidth).
 *   buf   device memory, 16-B aligned; bytes a non-zero multiple of 16.
 *   sink  a device word the kernel may overwrite (it almost never does); 4-B aligned.
 * Errors: W4_ERR_NULL, W4_ERR_SHAPE, W4_ERR_ALIGN, W4_ERR_ARCH, W4_ERR_HIP.
 */
w4_status w4_stream_read(const void* buf, size_t bytes, uint32_t* sink, hipStream_t stream);

/* Text of a status code (static storage). */
const char* w4_status_string(w4_status s);
/* Message of the last W4_ERR_HIP on the calling thread ("" if none). */
const char* w4_last_hip_error(void);
/* W4_FORMAT_VERSION of the library (prepared-layout version). */
int w4_format_version(void);

#ifdef __cplusplus
}
#endif

#endif /* W4A16_H */
