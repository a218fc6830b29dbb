// C-ABI entry points of libw4a16: argument validation, device check, launch.
// The kernels live in w4_quantize.hip, w4_gemv.hip, w4_gemv_mfma.hip, w4_gemm.hip and
// w4_w8a8.hip.
#include <atomic>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "w4a16.h"
#include "w4_internal.h"

namespace {

thread_local std::string g_last_hip_error;

constexpr int kMaxDevices = 64;
std::atomic<int> g_arch_state[kMaxDevices];  // 0 unknown, 1 gfx950, 2 other

w4_status hip_fail(hipError_t e) {
    g_last_hip_error = hipGetErrorString(e);
    return W4_ERR_HIP;
}

w4_status check_arch() {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e);
    if (dev < 0 || dev >= kMaxDevices) return W4_ERR_ARCH;
    int st = g_arch_state[dev].load(std::memory_order_acquire);
    if (st == 0) {
        hipDeviceProp_t prop;
        e = hipGetDeviceProperties(&prop, dev);
        if (e != hipSuccess) return hip_fail(e);
        st = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
        g_arch_state[dev].store(st, std::memory_order_release);
    }
    return st == 1 ? W4_OK : W4_ERR_ARCH;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

w4_status check_nk(int64_t n, int64_t k) {
    if (n < 1 || k < W4_GROUP || k % W4_GROUP != 0) return W4_ERR_SHAPE;
    if (n > (int64_t)0x7FFFFFFF || k > (int64_t)0x7FFFFFFF) return W4_ERR_SHAPE;
    return W4_OK;
}

w4_status to_fmt(const w4_format* in, w4::Fmt* out) {
    if (!in) return W4_ERR_NULL;
    if ((in->group != 32 && in->group != 64 && in->group != 128) ||
        (in->scale_bf16 != 0 && in->scale_bf16 != 1) ||
        (in->zero_bits != 4 && in->zero_bits != 8) || (in->symmetric != 0 && in->symmetric != 1))
        return W4_ERR_UNSUPPORTED;
    out->group = in->group;
    out->scale_bf16 = in->scale_bf16 == 1;
    out->zero4 = in->zero_bits == 4;
    out->symmetric = in->symmetric == 1;
    return W4_OK;
}

}  // namespace

// Workspace of w4_gemm_noalloc.  In host code this name is only a stand-in for the
// symbol: its device address (one per GPU) comes from hipGetSymbolAddress and is the
// only form passed to kernels.
static __device__ __align__(256) uint8_t scratch[W4_GEMM_NOALLOC_MAX_WORKSPACE];

namespace {

std::atomic<void*> g_scratch_addr[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of the current device's scratch, looked up once per device.
w4_status scratch_address(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e);
    if (dev < 0 || dev >= kMaxDevices) return W4_ERR_ARCH;
    void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch_addr[dev].load(std::memory_order_relaxed);
        if (!p) {
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess) return hip_fail(e);
            if (!p) return W4_ERR_WORKSPACE;
            g_scratch_addr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return W4_OK;
}

}  // namespace

extern "C" {

const char* w4_status_string(w4_status s) {
    switch (s) {
        case W4_OK: return "ok";
        case W4_ERR_NULL: return "null pointer";
        case W4_ERR_SHAPE: return "unsupported shape";
        case W4_ERR_ALIGN: return "misaligned pointer";
        case W4_ERR_DTYPE: return "unsupported dtype";
        case W4_ERR_UNSUPPORTED: return "unsupported format";
        case W4_ERR_ARCH: return "device is not gfx950";
        case W4_ERR_WORKSPACE: return "workspace missing or too small";
        case W4_ERR_HIP: return "HIP runtime error";
        case W4_ERR_BUFFER: return "destination buffer too small";
    }
    return "unknown status";
}

const char* w4_last_hip_error(void) { return g_last_hip_error.c_str(); }

int w4_format_version(void) { return W4_FORMAT_VERSION; }

static w4_status quantize_common(const void* W, w4_dtype wt, int64_t N, int64_t K,
                                 uint8_t* packed, uint16_t* scales_f16, uint8_t* zeros,
                                 uint32_t* d_status, bool symmetric, hipStream_t stream) {
    if (!W || !packed || !scales_f16 || !zeros) return W4_ERR_NULL;
    if (wt != W4_F32 && wt != W4_BF16) return W4_ERR_DTYPE;
    w4_status st = check_nk(N, K);
    if (st != W4_OK) return st;
    if (!aligned(W, 16) || !aligned(packed, 16) || !aligned(scales_f16, 2) ||
        (d_status && !aligned(d_status, 4)))
        return W4_ERR_ALIGN;
    st = check_arch();
    if (st != W4_OK) return st;
    w4::Fmt f;
    f.symmetric = symmetric;
    hipError_t e = w4::launch_quantize(W, wt == W4_BF16, f, N * (K / W4_GROUP), packed,
                                       scales_f16, zeros, d_status, stream);
    return e == hipSuccess ? W4_OK : hip_fail(e);
}

w4_status w4_quantize(const void* W, w4_dtype wt, int64_t N, int64_t K, uint8_t* packed,
                      uint16_t* scales_f16, uint8_t* zeros, uint32_t* d_status,
                      hipStream_t stream) {
    return quantize_common(W, wt, N, K, packed, scales_f16, zeros, d_status, false, stream);
}

w4_status w4_quantize_symmetric(const void* W, w4_dtype wt, int64_t N, int64_t K,
                                uint8_t* packed, uint16_t* scales_f16, uint8_t* zeros,
                                uint32_t* d_status, hipStream_t stream) {
    return quantize_common(W, wt, N, K, packed, scales_f16, zeros, d_status, true, stream);
}

size_t w4_prepared_bytes(int64_t N, int64_t K) {
    if (check_nk(N, K) != W4_OK) return 0;
    return (size_t)w4::prepared_total(N, K);
}

w4_status w4_prepare(const uint8_t* packed, const uint16_t* scales_f16, const uint8_t* zeros,
                     int64_t N, int64_t K, void* prepared, size_t prepared_bytes,
                     hipStream_t stream) {
    if (!packed || !scales_f16 || !zeros || !prepared) return W4_ERR_NULL;
    w4_status st = check_nk(N, K);
    if (st != W4_OK) return st;
    if (!aligned(packed, 16) || !aligned(scales_f16, 2) || !aligned(prepared, 256))
        return W4_ERR_ALIGN;
    if (prepared_bytes < w4_prepared_bytes(N, K)) return W4_ERR_BUFFER;
    st = check_arch();
    if (st != W4_OK) return st;
    hipError_t e = w4::launch_prepare(packed, scales_f16, zeros, N, K, w4::Fmt{},
                                      static_cast<uint8_t*>(prepared), stream);
    return e == hipSuccess ? W4_OK : hip_fail(e);
}

w4_status w4_unprepare(const void* prepared, int64_t N, int64_t K, uint8_t* packed,
                       uint16_t* scales_f16, uint8_t* zeros, hipStream_t stream) {
    if (!packed || !scales_f16 || !zeros || !prepared) return W4_ERR_NULL;
    w4_status st = check_nk(N, K);
    if (st != W4_OK) return st;
    if (!aligned(packed, 16) || !aligned(scales_f16, 2) || !aligned(prepared, 256))
        return W4_ERR_ALIGN;
    st = check_arch();
    if (st != W4_OK) return st;
    hipError_t e = w4::launch_unprepare(static_cast<const uint8_t*>(prepared), N, K, w4::Fmt{}, packed,
                                        scales_f16, zeros, stream);
    return e == hipSuccess ? W4_OK : hip_fail(e);
}

w4_status w4_gemv(const void* prepared, int64_t N, int64_t K, const void* x, w4_dtype xt,
                  int64_t M, void* y, w4_dtype yt, hipStream_t stream) {
    if (!prepared || !x || !y) return W4_ERR_NULL;
    if ((xt != W4_F32 && xt != W4_BF16) || (yt != W4_F32 && yt != W4_BF16)) return W4_ERR_DTYPE;
    w4_status st = check_nk(N, K);
    if (st != W4_OK) return st;
    if (K > W4_GEMV_MAX_K || M < 1 || M > W4_GEMV_MAX_M) return W4_ERR_SHAPE;
    if (!aligned(prepared, 256) || !aligned(x, 16) || !aligned(y, yt == W4_F32 ? 4 : 2))
        return W4_ERR_ALIGN;
    st = check_arch();
    if (st != W4_OK) return st;
    hipError_t e = w4::launch_gemv(static_cast<const uint8_t*>(prepared), N, K, x, xt == W4_F32,
                                   M, y, yt == W4_BF16, stream);
    return e == hipSuccess ? W4_OK : hip_fail(e);
}

size_t w4_zeros_bytes(int64_t N, int64_t K, const w4_format* fmt) {
    w4::Fmt f;
    if (to_fmt(fmt, &f) != W4_OK || check_nk(N, K) != W4_OK) return 0;
    const int64_t groups = N * (K / f.group);
    return (size_t)(f.zero4 ? (groups + 1) / 2 : groups);
}

w4_status w4_quantize_fmt(const void* W, w4_dtype wt, int64_t N, int64_t K,
                          const w4_format* fmt, uint8_t* packed, uint16_t* scales,
                          uint8_t* zeros, uint32_t* d_status, hipStream_t stream) {
    if (!W || !packed || !scales || !zeros || !fmt) return W4_ERR_NULL;
    w4::Fmt f;
    w4_status st = to_fmt(fmt, &f);
    if (st != W4_OK) return st;
    if (wt != W4_F32 && wt != W4_BF16) return W4_ERR_DTYPE;
    st = check_nk(N, K);
    if (st != W4_OK) return st;
    if (!aligned(W, 16) || !aligned(packed, 16) || !aligned(scales, 2) ||
        (d_status && !aligned(d_status, 4)))
        return W4_ERR_ALIGN;
    st = check_arch();
    if (st != W4_OK) return st;
    hipError_t e = w4::launch_quantize(W, wt == W4_BF16, f, N * (K / f.group), packed, scales,
                                       zeros, d_status, stream);
    return e == hipSuccess ? W4_OK : hip_fail(e);
}

size_t w4_prepared_bytes_fmt(int64_t N, int64_t K, const w4_format* fmt) {
    w4::Fmt f;
    if (to_fmt(fmt, &f) != W4_OK || check_nk(N, K) != W4_OK) return 0;
    return (size_t)w4::prepared_total_g(N, K, f.group);
}

w4_status w4_prepare_fmt(const uint8_t* packed, const uint16_t* scales, const uint8_t* zeros,
                         int64_t N, int64_t K, const w4_format* fmt, void* prepared,
                         size_t prepared_bytes, hipStream_t stream) {
    if (!packed || !scales || !zeros || !prepared || !fmt) return W4_ERR_NULL;
    w4::Fmt f;
    w4_status st = to_fmt(fmt, &f);
    if (st != W4_OK) return st;
    st = check_nk(N, K);
    if (st != W4_OK) return st;
    if (!aligned(packed, 16) || !aligned(scales, 2) || !aligned(prepared, 256))
        return W4_ERR_ALIGN;
    if (prepared_bytes < w4_prepared_bytes_fmt(N, K, fmt)) return W4_ERR_BUFFER;
    st = check_arch();
    if (st != W4_OK) return st;
    hipError_t e = w4::launch_prepare(packed, scales, zeros, N, K, f,
                                      static_cast<uint8_t*>(prepared), stream);
    return e == hipSuccess ? W4_OK : hip_fail(e);
}

w4_status w4_unprepare_fmt(const void* prepared, int64_t N, int64_t K, const w4_format* fmt,
                           uint8_t* packed, uint16_t* scales, uint8_t* zeros,
                           hipStream_t stream) {
    if (!packed || !scales || !zeros || !prepared || !fmt) return W4_ERR_NULL;
    w4::Fmt f;
    w4_status st = to_fmt(fmt, &f);
    if (st != W4_OK) return st;
    st = check_nk(N, K);
    if (st != W4_OK) return st;
    if (!aligned(packed, 16) || !aligned(scales, 2) || !aligned(prepared, 256))
        return W4_ERR_ALIGN;
    st = check_arch();
    if (st != W4_OK) return st;
    hipError_t e = w4::launch_unprepare(static_cast<const uint8_t*>(prepared), N, K, f, packed,
                                        scales, zeros, stream);
    return e == hipSuccess ? W4_OK : hip_fail(e);
}

w4_status w4_gemv_fmt(const void* prepared, int64_t N, int64_t K, const w4_format* fmt,
                      const void* x, w4_dtype xt, int64_t M, void* y, w4_dtype yt,
                      hipStream_t stream) {
    if (!fmt) return W4_ERR_NULL;
    w4::Fmt f;
    w4_status st = to_fmt(fmt, &f);
    if (st != W4_OK) return st;
    if (f.group == W4_GROUP && !f.scale_bf16)
        return w4_gemv(prepared, N, K, x, xt, M, y, yt, stream);
    if (!prepared || !x || !y) return W4_ERR_NULL;
    if ((xt != W4_F32 && xt != W4_BF16) || (yt != W4_F32 && yt != W4_BF16)) return W4_ERR_DTYPE;
    st = check_nk(N, K);
    if (st != W4_OK) return st;
    if (K > W4_GEMV_MAX_K || M < 1 || M > W4_GEMV_MAX_M) return W4_ERR_SHAPE;
    if (!aligned(prepared, 256) || !aligned(x, 16) || !aligned(y, yt == W4_F32 ? 4 : 2))
        return W4_ERR_ALIGN;
    st = check_arch();
    if (st != W4_OK) return st;
    hipError_t e = w4::launch_gemv_dot2(static_cast<const uint8_t*>(prepared), N, K, f.group,
                                        f.scale_bf16, x, xt == W4_F32, M, y, yt == W4_BF16,
                                        stream);
    return e == hipSuccess ? W4_OK : hip_fail(e);
}

size_t w4_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K) {
    if (M < 1 || check_nk(N, K) != W4_OK || K > W4_GEMM_MAX_K) return 0;
    return w4::gemm_workspace(M, K);
}

w4_status w4_gemm(const void* prepared, int64_t N, int64_t K, const void* X, int64_t M, void* Y,
                  w4_dtype yt, void* workspace, size_t workspace_bytes, hipStream_t stream) {
    if (!prepared || !X || !Y) return W4_ERR_NULL;
    if (yt != W4_F32 && yt != W4_BF16) return W4_ERR_DTYPE;
    w4_status st = check_nk(N, K);
    if (st != W4_OK) return st;
    if (K > W4_GEMM_MAX_K || M < 1 || (M + 127) / 128 > 65535) return W4_ERR_SHAPE;
    // the tile count (128 x 256 output tiles, padded to a multiple of 8) is a grid size
    if (((M + 127) / 128) * ((N + 255) / 256) > (int64_t)INT32_MAX - 8) return W4_ERR_SHAPE;
    if (!workspace || workspace_bytes < w4_gemm_workspace_bytes(M, N, K)) return W4_ERR_WORKSPACE;
    if (!aligned(prepared, 256) || !aligned(X, 16) || !aligned(Y, yt == W4_F32 ? 4 : 2) ||
        !aligned(workspace, 16))
        return W4_ERR_ALIGN;
    st = check_arch();
    if (st != W4_OK) return st;
    hipError_t e = w4::launch_gemm(static_cast<const uint8_t*>(prepared), N, K, X, M, Y,
                                   yt == W4_BF16, workspace, stream);
    return e == hipSuccess ? W4_OK : hip_fail(e);
}

w4_status w4_gemm_noalloc(const void* prepared, int64_t N, int64_t K, const void* X, int64_t M,
                          void* Y, w4_dtype yt, hipStream_t stream) {
    if (!prepared || !X || !Y) return W4_ERR_NULL;
    if (yt != W4_F32 && yt != W4_BF16) return W4_ERR_DTYPE;
    w4_status st = check_nk(N, K);
    if (st != W4_OK) return st;
    if (K > W4_GEMM_MAX_K || M < 1 || (M + 127) / 128 > 65535) return W4_ERR_SHAPE;
    if (((M + 127) / 128) * ((N + 255) / 256) > (int64_t)INT32_MAX - 8) return W4_ERR_SHAPE;
    if (w4_gemm_workspace_bytes(M, N, K) > W4_GEMM_NOALLOC_MAX_WORKSPACE) return W4_ERR_WORKSPACE;
    if (!aligned(prepared, 256) || !aligned(X, 16) || !aligned(Y, yt == W4_F32 ? 4 : 2))
        return W4_ERR_ALIGN;
    st = check_arch();
    if (st != W4_OK) return st;
    void* ws = nullptr;
    st = scratch_address(&ws);
    if (st != W4_OK) return st;
    hipError_t e = w4::launch_gemm(static_cast<const uint8_t*>(prepared), N, K, X, M, Y,
                                   yt == W4_BF16, ws, stream);
    return e == hipSuccess ? W4_OK : hip_fail(e);
}

w4_status w4_fp8_quantize_rows(const void* A, w4_dtype at, int64_t rows, int64_t K,
                               uint8_t* codes, float* scales, uint32_t* d_status,
                               hipStream_t stream) {
    if (!A || !codes || !scales) return W4_ERR_NULL;
    if (at != W4_F32 && at != W4_BF16) return W4_ERR_DTYPE;
    if (rows < 1 || rows > (int64_t)INT32_MAX || K < W4_GROUP || K % W4_GROUP != 0 ||
        K > W4_FP8_MAX_K)
        return W4_ERR_SHAPE;
    if (!aligned(A, 16) || !aligned(codes, 16) || !aligned(scales, 4) || !aligned(d_status, 4))
        return W4_ERR_ALIGN;
    w4_status st = check_arch();
    if (st != W4_OK) return st;
    hipError_t e = w4::launch_w8_quantize_rows(A, at == W4_BF16, rows, K, codes, scales,
                                                d_status, stream);
    return e == hipSuccess ? W4_OK : hip_fail(e);
}

w4_status w4_fp8_gemm(const uint8_t* xq, const float* sx, int64_t M, const uint8_t* wq,
                      const float* sw, int64_t N, int64_t K, void* Y, w4_dtype yt,
                      hipStream_t stream) {
    if (!xq || !sx || !wq || !sw || !Y) return W4_ERR_NULL;
    if (yt != W4_F32 && yt != W4_BF16) return W4_ERR_DTYPE;
    if (M < 1 || N < 1 || M > (int64_t)INT32_MAX || N > (int64_t)INT32_MAX || K < W4_GROUP ||
        K % W4_GROUP != 0 || K > W4_FP8_MAX_K)
        return W4_ERR_SHAPE;
    const int64_t tiles = ((M + 127) / 128) * ((N + 127) / 128);
    if (tiles > (int64_t)INT32_MAX) return W4_ERR_SHAPE;
    if (!aligned(xq, 16) || !aligned(wq, 16) || !aligned(sx, 4) || !aligned(sw, 4) ||
        !aligned(Y, yt == W4_F32 ? 4 : 2))
        return W4_ERR_ALIGN;
    w4_status st = check_arch();
    if (st != W4_OK) return st;
    hipError_t e = w4::launch_fp8_gemm(xq, sx, M, wq, sw, N, K, Y, yt == W4_BF16, stream);
    return e == hipSuccess ? W4_OK : hip_fail(e);
}

w4_status w4_int8_quantize_rows(const void* A, w4_dtype at, int64_t rows, int64_t K,
                                int8_t* codes, float* scales, uint32_t* d_status,
                                hipStream_t stream) {
    if (!A || !codes || !scales) return W4_ERR_NULL;
    if (at != W4_F32 && at != W4_BF16) return W4_ERR_DTYPE;
    if (rows < 1 || rows > (int64_t)INT32_MAX || K < W4_GROUP || K % W4_GROUP != 0 ||
        K > W4_FP8_MAX_K)
        return W4_ERR_SHAPE;
    if (!aligned(A, 16) || !aligned(codes, 16) || !aligned(scales, 4) || !aligned(d_status, 4))
        return W4_ERR_ALIGN;
    w4_status st = check_arch();
    if (st != W4_OK) return st;
    hipError_t e = w4::launch_w8_quantize_rows(A, at == W4_BF16, rows, K,
                                                reinterpret_cast<uint8_t*>(codes), scales,
                                                d_status, stream, true);
    return e == hipSuccess ? W4_OK : hip_fail(e);
}

w4_status w4_int8_gemm(const int8_t* xq, const float* sx, int64_t M, const int8_t* wq,
                       const float* sw, int64_t N, int64_t K, void* Y, w4_dtype yt,
                       hipStream_t stream) {
    if (!xq || !sx || !wq || !sw || !Y) return W4_ERR_NULL;
    if (yt != W4_F32 && yt != W4_BF16) return W4_ERR_DTYPE;
    if (M < 1 || N < 1 || M > (int64_t)INT32_MAX || N > (int64_t)INT32_MAX || K < W4_GROUP ||
        K % W4_GROUP != 0 || K > W4_FP8_MAX_K)
        return W4_ERR_SHAPE;
    const int64_t tiles = ((M + 127) / 128) * ((N + 255) / 256);
    if (tiles > (int64_t)INT32_MAX) return W4_ERR_SHAPE;
    if (!aligned(xq, 16) || !aligned(wq, 16) || !aligned(sx, 4) || !aligned(sw, 4) ||
        !aligned(Y, yt == W4_F32 ? 4 : 2))
        return W4_ERR_ALIGN;
    w4_status st = check_arch();
    if (st != W4_OK) return st;
    hipError_t e = w4::launch_int8_gemm(reinterpret_cast<const uint8_t*>(xq), sx, M,
                                        reinterpret_cast<const uint8_t*>(wq), sw, N, K, Y,
                                        yt == W4_BF16, stream);
    return e == hipSuccess ? W4_OK : hip_fail(e);
}

w4_status w4_stream_read(const void* buf, size_t bytes, uint32_t* sink, hipStream_t stream) {
    if (!buf || !sink) return W4_ERR_NULL;
    if (bytes == 0 || bytes % 16 != 0) return W4_ERR_SHAPE;
    if (!aligned(buf, 16) || !aligned(sink, 4)) return W4_ERR_ALIGN;
    w4_status st = check_arch();
    if (st != W4_OK) return st;
    hipError_t e = w4::launch_stream_read(buf, (int64_t)bytes, sink, stream);
    return e == hipSuccess ? W4_OK : hip_fail(e);
}

}  // extern "C"
