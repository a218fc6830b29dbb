// Read-bandwidth probe: a plain streaming read of a buffer, the measuring stick for the
// products.  Decode time is bytes read / bandwidth (page "Weight quantization", sections
// "Complexity and constants" and "Efficiency"), so a product's rate is judged against what
// a kernel that only reads the same bytes, in the same launch pattern, achieves on the
// same device.
//
// Each workgroup of 256 threads reads one contiguous share of the buffer with
// non-temporal 16-byte loads, eight in flight per thread, and folds the words with XOR;
// the fold is written only if it equals a fixed word, so the loads cannot be dropped and
// almost never produce a store.
#include "w4_internal.h"

namespace w4 {
namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 8;
constexpr int kProbeGrid = 8192;   // fastest of the grids measured on MI355X for 35-250 MB
constexpr uint32_t kProbeMagic = 0x9E3779B9u;

__global__ __launch_bounds__(kProbeThreads) void stream_read_kernel(const u32x4_t* __restrict__ p,
                                                                    int64_t n16, int64_t per_wg,
                                                                    uint32_t* __restrict__ sink) {
    const int64_t b = (int64_t)blockIdx.x * per_wg;
    const int64_t e = b + per_wg < n16 ? b + per_wg : n16;
    uint32_t acc = 0;
    int64_t i = b + threadIdx.x;
    for (; i + (kProbeUnroll - 1) * kProbeThreads < e; i += kProbeUnroll * kProbeThreads) {
        u32x4_t v[kProbeUnroll];
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) v[u] = __builtin_nontemporal_load(p + i + u * kProbeThreads);
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < e; i += kProbeThreads) {
        const u32x4_t v = __builtin_nontemporal_load(p + i);
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    if (acc == kProbeMagic) sink[0] = acc;
}

}  // namespace

hipError_t launch_stream_read(const void* buf, int64_t bytes, uint32_t* sink, hipStream_t s) {
    const int64_t n16 = bytes / 16;
    const int64_t per_wg = (n16 + kProbeGrid - 1) / kProbeGrid;
    const unsigned grid = (unsigned)((n16 + per_wg - 1) / per_wg);
    hipLaunchKernelGGL(stream_read_kernel, dim3(grid), dim3(kProbeThreads), 0, s,
                       static_cast<const u32x4_t*>(buf), n16, per_wg, sink);
    return hipGetLastError();
}

}  // namespace w4
