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
//   * a workgroup holds ceil(K/2048) waves and walks rows_per_wg rows in
//     chunks of CH steps of four rows; x is loaded first, then all loads of a
//     chunk are issued before any is used (a scheduling barrier keeps them
//     there), so step c computes while the later steps are still arriving and
//     the compiler's in-order wait counts stay exact (no load crosses a loop
//     iteration);
//   * groups of up to eight waves end the launch with a round of workgroups that take
//     half the rows of the others, which shortens the tail of the weight stream;
//   * the scale/zero words of the four rows of a step are one 16-byte load;
//   * unpack: v_and_or_b32((word >> 4j), 0x000F000F, 0x43004300) turns the two
//     codes of an input pair into the bf16 values 128+q, and v_dot2_f32_bf16
//     multiplies the pair by the matching x pair and accumulates in f32:
//     D = sum (128+q)*x.  The slice sum S = sum x is computed once per
//     workgroup by the same instruction sequence with the pair (1, 1), so the
//     slice's share of the group term is scale16 * (D - (128 + zero) * S) =
//     scale16 * (sum q*x - zero * sum x).  Because scaling by 128 commutes
//     with rounding, a slice whose codes are all 0 gives D = 128*S exactly and
//     contributes exactly 0, and a one-hot x gives exactly (q - zero)*scale16;
//   * reduction of the four rows across the wave: v_permlane32_swap and
//     v_permlane16_swap transpose-and-add (each lane ends with one row), DPP
//     row rotations finish the 16-lane sums; waves are combined through LDS.
//     No atomics, so results are deterministic.
// Binary32 activations are split into two bf16 parts (hi = bf16(x),
// lo = bf16(x - hi)) that are accumulated separately and added at the end.
#include <atomic>
#include <cstdlib>

#include "w4_internal.h"

namespace w4 {
namespace {

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kRowsPerStep = 4;

// one 16-byte weight slice, marked non-temporal: every byte is read exactly once
__device__ __forceinline__ u32x4_t load_stream(const u32x4_t* p) { return __builtin_nontemporal_load(p); }

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

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                                 0xF, 0xF, false));
}

// exchange the upper 32 lanes of a with the lower 32 lanes of b
__device__ __forceinline__ void swap32(float& a, float& b) {
    const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, a),
                                                    __builtin_bit_cast(uint32_t, b), false, false);
    a = __builtin_bit_cast(float, (uint32_t)r[0]);
    b = __builtin_bit_cast(float, (uint32_t)r[1]);
}

// exchange the odd 16-lane rows of a with the even 16-lane rows of b
__device__ __forceinline__ void swap16(float& a, float& b) {
    const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, a),
                                                    __builtin_bit_cast(uint32_t, b), false, false);
    a = __builtin_bit_cast(float, (uint32_t)r[0]);
    b = __builtin_bit_cast(float, (uint32_t)r[1]);
}

// four per-lane row values -> lane l holds the wave-wide sum of row (l >> 4) & 3
__device__ __forceinline__ float reduce4(float a0, float a1, float a2, float a3) {
    swap32(a0, a2);
    swap32(a1, a3);
    float k0 = a0 + a2;  // lanes 0-31: row 0, lanes 32-63: row 2
    float k1 = a1 + a3;  // lanes 0-31: row 1, lanes 32-63: row 3
    swap16(k0, k1);
    float k = k0 + k1;   // 16-lane row r of the wave holds output row r
    k += dpp<0x128>(k);  // row_ror:8
    k += dpp<0x124>(k);  // row_ror:4
    k += dpp<0x122>(k);  // row_ror:2
    k += dpp<0x121>(k);  // row_ror:1
    return k;
}

// SBF16: the scale bits are bfloat16 (else binary16); gshift: log2(group / 32), the slices
// of one group (a group of 32, 64 or 128 inputs has its own scale/zero word)
template <int MT, bool XF32, int SPT, int MAXT, int CH, bool RAGGED, bool SBF16>
__global__ __launch_bounds__(MAXT) void gemv_kernel(const u32x4_t* __restrict__ wq,
                                                    const u32x4_t* __restrict__ sz4,
                                                    const void* __restrict__ xv,
                                                    void* __restrict__ yv, int y_bf16, int N,
                                                    int K, int M, int rows_per_wg, int gshift,
                                                    int tail_first, int tail_rows) {
    constexpr int XE = XF32 ? 2 * MT : MT;  // bf16 operand rows
    constexpr int R = kRowsPerStep;
    extern __shared__ float red[];          // [waves][rows_per_wg][XE]

    const int S = K >> 5;
    const int Kg = K >> (5 + gshift);
    const int T = blockDim.x;
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int n_waves = T >> 6;
    // workgroups from tail_first on (the last ones dispatched) take tail_rows rows each, so
    // the launch ends on short workgroups; rows_per_wg is the LDS row stride of both kinds
    const int row_stride = rows_per_wg;
    const bool in_tail = (int)blockIdx.x >= tail_first;
    const int r0 = in_tail ? tail_first * rows_per_wg + ((int)blockIdx.x - tail_first) * tail_rows
                           : (int)blockIdx.x * rows_per_wg;
    if (in_tail) rows_per_wg = tail_rows;
    const int r_end = min(N, r0 + rows_per_wg);

    // slice j of this lane is threadIdx.x + j*T (16 bytes of every row).  With a ragged
    // K the lanes past the last slice read the last slice and their x is zero.
    int sl[SPT];
    bool act[SPT];
    uint32_t woff[SPT], soff[SPT];
#pragma unroll
    for (int j = 0; j < SPT; ++j) {
        sl[j] = threadIdx.x + j * T;
        act[j] = RAGGED ? sl[j] < S : true;
        const int slc = RAGGED ? min(sl[j], S - 1) : sl[j];
        woff[j] = (uint32_t)slc * 16u;
        soff[j] = (uint32_t)(slc >> gshift) * 16u;
    }

    // ---- x slices first: their loads complete before the weight stream that follows
    uint32_t xr[SPT][XE][16];
    float sx[SPT][XE];
#pragma unroll
    for (int j = 0; j < SPT; ++j) {
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            const bool ok = act[j] && (MT == 1 || m < M);  // zero x for idle lanes and absent rows
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
    }

    __builtin_amdgcn_sched_barrier(0);  // keep the x loads ahead of the weight stream

    // constants of the unpack kept in registers so v_and_or_b32 is selected
    uint32_t nib_mask, bias_bits;
    asm volatile("s_mov_b32 %0, 0x000F000F" : "=s"(nib_mask));
    asm volatile("v_mov_b32 %0, 0x43004300" : "=v"(bias_bits));

    const char* wbase = reinterpret_cast<const char*>(wq);
    const char* sbase = reinterpret_cast<const char*>(sz4);
    const int64_t row_bytes = (int64_t)S * 16;

    // rows_per_wg is a multiple of CH*4: every chunk is whole; rows past N repeat row N-1
    // (their sums are never stored)
    u32x4_t wb[CH][R][SPT];
    u32x4_t sb[CH][SPT];
    auto issue_chunk = [&](int c0) {
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const int rb = r0 + c0 + c * R;
            const char* srow = sbase + (int64_t)(min(rb, N - 1) >> 2) * Kg * 16;
#pragma unroll
            for (int j = 0; j < SPT; ++j) sb[c][j] = *reinterpret_cast<const u32x4_t*>(srow + soff[j]);
#pragma unroll
            for (int rr = 0; rr < R; ++rr) {
                const char* rowp = wbase + (int64_t)min(rb + rr, N - 1) * row_bytes;
#pragma unroll
                for (int j = 0; j < SPT; ++j)
                    wb[c][rr][j] = load_stream(reinterpret_cast<const u32x4_t*>(rowp + woff[j]));
            }
            // loads stay in step order, so step c only waits for its own loads
            __builtin_amdgcn_sched_barrier(0);
        }
        // every load of the chunk is issued before any of it is used: step c computes while
        // the loads of the later steps are still in flight
    };
    auto compute_chunk = [&](int c0) {
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            float acc[R][XE];
#pragma unroll
            for (int rr = 0; rr < R; ++rr)
#pragma unroll
                for (int e = 0; e < XE; ++e) acc[rr][e] = 0.0f;
#pragma unroll
            for (int j = 0; j < SPT; ++j) {
#pragma unroll
                for (int rr = 0; rr < R; ++rr) {
                    const uint32_t szw = sb[c][j][rr];
                    const float s = SBF16 ? __uint_as_float(szw << 16)
                                          : (float)__builtin_bit_cast(_Float16, (uint16_t)(szw & 0xFFFFu));
                    const float zb = (float)((szw >> 16) & 0xFFu);  // zero + 128
                    uint32_t pr[16];
#pragma unroll
                    for (int t = 0; t < 4; ++t)
#pragma unroll
                        for (int q = 0; q < 4; ++q)
                            pr[4 * t + q] = ((wb[c][rr][j][t] >> (4 * q)) & nib_mask) | bias_bits;
#pragma unroll
                    for (int e = 0; e < XE; ++e) {
                        float d = 0.0f;
#pragma unroll
                        for (int i = 0; i < 16; ++i) d = dot2(pr[i], xr[j][e][i], d);
                        acc[rr][e] = fmaf(s, fmaf(-zb, sx[j][e], d), acc[rr][e]);
                    }
                }
            }
            if constexpr (RAGGED) {
                // lanes past the last slice read real (unrelated) scales; drop their terms
                bool any_off = false;
#pragma unroll
                for (int j = 0; j < SPT; ++j) any_off |= !act[j];
                if (any_off)
#pragma unroll
                    for (int rr = 0; rr < R; ++rr)
#pragma unroll
                        for (int e = 0; e < XE; ++e) acc[rr][e] = 0.0f;
            }
            const int rbase = c0 + c * R;
#pragma unroll
            for (int e = 0; e < XE; ++e) {
                const float k = reduce4(acc[0][e], acc[1][e], acc[2][e], acc[3][e]);
                if ((lane & 15) == 0) red[(wave * row_stride + rbase + (lane >> 4)) * XE + e] = k;
            }
        }
    };

    issue_chunk(0);
#pragma unroll
    for (int j = 0; j < SPT; ++j)
#pragma unroll
        for (int e = 0; e < XE; ++e) sx[j][e] = pair_sum(xr[j][e]);
    compute_chunk(0);
    for (int c0 = CH * R; c0 < rows_per_wg; c0 += CH * R) {
        issue_chunk(c0);
        compute_chunk(c0);
    }
    __syncthreads();

    const int rows_here = r_end - r0;
    for (int t = threadIdx.x; t < rows_here * MT; t += T) {
        const int rloc = t / MT;
        const int m = t - rloc * MT;
        if (m >= M) continue;
        float v = 0.0f;
        for (int w = 0; w < n_waves; ++w) {
            const float* p = red + (w * row_stride + rloc) * XE;
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
    const u32x4_t* sz4;
    const void* x;
    void* y;
    int y_bf16, n, k, m, rows;
    int gshift;       // log2(group / 32)
    bool scale_bf16;
};

int env_int(const char* name, int dflt) {
    const char* e = getenv(name);
    return e ? atoi(e) : dflt;
}

constexpr int kMaxRowsPerWg = 64;

int compute_units() {
    static std::atomic<int> cached{0};
    int v = cached.load(std::memory_order_relaxed);
    if (v > 0) return v;
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
        cus = 256;
    cached.store(cus, std::memory_order_relaxed);
    return cus;
}

// Rows per workgroup chosen from the number of resident workgroups: a whole
// number of rounds (see below), rows a multiple of the chunk.
template <typename Kern>
int rows_for(Kern kernel, int block, int n, int xe, int chunk_rows, std::atomic<int>* cache) {
    const int waves = block / 64;
    int resident = cache[waves].load(std::memory_order_relaxed);
    if (resident == 0) {
        const size_t smem = (size_t)waves * kMaxRowsPerWg * xe * sizeof(float);
        int r = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&r, kernel, block, smem) != hipSuccess || r < 1)
            r = 1;
        cache[waves].store(r, std::memory_order_relaxed);
        resident = r;
    }
    static const int forced = env_int("W4A16_GEMV_ROWS", 0);
    static const int forced_rounds = env_int("W4A16_GEMV_ROUNDS", 0);
    // measured on MI355X: groups of up to 8 waves stream best with about three rounds of
    // resident groups (finer work, shorter tail); the 14-wave groups of K ~ 28K with one
    int rounds = forced_rounds > 0 ? forced_rounds : (waves <= 8 ? 3 : 1);
    int rows;
    if (forced > 0) {
        rows = forced;
    } else {
        const long wgs = (long)resident * compute_units() * rounds;
        rows = (int)((n + wgs - 1) / wgs);
    }
    rows = (rows + chunk_rows - 1) / chunk_rows * chunk_rows;
    if (rows < chunk_rows) rows = chunk_rows;
    if (rows > kMaxRowsPerWg) rows = kMaxRowsPerWg / chunk_rows * chunk_rows;
    return rows;
}

template <int MT, bool XF32, int SPT, int MAXT, int CH, bool RAGGED, bool SBF16>
hipError_t launch_var(GemvArgs a, dim3 block, hipStream_t s) {
    constexpr int XE = XF32 ? 2 * MT : MT;
    static std::atomic<int> cache[17];
    auto kern = gemv_kernel<MT, XF32, SPT, MAXT, CH, RAGGED, SBF16>;
    a.rows = rows_for(kern, (int)block.x, a.n, XE, CH * kRowsPerStep, cache);
    unsigned wgs = (unsigned)((a.n + a.rows - 1) / a.rows);
    // A short last round: the last round of resident workgroups takes 1/tail of the rows.
    // Workgroups start in index order as earlier ones finish, so the final ones otherwise
    // start late with a full share and stream alone at the end.  Measured on MI355X
    // (57344x8192 at M = 1): 38.3-38.4 us against 39.5-40.0 us; the one-round 14-wave
    // groups of K ~ 28K run slower with it, so they keep equal shares.
    int tail_first = (int)wgs, tail_rows = a.rows;
    static const int tail_env = env_int("W4A16_GEMV_TAIL", -1);
    const int tail = tail_env >= 0 ? tail_env : (block.x <= 512 ? 2 : 0);
    static const int tail_rounds = env_int("W4A16_GEMV_TAILROUNDS", 1);
    const int half = tail > 0 ? a.rows / tail : 0;
    if (tail > 1 && half * tail == a.rows && half >= CH * kRowsPerStep && half % (CH * kRowsPerStep) == 0) {
        const long round = (long)cache[block.x / 64].load(std::memory_order_relaxed) * compute_units();
        const long tail_rows_total = round * tail_rounds * half;
        const long main_wgs = ((long)a.n - tail_rows_total) / a.rows;
        if (main_wgs > 0) {
            tail_first = (int)main_wgs;
            tail_rows = half;
            const long rest = (long)a.n - main_wgs * a.rows;
            wgs = (unsigned)(main_wgs + (rest + half - 1) / half);
        }
    }
    const dim3 grid(wgs);
    const size_t shmem = (size_t)(block.x / 64) * a.rows * XE * sizeof(float);
    hipLaunchKernelGGL(kern, grid, block, shmem, s, a.wq, a.sz4, a.x, a.y, a.y_bf16, a.n, a.k, a.m,
                       a.rows, a.gshift, tail_first, tail_rows);
    return hipGetLastError();
}

template <int MT, bool XF32, int SPT, int MAXT, int CH, bool SBF16>
hipError_t launch_one(const GemvArgs& a, dim3 block, hipStream_t s) {
    const bool ragged = (int)block.x * SPT * 32 != a.k;
    return ragged ? launch_var<MT, XF32, SPT, MAXT, CH, true, SBF16>(a, block, s)
                  : launch_var<MT, XF32, SPT, MAXT, CH, false, SBF16>(a, block, s);
}

// Instantiated variants (MT = rows of x per launch, SPT = 16-byte slices per lane,
// CH = steps of four rows whose loads are issued together):
//   M=1 bf16:   SPT 1, up to 1024 threads (K <= 32768), CH 2 or 4
//   otherwise:  up to 512 threads; SPT 1 for K <= 16384, SPT 2 up to 32768; CH 2 (1 for
//               the SPT 2 variants with two x rows); MT up to 4 (bf16, SPT 1), 2 (bf16,
//               SPT 2 / f32, SPT 1), 1 (f32, SPT 2) so that the registers fit the
//               256-VGPR budget of a 512-thread group
int max_mt(bool x_f32, int spt) {
    if (!x_f32) return spt == 1 ? 4 : 2;
    return spt == 1 ? 2 : 1;
}

// SB: bfloat16 scale bits (the format variants take the default load chunk only)
template <bool SB>
hipError_t dispatch_t(bool x_f32, int spt, int mt, const GemvArgs& a, dim3 block, hipStream_t s) {
    static const int chunk = SB ? 2 : env_int("W4A16_GEMV_CHUNK", 2);
    if (!x_f32 && mt == 1 && spt == 1) {
        if constexpr (!SB) {
            if (block.x > 512) {
                if (chunk == 1) return launch_one<1, false, 1, 1024, 1, SB>(a, block, s);
                if (chunk == 4) return launch_one<1, false, 1, 1024, 4, SB>(a, block, s);
            } else {
                if (chunk == 1) return launch_one<1, false, 1, 512, 1, SB>(a, block, s);
                if (chunk == 4) return launch_one<1, false, 1, 512, 4, SB>(a, block, s);
            }
        }
        return block.x > 512 ? launch_one<1, false, 1, 1024, 2, SB>(a, block, s)
                             : launch_one<1, false, 1, 512, 2, SB>(a, block, s);
    }
#define W4_CASE(MTV, XF, SP, NB) \
    if (mt == MTV && x_f32 == XF && spt == SP) return launch_one<MTV, XF, SP, 512, NB, SB>(a, block, s);
    W4_CASE(2, false, 1, 2) W4_CASE(3, false, 1, 2) W4_CASE(4, false, 1, 2)
    W4_CASE(1, false, 2, 2) W4_CASE(2, false, 2, 1)
    W4_CASE(1, true, 1, 2) W4_CASE(2, true, 1, 2)
    W4_CASE(1, true, 2, 1)
#undef W4_CASE
    return hipErrorInvalidValue;
}

hipError_t dispatch(bool x_f32, int spt, int mt, const GemvArgs& a, dim3 block, hipStream_t s) {
    return a.scale_bf16 ? dispatch_t<true>(x_f32, spt, mt, a, block, s)
                        : dispatch_t<false>(x_f32, spt, mt, a, block, s);
}

}  // namespace

hipError_t launch_gemv(const uint8_t* prepared, int64_t n, int64_t k, const void* x, bool x_f32,
                       int64_t m, void* y, bool y_bf16, hipStream_t s) {
    // bf16 rows: the matrix-core kernels read the weights once for all rows.  The dot2
    // kernel below does M times the vector work per weight; it stays faster (measured on
    // MI355X at the 70B shapes) at one row, at two rows while it needs a single pass over
    // the weights (K <= 16384; down 8192x28672 at M = 2: 36.4 us here against 26.0 us on the
    // matrix cores), and at three rows on shapes with K and N <= 16384 that the ring kernel
    // takes (qkv 10240x8192: 14.4 against 15.3 us; o 8192x8192 streams faster, 11.2 against
    // 12.2 us).
    static const int use_mfma = env_int("W4A16_GEMV_MFMA", 1);
    const bool one_pass = k <= 16384;
    const bool dot2_wins = m == 1 || (m == 2 && one_pass) ||
                           (m == 3 && one_pass && n <= 16384 && gemv_ring_takes(n, k));
    if (!x_f32 && !dot2_wins && use_mfma)
        return launch_gemv_mfma(prepared, n, k, static_cast<const uint16_t*>(x), m, y, y_bf16, s);
    return launch_gemv_dot2(prepared, n, k, kGroup, false, x, x_f32, m, y, y_bf16, s);
}

hipError_t launch_gemv_dot2(const uint8_t* prepared, int64_t n, int64_t k, int group,
                            bool scale_bf16, const void* x, bool x_f32, int64_t m, void* y,
                            bool y_bf16, hipStream_t s) {
    const int S = (int)(k / 32);
    GemvArgs a;
    a.wq = reinterpret_cast<const u32x4_t*>(prepared);
    a.sz4 = reinterpret_cast<const u32x4_t*>(prepared + sz_offset(n, k));
    a.y_bf16 = y_bf16 ? 1 : 0;
    a.n = (int)n;
    a.k = (int)k;
    a.rows = 0;
    a.gshift = group == 32 ? 0 : group == 64 ? 1 : 2;
    a.scale_bf16 = scale_bf16;
    const bool wide = !x_f32 && m == 1;      // one slice per lane, up to 1024 threads
    const int spt = wide ? 1 : (S <= 512 ? 1 : 2);
    const int waves = (S + 64 * spt - 1) / (64 * spt);
    const dim3 block(64 * waves);
    const int mt_max = max_mt(x_f32, spt);
    for (int64_t m0 = 0; m0 < m; m0 += mt_max) {
        const int mc = (int)((m - m0) < mt_max ? (m - m0) : mt_max);
        a.x = x_f32 ? (const void*)(static_cast<const float*>(x) + m0 * k)
                    : (const void*)(static_cast<const uint16_t*>(x) + m0 * k);
        a.y = y_bf16 ? (void*)(static_cast<uint16_t*>(y) + m0 * n)
                     : (void*)(static_cast<float*>(y) + m0 * n);
        a.m = mc;
        hipError_t err = dispatch(x_f32, spt, mc, a, block, s);
        if (err != hipSuccess) return err;
    }
    return hipSuccess;
}

}  // namespace w4
