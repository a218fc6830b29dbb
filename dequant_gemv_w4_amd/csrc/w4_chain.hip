// A chain of decode GEMVs (M = 1) in one persistent launch.
//
// A decode step multiplies every quantized matrix once by its activation row,
// and the step time is bounded below by weight bytes / HBM bandwidth (page
// "Weight quantization", sections "Complexity and constants" and "Efficiency").
// Launching each product separately pays a launch, a ramp-up and a drain per
// matrix.  Here the products are stages of one launch: stage s may read what
// stage s-1 wrote (its x can be an earlier y), so a workgroup computes an item
// of stage s only after every item of stage s-1 has been stored, but it issues
// the weight loads of its next units before it waits.  The weight stream
// therefore keeps running through the stage boundaries.
//
// Work: each GEMV is cut into items of `rows` rows; items are numbered stage by
// stage and workgroup w takes items w, w+G, w+2G, ... in order (G = the grid,
// one round of resident workgroups, so every workgroup is running).  A unit is
// four rows times one 16-byte slice per lane (256 lanes = 8192 inputs); a row of
// K inputs takes ceil(K/8192) units.
//
// Loads: every wave has a ring of kRing units in LDS.  The codes and scale/zero
// words of a unit go straight from global memory to the ring (global_load_lds:
// lane l's bytes land at slot + 16 l and lane l reads them back, so the ring
// needs no barrier), kRing units ahead of the arithmetic, across item and stage
// boundaries.  A unit is five loads and the wait before a unit is an exact count.
//
// Per unit and lane the arithmetic is that of gemv_kernel: v_and_or_b32 builds
// bf16 128+q pairs, v_dot2c_f32_bf16 accumulates D = sum (128+q) x, the slice
// sum S (same dot2 sequence with the pair (1,1)) removes the offset and the
// zero, scale16 * (D - (128 + zero) * S) is the slice's share of the group term
// (page "Weight quantization", section "How it works": one multiply per group).
// x slices sit in registers (loaded when a GEMV starts); rows are reduced across
// the wave with permlane swaps and DPP, across waves through LDS; no
// floating-point atomics.
//
// Synchronisation across workgroups (on MI355X the L2 of each XCD is private):
// rows are stored with device-scope stores (written through), x is read with
// device-scope loads, and the per-stage counters are device-scope atomics, so no
// L2 write-back or invalidate is needed.  After its rows of a stage are stored a
// workgroup waits for those stores (an exact count: only ring loads issued after
// them may still be in flight) and adds its item count to done[stage]; before the
// first item of a new stage it waits until done[stage-1] equals that stage's item
// count.  The wait is bounded: after spin_limit polls it sets a status bit and
// continues, so no launch can hang.  The last workgroup to finish resets the
// counters, leaving the workspace zeroed for the next launch.
#include <atomic>
#include <cstdlib>
#include <cstring>
#include <type_traits>
#include <vector>

#include "w4_internal.h"

namespace w4 {
namespace {

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int CT = 256;   // threads per workgroup
constexpr int CW = CT / 64;
#ifndef W4_CHAIN_RING
#define W4_CHAIN_RING 7
#endif
constexpr int kRing = W4_CHAIN_RING;    // units in flight per wave
constexpr int kUnitBytes = 5 * 1024;    // per wave: codes of four rows + their scale/zero words
constexpr int kMaxItemRows = 64;
constexpr int kMaxPasses = 4;           // K <= 32768: at most four 16-byte slices per lane

__device__ __forceinline__ float dot2(uint32_t w, uint32_t x, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w),
                                           __builtin_bit_cast(bf16x2_t, x), acc, false);
}

__device__ __forceinline__ uint32_t bf16_bits_rne(float f) {
    const uint32_t u = __float_as_uint(f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                                 0xF, 0xF, false));
}

__device__ __forceinline__ void swap32(float& a, float& b) {
    const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, a),
                                                    __builtin_bit_cast(uint32_t, b), false, false);
    a = __builtin_bit_cast(float, (uint32_t)r[0]);
    b = __builtin_bit_cast(float, (uint32_t)r[1]);
}

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
    float k0 = a0 + a2;
    float k1 = a1 + a3;
    swap16(k0, k1);
    float k = k0 + k1;
    k += dpp<0x128>(k);
    k += dpp<0x124>(k);
    k += dpp<0x122>(k);
    k += dpp<0x121>(k);
    return k;
}

// position of the pipeline: unit (item, row step, slice pass) of this workgroup
struct Cursor {
    int item;   // global item index (-1 when exhausted)
    int d;      // descriptor of the item
    int step;   // row step (four rows) inside the item
    int pass;   // slice pass inside the row step
};

struct Geo {        // geometry of one descriptor (read from the plan)
    const uint8_t* w;
    const uint8_t* sz;
    const uint16_t* x;
    void* y;
    int n, k, rows, first, count, stage, y_bf16;
};

__device__ __forceinline__ Geo geo_of(const ChainDesc* __restrict__ descs, int d) {
    // the index is wave-uniform: scalar loads, which do not count against vmcnt
    const ChainDesc& c = descs[__builtin_amdgcn_readfirstlane(d)];
    Geo g;
    g.w = c.w;
    g.sz = c.sz;
    g.x = c.x;
    g.y = c.y;
    g.n = c.n;
    g.k = c.k;
    g.rows = c.rows;
    g.first = c.first_item;
    g.count = c.n_items;
    g.stage = c.stage;
    g.y_bf16 = c.y_bf16;
    return g;
}

__device__ __forceinline__ int item_rows(const Geo& g, int item) {
    const int r0 = (item - g.first) * g.rows;
    return min(g.rows, g.n - r0);
}

__device__ __forceinline__ int passes_of(const Geo& g) { return (g.k / 32 + CT - 1) / CT; }

// move the cursor to the descriptor that holds c.item (items grow monotonically)
__device__ __forceinline__ void seek(Cursor& c, Geo& g, const ChainDesc* __restrict__ descs,
                                     int n_desc, int total) {
    if (c.item >= total) {
        c.item = -1;
        return;
    }
    while (c.item >= g.first + g.count && c.d + 1 < n_desc) {
        ++c.d;
        g = geo_of(descs, c.d);
    }
}

__device__ __forceinline__ void advance(Cursor& c, Geo& g, const ChainDesc* __restrict__ descs,
                                        int n_desc, int total, int grid) {
    if (++c.pass < passes_of(g)) return;
    c.pass = 0;
    if (++c.step < (item_rows(g, c.item) + 3) / 4) return;
    c.step = 0;
    c.item += grid;
    seek(c, g, descs, n_desc, total);
}

// 16 bytes per lane from global memory straight into LDS: lane l of the wave writes
// bytes [16 l, 16 l + 16) after the wave-uniform LDS address.  Inline assembly, so the
// compiler neither orders other LDS reads behind it nor waits for it; the kernel counts
// these loads itself (vmcnt).
__device__ __forceinline__ void lds_dma16(const void* g, uint32_t lds_addr) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(g), "s"(lds_addr)
                 : "memory", "m0");
}

// wait until at most 5 n vector-memory operations of this wave are outstanding: the unit
// computed next was issued n units before the newest one, and every unit is five loads
__device__ __forceinline__ void wait_units(int n) {
    switch (n) {
        case 0: __builtin_amdgcn_s_waitcnt(0x0F70); break;             // vmcnt(0)
        case 1: __builtin_amdgcn_s_waitcnt(0x0F75); break;             // vmcnt(5)
        case 2: __builtin_amdgcn_s_waitcnt(0x0F7A); break;             // vmcnt(10)
        case 3: __builtin_amdgcn_s_waitcnt(0x0F7F); break;             // vmcnt(15)
        case 4: __builtin_amdgcn_s_waitcnt(0x4F74); break;             // vmcnt(20)
        case 5: __builtin_amdgcn_s_waitcnt(0x4F79); break;             // vmcnt(25)
        default: __builtin_amdgcn_s_waitcnt(0x4F7E); break;            // vmcnt(30)
    }
    asm volatile("" ::: "memory");  // LDS reads of the unit stay after the wait
}

// device-scope stores (write through to memory, so other XCDs read them with
// device-scope loads); inline assembly, like the ring loads, so the compiler's wait
// counts stay out of the unit loop; release_items waits for them explicitly
typedef __attribute__((address_space(1))) uint32_t gu32;
typedef __attribute__((address_space(1))) uint16_t gu16;
__device__ __forceinline__ void store_dev32(uint32_t* p, uint32_t v) {
    asm volatile("global_store_dword %0, %1, off sc1" : : "v"((gu32*)p), "v"(v) : "memory");
}
__device__ __forceinline__ void store_dev16(uint16_t* p, uint32_t v) {
    asm volatile("global_store_short %0, %1, off sc1" : : "v"((gu16*)p), "v"(v) : "memory");
}

// barrier for LDS data only (no fence: the ring's loads in flight are not waited for)
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

__global__ __launch_bounds__(CT) void chain_kernel(const ChainDesc* __restrict__ descs,
                                                   const int32_t* __restrict__ stage_items,
                                                   uint32_t* __restrict__ ws, int n_desc,
                                                   int n_stages, int total, int spin_limit) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];  // rings, then row sums

    uint32_t* status = ws;                // word 0: bit 0 = a stage wait gave up
    uint32_t* exit_count = ws + 1;        // word 1: workgroups that finished
    uint32_t* done = ws + 2;              // words 2..: items stored per stage

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int grid = gridDim.x;

    const uint32_t smem_lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)smem;
    const uint32_t ring = __builtin_amdgcn_readfirstlane(smem_lds + wave * kRing * kUnitBytes);
    const uint8_t* ring_p = smem + wave * kRing * kUnitBytes;
    float* red = reinterpret_cast<float*>(smem + CW * kRing * kUnitBytes);  // [CW][kMaxItemRows]

    uint32_t nib_mask, bias_bits;
    asm volatile("s_mov_b32 %0, 0x000F000F" : "=s"(nib_mask));
    asm volatile("v_mov_b32 %0, 0x43004300" : "=v"(bias_bits));

    // ---- issue cursor (loads run kRing units ahead) and compute cursor
    Cursor ic{(int)blockIdx.x, 0, 0, 0};
    Geo ig = geo_of(descs, 0);
    seek(ic, ig, descs, n_desc, total);
    Cursor cc = ic;
    Geo cg = ig;
    int issued = 0, computed = 0;   // units of this workgroup (the same in every wave)
    int units_since_store = 0;       // units issued after this wave's latest row stores

    auto issue_unit = [&]() {
        const int S = ig.k >> 5;
        const int r0 = (ic.item - ig.first) * ig.rows + ic.step * 4;
        const int sl = min(tid + ic.pass * CT, S - 1);   // lanes past the last slice repeat it
        const int64_t row_bytes = (int64_t)ig.k / 2;
        const uint32_t slot =
            __builtin_amdgcn_readfirstlane(ring + (uint32_t)(issued % kRing) * kUnitBytes);
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
            lds_dma16(ig.w + (int64_t)min(r0 + rr, ig.n - 1) * row_bytes + (uint32_t)sl * 16u,
                      slot + rr * 1024);
        lds_dma16(ig.sz + ((int64_t)(r0 >> 2) * (ig.k >> 7) + (sl >> 2)) * 16, slot + 4096);
        ++issued;
        ++units_since_store;
        advance(ic, ig, descs, n_desc, total, grid);
    };
    for (int b = 0; b < kRing && ic.item >= 0; ++b) issue_unit();

    int cur_stage = 0;
    const uint16_t* cur_x = nullptr;
    int items_this_stage = 0;
    uint32_t xr[kMaxPasses][16];   // x slices of this lane (bf16 pairs), one per pass
    float sx[kMaxPasses];          // their sums, by the same dot2 sequence as the weights
    float acc[4] = {0.f, 0.f, 0.f, 0.f};

    // stores of this workgroup are complete before the count that publishes them: only the
    // ring loads issued after the latest stores may still be in flight
    auto release_items = [&](int s, int count) {
        wait_units(min(units_since_store, kRing - 1));
        lds_barrier();
        if (tid == 0 && count > 0)
            __hip_atomic_fetch_add(done + s, (uint32_t)count, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
    };
    auto wait_stage = [&](int s) {  // every item of stage s stored
        if (tid == 0) {
            const uint32_t need = (uint32_t)stage_items[s];
            int polls = 0;
            while (__hip_atomic_load(done + s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < need) {
                __builtin_amdgcn_s_sleep(2);
                if (++polls > spin_limit) {
                    __hip_atomic_fetch_or(status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    break;
                }
            }
        }
        lds_barrier();
    };
    // x of the current GEMV: device-scope loads, which read what other workgroups stored
    auto load_x = [&]() {
        const int S = cg.k >> 5;
        const gu32* xw = (const gu32*)reinterpret_cast<const uint32_t*>(cg.x);
#pragma unroll
        for (int p = 0; p < kMaxPasses; ++p) {
            const int sl = tid + p * CT;
            const bool ok = sl < S;
#pragma unroll
            for (int i = 0; i < 16; ++i)
                xr[p][i] = ok ? __hip_atomic_load((gu32*)(xw + (int64_t)sl * 16 + i), __ATOMIC_RELAXED,
                                                  __HIP_MEMORY_SCOPE_AGENT)
                              : 0u;
            float d = 0.0f;
#pragma unroll
            for (int i = 0; i < 16; ++i) d = dot2(0x3F803F80u, xr[p][i], d);
            sx[p] = d;
        }
    };

    auto unit_math = [&](auto pass_c) {
        constexpr int P = decltype(pass_c)::value;
        const uint8_t* slot = ring_p + (computed % kRing) * kUnitBytes;
        const u32x4_t s4 = *reinterpret_cast<const u32x4_t*>(slot + 4096 + 16 * lane);
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const u32x4_t w4 = *reinterpret_cast<const u32x4_t*>(slot + rr * 1024 + 16 * lane);
            const uint32_t szw = s4[rr];
            const float sc = (float)__builtin_bit_cast(_Float16, (uint16_t)(szw & 0xFFFFu));
            const float zb = (float)((szw >> 16) & 0xFFu);
            float d = 0.0f;
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    d = dot2(((w4[t] >> (4 * q)) & nib_mask) | bias_bits, xr[P][4 * t + q], d);
            acc[rr] = fmaf(sc, fmaf(-zb, sx[P], d), acc[rr]);
        }
    };

    while (cc.item >= 0) {
        if (cc.step == 0 && cc.pass == 0) {
            // ---- first unit of an item: stage order, then x of this GEMV
            if (cg.stage != cur_stage) {
                release_items(cur_stage, items_this_stage);
                items_this_stage = 0;
                for (int st = cur_stage; st < cg.stage; ++st) wait_stage(st);
                cur_stage = cg.stage;
                cur_x = nullptr;  // x of a later stage may be written by an earlier one
            }
            if (cg.x != cur_x) {
                load_x();
                cur_x = cg.x;
            }
        }
        wait_units(issued - computed - 1);
        const int passes = passes_of(cg);
        switch (cc.pass) {
            case 0: unit_math(std::integral_constant<int, 0>{}); break;
            case 1: unit_math(std::integral_constant<int, 1>{}); break;
            case 2: unit_math(std::integral_constant<int, 2>{}); break;
            default: unit_math(std::integral_constant<int, 3>{}); break;
        }
        // a lane past the last slice of the row (ragged K) holds x = 0 and sum 0: it adds
        // exactly 0 to its rows
        ++computed;
        if (cc.pass == passes - 1) {
            const float k = reduce4(acc[0], acc[1], acc[2], acc[3]);
            if ((lane & 15) == 0) red[wave * kMaxItemRows + cc.step * 4 + (lane >> 4)] = k;
            acc[0] = acc[1] = acc[2] = acc[3] = 0.0f;
            const int nrows = item_rows(cg, cc.item);
            if (cc.step == (nrows + 3) / 4 - 1) {
                // ---- last unit of the item: combine the waves and store the rows
                lds_barrier();
                if (tid < nrows) {
                    float v = 0.0f;
#pragma unroll
                    for (int wv = 0; wv < CW; ++wv) v += red[wv * kMaxItemRows + tid];
                    const int64_t row = (int64_t)(cc.item - cg.first) * cg.rows + tid;
                    if (cg.y_bf16)
                        store_dev16(static_cast<uint16_t*>(cg.y) + row, bf16_bits_rne(v));
                    else
                        store_dev32(static_cast<uint32_t*>(cg.y) + row, __float_as_uint(v));
                }
                units_since_store = 0;
                lds_barrier();  // red is reused by the next item
                ++items_this_stage;
            }
        }
        // refill the slot just consumed (its LDS reads are complete: their values were used)
        if (ic.item >= 0) issue_unit();
        advance(cc, cg, descs, n_desc, total, grid);
    }
    release_items(cur_stage, items_this_stage);

    // ---- the last workgroup out resets the counters for the next launch
    __syncthreads();
    if (tid == 0) {
        const uint32_t prev = __hip_atomic_fetch_add(exit_count, 1u, __ATOMIC_ACQ_REL,
                                                     __HIP_MEMORY_SCOPE_AGENT);
        if (prev == (uint32_t)grid - 1) {
            for (int s = 0; s < n_stages; ++s)
                __hip_atomic_store(done + s, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(exit_count, 0u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

int chain_compute_units() {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
        cus = 256;
    return cus;
}

}  // namespace

size_t chain_lds_bytes(int) {
    return (size_t)CW * kRing * kUnitBytes + (size_t)CW * kMaxItemRows * 4;
}

static hipError_t allow_lds(size_t lds) {
    if (lds <= 65536) return hipSuccess;
    return hipFuncSetAttribute(reinterpret_cast<const void*>(chain_kernel),
                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
}

// Grid (one round of resident workgroups) for a chain whose largest K is max_k.
int chain_grid(int max_k) {
    if (allow_lds(chain_lds_bytes(max_k)) != hipSuccess) return 0;
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, chain_kernel, CT,
                                                     chain_lds_bytes(max_k)) != hipSuccess ||
        per_cu < 1)
        per_cu = 1;
    return per_cu * chain_compute_units();
}

hipError_t launch_chain(const ChainHeader& h, const uint8_t* plan_dev, uint32_t* ws,
                        hipStream_t s) {
    const ChainDesc* descs = reinterpret_cast<const ChainDesc*>(plan_dev + sizeof(ChainHeader));
    const int32_t* stage_items = reinterpret_cast<const int32_t*>(
        plan_dev + sizeof(ChainHeader) + sizeof(ChainDesc) * (size_t)h.n_desc);
    const size_t lds = chain_lds_bytes(h.max_k);
    hipError_t e = allow_lds(lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(chain_kernel, dim3((unsigned)h.grid), dim3(CT), lds, s, descs, stage_items,
                       ws, h.n_desc, h.n_stages, h.total_items, h.spin_limit);
    return hipGetLastError();
}

}  // namespace w4
