// hs_internal.h -- shared types of the gfx950 RESOLVE kernels and their host launchers.
//
// Device state of one handle (all arrays layer-major so that one layer's state
// is contiguous; `rl` below is layer * num_req + request):
//   cache      uint8  [layer][req][B][row_bytes]   the GPU hot cache (blog section 2, item 2)
//   slot_pos   int32  [layer][req][B]    logical position held by each slot, -1 = empty
//   ts         uint32 [layer][req][B]    recency stamp, 0 = never used; a miss fetched at
//                                        step t gets 2t+1, a hit 2t+2, so hits rank above
//                                        newly fetched misses (pith "What carries the argument")
//   page_table int32  [layer][req][L_ctx] slot of each logical position, -1 = host only
//                                        (blog section 2, item 3)
//   clock      uint32 [layer][req]       resolves done on this (request, layer)
//   plan       int4   [layer][req][B]    last step's misses {j, slot, evicted pos, new pos}
//   miss_count int32  [layer][req]
//   hit_mask   uint8  [layer][req][B]
//   status     int32  [layer][req]       0, or the device error code of the last step
//   length     int32  [layer][req]       positions of the history written so far (<= L_ctx)
//   stats      uint64 [layer][req][4]    hits, misses, miss bytes, resolves (each unit adds to
//                                        its own counters only, so no two units contend)
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hisparse.h"

namespace hs {

constexpr int kPlanThreads = 1024;           // one workgroup per (request, layer)
constexpr int kPlanWaves = kPlanThreads / 64;
constexpr int kFetchThreads = 256;
constexpr int kMaxBatch = 32;                // layers per batched launch
constexpr int kHistBins = 1024;              // radix-select digit of 10 bits
constexpr int kPhaseSlots = 16;              // phase stamps per (request, layer)

struct StateBase {
    uint8_t* cache;
    int32_t* slot_pos;
    uint32_t* ts;
    int32_t* page_table;
    uint32_t* clock;
    int4* plan;
    int32_t* miss_count;
    uint8_t* hit_mask;
    int32_t* status;
    int32_t* err;                   // sticky {code, layer, req, detail}
    unsigned long long* stats;      // [layer][req][4]: hits, misses, miss bytes, resolves
    unsigned long long* phase;      // [layer][req][kPhaseSlots] wall-clock stamps, or null (off)
    uint8_t* pool;                  // device-visible pointer to the host pool
    int32_t* length;                // [layer][req] positions written so far in each history
    uint32_t* arrive;               // [layer][req] workgroups of a split unit done (0 between launches)
    const int64_t* region_row;      // [req * num_layers + layer]
    int64_t L_ctx;
    int64_t row_bytes;
    int R, NL, B;
};

struct LayerBatch {
    const int32_t* sel[kMaxBatch];  // [R][k] per entry
    int32_t* out[kMaxBatch];        // [R][k] per entry
    const int32_t* anchor_sel[kMaxBatch];  // publish only: the anchor's selection [R][k]
    int layer[kMaxBatch];
    int n;
    int k;
    int hash_bits;
    int probe;    // HS_PROBE_PAGE_TABLE, HS_PROBE_SLOT_SCAN or HS_PROBE_SLOT_SCAN_HASH
    int lk_half;  // ints in each of the hash kernel's two lookup arrays (set by launch_plan)
    int ngroups;  // bitmap kernel: 16-byte groups of position bits, ceil(L_ctx / 128)
    int r1_ints;  // bitmap kernel: ints of its first LDS region
    int nt;       // non-temporal host loads and cache stores in the metadata kernel's own copy
    int copy;     // the metadata kernel copies the misses itself (set by launch_plan)
    int trace;    // phase stamps on (s.phase is set)
    int lanes;    // bitmap kernel: lanes a unit asked for (0: by launch size)
    int wgs;      // bitmap kernel: workgroups a unit (0: one, with a fetch launch after it; G >= 1:
                  // G workgroups plan it alike and copy its misses between them, set by plan_wgs)
};

struct FetchBatch {
    int layer[kMaxBatch];
    int n;
};

struct ReplayBatch {
    int anchor;
    int k;
    int shared[kMaxBatch];
    int n;
};

// Host launchers (defined in the .hip files).
size_t plan_lds_bytes(int k, int half, int B);
hipError_t launch_plan(const StateBase& s, const LayerBatch& lb, hipStream_t st);
// The bitmap metadata kernel (resolve_bitmap.hip): its LDS need, its lanes a
// unit, and its launch (vec: k and B multiples of 4, arrays 16-byte aligned).
size_t bitmap_lds_bytes(int k, int64_t L_ctx, bool wide);
int bitmap_lanes(int B, int k, bool wide, int asked);
hipError_t launch_bitmap_resolve(const StateBase& s, const LayerBatch& lb, bool wide, bool vec, hipStream_t st);
hipError_t launch_trim(const StateBase& s, hipStream_t st);
// Workgroups a unit of a metadata launch takes when it copies its own misses
// between several workgroups (0: it does not; a fetch launch follows).
// `asked`: -1 by launch size, 0 never, G >= 1 that many.
int plan_wgs(const StateBase& s, const LayerBatch& lb, int asked);
// Whether a metadata launch copies its own misses (a wide launch, or one
// whose units take several workgroups: no fetch launch follows it).
bool plan_copies_misses(const StateBase& s, const LayerBatch& lb);
hipError_t launch_publish(const StateBase& s, const LayerBatch& lb, hipStream_t st);
hipError_t launch_fetch(const StateBase& s, const FetchBatch& fb, int blocks, int unroll, bool nt, hipStream_t st);
hipError_t launch_replay_meta(const StateBase& s, const ReplayBatch& rb, hipStream_t st);
hipError_t launch_append(const StateBase& s, int layer, const uint8_t* rows, hipStream_t st);
hipError_t launch_gather_checksum(const StateBase& s, int layer, const int32_t* slot_idx, int k, uint64_t* out,
                                  hipStream_t st);
hipError_t launch_link_read(const void* src, void* dst, size_t bytes, hipStream_t st);
size_t attend_workspace_floats(int R, int H, int nchunk);
int attend_chunk(int R, int H, int k, int ht);
int attend_head_tiles(int R, int H, int k);
hipError_t launch_attend_mla(const StateBase& s, int layer, const uint16_t* q, int H, const int32_t* slot_idx, int k,
                             float scale, float* out, float* lse, float* workspace, int ht, int chunk,
                             hipStream_t st);
hipError_t launch_hbm_copy(const void* src, void* dst, size_t bytes, hipStream_t st);

// Largest dynamic-LDS limit already granted to one kernel, per device.
struct LdsGrants {
    static constexpr int kDevices = 64;
    size_t bytes[kDevices] = {};
};

// Raise a kernel's dynamic-LDS limit when a launch needs more than the default
// 64 KB.  The limit is set once per kernel and device (and again only for a
// larger need), so steady-state launches make no attribute call.  A handle is
// not thread-safe, and neither is this bookkeeping.
inline hipError_t ensure_lds_limit(const void* fn, size_t lds, LdsGrants& g) {
    if (lds <= 65536) return hipSuccess;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) dev = -1;
    const bool tracked = dev >= 0 && dev < LdsGrants::kDevices;
    if (tracked && lds <= g.bytes[dev]) return hipSuccess;
    const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (e == hipSuccess && tracked) g.bytes[dev] = lds;
    return e;
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// 16-byte load / store, non-temporal (streamed past the caches) when NT.
template <bool NT>
__device__ inline u32x4 ld16(const u32x4* p) {
    if constexpr (NT) return __builtin_nontemporal_load(p);
    else return *p;
}

template <bool NT>
__device__ inline void st16(u32x4* p, u32x4 v) {
    if constexpr (NT) __builtin_nontemporal_store(v, p);
    else *p = v;
}

// Record the first device-side data error in the sticky word.
__device__ inline void record_error(int32_t* err, int code, int layer, int req, int detail) {
    if (atomicCAS(err, 0, code) == 0) {
        err[1] = layer;
        err[2] = req;
        err[3] = detail;
    }
}

}  // namespace hs
