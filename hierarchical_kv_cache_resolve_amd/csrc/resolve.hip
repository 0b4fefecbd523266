// resolve.hip -- the metadata half of RESOLVE on gfx950 for histories whose
// positions do not fit the LDS as a bitmap (or when a probe is forced): hash
// build, cache probe, miss compaction, LRU victim choice, metadata update and
// publication; also the shared layers' publish-only resolve, the replay of an
// anchor's plan, and the trim of cached positions past a history's length.
//
// One 1024-lane workgroup (16 wave64s) per (request, layer); a batched launch
// covers several independent layers with grid.y.  The five stages follow the
// pith review's "Core claim" / "What carries the argument" (shared-memory hash
// table over the selected positions, a parallel probe and scan to mark hits and
// choose victims, page-table publication).  The default lookup structure, a
// bitmap over the history's positions, lives in resolve_bitmap.hip; launch_plan
// picks it whenever it fits the LDS.  The host fetch of the misses is the
// separate streaming kernel in fetch.hip, launched right after on the same
// stream, because the miss rows of all requests are best spread over the whole
// chip rather than over one workgroup per request.
//
// Determinism: victims are the m candidate slots with the smallest
// (stamp, slot) keys, assigned in ascending slot order to the misses in
// ascending selection order.  The kernel reaches that set with a radix select
// over the stamps (10-bit digits relative to the minimum candidate stamp) and
// one block-wide prefix scan that counts strictly-older slots and tied slots
// together, so the result does not depend on wave scheduling.
#include <algorithm>
#include <climits>

#include "hs_device.h"

namespace hs {

namespace {

constexpr int kEmpty = -1;
constexpr int kMisc = 128;  // LDS words for flags, per-wave partial counts and broadcasts

// Offsets inside the misc block (each scan owns its own words, so no barrier
// is needed before one scan's partials are overwritten by the next).
enum : int {
    M_FLAGS = 0,     // bit 0: a position out of range, bit 1: a repeated position
    M_BADAT = 1,     // largest offending selection index + 1
    M_MISS = 2,      // [16] misses per wave
    M_MIN = 18,      // [16] per-wave minimum candidate stamp
    M_MAX = 34,      // [16] per-wave maximum candidate stamp
    M_STRICT = 50,   // [16] strictly-older candidates per wave
    M_TIE = 66,      // [16] tied candidates per wave
    M_HIST = 82,     // [16] histogram-scan wave totals
    M_BIN = 98,      // crossing bin of the current radix pass
    M_BELOW = 99,    // candidates below the crossing bin
};

// How the slot-scan probe maps a cached position to its selection index.
enum : int {
    PROBE_TABLE = 0,   // no slot scan: page-table lookups
    PROBE_HASH = 1,    // bucketed LDS hash of the selection
};

__device__ inline unsigned hash_bucket(int p, int bucket_bits) {
    // multiplicative hashing with the golden-ratio constant (Knuth, TAOCP 6.4)
    return bucket_bits > 0 ? (static_cast<unsigned>(p) * 0x9E3779B1u) >> (32 - bucket_bits) : 0u;
}

// LDS carve-up of the metadata kernel (ints): the lookup structure's two
// arrays of `half` ints each (hash keys and values, or the position bitmap and
// its per-word ranks), slot per selection [k], miss list [k], selection copy
// [k], hit bitmap over slots [B/32 rounded up to 4], histogram [kHistBins],
// misc [kMisc].  Keys come first so 16-byte bucket reads are aligned.
struct PlanLds {
    int* bkey;
    int* bval;
    int* sidx;
    int* mlist;
    int* sel;
    unsigned* hitmap;
    int* hist;
    int* misc;
};

__device__ inline int hitmap_words(int B) { return ((B + 127) >> 7) << 2; }

__device__ inline PlanLds carve(int* base, int half, int k, int B) {
    PlanLds l;
    l.bkey = base;
    l.bval = l.bkey + half;
    l.sidx = l.bval + half;
    l.mlist = l.sidx + k;
    l.sel = l.mlist + k;
    l.hitmap = reinterpret_cast<unsigned*>(l.sel + k);
    l.hist = reinterpret_cast<int*>(l.hitmap) + hitmap_words(B);
    l.misc = l.hist + kHistBins;
    return l;
}

// Bucketed open addressing: 4 entries per bucket, filled in order, buckets
// probed linearly.  One 16-byte LDS read checks a whole bucket, which keeps
// the 64 lanes of a wave close together.  Returns false if p is already
// present.
__device__ inline bool bucket_insert(const PlanLds& l, unsigned nbm, int bucket_bits, int p, int j) {
    unsigned b = hash_bucket(p, bucket_bits);
    for (;;) {
        const int4 kk = *reinterpret_cast<const int4*>(l.bkey + 4 * b);
        if (kk.x == p || kk.y == p || kk.z == p || kk.w == p) return false;
        const int snap[4] = {kk.x, kk.y, kk.z, kk.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (snap[i] != kEmpty) continue;
            const int prev = atomicCAS(&l.bkey[4 * b + i], kEmpty, p);
            if (prev == kEmpty) {
                l.bval[4 * b + i] = j;
                return true;
            }
            if (prev == p) return false;
        }
        b = (b + 1) & nbm;
    }
}

__device__ inline int bucket_find(const PlanLds& l, unsigned nbm, int bucket_bits, int p) {
    unsigned b = hash_bucket(p, bucket_bits);
    for (;;) {
        const int4 kk = *reinterpret_cast<const int4*>(l.bkey + 4 * b);
        if (kk.x == p) return l.bval[4 * b];
        if (kk.y == p) return l.bval[4 * b + 1];
        if (kk.z == p) return l.bval[4 * b + 2];
        if (kk.w == p) return l.bval[4 * b + 3];
        if (kk.w == kEmpty) return -1;  // entries fill in order: a bucket with room ends the chain
        b = (b + 1) & nbm;
    }
}

// Per-lane contiguous slot range [tid*PER, tid*PER + PER), moved as 16-byte
// vectors when the whole range is in bounds and 16-byte aligned (B % 4 == 0).
// Per-lane contiguous slot run [tid*PER, tid*PER + PER).  VEC (B % 4 == 0)
// moves it as 16-byte pieces, each of which lies wholly inside or wholly
// outside [0, B); the scalar form handles any B.  The two forms are separate
// instantiations so that no load result has to be merged across a branch.
template <int PER, bool VEC, typename T>
__device__ inline void load_run(const T* g, int s0, int B, T (&v)[PER], T fill) {
    if constexpr (VEC && (PER % 4) == 0) {
#pragma unroll
        for (int q = 0; q < PER; q += 4) {
            int4 w = make_int4(static_cast<int>(fill), static_cast<int>(fill), static_cast<int>(fill),
                               static_cast<int>(fill));
            if (s0 + q < B) w = *reinterpret_cast<const int4*>(g + s0 + q);
            v[q] = static_cast<T>(w.x);
            v[q + 1] = static_cast<T>(w.y);
            v[q + 2] = static_cast<T>(w.z);
            v[q + 3] = static_cast<T>(w.w);
        }
    } else {
#pragma unroll
        for (int q = 0; q < PER; ++q) v[q] = (s0 + q < B) ? g[s0 + q] : fill;
    }
}

template <int PER, bool VEC, typename T>
__device__ inline void store_run(T* g, int s0, int B, const T (&v)[PER]) {
    if constexpr (VEC && (PER % 4) == 0) {
#pragma unroll
        for (int q = 0; q < PER; q += 4) {
            if (s0 + q < B) {
                int4 w;
                w.x = static_cast<int>(v[q]);
                w.y = static_cast<int>(v[q + 1]);
                w.z = static_cast<int>(v[q + 2]);
                w.w = static_cast<int>(v[q + 3]);
                *reinterpret_cast<int4*>(g + s0 + q) = w;
            }
        }
    } else {
#pragma unroll
        for (int q = 0; q < PER; ++q)
            if (s0 + q < B) g[s0 + q] = v[q];
    }
}

// Reject one request: publish -1, leave its state unchanged.
__device__ inline void reject(const StateBase& s, int32_t* out, int k, int64_t rl, int layer, int r, int code,
                              int detail) {
    for (int j = threadIdx.x; j < k; j += kPlanThreads) {
        out[j] = -1;
        s.hit_mask[rl * s.B + j] = 0;
    }
    if (threadIdx.x == 0) {
        s.miss_count[rl] = 0;
        s.status[rl] = code;
        record_error(s.err, code, layer, r, detail);
    }
}

// Optional per-phase wall-clock stamps (constant-rate clock).  Every wave
// takes them (the clock read is a scalar instruction, so they stay in scalar
// registers) and lane 0 writes its wave's once at the end, so tracing adds no
// global store that a later barrier would have to wait for.  Slots: 0 start,
// 1 global reads issued and LDS cleared, 2 selection inserted, 3 probe done,
// 4 miss list, 5-8 victim stages, 9 metadata written, 10 published; the
// bitmap probe also stamps 11 word counts and 12 ranks.
#define HS_PHASE(i)                                          \
    do {                                                     \
        if (s.phase != nullptr) stamp[(i)] = wall_clock64(); \
    } while (0)
#define HS_PHASE_FLUSH()                                                                \
    do {                                                                                \
        if (s.phase != nullptr && tid == 0)                                             \
            for (int i_ = 0; i_ < 13; ++i_) s.phase[rl * kPhaseSlots + i_] = stamp[i_]; \
    } while (0)


// With l.hist holding counts per bin (bin b at index b), find the bin where
// the count taken from the top bin downwards first reaches `need`; `below`
// is the count of the bins above it.  Leaves l.hist zeroed.  Barriers inside.
__device__ inline void find_crossing_from_top(const PlanLds& l, int need, int& bin, int& below) {
    const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
    const int my_bin = kHistBins - 1 - tid;
    const int hb = l.hist[my_bin];
    l.hist[my_bin] = 0;
    const int incl = wave_incl_scan(hb);
    if (lane == 63) l.misc[M_HIST + wave] = incl;
    __syncthreads();
    const int excl = incl - hb + sum_before(l.misc + M_HIST, wave);
    if (excl < need && need <= excl + hb) {
        l.misc[M_BIN] = my_bin;
        l.misc[M_BELOW] = excl;
    }
    __syncthreads();
    bin = l.misc[M_BIN];
    below = l.misc[M_BELOW];
}

// General threshold search among the slots flagged in `elig` (this lane's
// run): the m-th smallest stamp T and how many slots stamped exactly T are
// taken.  Min/max reduction, then a radix select over stamps relative to the
// minimum in 10-bit digits from the top.  Expects l.hist zeroed; leaves it
// zeroed.  Barriers inside.
template <int PER>
__device__ inline void radix_select(const PlanLds& l, const uint32_t (&tsv)[PER], unsigned elig, int m,
                                    uint32_t& T, int& need_eq) {
    const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
    unsigned mn = 0xFFFFFFFFu, mx = 0u;
#pragma unroll
    for (int q = 0; q < PER; ++q) {
        if ((elig >> q) & 1u) {
            mn = min(mn, tsv[q]);
            mx = max(mx, tsv[q]);
        }
    }
    mn = wave_min(mn);
    mx = wave_max(mx);
    if (lane == 0) {
        l.misc[M_MIN + wave] = static_cast<int>(mn);
        l.misc[M_MAX + wave] = static_cast<int>(mx);
    }
    __syncthreads();
    mn = 0xFFFFFFFFu;
    mx = 0u;
#pragma unroll
    for (int w = 0; w < kPlanWaves; ++w) {
        mn = min(mn, static_cast<unsigned>(l.misc[M_MIN + w]));
        mx = max(mx, static_cast<unsigned>(l.misc[M_MAX + w]));
    }
    if (mn == mx) {
        T = mn;
        need_eq = m;
        return;
    }
    const int nbits = 32 - __clz(static_cast<int>(mx - mn));
    uint64_t prefix = 0;
    int remaining = m, pos = nbits;
    while (pos > 0) {
        const int d = pos < 10 ? pos : 10;
        pos -= d;
#pragma unroll
        for (int q = 0; q < PER; ++q) {
            int bin = -1;
            if ((elig >> q) & 1u) {
                const uint64_t rel = static_cast<uint64_t>(tsv[q] - mn);
                if ((rel >> (pos + d)) == prefix) bin = static_cast<int>((rel >> pos) & ((1u << d) - 1u));
            }
            hist_add(l.hist, bin);
        }
        __syncthreads();
        const int hb = l.hist[tid];
        l.hist[tid] = 0;
        const int incl = wave_incl_scan(hb);
        if (lane == 63) l.misc[M_HIST + wave] = incl;
        __syncthreads();
        const int bl = incl - hb + sum_before(l.misc + M_HIST, wave);
        if (bl < remaining && remaining <= bl + hb) {
            l.misc[M_BIN] = tid;
            l.misc[M_BELOW] = bl;
        }
        __syncthreads();
        prefix = (prefix << d) | static_cast<uint64_t>(l.misc[M_BIN]);
        remaining -= l.misc[M_BELOW];
    }
    T = mn + static_cast<uint32_t>(prefix);
    need_eq = remaining;
}

// Copy the m missed rows of one (request, layer) from the host pool into their
// victim slots: miss i (ascending selection index) is selection j =
// l.mlist[i], whose position l.sel[j] goes to slot -2 - l.sidx[j].  Each lane
// keeps four 16-byte host loads in flight.
template <bool NT>
__device__ inline void copy_misses(const StateBase& s, const PlanLds& l, int64_t rl, int r, int layer, int m) {
    constexpr int U = 4;
    const int row16 = static_cast<int>(s.row_bytes >> 4);
    const int total = m * row16;
    const uint8_t* src_base = s.pool + s.region_row[static_cast<int64_t>(r) * s.NL + layer] * s.row_bytes;
    uint8_t* dst_base = s.cache + rl * s.B * s.row_bytes;
    for (int c0 = threadIdx.x; c0 < total; c0 += kPlanThreads * U) {
        u32x4 v[U];
        u32x4* dst[U];
#pragma unroll
        for (int x = 0; x < U; ++x) {
            const int c = c0 + x * kPlanThreads;
            dst[x] = nullptr;
            if (c < total) {
                const int i = c / row16, off = c - i * row16;
                const int j = l.mlist[i];
                const int slot = -2 - l.sidx[j];
                const u32x4* src = reinterpret_cast<const u32x4*>(src_base + static_cast<int64_t>(l.sel[j]) * s.row_bytes) + off;
                dst[x] = reinterpret_cast<u32x4*>(dst_base + static_cast<int64_t>(slot) * s.row_bytes) + off;
                v[x] = ld16<NT>(src);
            }
        }
#pragma unroll
        for (int x = 0; x < U; ++x)
            if (dst[x]) st16<NT>(dst[x], v[x]);
    }
}

// The metadata half of RESOLVE for one (request, layer).
//   1. every global read is issued up front: clock, selection, slot map and
//      stamps of this lane's slot run, then (page-table probe) the page-table
//      entry of each selected position (which says where the position is
//      cached, if at all);
//   2. page-table probe: hits are marked in an LDS bitmap over the slots (a
//      slot claimed twice means a repeated position); the positions that
//      missed go into an LDS hash table, which catches repeats among them.
//      Slot-scan probe: every selected position goes into the LDS hash (a
//      repeat is caught on insertion) and every cached slot's position is
//      looked up in it;
//   3. misses are compacted in ascending j with wave ballots;
//   4. the m victims are the non-hit slots with the smallest (stamp, slot)
//      keys (radix select on the stamps, then one ballot-counted pass);
//   5. the i-th miss takes the i-th victim in slot order; slot map, stamps
//      (2t+1 for misses, 2t+2 for hits), page table and plan are written and
//      every selection's slot is published.
// SPL: selections a lane holds at most (k <= SPL * 1024); 2 covers k up to
// 2048 without carrying the empty iterations of the 4096 build.
// WIDE: the instantiation for launches over many (request, layer) units.  Up
// to B = 4096 (PER <= 4) it is held to 8 waves per SIMD, so two workgroups
// share a CU; per-layer launches (a few units) use the unconstrained build,
// whose scalar registers need not spill.
template <int PER, bool VEC, int PROBE, bool WIDE, int SPL>
__global__ __launch_bounds__(kPlanThreads) __attribute__((amdgpu_waves_per_eu(WIDE && PER <= 4 ? 8 : 1)))
void plan_kernel(StateBase s, LayerBatch lb) {
    constexpr bool SCAN = PROBE != PROBE_TABLE;
    extern __shared__ int lds_raw[];
    const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
    const int r = blockIdx.x;
    const int layer = lb.layer[blockIdx.y];
    const int k = lb.k, B = s.B, H = 1 << lb.hash_bits;
    const int bucket_bits = lb.hash_bits - 2;
    const unsigned nbm = static_cast<unsigned>((H >> 2) - 1);
    const int64_t rl = static_cast<int64_t>(layer) * s.R + r;
    const int32_t* sel = lb.sel[blockIdx.y] + static_cast<int64_t>(r) * k;
    int32_t* out = lb.out[blockIdx.y] + static_cast<int64_t>(r) * k;
    int32_t* spos_g = s.slot_pos + rl * B;
    uint32_t* ts_g = s.ts + rl * B;
    int32_t* pt = s.page_table + rl * s.L_ctx;
    const PlanLds l = carve(lds_raw, lb.lk_half, k, B);
    const unsigned long long lt = lanemask_lt();
    unsigned long long stamp[13] = {0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
    HS_PHASE(0);

    // 1. global reads
    const uint32_t t = s.clock[rl];
    const int64_t hist_len = s.length[rl];
    int selv[SPL];
#pragma unroll
    for (int q = 0; q < SPL; ++q) {
        const int j = tid + q * kPlanThreads;
        selv[q] = j < k ? sel[j] : 0;
    }
    const int s0 = tid * PER;
    int spos[PER];
    uint32_t tsv[PER];
    load_run<PER, VEC, int>(spos_g, s0, B, spos, kEmpty);
    if constexpr (!SCAN) load_run<PER, VEC, uint32_t>(ts_g, s0, B, tsv, 0xFFFFFFFFu);
    int bad = 0, bad_at = 0;
    int ptv[SPL];
#pragma unroll
    for (int q = 0; q < SPL; ++q) {
        const int j = tid + q * kPlanThreads;
        ptv[q] = -1;
        if (j < k) {
            // the page-table load depends on the static table bound only, so it
            // does not wait for the history length
            const int p = selv[q];
            const bool in_table = p >= 0 && static_cast<int64_t>(p) < s.L_ctx;
            if (!in_table || static_cast<int64_t>(p) >= hist_len) {
                bad |= 1;
                bad_at = j + 1;
            }
            if constexpr (!SCAN) {
                if (in_table) ptv[q] = pt[p];
            }
        }
    }

    for (int i = tid; i < H; i += kPlanThreads) l.bkey[i] = kEmpty;
    if constexpr (PROBE == PROBE_HASH) {
        for (int j = tid; j < k; j += kPlanThreads) l.sidx[j] = -1;
    } else {
        for (int i = tid; i < hitmap_words(B); i += kPlanThreads) l.hitmap[i] = 0u;
    }
    l.hist[tid] = 0;
    if (tid < kMisc) l.misc[tid] = 0;
    __syncthreads();
    HS_PHASE(1);

    // 2. page-table probe: hits into the slot bitmap, misses into the hash.
    //    slot-scan probe: every selected position into the lookup structure.
#pragma unroll
    for (int q = 0; q < SPL; ++q) {
        const int j = tid + q * kPlanThreads;
        if (j < k && !(bad & 1)) {
            const int p = selv[q];
            const int slot = ptv[q];
            l.sel[j] = p;
            if constexpr (PROBE == PROBE_HASH) {
                if (!bucket_insert(l, nbm, bucket_bits, p, j)) {
                    bad |= 2;
                    bad_at = j + 1;
                }
            } else if (slot >= 0) {
                l.sidx[j] = slot;
                if (slot >= B) {
                    bad |= 1;  // a page-table entry outside the cache: treat like a bad position
                    bad_at = j + 1;
                } else {
                    const unsigned bit = 1u << (slot & 31);
                    if (atomicOr(&l.hitmap[slot >> 5], bit) & bit) {
                        bad |= 2;
                        bad_at = j + 1;
                    }
                }
            } else {
                l.sidx[j] = -1;
                if (!bucket_insert(l, nbm, bucket_bits, p, j)) {
                    bad |= 2;
                    bad_at = j + 1;
                }
            }
        }
    }
    block_or_into(&l.misc[M_FLAGS], bad);
    if (bad) atomicMax(&l.misc[M_BADAT], bad_at);
    __syncthreads();
    HS_PHASE(2);
    const int flags = l.misc[M_FLAGS];
    if (flags) {
        reject(s, out, k, rl, layer, r, (flags & 1) ? HS_DEV_RANGE : HS_DEV_DUP, l.misc[M_BADAT] - 1);
        return;
    }
    // this lane's slots that hold a selected position
    unsigned hitbits = 0;
    if constexpr (PROBE == PROBE_HASH) {
        // the pages' probe: every cached position looked up in the hash
#pragma unroll
        for (int q = 0; q < PER; ++q) {
            if (s0 + q < B && spos[q] >= 0) {
                const int j = bucket_find(l, nbm, bucket_bits, spos[q]);
                if (j >= 0) {
                    l.sidx[j] = s0 + q;
                    hitbits |= 1u << q;
                }
            }
        }
        __syncthreads();
    } else {
        // PER divides 32, so the run's bits lie in one word
        hitbits = s0 < B ? (l.hitmap[s0 >> 5] >> (s0 & 31)) & ((PER == 32) ? 0xFFFFFFFFu : ((1u << PER) - 1u)) : 0u;
    }
    HS_PHASE(3);

    // 3. miss list in ascending j: each lane owns the contiguous run
    // [tid*kper, tid*kper + kper); prefix counts come from wave ballots.
    const int kper = (k + kPlanThreads - 1) / kPlanThreads;
    const int j0 = tid * kper;
    unsigned mflags = 0;
    int mpre = 0, mtot = 0;
#pragma unroll
    for (int q = 0; q < SPL; ++q) {
        if (q < kper) {
            const int j = j0 + q;
            const bool f = j < k && l.sidx[j] < 0;
            mflags |= static_cast<unsigned>(f) << q;
            const unsigned long long bm = __ballot(f);
            mpre += __popcll(bm & lt);
            mtot += __popcll(bm);
        }
    }
    if (lane == 0) l.misc[M_MISS + wave] = mtot;
    __syncthreads();
    const int m = sum_before(l.misc + M_MISS, kPlanWaves);
    int base = mpre + sum_before(l.misc + M_MISS, wave);
#pragma unroll
    for (int q = 0; q < SPL; ++q)
        if ((mflags >> q) & 1u) l.mlist[base++] = j0 + q;
    HS_PHASE(4);
    const int h = k - m;
    const uint32_t ts_miss = 2u * t + 1u, ts_hit = 2u * t + 2u;

    if (m == 0) {
        // Every selection hit: only the hit stamps change.
        if (hitbits) {
            if constexpr (SCAN) {
#pragma unroll
                for (int q = 0; q < PER; ++q)
                    if ((hitbits >> q) & 1u) ts_g[s0 + q] = ts_hit;
            } else {
#pragma unroll
                for (int q = 0; q < PER; ++q)
                    if ((hitbits >> q) & 1u) tsv[q] = ts_hit;
                store_run<PER, VEC, uint32_t>(ts_g, s0, B, tsv);
            }
        }
    } else {
        if constexpr (SCAN) load_run<PER, VEC, uint32_t>(ts_g, s0, B, tsv, 0xFFFFFFFFu);
        __syncthreads();  // miss list complete
        HS_PHASE(5);
        const int ncand = B - h;
        // 4. threshold stamp T and how many candidates stamped exactly T must
        // go (lowest slots first); the rest of the victims are older than T.
        uint32_t T;
        int need_eq;
        if (m == ncand) {
            T = 0xFFFFFFFFu;  // every candidate is a victim (stamps never reach this value)
            need_eq = 0;
        } else {
            // Histogram of candidate ages a = 2t - stamp (no stamp exceeds 2t
            // before step t); ages of 1023 and more share the top bin.  The m
            // victims are the oldest, so the crossing is counted from the top.
            const uint32_t top = 2u * t;
            unsigned cand_bits = 0;
#pragma unroll
            for (int q = 0; q < PER; ++q) {
                int bin = -1;
                if (s0 + q < B && !((hitbits >> q) & 1u)) {
                    cand_bits |= 1u << q;
                    const uint32_t age = top - tsv[q];
                    bin = age < kHistBins - 1 ? static_cast<int>(age) : kHistBins - 1;
                }
                hist_add(l.hist, bin);
            }
            __syncthreads();
            int bin, below;
            find_crossing_from_top(l, m, bin, below);
            if (bin < kHistBins - 1) {
                T = top - static_cast<uint32_t>(bin);
                need_eq = m - below;
            } else {
                // All m victims are at least 1023 ages old: select among those
                // with a radix select on their stamps.
                unsigned old_bits = 0;
#pragma unroll
                for (int q = 0; q < PER; ++q)
                    if (((cand_bits >> q) & 1u) && top - tsv[q] >= static_cast<uint32_t>(kHistBins - 1))
                        old_bits |= 1u << q;
                radix_select<PER>(l, tsv, old_bits, m, T, need_eq);
            }
        }
        HS_PHASE(6);

        // Victim ranks in slot order: strictly older candidates and tied
        // candidates are counted together with two ballots per slot column.
        unsigned strict_bits = 0, tie_bits = 0;
        int spre = 0, tpre = 0, stot = 0, ttot = 0;
#pragma unroll
        for (int q = 0; q < PER; ++q) {
            const bool cand = s0 + q < B && !((hitbits >> q) & 1u);
            const bool st = cand && tsv[q] < T;
            const bool ti = cand && tsv[q] == T;
            strict_bits |= static_cast<unsigned>(st) << q;
            tie_bits |= static_cast<unsigned>(ti) << q;
            const unsigned long long bs = __ballot(st), bt = __ballot(ti);
            spre += __popcll(bs & lt);
            tpre += __popcll(bt & lt);
            stot += __popcll(bs);
            ttot += __popcll(bt);
        }
        if (lane == 0) {
            l.misc[M_STRICT + wave] = stot;
            l.misc[M_TIE + wave] = ttot;
        }
        __syncthreads();
        int sb = spre + sum_before(l.misc + M_STRICT, wave);
        int tb = tpre + sum_before(l.misc + M_TIE, wave);
        HS_PHASE(7);
        // 5. assignment and metadata update
        bool any_victim = false;
#pragma unroll
        for (int q = 0; q < PER; ++q) {
            const int slot = s0 + q;
            if (slot >= B) continue;
            if ((hitbits >> q) & 1u) {
                tsv[q] = ts_hit;
                continue;
            }
            int rank = -1;
            if ((strict_bits >> q) & 1u) {
                rank = sb + min(tb, need_eq);
                ++sb;
            } else if ((tie_bits >> q) & 1u) {
                if (tb < need_eq) rank = sb + tb;
                ++tb;
            }
            if (rank >= 0 && rank < m) {
                // the rank-th miss (ascending j) takes this slot; the evicted
                // position goes back to host-only (no write-back: the host copy
                // is authoritative)
                const int j = l.mlist[rank];
                const int newp = l.sel[j];
                const int old = spos[q];
                s.plan[rl * B + rank] = make_int4(j, slot, old, newp);
                if (old >= 0) pt[old] = -1;
                pt[newp] = slot;
                l.sidx[j] = -2 - slot;
                spos[q] = newp;
                tsv[q] = ts_miss;
                any_victim = true;
            }
        }
        if (any_victim) store_run<PER, VEC, int>(spos_g, s0, B, spos);
        if (any_victim || hitbits) store_run<PER, VEC, uint32_t>(ts_g, s0, B, tsv);
        HS_PHASE(8);
        __syncthreads();  // every miss's slot is in l.sidx
    }
    // (all hit: l.sidx has not changed since the miss list's barrier, so the
    // stamp stores need not drain before publication)
    HS_PHASE(9);

    // publication of every selection's slot
    for (int j = tid; j < k; j += kPlanThreads) {
        const int v = l.sidx[j];
        out[j] = v >= 0 ? v : -2 - v;
        s.hit_mask[rl * B + j] = v >= 0 ? 1 : 0;
    }
    if (tid == 0) {
        s.miss_count[rl] = m;
        s.status[rl] = 0;
        s.clock[rl] = t + 1u;
        unsigned long long* st = s.stats + 4 * rl;
        atomicAdd(st + 0, static_cast<unsigned long long>(h));
        atomicAdd(st + 1, static_cast<unsigned long long>(m));
        atomicAdd(st + 2, static_cast<unsigned long long>(m) * static_cast<unsigned long long>(s.row_bytes));
        atomicAdd(st + 3, 1ull);
    }
    if constexpr (WIDE) {
        // a wide launch copies its own misses: with hundreds of workgroups
        // copying at once the link is as busy as under the chip-wide fetch
        // kernel, and the launch after it is saved.  Same flat (row, 16-byte
        // piece) order as the fetch kernel; l.sidx and l.sel are final here.
        if (lb.copy && m > 0) {
            if (lb.nt) copy_misses<true>(s, l, rl, r, layer, m);
            else copy_misses<false>(s, l, rl, r, layer, m);
        }
    }
    HS_PHASE(10);
    HS_PHASE_FLUSH();
}

// Publish-only resolve of a shared layer whose plan was replayed from its
// anchor: look up each selected position in the layer's page table, check the
// slot really holds it, and publish.  LDS: one bit per slot to catch repeats.
__global__ __launch_bounds__(kPlanThreads) void publish_kernel(StateBase s, LayerBatch lb) {
    extern __shared__ unsigned pub_bits[];
    const int tid = threadIdx.x, r = blockIdx.x;
    const int layer = lb.layer[blockIdx.y];
    const int k = lb.k, B = s.B;
    const int64_t rl = static_cast<int64_t>(layer) * s.R + r;
    const int32_t* sel = lb.sel[blockIdx.y] + static_cast<int64_t>(r) * k;
    int32_t* out = lb.out[blockIdx.y] + static_cast<int64_t>(r) * k;
    const int32_t* pt = s.page_table + rl * s.L_ctx;
    const int32_t* spos = s.slot_pos + rl * B;
    __shared__ int pub_flags;
    for (int i = tid; i < (B + 31) / 32; i += kPlanThreads) pub_bits[i] = 0u;
    if (tid == 0) pub_flags = 0;
    __syncthreads();
    int bad_range = 0, bad_dup = 0, bad_res = 0, bad_div = 0, bad_at = -1;
    const int64_t hist_len = s.length[rl];
    const int32_t* asel = lb.anchor_sel[blockIdx.y] + static_cast<int64_t>(r) * k;
    for (int j = tid; j < k; j += kPlanThreads) {
        const int p = sel[j];
        if (p != asel[j]) {
            // not the selection the anchor resolved (another order or another
            // set): its hit mask and stamps would not be this layer's own
            bad_div = 1;
            bad_at = j;
        }
        if (p < 0 || static_cast<int64_t>(p) >= s.L_ctx) {
            bad_range = 1;
            bad_at = j;
            continue;
        }
        const int slot = pt[p];                    // issued before the length check resolves
        if (static_cast<int64_t>(p) >= hist_len) {
            bad_range = 1;
            bad_at = j;
            continue;
        }
        if (slot < 0 || slot >= B || spos[slot] != p) {
            bad_res = 1;
            bad_at = j;
            continue;
        }
        const unsigned bit = 1u << (slot & 31);
        if (atomicOr(&pub_bits[slot >> 5], bit) & bit) {
            bad_dup = 1;
            bad_at = j;
        }
    }
    block_or_into(&pub_flags, bad_range | (bad_dup << 1) | (bad_res << 2) | (bad_div << 3));
    __syncthreads();
    const int fl = pub_flags;
    if (fl) {
        const int code = (fl & 1)   ? HS_DEV_RANGE
                         : (fl & 2) ? HS_DEV_DUP
                         : (fl & 8) ? HS_DEV_DIVERGED
                                    : HS_DEV_NOT_RESIDENT;
        for (int j = tid; j < k; j += kPlanThreads) out[j] = -1;
        if (tid == 0) record_error(s.err, code, layer, r, bad_at);
        return;
    }
    for (int j = tid; j < k; j += kPlanThreads) out[j] = pt[sel[j]];
}

// Mirror the anchor's step into each shared layer (metadata half of the
// replay; the rows are copied by the fetch kernel afterwards).  Before the
// mirror, the shared layer's slot map must equal the anchor's map as it was
// before this step (the anchor's map with every victim's evicted position put
// back) and its clock must be one behind; otherwise the shared layer gets no
// plan (miss_count 0) and HS_DEV_DIVERGED is recorded.
__global__ __launch_bounds__(kPlanThreads) void replay_meta_kernel(StateBase s, ReplayBatch rb) {
    extern __shared__ int prev_pos[];  // [B]: evicted position of victim slots, INT_MIN elsewhere
    const int tid = threadIdx.x, r = blockIdx.x;
    const int A = rb.anchor, L2 = rb.shared[blockIdx.y];
    const int B = s.B;
    const int64_t ra = static_cast<int64_t>(A) * s.R + r;
    const int64_t rs = static_cast<int64_t>(L2) * s.R + r;
    if (s.status[ra] != 0) {
        // The anchor rejected this request's selection; the shared layer's own
        // publish will reject the same selection.
        if (tid == 0) s.miss_count[rs] = 0;
        return;
    }
    const int m = s.miss_count[ra];
    const int4* pa = s.plan + ra * B;
    __shared__ int div_flag;
    for (int i = tid; i < B; i += kPlanThreads) prev_pos[i] = INT_MIN;
    if (tid == 0) div_flag = 0;
    __syncthreads();
    for (int i = tid; i < m; i += kPlanThreads) {
        const int4 e = pa[i];
        prev_pos[e.y] = e.z;
    }
    __syncthreads();
    int diverged = 0;
    const int32_t* spa = s.slot_pos + ra * B;
    int32_t* sps = s.slot_pos + rs * B;
    for (int i = tid; i < B; i += kPlanThreads) {
        const int expect = prev_pos[i] != INT_MIN ? prev_pos[i] : spa[i];
        if (sps[i] != expect) diverged = 1;
    }
    if (tid == 0 && s.clock[rs] + 1u != s.clock[ra]) diverged = 1;
    block_or_into(&div_flag, diverged);
    __syncthreads();
    if (div_flag) {
        if (tid == 0) {
            s.miss_count[rs] = 0;
            record_error(s.err, HS_DEV_DIVERGED, L2, r, A);
        }
        return;
    }
    const uint32_t* tsa = s.ts + ra * B;
    uint32_t* tss = s.ts + rs * B;
    int32_t* pts = s.page_table + rs * s.L_ctx;
    int4* ps = s.plan + rs * B;
    for (int i = tid; i < B; i += kPlanThreads) {
        sps[i] = spa[i];
        tss[i] = tsa[i];
        s.hit_mask[rs * B + i] = s.hit_mask[ra * B + i];
    }
    for (int i = tid; i < m; i += kPlanThreads) {
        const int4 e = pa[i];
        ps[i] = e;
        if (e.z >= 0) pts[e.z] = -1;
        pts[e.w] = e.y;
    }
    if (tid == 0) {
        s.miss_count[rs] = m;
        s.status[rs] = 0;
        s.clock[rs] = s.clock[ra];
        unsigned long long* st = s.stats + 4 * rs;
        atomicAdd(st + 0, static_cast<unsigned long long>(rb.k - m));
        atomicAdd(st + 1, static_cast<unsigned long long>(m));
        atomicAdd(st + 2, static_cast<unsigned long long>(m) * static_cast<unsigned long long>(s.row_bytes));
        atomicAdd(st + 3, 1ull);
    }
}

// Drop every cached position at or past its history's length (after the
// lengths were lowered): the slot becomes empty (stamp 0) and the position
// host-only, so a record later rewritten at that position is fetched again
// rather than served from the old copy -- the host pool is the authoritative
// copy (blog section 2, item 1).  One workgroup per (request, layer).
__global__ __launch_bounds__(256) void trim_kernel(StateBase s) {
    const int r = blockIdx.x, layer = blockIdx.y;
    const int64_t rl = static_cast<int64_t>(layer) * s.R + r;
    const int len = s.length[rl];
    int32_t* spos = s.slot_pos + rl * s.B;
    uint32_t* ts = s.ts + rl * s.B;
    int32_t* pt = s.page_table + rl * s.L_ctx;
    for (int i = threadIdx.x; i < s.B; i += 256) {
        const int p = spos[i];
        if (p >= len) {
            pt[p] = -1;
            spos[i] = kEmpty;
            ts[i] = 0u;
        }
    }
}

}  // namespace

size_t plan_lds_bytes(int k, int half, int B) {
    const size_t hit_words = static_cast<size_t>(((B + 127) >> 7) << 2);
    return sizeof(int) * (2 * static_cast<size_t>(half) + 3 * static_cast<size_t>(k) + hit_words + kHistBins + kMisc);
}

template <int PER, bool VEC, int PROBE, bool WIDE, int SPL>
static hipError_t launch_plan_k(const StateBase& s, const LayerBatch& lb, size_t lds, hipStream_t st) {
    static LdsGrants granted;  // per instantiation
    const hipError_t e =
        ensure_lds_limit(reinterpret_cast<const void*>(&plan_kernel<PER, VEC, PROBE, WIDE, SPL>), lds, granted);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((plan_kernel<PER, VEC, PROBE, WIDE, SPL>), dim3(s.R, lb.n), dim3(kPlanThreads), lds, st, s,
                       lb);
    return hipGetLastError();
}

template <int PER, bool VEC, int PROBE, bool WIDE>
static hipError_t launch_plan_w(const StateBase& s, const LayerBatch& lb, size_t lds, hipStream_t st) {
    static_assert(HS_MAX_K <= 4 * kPlanThreads, "a lane holds at most four selections");
    return lb.k <= 2 * kPlanThreads ? launch_plan_k<PER, VEC, PROBE, WIDE, 2>(s, lb, lds, st)
                                    : launch_plan_k<PER, VEC, PROBE, WIDE, 4>(s, lb, lds, st);
}

template <int PER, bool VEC, int PROBE>
static hipError_t launch_plan_t(const StateBase& s, const LayerBatch& lb, size_t lds, bool wide, hipStream_t st) {
    return wide ? launch_plan_w<PER, VEC, PROBE, true>(s, lb, lds, st)
                : launch_plan_w<PER, VEC, PROBE, false>(s, lb, lds, st);
}

template <int PER, int PROBE>
static hipError_t launch_plan_s(const StateBase& s, const LayerBatch& lb, size_t lds, bool wide, hipStream_t st) {
    return (s.B & 3) == 0 ? launch_plan_t<PER, true, PROBE>(s, lb, lds, wide, st)
                          : launch_plan_t<PER, false, PROBE>(s, lb, lds, wide, st);
}

template <int PER>
static hipError_t launch_plan_p(const StateBase& s, const LayerBatch& lb, size_t lds, int probe, bool wide,
                                hipStream_t st) {
    switch (probe) {
        case PROBE_HASH: return launch_plan_s<PER, PROBE_HASH>(s, lb, lds, wide, st);
        default: return launch_plan_s<PER, PROBE_TABLE>(s, lb, lds, wide, st);
    }
}

static bool plan_is_wide(const StateBase& s, int n) {
    // enough units that two per CU matter: more than one workgroup per CU
    return static_cast<int64_t>(s.R) * n > 256;
}

// Runs of the bitmap kernel move as 16-byte vectors when k and B are
// multiples of 4 and the caller's selection and output arrays are aligned.
static bool bitmap_vec(const StateBase& s, const LayerBatch& lb) {
    bool vec = (lb.k & 3) == 0 && (s.B & 3) == 0;
    for (int i = 0; i < lb.n && vec; ++i)
        vec = (reinterpret_cast<uintptr_t>(lb.sel[i]) & 15u) == 0 && (reinterpret_cast<uintptr_t>(lb.out[i]) & 15u) == 0;
    return vec;
}

int plan_wgs(const StateBase& s, const LayerBatch& lb, int asked) {
    if (asked == 0 || lb.probe != HS_PROBE_SLOT_SCAN || plan_is_wide(s, lb.n)) return 0;
    if (bitmap_lds_bytes(lb.k, s.L_ctx, false) > 160 * 1024) return 0;
    if (bitmap_lanes(s.B, lb.k, false, lb.lanes) != 1024 || !bitmap_vec(s, lb)) return 0;
    if (s.row_bytes > (static_cast<int64_t>(1) << 20)) return 0;  // (piece indices stay inside 32 bits)
    if (asked > 0) return asked;
    // by launch size.  A split unit copies only its own misses, so the units
    // with the most misses set the end of the launch, where the fetch kernel
    // spreads all of a launch's misses evenly over the chip: measured, the
    // split launch saves time where a layer's misses are a few MB (16
    // requests of 1152-byte records) and loses 2 % where they are tens of MB
    // (64 requests of 4 KB records).  Split only launches whose misses cannot
    // exceed 64 MB, into about 64 workgroups: fewer, longer copiers than one
    // per CU kept the host link busier (workgroups per unit measured at
    // 16 requests x 8 layers of 1152-byte records: 0.753 ms a step at 2-4,
    // 0.782 at 16, 0.812 at 32; 18 KB records 0.715 at 3-4 against 0.749 at
    // 16; 8 requests 0.420 at 4-8 against 0.456 at 32).
    const int units = s.R * lb.n;
    if (static_cast<int64_t>(units) * lb.k * s.row_bytes > (static_cast<int64_t>(64) << 20)) return 0;
    return std::max(1, std::min(32, (64 + units - 1) / units));
}

bool plan_copies_misses(const StateBase& s, const LayerBatch& lb) {
    // (rows up to 8 MB keep the wide copy's piece index inside 32 bits)
    return lb.wgs > 0 || (plan_is_wide(s, lb.n) && s.row_bytes <= (static_cast<int64_t>(1) << 23));
}

hipError_t launch_plan(const StateBase& s, const LayerBatch& lb_in, hipStream_t st) {
    LayerBatch lb = lb_in;
    const bool wide = plan_is_wide(s, lb.n);
    lb.copy = plan_copies_misses(s, lb) ? 1 : 0;
    lb.trace = s.phase != nullptr ? 1 : 0;
    if (lb.probe == HS_PROBE_SLOT_SCAN && bitmap_lds_bytes(lb.k, s.L_ctx, wide) <= 160 * 1024) {
        // the default: a bitmap over the history's positions, whenever it
        // fits the LDS of one CU.  Runs move as 16-byte vectors when k and B
        // are multiples of 4 and the caller's arrays are 16-byte aligned.
        return launch_bitmap_resolve(s, lb, wide, bitmap_vec(s, lb), st);
    }
    const int H = 1 << lb.hash_bits;
    const int probe = lb.probe == HS_PROBE_PAGE_TABLE ? PROBE_TABLE : PROBE_HASH;
    lb.lk_half = H;
    const size_t lds = plan_lds_bytes(lb.k, lb.lk_half, s.B);
    const int per = (s.B + kPlanThreads - 1) / kPlanThreads;
    if (per <= 1) return launch_plan_p<1>(s, lb, lds, probe, wide, st);
    if (per <= 2) return launch_plan_p<2>(s, lb, lds, probe, wide, st);
    if (per <= 4) return launch_plan_p<4>(s, lb, lds, probe, wide, st);
    if (per <= 8) return launch_plan_p<8>(s, lb, lds, probe, wide, st);
    if (per <= 16) return launch_plan_p<16>(s, lb, lds, probe, wide, st);
    return hipErrorInvalidValue;
}

hipError_t launch_publish(const StateBase& s, const LayerBatch& lb, hipStream_t st) {
    const size_t lds = sizeof(unsigned) * static_cast<size_t>((s.B + 31) / 32);
    hipLaunchKernelGGL(publish_kernel, dim3(s.R, lb.n), dim3(kPlanThreads), lds, st, s, lb);
    return hipGetLastError();
}

hipError_t launch_replay_meta(const StateBase& s, const ReplayBatch& rb, hipStream_t st) {
    const size_t lds = sizeof(int) * static_cast<size_t>(s.B);
    static LdsGrants granted;
    const hipError_t e = ensure_lds_limit(reinterpret_cast<const void*>(&replay_meta_kernel), lds, granted);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(replay_meta_kernel, dim3(s.R, rb.n), dim3(kPlanThreads), lds, st, s, rb);
    return hipGetLastError();
}

hipError_t launch_trim(const StateBase& s, hipStream_t st) {
    hipLaunchKernelGGL(trim_kernel, dim3(s.R, s.NL), dim3(256), 0, st, s);
    return hipGetLastError();
}

}  // namespace hs
