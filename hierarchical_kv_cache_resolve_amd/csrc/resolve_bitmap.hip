// resolve_bitmap.hip -- the metadata half of RESOLVE on gfx950 when the
// history's positions fit the LDS as a bitmap (every workload here).
//
// One workgroup of NT lanes (512 or 1024) per (request, layer); a batched
// launch covers several independent layers with grid.y.  The stages follow
// the pith review's "Core claim" and "What carries the argument" and the
// blog's section 3 ("RESOLVE: Five Stages in One Launch"): a lookup
// structure over the selected positions in shared memory, every cached slot
// probed against it to mark hits, LRU victims for the misses (hits ranked
// above newly fetched misses), then metadata update and publication.  The
// lookup structure is a bitmap over the history's positions plus a 16-bit
// rank for each 32-bit bitmap word: the rank of a selected position is its
// index among the selected positions, so a position maps to its selection in
// O(1) with no probe chains.
//
// The kernel is laid out for the all-hit case, which decides the cost of a
// layer whose selection barely moves: four barriers, hits found on the slot
// side by one bit test each, every hit published as soon as the selection
// side reads its slot, each lane's run of hit stamps written back as whole
// 16-byte pieces.  Only a unit with misses goes on to the victim search (age
// histogram, threshold, slot-order ranking; one more barrier), and there the
// lane of each miss publishes it from the victim list.
//
// Determinism: victims are the m candidate slots with the smallest
// (stamp, slot) keys, assigned in ascending slot order to the misses in
// ascending selection order, whatever the order in which waves run.
#include <type_traits>

#include "hs_device.h"

namespace hs {

namespace {

constexpr int kEmpty = -1;
constexpr int kHistQ = kHistBins / 64;  // histogram bins per lane of a wave that scans all of them

// Words of the misc block (each scan owns its own words, so one scan's
// partials never have to be drained before the next scan writes its own).
enum : int {
    X_FLAGS = 0,    // bit 0: a position outside the history, bit 1: a repeated position
    X_BADAT = 1,    // largest offending selection index + 1
    X_RANK = 2,     // first group rank not yet handed to a wave
    X_BIN = 3,      // radix select: crossing bin of the current pass
    X_BELOW = 4,    // radix select: candidates below it
    X_LAST = 5,     // split unit: this workgroup arrived last
    X_TBIN = 6,     // victim threshold: crossing bin found by wave 0
    X_TBELOW = 7,   // victim threshold: candidates in the bins above it
    X_MISS = 16,    // [16] per-wave inclusive miss counts
    X_VICT = 32,    // [16] per-wave packed (strict | tie << 16) victim counts
    X_HIST = 48,    // [16] radix-scan partials
    X_MIN = 64,     // [16] per-wave minimum candidate stamp
    X_MAX = 80,     // [16] per-wave maximum candidate stamp
    X_HITS = 96,    // [16] per-wave inclusive hit counts
    X_STAMP = 112,  // [2 * 11] phase stamps of wave 0 while tracing
    kMiscWords = 144,
};

// A lane's contiguous run v[0..N) of elements i0 .. i0+N-1 of g, in pieces of
// W = min(N, 4) elements when VEC (the caller guarantees n % 4 == 0 and
// 16-byte alignment, so each piece lies wholly inside or outside [0, n));
// element by element otherwise.  Elements outside [0, n) read as `fill`.
// The loads are unconditional, from an address clamped into [0, n), so no
// loaded value is merged across a branch (which would make the wave wait for
// it on the spot instead of where it is used).
template <int N, bool VEC, typename T>
__device__ inline void load_run(const T* g, int i0, int n, T (&v)[N], T fill) {
    constexpr int W = N < 4 ? N : 4;
    if constexpr (VEC && W == 4) {
#pragma unroll
        for (int q = 0; q < N; q += 4) {
            const bool in = i0 + q < n;
            const uint4 w = *reinterpret_cast<const uint4*>(g + (in ? i0 + q : n - 4));
            v[q] = in ? static_cast<T>(w.x) : fill;
            v[q + 1] = in ? static_cast<T>(w.y) : fill;
            v[q + 2] = in ? static_cast<T>(w.z) : fill;
            v[q + 3] = in ? static_cast<T>(w.w) : fill;
        }
    } else if constexpr (VEC && W == 2) {
        const bool in = i0 < n;
        const uint2 w = *reinterpret_cast<const uint2*>(g + (in ? i0 : n - 2));
        v[0] = in ? static_cast<T>(w.x) : fill;
        v[1] = in ? static_cast<T>(w.y) : fill;
    } else {
#pragma unroll
        for (int q = 0; q < N; ++q) {
            const bool in = i0 + q < n;
            const T w = g[in ? i0 + q : n - 1];
            v[q] = in ? w : fill;
        }
    }
}

// Store the pieces of a run that hold at least one element flagged in
// `mask` (bit q: element q); same piece layout as load_run.
template <int N, bool VEC, typename T>
__device__ inline void store_run_masked(T* g, int i0, int n, const T (&v)[N], unsigned mask) {
    constexpr int W = N < 4 ? N : 4;
    if constexpr (VEC && W == 4) {
#pragma unroll
        for (int q = 0; q < N; q += 4) {
            if ((mask >> q) & 0xFu) {
                *reinterpret_cast<uint4*>(g + i0 + q) =
                    make_uint4(static_cast<unsigned>(v[q]), static_cast<unsigned>(v[q + 1]),
                               static_cast<unsigned>(v[q + 2]), static_cast<unsigned>(v[q + 3]));
            }
        }
    } else if constexpr (VEC && W == 2) {
        if (mask & 3u)
            *reinterpret_cast<uint2*>(g + i0) = make_uint2(static_cast<unsigned>(v[0]), static_cast<unsigned>(v[1]));
    } else {
#pragma unroll
        for (int q = 0; q < N; ++q)
            if (((mask >> q) & 1u) && i0 + q < n) g[i0 + q] = v[q];
    }
}

// Bits 0 .. min(N, avail) - 1: which elements of a lane's run of N exist.
// Per-element existence is carried as a bit mask in one register and tested
// where it is used, rather than as N predicates the compiler would keep (or
// spill) as scalar lane masks.
template <int N>
__device__ inline unsigned run_mask(int avail) {
    static_assert(N <= 16, "runs of at most 16");
    const int c = avail < 0 ? 0 : (avail > N ? N : avail);
    return (1u << c) - 1u;
}

// Ranks of positions p[0..N) among the selected positions, and which of them
// are selected: each 32-bit word of the bitmap carries the rank of its first
// bit (16-bit ranks: k <= 4096), so rank = the word's rank + the set bits
// below p in the word -- two LDS reads and a handful of ALU instructions.
// All N lookups' reads are issued before any rank is computed.
template <int N>
__device__ inline void bitmap_ranks(const unsigned* bits, const uint16_t* wrank, const int (&p)[N], int (&rank)[N],
                                    unsigned& isset) {
    unsigned w[N];
    int base[N];
#pragma unroll
    for (int i = 0; i < N; ++i) {
        w[i] = bits[p[i] >> 5];
        base[i] = wrank[p[i] >> 5];
    }
    // (the empty asm uses every read unconditionally, so no read is moved
    // into a branch of its own that would wait for it on the spot)
#pragma unroll
    for (int i = 0; i < N; ++i) asm volatile("" : "+v"(w[i]), "+v"(base[i]));
    isset = 0;
#pragma unroll
    for (int i = 0; i < N; ++i) {
        const unsigned sh = static_cast<unsigned>(p[i]) & 31u;
        rank[i] = base[i] + __popc(w[i] & ((1u << sh) - 1u));
        isset |= ((w[i] >> sh) & 1u) << i;
    }
}

// The age bin where the count taken from the oldest bin downwards first
// reaches `need`, and the count of the bins above it, found by one wave from
// the finished histogram: lane i sums the 16 bins [1008 - 16i, 1023 - 16i],
// one wave scan orders the lanes from the top and a ballot finds the lane L
// where the count crosses `need`; then lanes 0..15 take L's bins from the top
// down, one each, and a scan over that row of 16 lanes finds the bin.
// Requires 0 < need <= the histogram's total.
__device__ inline void crossing_from_top(const int* hist, int need, int& bin, int& below) {
    const int lane = threadIdx.x & 63;
    const int lo = kHistBins - kHistQ * (lane + 1);
    int c = 0;
#pragma unroll
    for (int i = 0; i < kHistQ; i += 4) {
        const int4 v = *reinterpret_cast<const int4*>(hist + lo + i);
        c += v.x + v.y + v.z + v.w;
    }
    const int incl = wave_incl_scan(c);
    const int L = __ffsll(static_cast<long long>(__ballot(incl - c < need && need <= incl))) - 1;  // wave-uniform
    const int loL = kHistBins - kHistQ * (L + 1);
    const int aboveL = __builtin_amdgcn_readlane(incl - c, L);
    const int hb = lane < kHistQ ? hist[loL + kHistQ - 1 - lane] : 0;
    const int x = row_incl_scan(hb);
    const int F = __ffsll(static_cast<long long>(__ballot(lane < kHistQ && need <= aboveL + x))) - 1;
    bin = loL + kHistQ - 1 - F;
    below = aboveL + __builtin_amdgcn_readlane(x - hb, F);
}

// Fallback threshold search among the slots flagged in `elig` (this lane's
// run): the m-th smallest stamp T and how many slots stamped exactly T are
// taken.  Min/max reduction, then a radix select over stamps relative to the
// minimum in 10-bit digits from the top.  Expects hist zeroed; leaves it
// zeroed.  Barriers inside; every lane of the workgroup must call it.
template <int NT, int PER>
__device__ inline void radix_select(int* hist, int* misc, const uint32_t (&tsv)[PER], unsigned elig, int m,
                                    uint32_t& T, int& need_eq) {
    constexpr int NW = NT / 64, BPL = kHistBins / NT;
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
        misc[X_MIN + wave] = static_cast<int>(mn);
        misc[X_MAX + wave] = static_cast<int>(mx);
    }
    __syncthreads();
    mn = 0xFFFFFFFFu;
    mx = 0u;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        mn = min(mn, static_cast<unsigned>(misc[X_MIN + w]));
        mx = max(mx, static_cast<unsigned>(misc[X_MAX + w]));
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
            hist_add(hist, bin);
        }
        __syncthreads();
        // lane tid owns bins [tid*BPL, tid*BPL + BPL): read and zero them, then
        // a block scan finds the bin where the count from the bottom reaches
        // `remaining`
        int hb[BPL], c = 0;
#pragma unroll
        for (int i = 0; i < BPL; ++i) {
            hb[i] = hist[tid * BPL + i];
            hist[tid * BPL + i] = 0;
            c += hb[i];
        }
        const int incl = wave_incl_scan(c);
        if (lane == 63) misc[X_HIST + wave] = incl;
        __syncthreads();
        int acc = incl - c + sum_before(misc + X_HIST, wave);
#pragma unroll
        for (int i = 0; i < BPL; ++i) {
            if (acc < remaining && remaining <= acc + hb[i]) {
                misc[X_BIN] = tid * BPL + i;
                misc[X_BELOW] = acc;
            }
            acc += hb[i];
        }
        __syncthreads();
        prefix = (prefix << d) | static_cast<uint64_t>(misc[X_BIN]);
        remaining -= misc[X_BELOW];
    }
    T = mn + static_cast<uint32_t>(prefix);
    need_eq = remaining;
}

// Phase stamps (constant-rate clock) while tracing is on: lane 0 of wave 0
// keeps them in the misc block (no long-lived scalar registers) and writes
// them out at the end.  Slots in program order: 0 start, 1 reads issued and
// LDS cleared, 2 selection inserted, 3 ranks and hit test, 4 threshold, 5 slot
// by rank and victim counts, 7 selection side looked up, 8 hits published,
// 6 victim lists, 9 metadata written, 10 end; split units take 7 and 8
// (and their host loads) before 4 and 5.
#define HB_PHASE(i)                                                                      \
    do {                                                                                 \
        if (HB_ARG(trace) && tid == 0 && lead)                                                \
            reinterpret_cast<unsigned long long*>(misc + X_STAMP)[(i)] = wall_clock64(); \
    } while (0)
#define HB_PHASE_FLUSH()                                                                                 \
    do {                                                                                                 \
        if (HB_ARG(trace) && tid == 0 && lead) {                                                              \
            const unsigned long long* st_ = reinterpret_cast<const unsigned long long*>(misc + X_STAMP); \
            for (int i_ = 0; i_ < 11; ++i_) s.phase[rl * kPhaseSlots + i_] = st_[i_];                    \
        }                                                                                                \
    } while (0)

// Per-unit counters and the end of a step: miss count, status, clock.  The
// status and counter arrays are read from the arguments here, at the end, so
// they hold no registers before.
__device__ inline void finish_unit(const StateBase& s, uint32_t* clock_u, int32_t* mc_u, int64_t rl, uint32_t t,
                                   int k, int m) {
    *mc_u = m;
    s.status[rl] = 0;
    *clock_u = t + 1u;
    unsigned long long* st = s.stats + 4 * rl;
    atomicAdd(st + 0, static_cast<unsigned long long>(k - m));
    if (m > 0) {
        atomicAdd(st + 1, static_cast<unsigned long long>(m));
        atomicAdd(st + 2, static_cast<unsigned long long>(m) * static_cast<unsigned long long>(s.row_bytes));
    }
    atomicAdd(st + 3, 1ull);
}

// Copy missed rows of one (request, layer) from the host pool into their
// victim slots (launches where no separate fetch launch follows): miss i
// reads position mpos[i] into slot msl[i].  The pieces [c_begin, c_end) of the
// flat (row, 16-byte piece) space of the unit's misses are copied, in the
// fetch kernel's order and with its 16-byte loads, U pieces a lane a round.
template <int NT, bool NTL, int U>
__device__ inline void copy_misses(const StateBase& s, const int* mpos, const int* msl, int64_t rl, int r, int layer,
                                   int c_begin, int c_end) {
    const int row16 = static_cast<int>(s.row_bytes >> 4);
    const uint8_t* src_base = s.pool + s.region_row[static_cast<int64_t>(r) * s.NL + layer] * s.row_bytes;
    uint8_t* dst_base = s.cache + rl * s.B * s.row_bytes;
    for (int c0 = c_begin + static_cast<int>(threadIdx.x); c0 < c_end; c0 += NT * U) {
        u32x4 v[U];
        u32x4* dst[U];
#pragma unroll
        for (int x = 0; x < U; ++x) {
            const int c = c0 + x * NT;
            dst[x] = nullptr;
            if (c < c_end) {
                const int i = c / row16, off = c - i * row16;
                const u32x4* src = reinterpret_cast<const u32x4*>(src_base + static_cast<int64_t>(mpos[i]) * s.row_bytes) + off;
                dst[x] = reinterpret_cast<u32x4*>(dst_base + static_cast<int64_t>(msl[i]) * s.row_bytes) + off;
                v[x] = ld16<NTL>(src);
            }
        }
#pragma unroll
        for (int x = 0; x < U; ++x)
            if (dst[x]) st16<NTL>(dst[x], v[x]);
    }
}

// The victim threshold of a unit with misses (the kernel's step 4, in the
// kernel's own variables): the age histogram unless built speculatively, its
// crossing bin or the radix select, the strict and tied victim bits and
// their packed scan.  Wave 0 alone finds the crossing bin and hands it to
// the others through LDS (one more barrier): every wave finding it on its own
// cost more issue slots than the barrier (per-layer launch of 64 request-
// layers of 4 KB records: 11.9 against 12.3 us by events).
#define HB_FIND_THRESHOLD()                                                                   \
    do {                                                                                      \
        if (!spec) {                                                                          \
        _Pragma("unroll")                                                                     \
            for (int q = 0; q < PER; ++q) {                                                   \
                int bin = -1;                                                                 \
                if ((candbits >> q) & 1u) {                                                   \
                    const uint32_t age = 2u * t - tsv[q];                                     \
                    bin = age < kHistBins - 1 ? static_cast<int>(age) : kHistBins - 1;        \
                }                                                                             \
                hist_add(hist, bin);                                                          \
            }                                                                                 \
            __syncthreads();                                                                  \
        }                                                                                     \
        const int ncand = B - h;                                                              \
        if (m == ncand) {                                                                     \
            T = 0xFFFFFFFFu; /* every candidate is a victim (stamps never reach this value) */\
        } else {                                                                              \
            int bin, below;                                                                   \
            if (wave == 0) {                                                                  \
                crossing_from_top(hist, m, bin, below);                                       \
                if (lane == 0) {                                                              \
                    misc[X_TBIN] = bin;                                                       \
                    misc[X_TBELOW] = below;                                                   \
                }                                                                             \
            }                                                                                 \
            __syncthreads();                                                                  \
            bin = misc[X_TBIN];                                                               \
            below = misc[X_TBELOW];                                                           \
            if (bin < kHistBins - 1) {                                                        \
                T = 2u * t - static_cast<uint32_t>(bin);                                      \
                need_eq = m - below;                                                          \
            } else {                                                                          \
                /* All m victims are at least 1023 ages old: select among those               \
                   with a radix select on their stamps (hist must start at zero). */          \
                __syncthreads();                                                              \
                for (int i = tid; i < kHistBins; i += NT) hist[i] = 0;                        \
                unsigned old_bits = 0;                                                        \
        _Pragma("unroll")                                                                     \
                for (int q = 0; q < PER; ++q)                                                 \
                    if (((candbits >> q) & 1u) &&                                             \
                        2u * t - tsv[q] >= static_cast<uint32_t>(kHistBins - 1))              \
                        old_bits |= 1u << q;                                                  \
                __syncthreads();                                                              \
                radix_select<NT, PER>(hist, misc, tsv, old_bits, m, T, need_eq);              \
            }                                                                                 \
        }                                                                                     \
        _Pragma("unroll")                                                                     \
        for (int q = 0; q < PER; ++q) {                                                       \
            const bool cand = (candbits >> q) & 1u;                                           \
            strict_bits |= static_cast<unsigned>(cand && tsv[q] < T) << q;                    \
            tie_bits |= static_cast<unsigned>(cand && tsv[q] == T) << q;                      \
        }                                                                                     \
        packed = __popc(strict_bits) | (__popc(tie_bits) << 16);                              \
        vincl = wave_incl_scan(packed);                                                       \
        if (lane == 63) misc[X_VICT + wave] = vincl;                                          \
        HB_PHASE(4);                                                                          \
    } while (0)

// LDS layout (ints): region 1 -- bitmap [4*NG words as NG 16-byte groups],
// 16-bit rank of each word [4*NG halves], slot by rank [k] with a spare word
// per lane [64], then victim slot by victim rank [k] and evicted position by
// victim rank [k], each with a spare word per lane [64] (wide launches: the
// two victim lists start at word 0 and overlay the rest of region 1) -- then
// the histogram [kHistBins] and the misc block [kMiscWords].
//
// Template parameters: NT lanes a unit; SPL selections and PER slots a lane
// (contiguous runs j0 = tid*SPL, s0 = tid*PER); VEC: k and B multiples of 4
// and 16-byte aligned selection / output arrays, so runs move as vectors;
// WIDE: a launch over many units (held to eight waves per SIMD at 512 lanes,
// and it copies its own misses); SPLIT: each unit takes lb.wgs workgroups,
// which all plan it alike (the plan is deterministic) and copy its misses
// between them, so no fetch launch follows.  A split unit's workgroups read
// the old slot map, stamps and clock; only the last one to be done reading
// them (a counter per unit, bumped before the copy and looked at after it; no
// workgroup ever waits for another) writes the new metadata, after its copy,
// so none is overwritten while another workgroup may still read it.  A unit
// without misses is the exception: the lead workgroup ends it at once, as
// what it writes (hit stamps, clock) changes nothing the others need when
// every selection hits.
//
// Barriers: B1 LDS cleared; B2 selection inserted; B3 word ranks, hit test of
// every slot (a bit test, no rank needed), hit count -- so m = k - h is known
// here -- and, when the unit missed at its last step, the age histogram of
// the candidates; B4 slot by rank, and (m > 0) threshold and packed victim
// counts; (m > 0 only) hits published and miss counts, then -- wide launches:
// after one more barrier, as the lists overlay the bitmap -- victims listed
// by rank, B5.  After B5 each missing selection takes the victim of its own
// rank.  A split unit with misses takes B4 for the slot by rank alone, looks
// its selections up, lists each miss's position by rank (two barriers),
// issues its first host loads, and only then finds the threshold and victim
// counts (one barrier) before the victim lists and B5.
// a split unit's first host piece of each lane, loaded before its victims are
// found, and its share of the flat (row, piece) space of the unit's misses
// host pieces a lane loads before the victims are found (two or four, at the
// same ~64 workgroups a launch, measured slower: 0.764 and 0.786 against
// 0.753 ms a step of 16 requests x 8 layers of 1152-byte records)
constexpr int kSplitEarly = 1;
struct SplitEarly {
    u32x4 v[kSplitEarly];
    int i[kSplitEarly], off[kSplitEarly];  // miss row (by rank; -1: none) and piece of each
    int i0;                                // this lane's first miss (by rank)
    int c_begin, c_end;
};
struct NoSplitEarly {};

// Where a kernel's first phase takes its scalars from: the argument structs,
// read at each use (wide and split launches), or separate arguments that the
// build preloads into scalar registers at wave launch (per-layer launches).
#define HB_STRUCT_k lb.k
#define HB_STRUCT_B s.B
#define HB_STRUCT_R s.R
#define HB_STRUCT_ngroups lb.ngroups
#define HB_STRUCT_r1_ints lb.r1_ints
#define HB_STRUCT_trace lb.trace
#define HB_STRUCT_clock s.clock
#define HB_STRUCT_length s.length
#define HB_STRUCT_miss_count s.miss_count
#define HB_STRUCT_slot_pos s.slot_pos
#define HB_STRUCT_ts s.ts
#define HB_PRELOADED(x) x##_arg

// Wide and split launches: every argument read from the argument block (these
// builds are short of scalar registers; preloading measured slower there).
template <int NT, int SPL, int PER, bool VEC, bool WIDE, bool SPLIT>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(WIDE ? (NT == 512 ? 8 : 6) : 1)))
void bitmap_resolve_kernel(StateBase s, LayerBatch lb) {
#define HB_ARG(x) HB_STRUCT_##x
#include "resolve_bitmap_unit.inc"
#undef HB_ARG
}

// Per-layer launches, one workgroup a unit: the first phase's values lead the
// arguments, and the build preloads them into scalar registers at wave launch
// (the per-layer launch at 64 request-layers of 4 KB records: 11.4 against
// 11.8 us by events over three interleaved runs).
template <int NT, int SPL, int PER, bool VEC, bool WIDE = false, bool SPLIT = false>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(1)))
void bitmap_resolve_layer_kernel(int k_arg, int B_arg, int R_arg, int ngroups_arg, int r1_ints_arg, int trace_arg,
                                 uint32_t* clock_arg, int32_t* length_arg, int32_t* miss_count_arg,
                                 int32_t* slot_pos_arg, uint32_t* ts_arg, StateBase s, LayerBatch lb) {
    static_assert(!WIDE && !SPLIT, "one workgroup a unit, one unit a workgroup");
#define HB_ARG(x) HB_PRELOADED(x)
#include "resolve_bitmap_unit.inc"
#undef HB_ARG
}

template <int NT, int SPL, int PER, bool VEC, bool WIDE, bool SPLIT>
hipError_t launch_b(const StateBase& s, const LayerBatch& lb, size_t lds, hipStream_t st) {
    static LdsGrants granted;  // per instantiation
    const unsigned gx = SPLIT ? static_cast<unsigned>(s.R) * static_cast<unsigned>(lb.wgs) : static_cast<unsigned>(s.R);
    if constexpr (!WIDE && !SPLIT) {
        const void* fn = reinterpret_cast<const void*>(&bitmap_resolve_layer_kernel<NT, SPL, PER, VEC>);
        const hipError_t e = ensure_lds_limit(fn, lds, granted);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL((bitmap_resolve_layer_kernel<NT, SPL, PER, VEC>), dim3(gx, lb.n), dim3(NT), lds, st, lb.k,
                           s.B, s.R, lb.ngroups, lb.r1_ints, lb.trace, s.clock, s.length, s.miss_count, s.slot_pos,
                           s.ts, s, lb);
    } else {
        const void* fn = reinterpret_cast<const void*>(&bitmap_resolve_kernel<NT, SPL, PER, VEC, WIDE, SPLIT>);
        const hipError_t e = ensure_lds_limit(fn, lds, granted);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL((bitmap_resolve_kernel<NT, SPL, PER, VEC, WIDE, SPLIT>), dim3(gx, lb.n), dim3(NT), lds, st,
                           s, lb);
    }
    return hipGetLastError();
}

template <int NT, int SPL, int PER, bool WIDE>
hipError_t launch_v(const StateBase& s, const LayerBatch& lb, size_t lds, bool vec, hipStream_t st) {
    if (lb.wgs > 0) {
        // split units: 1024 lanes, vector runs (plan_wgs checks both)
        if constexpr (NT == 1024 && !WIDE) {
            if (vec) return launch_b<NT, SPL, PER, true, false, true>(s, lb, lds, st);
        }
        return hipErrorInvalidValue;
    }
    return vec ? launch_b<NT, SPL, PER, true, WIDE, false>(s, lb, lds, st)
               : launch_b<NT, SPL, PER, false, WIDE, false>(s, lb, lds, st);
}

template <int NT, int SPL, bool WIDE>
hipError_t launch_p(const StateBase& s, const LayerBatch& lb, size_t lds, bool vec, hipStream_t st) {
    const int per = (s.B + NT - 1) / NT;
    if (per <= 1) return launch_v<NT, SPL, 1, WIDE>(s, lb, lds, vec, st);
    if (per <= 2) return launch_v<NT, SPL, 2, WIDE>(s, lb, lds, vec, st);
    if (per <= 4) return launch_v<NT, SPL, 4, WIDE>(s, lb, lds, vec, st);
    if (per <= 8) return launch_v<NT, SPL, 8, WIDE>(s, lb, lds, vec, st);
    if constexpr (NT == 1024) {
        if (per <= 16) return launch_v<NT, SPL, 16, WIDE>(s, lb, lds, vec, st);
    }
    return hipErrorInvalidValue;
}

template <int NT, bool WIDE>
hipError_t launch_s(const StateBase& s, const LayerBatch& lb, size_t lds, bool vec, hipStream_t st) {
    const int spl = (lb.k + NT - 1) / NT;
    if (spl <= 1) return launch_p<NT, 1, WIDE>(s, lb, lds, vec, st);
    if (spl <= 2) return launch_p<NT, 2, WIDE>(s, lb, lds, vec, st);
    if (spl <= 4) return launch_p<NT, 4, WIDE>(s, lb, lds, vec, st);
    return hipErrorInvalidValue;
}

}  // namespace

// Ints of region 1 of the bitmap kernel's LDS, rounded to 16 bytes: bitmap
// (4 per group), 16-bit word ranks (2 per group), slot by rank with a spare
// word per lane, victim lists (after the rest, or over it in wide launches).
static size_t bitmap_r1_ints(int k, int ngroups, bool wide) {
    const size_t base = 6 * static_cast<size_t>(ngroups) + static_cast<size_t>(k) + 64;
    const size_t lists = 2 * (static_cast<size_t>(k) + 64);
    const size_t r1 = wide ? std::max(base, lists) : base + lists;
    return (r1 + 3) & ~static_cast<size_t>(3);
}

size_t bitmap_lds_bytes(int k, int64_t L_ctx, bool wide) {
    const int ng = static_cast<int>((L_ctx + 127) >> 7);
    return sizeof(int) * (bitmap_r1_ints(k, ng, wide) + kHistBins + kMiscWords);
}

int bitmap_lanes(int B, int k, bool wide, int asked) {
    // 512 lanes let four units share a CU in wide launches; a few units per
    // launch take 1024 lanes unless asked otherwise
    const bool can512 = B <= 8 * 512 && k <= 4 * 512;
    if (asked == 512) return can512 ? 512 : 1024;
    if (asked == 1024) return 1024;
    return (wide && can512) ? 512 : 1024;
}

hipError_t launch_bitmap_resolve(const StateBase& s, const LayerBatch& lb_in, bool wide, bool vec, hipStream_t st) {
    LayerBatch lb = lb_in;
    lb.ngroups = static_cast<int>((s.L_ctx + 127) >> 7);
    lb.r1_ints = static_cast<int>(bitmap_r1_ints(lb.k, lb.ngroups, wide));
    const size_t lds = bitmap_lds_bytes(lb.k, s.L_ctx, wide);
    if (bitmap_lanes(s.B, lb.k, wide, lb.lanes) == 512) {
        return wide ? launch_s<512, true>(s, lb, lds, vec, st) : launch_s<512, false>(s, lb, lds, vec, st);
    }
    return wide ? launch_s<1024, true>(s, lb, lds, vec, st) : launch_s<1024, false>(s, lb, lds, vec, st);
}

}  // namespace hs
