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
        if (lb.trace && tid == 0 && lead)                                                \
            reinterpret_cast<unsigned long long*>(misc + X_STAMP)[(i)] = wall_clock64(); \
    } while (0)
#define HB_PHASE_FLUSH()                                                                                 \
    do {                                                                                                 \
        if (lb.trace && tid == 0 && lead) {                                                              \
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

template <int NT, int SPL, int PER, bool VEC, bool WIDE, bool SPLIT>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(WIDE ? (NT == 512 ? 8 : 6) : 1)))
void bitmap_resolve_kernel(StateBase s, LayerBatch lb) {
    constexpr int NW = NT / 64;
    static_assert(NW <= 16, "per-wave partials fit one row of 16 lanes");
    static_assert(!(WIDE && SPLIT), "a wide launch has one workgroup a unit");
    extern __shared__ int lds[];
    const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
    const int G = SPLIT ? lb.wgs : 1;
    const int r = SPLIT ? static_cast<int>(blockIdx.x) / G : static_cast<int>(blockIdx.x);
    const int g = SPLIT ? static_cast<int>(blockIdx.x) - r * G : 0;
    const bool lead = g == 0;  // publishes slot_idx and the hit mask, stamps phases
    const int layer = lb.layer[blockIdx.y];
    const int k = lb.k, B = s.B, NG = lb.ngroups;
    const int64_t rl = static_cast<int64_t>(layer) * s.R + r;
    const int32_t* sel = lb.sel[blockIdx.y] + static_cast<int64_t>(r) * k;
    int32_t* out = lb.out[blockIdx.y] + static_cast<int64_t>(r) * k;
    int32_t* spos_g = s.slot_pos + rl * B;
    uint32_t* ts_g = s.ts + rl * B;
    uint32_t* clock_u = s.clock + rl;
    int32_t* mc_u = s.miss_count + rl;
    uint4* const bits4 = reinterpret_cast<uint4*>(lds);
    unsigned* const bits = reinterpret_cast<unsigned*>(lds);
    uint16_t* const wrank = reinterpret_cast<uint16_t*>(lds + 4 * NG);  // [4*NG] rank of each word
    int* const byrank = lds + 6 * NG;
    // victim lists: a wide launch lays them over the bitmap, its ranks and
    // the slot by rank once every wave is done reading those (one more
    // barrier, only in units with misses), so four units fit a CU's LDS
    int* const vlist = WIDE ? lds : byrank + k + 64;
    int* const vold = vlist + k + 64;  // (each list has a spare word per lane)
    int* const hist = lds + lb.r1_ints;
    int* const misc = hist + kHistBins;
    if (lb.trace && tid == 0 && lead) {
        // the stamp words lie outside the part of the misc block cleared below
        unsigned long long* st0 = reinterpret_cast<unsigned long long*>(misc + X_STAMP);
        st0[0] = wall_clock64();
        for (int i = 1; i < 11; ++i) st0[i] = 0ull;
    }

    // 1. every global read up front: clock, history length, last step's miss
    // count, this lane's runs of the selection, the slot map and the stamps
    const uint32_t t = *clock_u;
    const int hist_len = s.length[rl];
    const bool spec = *mc_u > 0;  // expect misses: build the age histogram early
    const int j0 = tid * SPL, s0 = tid * PER;
    const unsigned insel = run_mask<SPL>(k - j0), inslot = run_mask<PER>(B - s0);
    int selv[SPL];
    load_run<SPL, VEC, int>(sel, j0, k, selv, kEmpty);
    int spos[PER];
    load_run<PER, VEC, int>(spos_g, s0, B, spos, kEmpty);
    // (the stamp run is read even by a unit that will hit everywhere: its
    // hit stamps go back as whole 16-byte pieces, which measured faster than
    // scattered 4-byte stores without the read)
    uint32_t tsv[PER];
    load_run<PER, VEC, uint32_t>(ts_g, s0, B, tsv, 0u);
    for (int g = tid; g < NG; g += NT) bits4[g] = make_uint4(0u, 0u, 0u, 0u);
    for (int i = tid; i < k; i += NT) byrank[i] = kEmpty;
    for (int i = tid; i < kHistBins; i += NT) hist[i] = 0;
    if (tid < X_STAMP) misc[tid] = 0;
    __syncthreads();
    HB_PHASE(1);

    // 2. every selected position sets its bit; a bit already set is a
    // repeated position, a position outside the history rejects the request
    // (straight-line: a lane without a valid selection ORs nothing into word 0)
    {
        int bad = 0, bad_at = 0;
#pragma unroll
        for (int q = 0; q < SPL; ++q) {
            const int j = j0 + q;
            const int p = selv[q];
            const bool live = (insel >> q) & 1u;
            const bool inr = live && static_cast<unsigned>(p) < static_cast<unsigned>(hist_len);
            const unsigned bit = inr ? 1u << (p & 31) : 0u;
            const unsigned old = atomicOr(&bits[inr ? p >> 5 : 0], bit);
            const int bb = ((live && !inr) ? 1 : 0) | ((old & bit) ? 2 : 0);
            bad |= bb;
            bad_at = bb ? j + 1 : bad_at;
        }
        block_or_into(&misc[X_FLAGS], bad);
        if (bad) atomicMax(&misc[X_BADAT], bad_at);
    }
    __syncthreads();
    HB_PHASE(2);
    const int flags = misc[X_FLAGS];
    if (flags) {
        // reject: -1 everywhere, state unchanged
        if (!lead) return;
        for (int j = tid; j < k; j += NT) {
            out[j] = -1;
            s.hit_mask[rl * B + j] = 0;
        }
        if (tid == 0) {
            *mc_u = 0;
            s.status[rl] = (flags & 1) ? HS_DEV_RANGE : HS_DEV_DUP;
            record_error(s.err, (flags & 1) ? HS_DEV_RANGE : HS_DEV_DUP, layer, r, misc[X_BADAT] - 1);
        }
        return;
    }

    // 3. group ranks: lane tid owns groups tid, tid + NT, ... (consecutive
    // lanes, consecutive 16-byte pieces); each wave takes its run of ranks
    // with one LDS atomic, so ranks map the selected positions one to one
    // onto [0, k) whatever order the waves' atomics land in
    {
        int cnt = 0;
        for (int g = tid; g < NG; g += NT) {
            const uint4 v = bits4[g];
            cnt += __popc(v.x) + __popc(v.y) + __popc(v.z) + __popc(v.w);
        }
        const int incl = wave_incl_scan(cnt);
        int wb = 0;
        if (lane == 63) wb = atomicAdd(&misc[X_RANK], incl);
        int base = __builtin_amdgcn_readlane(wb, 63) + incl - cnt;
        for (int g = tid; g < NG; g += NT) {
            const uint4 v = bits4[g];
            const unsigned r0 = static_cast<unsigned>(base);
            const unsigned r1 = r0 + __popc(v.x), r2 = r1 + __popc(v.y), r3 = r2 + __popc(v.z);
            reinterpret_cast<uint2*>(wrank)[g] = make_uint2(r0 | (r1 << 16), r2 | (r3 << 16));
            base = static_cast<int>(r3) + __popc(v.w);
        }
    }
    // hit test of this lane's slots (one bit each: a cached position whose
    // bit is set is selected), the hit stamps 2t+2 written back as whole
    // pieces of the stamp run, and the hit count
    const uint32_t ts_hit = 2u * t + 2u, ts_miss = 2u * t + 1u;
    const int nbits_pos = NG * 128;
    unsigned hitbits = 0;
    {
        unsigned w[PER];
#pragma unroll
        for (int q = 0; q < PER; ++q) {
            // (a slot past the end of the run holds -1, as does an empty one)
            const int p = spos[q];
            const bool live = static_cast<unsigned>(p) < static_cast<unsigned>(nbits_pos);
            w[q] = bits[live ? p >> 5 : 0];
        }
        // every word is read whether or not its slot is live (the empty asm
        // uses each one unconditionally), so no read sits in a branch of its
        // own that waits for it on the spot
#pragma unroll
        for (int q = 0; q < PER; ++q) asm volatile("" : "+v"(w[q]));
#pragma unroll
        for (int q = 0; q < PER; ++q) {
            const int p = spos[q];
            const bool live = static_cast<unsigned>(p) < static_cast<unsigned>(nbits_pos);
            hitbits |= static_cast<unsigned>(live && ((w[q] >> (p & 31)) & 1u)) << q;
        }
    }
    const unsigned candbits = inslot & ~hitbits;  // slots that may be evicted
    if (!SPLIT && hitbits) {
        uint32_t tsn[PER];
#pragma unroll
        for (int q = 0; q < PER; ++q) tsn[q] = ((hitbits >> q) & 1u) ? ts_hit : tsv[q];
        store_run_masked<PER, VEC, uint32_t>(ts_g, s0, B, tsn, hitbits);
    }
    {
        const int hincl = wave_incl_scan(__popc(hitbits));
        if (lane == 63) misc[X_HITS + wave] = hincl;
    }
    if (spec) {
        // candidate ages (2t - stamp; no stamp exceeds 2t before step t);
        // ages of 1023 and more share the top bin
#pragma unroll
        for (int q = 0; q < PER; ++q) {
            int bin = -1;
            if ((candbits >> q) & 1u) {
                const uint32_t age = 2u * t - tsv[q];
                bin = age < kHistBins - 1 ? static_cast<int>(age) : kHistBins - 1;
            }
            hist_add(hist, bin);
        }
    }
    __syncthreads();
    HB_PHASE(3);
    const int h = sum_before(misc + X_HITS, NW);
    const int m = k - h;

    // 4. each hit slot records itself at its position's rank (a slot that is
    // not a hit writes its lane's spare word byrank[k + lane] instead)
    {
        constexpr int NB = PER < 4 ? PER : 4;
#pragma unroll
        for (int q0 = 0; q0 < PER; q0 += NB) {
            int pp[NB], rk[NB];
            unsigned isset;
#pragma unroll
            for (int i = 0; i < NB; ++i) pp[i] = ((hitbits >> (q0 + i)) & 1u) ? spos[q0 + i] : 0;
            bitmap_ranks<NB>(bits, wrank, pp, rk, isset);
#pragma unroll
            for (int i = 0; i < NB; ++i) {
                const bool hit = (hitbits >> (q0 + i)) & 1u;
                byrank[hit ? rk[i] : k + lane] = s0 + q0 + i;
            }
        }
    }
    // threshold stamp T and how many candidates stamped exactly T go (lowest
    // slots first; every other victim is older than T), then the victim
    // counts in slot order, strict and tied packed into one scan (strict in
    // the low 16 bits, tied in the high; both at most B <= 16384).  A split
    // unit finds it later, after its selections are looked up and its host
    // loads issued, so that they are in flight meanwhile.
    uint32_t T = 0;
    int need_eq = 0, packed = 0, vincl = 0;
    unsigned strict_bits = 0, tie_bits = 0;
    if constexpr (!SPLIT) {
        if (m > 0) HB_FIND_THRESHOLD();
    }
    __syncthreads();
    if constexpr (!SPLIT) HB_PHASE(5);

    // 5. selection side: the slot recorded at each selection's rank is its
    // hit, published now, or nothing (a miss)
    int slv[SPL];
    unsigned mf = 0;
    {
        // (a lane past the end looks up position 0; its rank stays within
        // [0, k], so the read stays inside byrank and is discarded)
        int pp[SPL], rk[SPL];
        unsigned isset;
#pragma unroll
        for (int q = 0; q < SPL; ++q) pp[q] = ((insel >> q) & 1u) ? selv[q] : 0;
        bitmap_ranks<SPL>(bits, wrank, pp, rk, isset);
        (void)isset;
        int v[SPL];
#pragma unroll
        for (int q = 0; q < SPL; ++q) v[q] = byrank[rk[q]];
#pragma unroll
        for (int q = 0; q < SPL; ++q) asm volatile("" : "+v"(v[q]));
#pragma unroll
        for (int q = 0; q < SPL; ++q) {
            const bool live = (insel >> q) & 1u;
            slv[q] = live ? v[q] : kEmpty;
            mf |= static_cast<unsigned>(live && v[q] < 0) << q;
        }
    }
    HB_PHASE(7);
    if (lead) {
        constexpr int W = SPL < 4 ? SPL : 4;
        constexpr unsigned PM = (1u << W) - 1u;
        uint8_t* hm = s.hit_mask + rl * B;
        if constexpr (VEC && W >= 2) {
#pragma unroll
            for (int q = 0; q < SPL; q += W) {
                if (j0 + q < k) {
                    if (((mf >> q) & PM) == 0u) {
                        if constexpr (W == 4)
                            *reinterpret_cast<int4*>(out + j0 + q) = make_int4(slv[q], slv[q + 1], slv[q + 2], slv[q + 3]);
                        else
                            *reinterpret_cast<int2*>(out + j0 + q) = make_int2(slv[q], slv[q + 1]);
                    } else {
#pragma unroll
                        for (int e = 0; e < W; ++e)
                            if (!((mf >> (q + e)) & 1u)) out[j0 + q + e] = slv[q + e];
                    }
                    unsigned hw = 0;
#pragma unroll
                    for (int e = 0; e < W; ++e) hw |= static_cast<unsigned>(!((mf >> (q + e)) & 1u)) << (8 * e);
                    if constexpr (W == 4) *reinterpret_cast<uint32_t*>(hm + j0 + q) = hw;
                    else *reinterpret_cast<uint16_t*>(hm + j0 + q) = static_cast<uint16_t>(hw);
                }
            }
        } else {
#pragma unroll
            for (int q = 0; q < SPL; ++q) {
                const int j = j0 + q;
                if (j < k) {
                    if (!((mf >> q) & 1u)) out[j] = slv[q];
                    hm[j] = ((mf >> q) & 1u) ? 0 : 1;
                }
            }
        }
    }
    HB_PHASE(8);
    if (m == 0) {
        // every selection hit: the hit stamps are written, nothing else changes
        if constexpr (SPLIT) {
            // (the other workgroups of the unit find no miss either: the slot
            // map does not change, and stamps and clock only matter to misses)
            if (!lead) return;
            if (hitbits) {
                uint32_t tsn[PER];
#pragma unroll
                for (int q = 0; q < PER; ++q) tsn[q] = ((hitbits >> q) & 1u) ? ts_hit : tsv[q];
                store_run_masked<PER, VEC, uint32_t>(ts_g, s0, B, tsn, hitbits);
            }
        }
        if (tid == 0) finish_unit(s, clock_u, mc_u, rl, t, k, 0);
        HB_PHASE(10);
        HB_PHASE_FLUSH();
        return;
    }
    // misses per wave (for each miss's rank), and the victims: the slot of
    // victim rank i goes to vlist[i], its evicted position to vold[i] (and
    // back to host-only: no write-back, the host copy is authoritative); its
    // stamp becomes 2t+1 in this lane's run, written back whole
    const int mc = __popc(mf);
    const int mincl = wave_incl_scan(mc);
    if (lane == 63) misc[X_MISS + wave] = mincl;
    if constexpr (WIDE) __syncthreads();  // the victim lists overwrite the bitmap
    // a split unit: the position of each miss is listed by rank (over the slot
    // by rank, read by nobody any more) and this workgroup's first pieces of
    // the unit's flat (row, piece) space of misses are loaded from the host
    // into registers now; the victim slots they go to are found meanwhile
    // (kSplitEarly pieces a lane, as in the copy; the state exists in split
    // builds only, so the others keep their registers)
    std::conditional_t<SPLIT, SplitEarly, NoSplitEarly> early;
    if constexpr (SPLIT) {
        __syncthreads();  // miss counts visible; every read of the slot by rank done
        const int i0 = mincl - mc + sum_before(misc + X_MISS, wave);
        early.i0 = i0;
        int* const mpos = byrank;
        {
            int i = i0;
#pragma unroll
            for (int q = 0; q < SPL; ++q) {
                if ((mf >> q) & 1u) {
                    mpos[i] = selv[q];
                    ++i;
                }
            }
        }
        __syncthreads();  // every miss's position is listed
        const int row16 = static_cast<int>(s.row_bytes >> 4);
        const int total = m * row16;
        early.c_begin = static_cast<int>(static_cast<int64_t>(total) * g / G);
        early.c_end = static_cast<int>(static_cast<int64_t>(total) * (g + 1) / G);
        const uint8_t* src_base = s.pool + s.region_row[static_cast<int64_t>(r) * s.NL + layer] * s.row_bytes;
#pragma unroll
        for (int x = 0; x < kSplitEarly; ++x) {
            const int c = early.c_begin + tid + x * NT;
            early.i[x] = -1;
            early.off[x] = 0;
            if (c < early.c_end) {
                const int i = c / row16, off = c - i * row16;
                const u32x4* src = reinterpret_cast<const u32x4*>(src_base + static_cast<int64_t>(mpos[i]) * s.row_bytes) + off;
                early.i[x] = i;
                early.off[x] = off;
                early.v[x] = lb.nt ? ld16<true>(src) : ld16<false>(src);
            }
        }
        HB_FIND_THRESHOLD();
        __syncthreads();  // victim counts visible
        HB_PHASE(5);
    }
    unsigned vbits = 0;
    {
        const int vpre = vincl - packed + sum_before(misc + X_VICT, wave);
        int sb = vpre & 0xFFFF, tb = vpre >> 16;
        int32_t* pt = s.page_table + rl * s.L_ctx;
#pragma unroll
        for (int q = 0; q < PER; ++q) {
            const bool st = (strict_bits >> q) & 1u, ti = (tie_bits >> q) & 1u;
            const int rank = st ? sb + min(tb, need_eq) : ((ti && tb < need_eq) ? sb + tb : -1);
            sb += st ? 1 : 0;
            tb += ti ? 1 : 0;
            const bool victim = rank >= 0 && rank < m;
            // (straight-line: a slot that is not a victim writes its lane's
            // spare words past the lists instead)
            const int at = victim ? rank : k + lane;
            vlist[at] = s0 + q;
            vold[at] = spos[q];
            vbits |= static_cast<unsigned>(victim) << q;
        }
        if constexpr (!SPLIT) {
#pragma unroll
            for (int q = 0; q < PER; ++q) {
                if (((vbits >> q) & 1u) && spos[q] >= 0) pt[spos[q]] = -1;
                if constexpr (WIDE)
                    if ((vbits >> q) & 1u) ts_g[s0 + q] = ts_miss;  // (the stamp run is not kept live this far)
            }
        }
        if (!WIDE && !SPLIT && vbits) {
            uint32_t tsn[PER];
#pragma unroll
            for (int q = 0; q < PER; ++q)
                tsn[q] = ((vbits >> q) & 1u) ? ts_miss : (((hitbits >> q) & 1u) ? ts_hit : tsv[q]);
            store_run_masked<PER, VEC, uint32_t>(ts_g, s0, B, tsn, vbits | hitbits);
        }
    }
    __syncthreads();
    HB_PHASE(6);

    // 6. the i-th miss (ascending selection index) takes the victim of rank i
    // (ascending slot): plan entry, page table, slot map and publication
    if constexpr (!SPLIT) {
        const int i0 = mincl - mc + sum_before(misc + X_MISS, wave);  // this lane's first miss
        int32_t* pt = s.page_table + rl * s.L_ctx;
        int4* plan = s.plan + rl * B;
        int i = i0;
#pragma unroll
        for (int q = 0; q < SPL; ++q) {
            if ((mf >> q) & 1u) {
                const int j = j0 + q, p = selv[q];
                const int v = vlist[i], old = vold[i];
                plan[i] = make_int4(j, v, old, p);
                pt[p] = v;
                spos_g[v] = p;
                out[j] = v;
                if constexpr (WIDE) vold[i] = p;  // the copy reads positions from here
                ++i;
            }
        }
        HB_PHASE(9);
        if (tid == 0) finish_unit(s, clock_u, mc_u, rl, t, k, m);
        if constexpr (WIDE) {
            // a wide launch copies its own misses: with hundreds of workgroups
            // copying at once the link is as busy as under the chip-wide fetch
            // kernel, and the launch after it is saved
            if (lb.copy) {
                __syncthreads();  // every miss's position is in vold
                const int total = m * static_cast<int>(s.row_bytes >> 4);
                if (lb.nt) copy_misses<NT, true, 4>(s, vold, vlist, rl, r, layer, 0, total);
                else copy_misses<NT, false, 4>(s, vold, vlist, rl, r, layer, 0, total);
            }
        }
        HB_PHASE(10);
        HB_PHASE_FLUSH();
    } else {
        const int i0 = early.i0;  // this lane's first miss
        // the lead publishes the misses' slots
        if (lead) {
            int i = i0;
#pragma unroll
            for (int q = 0; q < SPL; ++q) {
                if ((mf >> q) & 1u) {
                    out[j0 + q] = vlist[i];
                    ++i;
                }
            }
        }
        HB_PHASE(9);
        // arrival, before the copy (which reads no metadata): every read of
        // the old metadata is long done, its values used before the barriers
        // above.  The counter's answer is only looked at after the copy, so
        // its round trip overlaps the copy instead of following it.
        unsigned arrived_before = 0;
        if (tid == 0) arrived_before = atomicAdd(&s.arrive[rl], 1u);
        {
            // the pieces loaded early go to their victim slots, then the rest
            // of this workgroup's share, one host load a lane in flight as in
            // the fetch kernel (about a megabyte over the launch's ~64
            // workgroups; more per lane measured slower over the host link)
            uint8_t* dst_base = s.cache + rl * s.B * s.row_bytes;
#pragma unroll
            for (int x = 0; x < kSplitEarly; ++x) {
                if (early.i[x] >= 0) {
                    u32x4* dst = reinterpret_cast<u32x4*>(dst_base + static_cast<int64_t>(vlist[early.i[x]]) * s.row_bytes) +
                                 early.off[x];
                    if (lb.nt) st16<true>(dst, early.v[x]);
                    else st16<false>(dst, early.v[x]);
                }
            }
            const int c_rest = min(early.c_end, early.c_begin + kSplitEarly * NT);
            if (lb.nt) copy_misses<NT, true, 1>(s, byrank, vlist, rl, r, layer, c_rest, early.c_end);
            else copy_misses<NT, false, 1>(s, byrank, vlist, rl, r, layer, c_rest, early.c_end);
        }
        // the last workgroup to arrive writes the new metadata
        if (tid == 0) misc[X_LAST] = arrived_before == static_cast<unsigned>(G - 1) ? 1 : 0;
        __syncthreads();
        if (!misc[X_LAST]) {
            HB_PHASE(10);
            HB_PHASE_FLUSH();
            return;
        }
        if (tid == 0) s.arrive[rl] = 0u;  // ready for the next launch
        // the unit's new metadata: evicted positions back to host only (no
        // write-back, the host copy is authoritative), the stamp run with the
        // hits at 2t+2 and the victims at 2t+1, then per miss the plan entry,
        // the page table and the slot map
        int32_t* pt = s.page_table + rl * s.L_ctx;
#pragma unroll
        for (int q = 0; q < PER; ++q)
            if (((vbits >> q) & 1u) && spos[q] >= 0) pt[spos[q]] = -1;
        if (vbits | hitbits) {
            uint32_t tsn[PER];
#pragma unroll
            for (int q = 0; q < PER; ++q)
                tsn[q] = ((vbits >> q) & 1u) ? ts_miss : (((hitbits >> q) & 1u) ? ts_hit : tsv[q]);
            store_run_masked<PER, VEC, uint32_t>(ts_g, s0, B, tsn, vbits | hitbits);
        }
        int4* plan = s.plan + rl * B;
        int i = i0;
#pragma unroll
        for (int q = 0; q < SPL; ++q) {
            if ((mf >> q) & 1u) {
                const int j = j0 + q, p = selv[q];
                const int v = vlist[i], old = vold[i];
                plan[i] = make_int4(j, v, old, p);
                pt[p] = v;
                spos_g[v] = p;
                ++i;
            }
        }
        if (tid == 0) finish_unit(s, clock_u, mc_u, rl, t, k, m);
        HB_PHASE(10);
        HB_PHASE_FLUSH();
    }
}

template <int NT, int SPL, int PER, bool VEC, bool WIDE, bool SPLIT>
hipError_t launch_b(const StateBase& s, const LayerBatch& lb, size_t lds, hipStream_t st) {
    static LdsGrants granted;  // per instantiation
    const void* fn = reinterpret_cast<const void*>(&bitmap_resolve_kernel<NT, SPL, PER, VEC, WIDE, SPLIT>);
    const hipError_t e = ensure_lds_limit(fn, lds, granted);
    if (e != hipSuccess) return e;
    const unsigned gx = SPLIT ? static_cast<unsigned>(s.R) * static_cast<unsigned>(lb.wgs) : static_cast<unsigned>(s.R);
    hipLaunchKernelGGL((bitmap_resolve_kernel<NT, SPL, PER, VEC, WIDE, SPLIT>), dim3(gx, lb.n), dim3(NT), lds, st, s,
                       lb);
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
