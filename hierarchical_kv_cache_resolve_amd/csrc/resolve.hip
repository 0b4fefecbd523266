// resolve.hip -- metadata half of RESOLVE on gfx950: hash build, cache probe,
// miss compaction, LRU victim choice, metadata update and publication.
//
// One 1024-lane workgroup (16 wave64s) per (request, layer); a batched launch
// covers several independent layers with grid.y.  The five stages follow the
// pith review's "Core claim" / "What carries the argument" (shared-memory hash
// table over the selected positions, a parallel probe and scan to mark hits and
// choose victims, page-table publication); the host fetch of the misses is the
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
#include <climits>

#include "hs_internal.h"

namespace hs {

namespace {

constexpr int kEmpty = -1;

__device__ inline unsigned hash_pos(int p, int bits) {
    // multiplicative hashing with the golden-ratio constant (Knuth, TAOCP 6.4)
    return (static_cast<unsigned>(p) * 0x9E3779B1u) >> (32 - bits);
}

// Block-wide exclusive scan of one int per lane (1024 lanes).  `scratch`
// holds kPlanWaves + 1 ints of LDS.  Ends with a barrier, so the scratch may
// be reused by the next call.
__device__ inline int block_excl_scan(int v, int* total, int* scratch) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int x = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
    }
    if (lane == 63) scratch[wave] = x;
    __syncthreads();
    if (wave == 0) {
        int w = lane < kPlanWaves ? scratch[lane] : 0;
#pragma unroll
        for (int off = 1; off < kPlanWaves; off <<= 1) {
            const int y = __shfl_up(w, off, 64);
            if (lane >= off) w += y;
        }
        if (lane < kPlanWaves) scratch[lane] = w;
    }
    __syncthreads();
    const int base = wave ? scratch[wave - 1] : 0;
    *total = scratch[kPlanWaves - 1];
    __syncthreads();
    return base + x - v;
}

__device__ inline unsigned wave_min(unsigned v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v = min(v, static_cast<unsigned>(__shfl_xor(static_cast<int>(v), off, 64)));
    return v;
}

__device__ inline unsigned wave_max(unsigned v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v = max(v, static_cast<unsigned>(__shfl_xor(static_cast<int>(v), off, 64)));
    return v;
}

// LDS carve-up of the plan kernel (ints): hash keys [H], hash values [H],
// slot per selection [k], miss list [k], selection copy [k], histogram
// [kHistBins], scan scratch [32].
struct PlanLds {
    int* hkey;
    int* hval;
    int* sidx;
    int* mlist;
    int* sel;
    int* hist;
    int* scratch;
};

__device__ inline PlanLds carve(int* base, int H, int k) {
    PlanLds l;
    l.hkey = base;
    l.hval = l.hkey + H;
    l.sidx = l.hval + H;
    l.mlist = l.sidx + k;
    l.sel = l.mlist + k;
    l.hist = l.sel + k;
    l.scratch = l.hist + kHistBins;
    return l;
}

// Insert (p -> j) with linear probing.  Returns false if p is already present.
__device__ inline bool hash_insert(const PlanLds& l, int H, int bits, int p, int j) {
    unsigned h = hash_pos(p, bits);
    for (;;) {
        const int prev = atomicCAS(&l.hkey[h], kEmpty, p);
        if (prev == kEmpty) {
            l.hval[h] = j;
            return true;
        }
        if (prev == p) return false;
        h = (h + 1) & static_cast<unsigned>(H - 1);
    }
}

__device__ inline int hash_find(const PlanLds& l, int H, int bits, int p) {
    unsigned h = hash_pos(p, bits);
    for (;;) {
        const int key = l.hkey[h];
        if (key == p) return l.hval[h];
        if (key == kEmpty) return -1;
        h = (h + 1) & static_cast<unsigned>(H - 1);
    }
}

// Per-lane contiguous slot range [tid*PER, tid*PER + PER), moved as 16-byte
// vectors when the whole range is in bounds and 16-byte aligned (B % 4 == 0).
template <int PER, typename T>
__device__ inline void load_run(const T* g, int s0, int B, T (&v)[PER], T fill) {
    if (s0 + PER <= B && (PER % 4) == 0 && (B & 3) == 0) {
#pragma unroll
        for (int q = 0; q < PER; q += 4) {
            const int4 w = *reinterpret_cast<const int4*>(g + s0 + q);
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

template <int PER, typename T>
__device__ inline void store_run(T* g, int s0, int B, const T (&v)[PER]) {
    if (s0 + PER <= B && (PER % 4) == 0 && (B & 3) == 0) {
#pragma unroll
        for (int q = 0; q < PER; q += 4) {
            int4 w;
            w.x = static_cast<int>(v[q]);
            w.y = static_cast<int>(v[q + 1]);
            w.z = static_cast<int>(v[q + 2]);
            w.w = static_cast<int>(v[q + 3]);
            *reinterpret_cast<int4*>(g + s0 + q) = w;
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

template <int PER>
__global__ __launch_bounds__(kPlanThreads) void plan_kernel(StateBase s, LayerBatch lb) {
    extern __shared__ int lds_raw[];
    const int tid = threadIdx.x;
    const int r = blockIdx.x;
    const int layer = lb.layer[blockIdx.y];
    const int k = lb.k, B = s.B, bits = lb.hash_bits, H = 1 << bits;
    const int64_t rl = static_cast<int64_t>(layer) * s.R + r;
    const int32_t* sel = lb.sel[blockIdx.y] + static_cast<int64_t>(r) * k;
    int32_t* out = lb.out[blockIdx.y] + static_cast<int64_t>(r) * k;
    int32_t* spos_g = s.slot_pos + rl * B;
    uint32_t* ts_g = s.ts + rl * B;
    int32_t* pt = s.page_table + rl * s.L_ctx;
    const PlanLds l = carve(lds_raw, H, k);

    // Independent global loads first: step clock and this lane's slot run.
    const uint32_t t = s.clock[rl];
    const int s0 = tid * PER;
    int spos[PER];
    load_run<PER, int>(spos_g, s0, B, spos, kEmpty);

    for (int i = tid; i < H; i += kPlanThreads) l.hkey[i] = kEmpty;
    for (int j = tid; j < k; j += kPlanThreads) l.sidx[j] = -1;
    __syncthreads();

    // Stage 1: hash table over the selected positions.
    int bad_range = 0, bad_dup = 0, bad_at = -1;
    for (int j = tid; j < k; j += kPlanThreads) {
        const int p = sel[j];
        l.sel[j] = p;
        if (p < 0 || static_cast<int64_t>(p) >= s.L_ctx) {
            bad_range = 1;
            bad_at = j;
        } else if (!hash_insert(l, H, bits, p, j)) {
            bad_dup = 1;
            bad_at = j;
        }
    }
    const int any_range = __syncthreads_or(bad_range);
    const int any_dup = __syncthreads_or(bad_dup);
    if (any_range || any_dup) {
        const int code = any_range ? HS_DEV_RANGE : HS_DEV_DUP;
        reject(s, out, k, rl, layer, r, code, bad_at);
        return;
    }

    // Stage 2: probe every cached position against the hash to mark hits.
    unsigned hitbits = 0;
#pragma unroll
    for (int q = 0; q < PER; ++q) {
        if (s0 + q < B && spos[q] >= 0) {
            const int j = hash_find(l, H, bits, spos[q]);
            if (j >= 0) {
                l.sidx[j] = s0 + q;
                hitbits |= 1u << q;
            }
        }
    }
    __syncthreads();

    // Miss list in ascending j: each lane owns a contiguous run of j.
    const int kper = (k + kPlanThreads - 1) / kPlanThreads;
    const int j0 = tid * kper;
    int cnt = 0;
    for (int q = 0; q < kper; ++q) {
        const int j = j0 + q;
        if (j < k && l.sidx[j] < 0) ++cnt;
    }
    int m;
    int base = block_excl_scan(cnt, &m, l.scratch);
    for (int q = 0; q < kper; ++q) {
        const int j = j0 + q;
        if (j < k && l.sidx[j] < 0) l.mlist[base++] = j;
    }
    const int h = k - m;
    const uint32_t ts_miss = 2u * t + 1u, ts_hit = 2u * t + 2u;

    if (m == 0) {
        // Every selection hit: only the hit stamps change.
#pragma unroll
        for (int q = 0; q < PER; ++q)
            if ((hitbits >> q) & 1u) ts_g[s0 + q] = ts_hit;
    } else {
        __syncthreads();  // miss list complete
        uint32_t tsv[PER];
        load_run<PER, uint32_t>(ts_g, s0, B, tsv, 0xFFFFFFFFu);
        const int ncand = B - h;
        // Stage 3: threshold stamp T and the number of slots stamped exactly T
        // that must go (lowest slots first).
        uint32_t T;
        int need_eq;
        if (m == ncand) {
            T = 0xFFFFFFFFu;  // every candidate is a victim (stamps never reach this value)
            need_eq = 0;
        } else {
            unsigned mn = 0xFFFFFFFFu, mx = 0u;
#pragma unroll
            for (int q = 0; q < PER; ++q) {
                if (s0 + q < B && !((hitbits >> q) & 1u)) {
                    mn = min(mn, tsv[q]);
                    mx = max(mx, tsv[q]);
                }
            }
            mn = wave_min(mn);
            mx = wave_max(mx);
            const int lane = tid & 63, wave = tid >> 6;
            if (lane == 0) {
                l.hist[wave] = static_cast<int>(mn);
                l.hist[kPlanWaves + wave] = static_cast<int>(mx);
            }
            __syncthreads();
            mn = 0xFFFFFFFFu;
            mx = 0u;
            for (int w = 0; w < kPlanWaves; ++w) {
                mn = min(mn, static_cast<unsigned>(l.hist[w]));
                mx = max(mx, static_cast<unsigned>(l.hist[kPlanWaves + w]));
            }
            __syncthreads();
            if (mn == mx) {
                T = mn;
                need_eq = m;
            } else {
                const int nbits = 32 - __clz(static_cast<int>(mx - mn));
                uint64_t prefix = 0;
                int remaining = m, pos = nbits;
                while (pos > 0) {
                    const int d = pos < 10 ? pos : 10;
                    pos -= d;
                    l.hist[tid] = 0;
                    __syncthreads();
#pragma unroll
                    for (int q = 0; q < PER; ++q) {
                        if (s0 + q < B && !((hitbits >> q) & 1u)) {
                            const uint64_t rel = static_cast<uint64_t>(tsv[q] - mn);
                            if ((rel >> (pos + d)) == prefix)
                                atomicAdd(&l.hist[static_cast<int>((rel >> pos) & ((1u << d) - 1u))], 1);
                        }
                    }
                    __syncthreads();
                    const int hb = l.hist[tid];
                    int tot;
                    const int below = block_excl_scan(hb, &tot, l.scratch);
                    if (below < remaining && remaining <= below + hb) {
                        l.scratch[kPlanWaves + 1] = tid;
                        l.scratch[kPlanWaves + 2] = below;
                    }
                    __syncthreads();
                    prefix = (prefix << d) | static_cast<uint64_t>(l.scratch[kPlanWaves + 1]);
                    remaining -= l.scratch[kPlanWaves + 2];
                    __syncthreads();
                }
                T = mn + static_cast<uint32_t>(prefix);
                need_eq = remaining;
            }
        }

        // Victim ranks in slot order: one scan counts strictly older
        // candidates (high 16 bits) and tied candidates (low 16 bits).
        int strict = 0, tie = 0;
#pragma unroll
        for (int q = 0; q < PER; ++q) {
            if (s0 + q < B && !((hitbits >> q) & 1u)) {
                if (tsv[q] < T) ++strict;
                else if (tsv[q] == T) ++tie;
            }
        }
        int tot;
        const int ex = block_excl_scan((strict << 16) | tie, &tot, l.scratch);
        int sb = ex >> 16, tb = ex & 0xFFFF;
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
            if (tsv[q] < T) {
                rank = sb + min(tb, need_eq);
                ++sb;
            } else if (tsv[q] == T) {
                if (tb < need_eq) rank = sb + tb;
                ++tb;
            }
            if (rank >= 0 && rank < m) {
                // Stage 4 bookkeeping and metadata update: the rank-th miss (in
                // ascending j) takes this slot; the evicted position goes back to
                // host-only (no write-back: the host copy is authoritative).
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
        if (any_victim) store_run<PER, int>(spos_g, s0, B, spos);
        if (any_victim || hitbits) store_run<PER, uint32_t>(ts_g, s0, B, tsv);
    }
    __syncthreads();

    // Stage 5: publish the slot of every selection.
    for (int j = tid; j < k; j += kPlanThreads) {
        const int v = l.sidx[j];
        out[j] = v >= 0 ? v : -2 - v;
        s.hit_mask[rl * B + j] = v >= 0 ? 1 : 0;
    }
    if (tid == 0) {
        s.miss_count[rl] = m;
        s.status[rl] = 0;
        s.clock[rl] = t + 1u;
        unsigned long long* st = s.stats + 4 * layer;
        atomicAdd(st + 0, static_cast<unsigned long long>(h));
        atomicAdd(st + 1, static_cast<unsigned long long>(m));
        atomicAdd(st + 2, static_cast<unsigned long long>(m) * static_cast<unsigned long long>(s.row_bytes));
        atomicAdd(st + 3, 1ull);
    }
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
    for (int i = tid; i < (B + 31) / 32; i += kPlanThreads) pub_bits[i] = 0u;
    __syncthreads();
    int bad_range = 0, bad_dup = 0, bad_res = 0, bad_at = -1;
    for (int j = tid; j < k; j += kPlanThreads) {
        const int p = sel[j];
        if (p < 0 || static_cast<int64_t>(p) >= s.L_ctx) {
            bad_range = 1;
            bad_at = j;
            continue;
        }
        const int slot = pt[p];
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
    const int any_range = __syncthreads_or(bad_range);
    const int any_dup = __syncthreads_or(bad_dup);
    const int any_res = __syncthreads_or(bad_res);
    if (any_range || any_dup || any_res) {
        const int code = any_range ? HS_DEV_RANGE : (any_dup ? HS_DEV_DUP : HS_DEV_NOT_RESIDENT);
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
    for (int i = tid; i < B; i += kPlanThreads) prev_pos[i] = INT_MIN;
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
    if (__syncthreads_or(diverged)) {
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
        unsigned long long* st = s.stats + 4 * L2;
        atomicAdd(st + 0, static_cast<unsigned long long>(rb.k - m));
        atomicAdd(st + 1, static_cast<unsigned long long>(m));
        atomicAdd(st + 2, static_cast<unsigned long long>(m) * static_cast<unsigned long long>(s.row_bytes));
        atomicAdd(st + 3, 1ull);
    }
}

}  // namespace

size_t plan_lds_bytes(int k, int hash_bits) {
    return sizeof(int) * (2 * (static_cast<size_t>(1) << hash_bits) + 3 * static_cast<size_t>(k) + kHistBins + 32);
}

hipError_t launch_plan(const StateBase& s, const LayerBatch& lb, hipStream_t st) {
    const dim3 grid(s.R, lb.n), block(kPlanThreads);
    const size_t lds = plan_lds_bytes(lb.k, lb.hash_bits);
    const int per = (s.B + kPlanThreads - 1) / kPlanThreads;
#define HS_PLAN_CASE(P)                                                                          \
    case P:                                                                                      \
        if (lds > 65536) {                                                                       \
            hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&plan_kernel<P>),   \
                                               hipFuncAttributeMaxDynamicSharedMemorySize,       \
                                               static_cast<int>(lds));                           \
            if (e != hipSuccess) return e;                                                       \
        }                                                                                        \
        hipLaunchKernelGGL(plan_kernel<P>, grid, block, lds, st, s, lb);                         \
        break;
    switch (per <= 1 ? 1 : per <= 2 ? 2 : per <= 4 ? 4 : per <= 8 ? 8 : 16) {
        HS_PLAN_CASE(1)
        HS_PLAN_CASE(2)
        HS_PLAN_CASE(4)
        HS_PLAN_CASE(8)
        HS_PLAN_CASE(16)
        default:
            return hipErrorInvalidValue;
    }
#undef HS_PLAN_CASE
    return hipGetLastError();
}

hipError_t launch_publish(const StateBase& s, const LayerBatch& lb, hipStream_t st) {
    const size_t lds = sizeof(unsigned) * static_cast<size_t>((s.B + 31) / 32);
    hipLaunchKernelGGL(publish_kernel, dim3(s.R, lb.n), dim3(kPlanThreads), lds, st, s, lb);
    return hipGetLastError();
}

hipError_t launch_replay_meta(const StateBase& s, const ReplayBatch& rb, hipStream_t st) {
    const size_t lds = sizeof(int) * static_cast<size_t>(s.B);
    if (lds > 65536) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&replay_meta_kernel),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(replay_meta_kernel, dim3(s.R, rb.n), dim3(kPlanThreads), lds, st, s, rb);
    return hipGetLastError();
}

}  // namespace hs
