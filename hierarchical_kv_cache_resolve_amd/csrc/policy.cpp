// policy.cpp -- CPU replay of selection traces under cache replacement
// policies (the cache-policy trace study: pith.science review of HiSparse,
// Figure 6 caption and "What carries the argument"; Belady's offline-optimal
// policy as the bound, the review's supporting citation [3]).  The policies and
// the batch semantics are stated in include/hspolicy.h.
#include "hspolicy.h"

#include <algorithm>
#include <atomic>
#include <cstdint>
#include <limits>
#include <new>
#include <thread>
#include <vector>

namespace {

constexpr int64_t kNever = std::numeric_limits<int64_t>::max() / 4;   // next use of a record never selected again

struct History {
    int policy, B, k, steps;
    int64_t L_ctx;
    const int32_t* sel;     // step t, entry j at sel[t * stride + j]
    int64_t stride;
};

// next_use[t*k + j]: the first step after t that selects sel[t][j] again, or kNever
int validate_and_next_use(const History& h, std::vector<int64_t>* next_use) {
    std::vector<int64_t> last(static_cast<size_t>(h.L_ctx), kNever);
    std::vector<int32_t> seen(static_cast<size_t>(h.L_ctx), -1);
    if (next_use) next_use->assign(static_cast<size_t>(h.steps) * h.k, kNever);
    for (int t = 0; t < h.steps; ++t) {
        const int32_t* s = h.sel + t * h.stride;
        for (int j = 0; j < h.k; ++j) {
            if (s[j] < 0 || s[j] >= h.L_ctx) return HS_POLICY_E_RANGE;
            if (seen[s[j]] == t) return HS_POLICY_E_DUP;
            seen[s[j]] = t;
        }
    }
    if (next_use) {
        for (int t = h.steps - 1; t >= 0; --t) {
            const int32_t* s = h.sel + t * h.stride;
            for (int j = 0; j < h.k; ++j) {
                (*next_use)[static_cast<size_t>(t) * h.k + j] = last[s[j]];
                last[s[j]] = t;
            }
        }
    }
    return HS_POLICY_OK;
}

// Replay one validated history; misses[t] (if non-null) gets the misses of step t.
int64_t replay(const History& h, const std::vector<int64_t>& next_use, int32_t* misses) {
    const int B = h.B, k = h.k;
    std::vector<int32_t> where(static_cast<size_t>(h.L_ctx), -1);   // position -> slot
    std::vector<int32_t> pos(B, -1);                                // slot -> position, -1 empty
    std::vector<int64_t> key(B, 0);                                 // stamp, or next use for Belady
    std::vector<int32_t> used_at(B, -1);                            // last step that selected the slot
    std::vector<int32_t> miss_j;
    std::vector<int32_t> cand;
    miss_j.reserve(k);
    cand.reserve(B);
    const bool belady = h.policy == HS_POLICY_BELADY;
    // eviction order: true if slot a goes before slot b
    auto before = [&](int32_t a, int32_t b) {
        const bool ea = pos[a] < 0, eb = pos[b] < 0;
        if (ea != eb) return ea;                     // empty slots first
        if (!ea && key[a] != key[b]) return belady ? key[a] > key[b] : key[a] < key[b];
        return a < b;
    };
    int64_t total = 0;
    for (int t = 0; t < h.steps; ++t) {
        const int32_t* s = h.sel + t * h.stride;
        miss_j.clear();
        for (int j = 0; j < k; ++j) {
            const int32_t slot = where[s[j]];
            if (slot < 0) {
                miss_j.push_back(j);
                continue;
            }
            used_at[slot] = t;
            switch (h.policy) {
                case HS_POLICY_LRU_PROMOTE: key[slot] = 2 * static_cast<int64_t>(t) + 2; break;
                case HS_POLICY_LRU: key[slot] = t + 1; break;
                case HS_POLICY_FIFO: break;
                default: key[slot] = next_use[static_cast<size_t>(t) * k + j]; break;
            }
        }
        const int m = static_cast<int>(miss_j.size());
        if (misses) misses[t] = m;
        total += m;
        if (m == 0) continue;
        cand.clear();
        for (int32_t v = 0; v < B; ++v)
            if (used_at[v] != t) cand.push_back(v);
        // B >= k guarantees at least m candidates: at most k - m slots were hit
        std::nth_element(cand.begin(), cand.begin() + (m - 1), cand.end(), before);
        std::sort(cand.begin(), cand.begin() + m);   // victims in ascending slot order
        for (int i = 0; i < m; ++i) {
            const int32_t v = cand[i];
            const int j = miss_j[i];
            if (pos[v] >= 0) where[pos[v]] = -1;
            pos[v] = s[j];
            where[s[j]] = v;
            used_at[v] = t;
            switch (h.policy) {
                case HS_POLICY_LRU_PROMOTE: key[v] = 2 * static_cast<int64_t>(t) + 1; break;
                case HS_POLICY_LRU:
                case HS_POLICY_FIFO: key[v] = t + 1; break;
                default: key[v] = next_use[static_cast<size_t>(t) * k + j]; break;
            }
        }
    }
    return total;
}

int check_args(int policy, int B, int k, int steps, int64_t L_ctx) {
    if (policy < 0 || policy >= HS_POLICY_COUNT || k < 1 || B < k || steps < 0 || L_ctx < k) return HS_POLICY_E_INVAL;
    return HS_POLICY_OK;
}

int replay_many(int policy, int B, int k, int steps, int64_t L_ctx, int n_hist, const int32_t* sel, int64_t* misses,
                int threads);

}  // namespace

extern "C" int hs_policy_replay(int policy, int B, int k, int steps, int64_t L_ctx, const int32_t* sel,
                                int32_t* misses) {
    int rc = check_args(policy, B, k, steps, L_ctx);
    if (rc) return rc;
    if (steps > 0 && (!sel || !misses)) return HS_POLICY_E_INVAL;
    try {
        const History h{policy, B, k, steps, L_ctx, sel, k};
        std::vector<int64_t> next_use;
        rc = validate_and_next_use(h, policy == HS_POLICY_BELADY ? &next_use : nullptr);
        if (rc) return rc;
        replay(h, next_use, misses);
    } catch (const std::bad_alloc&) {
        return HS_POLICY_E_NOMEM;
    }
    return HS_POLICY_OK;
}

extern "C" int hs_policy_replay_many(int policy, int B, int k, int steps, int64_t L_ctx, int n_hist,
                                     const int32_t* sel, int64_t* misses, int threads) {
    int rc = check_args(policy, B, k, steps, L_ctx);
    if (rc) return rc;
    if (n_hist < 0 || (n_hist > 0 && (!misses || (steps > 0 && !sel)))) return HS_POLICY_E_INVAL;
    if (threads < 1) threads = 1;
    threads = std::min(threads, std::max(n_hist, 1));
    try {
        return replay_many(policy, B, k, steps, L_ctx, n_hist, sel, misses, threads);
    } catch (const std::bad_alloc&) {
        return HS_POLICY_E_NOMEM;
    }
}

namespace {

int replay_many(int policy, int B, int k, int steps, int64_t L_ctx, int n_hist, const int32_t* sel, int64_t* misses,
                int threads) {
    std::vector<int> status(n_hist, HS_POLICY_OK);
    std::vector<int64_t> out(n_hist, 0);
    std::atomic<int> next{0};
    auto work = [&]() {
        for (int i = next.fetch_add(1); i < n_hist; i = next.fetch_add(1)) {
            try {
                const History h{policy, B, k, steps, L_ctx, sel + static_cast<int64_t>(i) * k,
                                static_cast<int64_t>(n_hist) * k};
                std::vector<int64_t> next_use;
                status[i] = validate_and_next_use(h, policy == HS_POLICY_BELADY ? &next_use : nullptr);
                if (status[i] == HS_POLICY_OK) out[i] = replay(h, next_use, nullptr);
            } catch (const std::bad_alloc&) {
                status[i] = HS_POLICY_E_NOMEM;
            }
        }
    };
    std::vector<std::thread> pool;
    for (int w = 1; w < threads; ++w) {
        try {
            pool.emplace_back(work);
        } catch (const std::exception&) {
            break;                                   // fewer helpers; the work still completes
        }
    }
    work();
    for (auto& th : pool) th.join();
    for (int i = 0; i < n_hist; ++i)
        if (status[i]) return status[i];
    std::copy(out.begin(), out.end(), misses);
    return HS_POLICY_OK;
}

}  // namespace
