/*
 * hspolicy.h -- C ABI of libhspolicy.so, the CPU replay of selection traces
 * under cache replacement policies (the cache-policy trace study).
 *
 * The study replays one sparse-selection trace under several cache
 * configurations and reports the per-step miss rate (pith.science review of
 * "HiSparse: Scaling Sparse-Attention Decoding with Hierarchical KV Cache
 * Management", Figure 6 caption: top-k-only staging at B = k against LRU
 * caches of B record slots per request and layer; "What carries the
 * argument": 13.4 % misses at B = 2k against 30 % for top-k-only).  Belady's
 * offline-optimal replacement is the upper bound of the comparison (the
 * review's record, supporting citation [3]).
 *
 * One history = one (request, layer) pair: a sequence of `steps` selections
 * of k distinct positions in [0, L_ctx).  A step is a batch: all k selected
 * records must be resident after it, so a victim is never a record selected
 * in the same step.  Empty slots are used first, lowest first.
 *
 * Policies (each a total order on the non-selected resident records; the
 * first m in that order are evicted for m misses):
 *   HS_POLICY_LRU_PROMOTE  the RESOLVE contract: a record fetched at step t is
 *                          stamped 2t+1, a hit 2t+2; evict smallest
 *                          (stamp, slot) first -- hits rank above the
 *                          step's newly fetched misses.
 *   HS_POLICY_LRU          plain LRU at step granularity: hits and misses of
 *                          step t both stamped t+1; smallest (stamp, slot).
 *   HS_POLICY_FIFO         no refresh on a hit: stamp t+1 at fetch only.
 *   HS_POLICY_BELADY       evict the record whose next selection is farthest
 *                          in the future (never again first), ties to the
 *                          lower slot; needs the whole trace (offline).
 * At B = k every policy reduces to top-k-only staging: misses at step t are
 * |S_t \ S_{t-1}|.
 *
 * All functions are plain CPU code; pointers are host pointers owned by the
 * caller.  Return value: 0, or a negative HS_POLICY_E_* code (nothing is
 * written to the outputs on an error).
 */
#ifndef HSPOLICY_H
#define HSPOLICY_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    HS_POLICY_LRU_PROMOTE = 0,
    HS_POLICY_LRU = 1,
    HS_POLICY_FIFO = 2,
    HS_POLICY_BELADY = 3,
    HS_POLICY_COUNT = 4
};

enum {
    HS_POLICY_OK = 0,
    HS_POLICY_E_INVAL = -1,   /* unknown policy, k < 1, B < k, steps < 0, L_ctx < k, NULL pointer */
    HS_POLICY_E_RANGE = -2,   /* a position outside [0, L_ctx) */
    HS_POLICY_E_DUP = -3,     /* a position repeated inside one step */
    HS_POLICY_E_NOMEM = -4
};

/* Replay one history.
 *   sel     int32 [steps][k]   selected positions, distinct within a step
 *   misses  int32 [steps]      out: records fetched at each step */
int hs_policy_replay(int policy, int B, int k, int steps, int64_t L_ctx, const int32_t* sel, int32_t* misses);

/* Replay n_hist independent histories laid out as [steps][n_hist][k] (the
 * layout of a [steps][layers][requests][k] trace flattened over layers and
 * requests), on up to `threads` host threads.
 *   misses  int64 [n_hist]     out: total misses of each history over all steps */
int hs_policy_replay_many(int policy, int B, int k, int steps, int64_t L_ctx, int n_hist, const int32_t* sel,
                          int64_t* misses, int threads);

#ifdef __cplusplus
}
#endif

#endif
