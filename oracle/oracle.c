/*
 * oracle.c -- plain, single-threaded CPU oracle of the HiSparse RESOLVE step.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file; it exists so tests, the smoke check and the CPU baseline
 * of the benchmark can compare the GPU library against an implementation
 * that can be checked against the pages by eye.  It shares no code, header
 * or table with the GPU library.
 *
 * Source: "HiSparse: Scaling Sparse-Attention Decoding with Hierarchical KV
 * Cache Management" as described by
 *   [blog]  "Inference Systems Infrastructure Notes (6): HiSparse", sections
 *           2 ("Two-Level Hierarchy"), 2.1 ("How Slots Are Actually
 *           Allocated"), 3 ("RESOLVE: Five Stages in One Launch");
 *   [pith]  the pith.science review of arXiv 2608.07009, blocks "What carries
 *           the argument" and "Core claim" (the five RESOLVE stages: hash
 *           table over the selected positions, probe of the cache to mark
 *           hits, LRU victims with hits promoted above newly fetched misses,
 *           fetch of misses from pinned host memory, publication of slots).
 *
 * State per (request r, layer l), exactly as the blog's section 2 lists it:
 *   slot_pos[B]      logical position held by each GPU slot, -1 = empty
 *   ts[B]            recency stamp of each slot, 0 = never used
 *   page_table[L]    GPU slot of each logical position, -1 = host only
 *   clock            number of resolves already done on this (r, l)
 *   cache[B][row]    (optional) the bytes each slot holds
 * The cache starts empty: prefill writes only to the host pool, which is the
 * sole authoritative copy (blog section 2, item 1).
 *
 * Readings where the pages leave a step open (each is also listed in the
 * design notes):
 *   - recency: the per-slot recency information that the blog's section 2
 *     (item 3, metadata) keeps for LRU is read as a 32-bit stamp per slot; a
 *     miss fetched at step t is stamped 2t+1 and a hit 2t+2, so a step's hits
 *     rank above the records it fetched and both above anything older (the
 *     per-step refinement of LRU in the pith review's "What carries the
 *     argument").
 *   - ties between equal stamps are broken by the lower slot index; empty
 *     slots (stamp 0) therefore go first, lowest slot first.
 *   - the i-th miss in ascending selection index j receives the i-th victim
 *     in ascending slot order.
 *   - a request whose selection holds an out-of-range or repeated position
 *     is rejected: its slots publish -1 and its state is left unchanged.
 *   - decode-time append (the pages describe only prefill writes): a new
 *     token's record goes to the next position of its history in the host
 *     pool, the authoritative copy, like prefill records (blog section 2,
 *     item 1); positions at or beyond a history's length are out of range;
 *     the record enters the GPU cache only when a later selection names it.
 *   - lowering a history's length drops the cached copies of the positions
 *     it cuts off (their slots become empty), so a record appended again at
 *     such a position is fetched from the pool, never served stale.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    int num_req, num_layers, B;
    int64_t L_ctx, row_bytes;
    int32_t* slot_pos;    /* [l][r][B] */
    uint32_t* ts;         /* [l][r][B] */
    int32_t* page_table;  /* [l][r][L_ctx] */
    uint32_t* clock;      /* [l][r] */
    int64_t* length;      /* [l][r] positions written in each history */
    uint8_t* cache;       /* [l][r][B][row_bytes], or NULL when bytes are not modelled */
} oracle_t;

enum { OR_OK = 0, OR_E_RANGE = 1, OR_E_DUP = 2, OR_E_K = 3, OR_E_FULL = 4 };

void oracle_reset(oracle_t* o) {
    const int64_t nrl = (int64_t)o->num_req * o->num_layers;
    for (int64_t i = 0; i < nrl * o->B; ++i) { o->slot_pos[i] = -1; o->ts[i] = 0; }
    for (int64_t i = 0; i < nrl * o->L_ctx; ++i) o->page_table[i] = -1;
    for (int64_t i = 0; i < nrl; ++i) o->clock[i] = 0;
    if (o->cache) memset(o->cache, 0, (size_t)(nrl * o->B * o->row_bytes));
}

void oracle_destroy(oracle_t* o) {
    if (!o) return;
    free(o->slot_pos); free(o->ts); free(o->page_table); free(o->clock); free(o->length); free(o->cache);
    free(o);
}

oracle_t* oracle_create(int num_req, int num_layers, int B, int64_t L_ctx, int64_t row_bytes, int model_bytes) {
    if (num_req < 1 || num_layers < 1 || B < 1 || L_ctx < 1 || row_bytes < 1) return NULL;
    oracle_t* o = (oracle_t*)calloc(1, sizeof *o);
    if (!o) return NULL;
    const int64_t nrl = (int64_t)num_req * num_layers;
    o->num_req = num_req; o->num_layers = num_layers; o->B = B; o->L_ctx = L_ctx; o->row_bytes = row_bytes;
    o->slot_pos = (int32_t*)malloc(sizeof(int32_t) * (size_t)(nrl * B));
    o->ts = (uint32_t*)malloc(sizeof(uint32_t) * (size_t)(nrl * B));
    o->page_table = (int32_t*)malloc(sizeof(int32_t) * (size_t)(nrl * L_ctx));
    o->clock = (uint32_t*)malloc(sizeof(uint32_t) * (size_t)nrl);
    o->length = (int64_t*)malloc(sizeof(int64_t) * (size_t)nrl);
    o->cache = model_bytes ? (uint8_t*)malloc((size_t)(nrl * B * row_bytes)) : NULL;
    if (!o->slot_pos || !o->ts || !o->page_table || !o->clock || !o->length || (model_bytes && !o->cache)) {
        oracle_destroy(o);
        return NULL;
    }
    for (int64_t i = 0; i < nrl; ++i) o->length[i] = L_ctx;
    oracle_reset(o);
    return o;
}

/* Accessors for tests. */
int32_t* oracle_slot_pos(oracle_t* o) { return o->slot_pos; }
uint32_t* oracle_ts(oracle_t* o) { return o->ts; }
int32_t* oracle_page_table(oracle_t* o) { return o->page_table; }
uint32_t* oracle_clock(oracle_t* o) { return o->clock; }
uint8_t* oracle_cache(oracle_t* o) { return o->cache; }
int64_t* oracle_length(oracle_t* o) { return o->length; }

/* Set the length of the (request, layer) history to n (0 <= n <= L_ctx).
 * A record at a position at or beyond n is no longer part of the history,
 * and a later append may write a different record there; since the host
 * pool is the authoritative copy (blog section 2, item 1), a cached copy of
 * such a position leaves the cache: its slot becomes empty (position -1,
 * stamp 0, as at creation) and the position host-only.  Returns OR_E_RANGE
 * for n outside [0, L_ctx], else OR_OK. */
int oracle_set_length(oracle_t* o, int layer, int req, int64_t n) {
    if (n < 0 || n > o->L_ctx) return OR_E_RANGE;
    const int64_t rl = (int64_t)layer * o->num_req + req;
    int32_t* spos = o->slot_pos + rl * o->B;
    uint32_t* ts = o->ts + rl * o->B;
    int32_t* pt = o->page_table + rl * o->L_ctx;
    for (int s = 0; s < o->B; ++s) {
        if (spos[s] >= 0 && (int64_t)spos[s] >= n) {
            pt[spos[s]] = -1;
            spos[s] = -1;
            ts[s] = 0;
        }
    }
    o->length[rl] = n;
    return OR_OK;
}

/* Decode-time append: rows [num_req][row_bytes] go to position length of
 * each (request, layer) history in `pool`; err[r] = OR_E_FULL for a history
 * that already holds L_ctx positions (nothing written).  Returns the number
 * of full histories. */
int oracle_append(oracle_t* o, int layer, const uint8_t* rows, uint8_t* pool, const int64_t* region_row,
                  int32_t* err) {
    int n_full = 0;
    for (int r = 0; r < o->num_req; ++r) {
        const int64_t rl = (int64_t)layer * o->num_req + r;
        const int64_t pos = o->length[rl];
        if (pos >= o->L_ctx) {
            err[r] = OR_E_FULL;
            ++n_full;
            continue;
        }
        const int64_t base = region_row ? region_row[(int64_t)r * o->num_layers + layer]
                                        : ((int64_t)r * o->num_layers + layer) * o->L_ctx;
        memcpy(pool + (base + pos) * o->row_bytes, rows + (int64_t)r * o->row_bytes, (size_t)o->row_bytes);
        o->length[rl] = pos + 1;
        err[r] = OR_OK;
    }
    return n_full;
}

/* The set of selected positions, kept as (position, j) pairs sorted by
 * position; membership is a binary search.  It plays the part of the hash
 * table the pages build over the selected positions: how the set is stored
 * does not change any result because the positions are distinct. */
typedef struct { int32_t pos, j; } sel_entry;

static int cmp_sel(const void* a, const void* b) {
    const sel_entry* x = (const sel_entry*)a;
    const sel_entry* y = (const sel_entry*)b;
    return (x->pos > y->pos) - (x->pos < y->pos);
}

/* LRU order: older stamp first, lower slot first among equal stamps. */
typedef struct { uint32_t ts; int32_t slot; } lru_key;

static int cmp_lru(const void* a, const void* b) {
    const lru_key* x = (const lru_key*)a;
    const lru_key* y = (const lru_key*)b;
    if (x->ts != y->ts) return x->ts < y->ts ? -1 : 1;
    return (x->slot > y->slot) - (x->slot < y->slot);
}

static int cmp_int(const void* a, const void* b) {
    const int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
    return (x > y) - (x < y);
}

/*
 * RESOLVE of one layer for every request.
 *   sel        [num_req][k] selected logical positions (the indexer output)
 *   pool       host KV pool base; row (r, l, p) is pool row region_row[r*num_layers+l] + p,
 *              or (r*num_layers+l)*L_ctx + p when region_row is NULL
 *   slot_idx   [num_req][k] out: GPU slot of each selection
 *   hit_mask   [num_req][k] out: 1 where the selection was already resident
 *   miss_count [num_req]    out
 *   plan       [num_req][k][4] out: per miss i, {j, victim slot, evicted position or -1, new position}
 *   err        [num_req]    out: 0, or OR_E_* for a rejected request
 * Returns the number of rejected requests.
 */
int oracle_resolve(oracle_t* o, int layer, const int32_t* sel, int k, const uint8_t* pool,
                   const int64_t* region_row, int32_t* slot_idx, uint8_t* hit_mask, int32_t* miss_count,
                   int32_t* plan, int32_t* err) {
    const int B = o->B;
    int n_err = 0;
    sel_entry* set = (sel_entry*)malloc(sizeof(sel_entry) * (size_t)(k > 0 ? k : 1));
    uint8_t* slot_hit = (uint8_t*)malloc((size_t)B);
    int32_t* misses = (int32_t*)malloc(sizeof(int32_t) * (size_t)(k > 0 ? k : 1));
    lru_key* cand = (lru_key*)malloc(sizeof(lru_key) * (size_t)B);
    int32_t* victims = (int32_t*)malloc(sizeof(int32_t) * (size_t)B);
    for (int r = 0; r < o->num_req; ++r) {
        const int32_t* S = sel + (int64_t)r * k;
        int32_t* out_idx = slot_idx + (int64_t)r * k;
        uint8_t* out_hit = hit_mask + (int64_t)r * k;
        int32_t* out_plan = plan + (int64_t)r * k * 4;
        const int64_t rl = (int64_t)layer * o->num_req + r;
        int32_t* spos = o->slot_pos + rl * B;
        uint32_t* ts = o->ts + rl * B;
        int32_t* pt = o->page_table + rl * o->L_ctx;
        const uint32_t t = o->clock[rl];

        /* Validate: B >= k (blog section 2, item 2), every position already
         * written in this history, all positions distinct. */
        int code = OR_OK;
        if (k < 1 || k > B) code = OR_E_K;
        for (int j = 0; code == OR_OK && j < k; ++j)
            if (S[j] < 0 || (int64_t)S[j] >= o->length[rl]) code = OR_E_RANGE;
        /* Stage 1: the set of selected positions. */
        for (int j = 0; code == OR_OK && j < k; ++j) { set[j].pos = S[j]; set[j].j = j; }
        if (code == OR_OK) {
            qsort(set, (size_t)k, sizeof(sel_entry), cmp_sel);
            for (int j = 1; j < k; ++j)
                if (set[j].pos == set[j - 1].pos) { code = OR_E_DUP; break; }
        }
        err[r] = code;
        if (code != OR_OK) {
            for (int j = 0; j < k; ++j) { out_idx[j] = -1; out_hit[j] = 0; }
            miss_count[r] = 0;
            ++n_err;
            continue;
        }

        /* Stage 2: probe every cache slot against the set to mark hits. */
        for (int j = 0; j < k; ++j) { out_idx[j] = -1; out_hit[j] = 0; }
        for (int s = 0; s < B; ++s) {
            slot_hit[s] = 0;
            if (spos[s] < 0) continue;
            sel_entry key = { spos[s], 0 };
            const sel_entry* f = (const sel_entry*)bsearch(&key, set, (size_t)k, sizeof(sel_entry), cmp_sel);
            if (f) { out_idx[f->j] = s; out_hit[f->j] = 1; slot_hit[s] = 1; }
        }

        /* Misses, in ascending selection index. */
        int m = 0;
        for (int j = 0; j < k; ++j)
            if (!out_hit[j]) misses[m++] = j;

        /* Stage 3: LRU victims.  Candidates are the slots not holding a
         * selected position (empty slots included); the m oldest by
         * (stamp, slot) are evicted.  B >= k guarantees enough candidates. */
        int nc = 0;
        for (int s = 0; s < B; ++s)
            if (!slot_hit[s]) { cand[nc].ts = ts[s]; cand[nc].slot = s; ++nc; }
        qsort(cand, (size_t)nc, sizeof(lru_key), cmp_lru);
        for (int i = 0; i < m; ++i) victims[i] = cand[i].slot;
        qsort(victims, (size_t)m, sizeof(int32_t), cmp_int);

        /* Stages 4-5 and metadata: the i-th miss takes the i-th victim; evict
         * (no write-back: the host copy is authoritative), fetch the host row,
         * update the maps and stamps, publish the slot. */
        for (int i = 0; i < m; ++i) {
            const int j = misses[i];
            const int32_t v = victims[i];
            const int32_t old = spos[v];
            if (old >= 0) pt[old] = -1;
            spos[v] = S[j];
            pt[S[j]] = v;
            ts[v] = 2u * t + 1u;
            out_idx[j] = v;
            out_plan[4 * i + 0] = j;
            out_plan[4 * i + 1] = v;
            out_plan[4 * i + 2] = old;
            out_plan[4 * i + 3] = S[j];
            if (o->cache && pool) {
                const int64_t base = region_row ? region_row[(int64_t)r * o->num_layers + layer]
                                                : ((int64_t)r * o->num_layers + layer) * o->L_ctx;
                memcpy(o->cache + (rl * B + v) * o->row_bytes, pool + (base + S[j]) * o->row_bytes,
                       (size_t)o->row_bytes);
            }
        }
        for (int j = 0; j < k; ++j)
            if (out_hit[j]) ts[out_idx[j]] = 2u * t + 2u;
        o->clock[rl] = t + 1u;
        miss_count[r] = m;
    }
    free(set); free(slot_hit); free(misses); free(cand); free(victims);
    return n_err;
}
