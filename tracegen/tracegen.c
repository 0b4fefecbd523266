/*
 * tracegen.c -- seeded synthetic inputs for the hierarchical KV cache RESOLVE step.
 *
 * This module holds no part of the cache method itself: it only draws
 * selection traces (which logical positions a sparse indexer picks at each
 * decode step) and fills a host KV pool with seeded normal bf16 values.
 * Both the CPU oracle and the GPU path consume its output; neither is
 * linked into it.
 *
 * Generators, written from their published definitions:
 *   - splitmix64: Steele, Lea & Flood, "Fast splittable pseudorandom number
 *     generators", OOPSLA 2014 (increment 0x9E3779B97F4A7C15 and the
 *     two xor-shift-multiply finalisation rounds).
 *   - xoshiro256**: Blackman & Vigna, "Scrambled linear pseudorandom number
 *     generators", ACM TOMS 2021 (the ** scrambler on state word 1).
 *   - Box-Muller transform: Box & Muller, Ann. Math. Statist. 1958.
 *
 * Trace recipe (stands in for the one-request GLM-5.1 selection trace of the
 * HiSparse trace study, "Per-step top-k miss rate", Figure 6, which is not
 * available; only its shape is taken: k selected positions per step out of
 * L_ctx, strong step-to-step retention):
 *   step 0     : k distinct uniform positions, array order = draw order.
 *   step t >= 1: each S_{t-1}[j] is kept in place with probability p (one
 *                Bernoulli draw per j, ascending j).  Every dropped j, in
 *                ascending order, is redrawn: a fair coin chooses between a
 *                uniform position and a position within +-W (W = window,
 *                zero excluded) of a uniformly chosen kept position; a
 *                candidate outside [0, L_ctx) or already in this step's set is
 *                rejected and the coin is thrown again.  With no kept
 *                position the draw is uniform.
 *   mode UNIFORM : k fresh distinct uniform positions every step (the
 *                  "uniformly random selection" falsifier of the review).
 *   mode HITONLY : p = 1 after step 0, so every later step repeats step 0.
 *
 * Layout of a trace: int32 [steps][num_layers][num_req][k].  Each
 * (request, stream) pair owns an independent xoshiro256** stream; layers of
 * one sharing group (group > 1) replay the same stream, which models
 * indexer output shared across a group of layers.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <math.h>
#include <pthread.h>

#define TG_GAMMA 0x9E3779B97F4A7C15ull

static inline uint64_t sm64_out(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

/* i-th output (i >= 0) of the splitmix64 sequence started at `seed`. */
static inline uint64_t sm64_at(uint64_t seed, uint64_t i) {
    return sm64_out(seed + (i + 1) * TG_GAMMA);
}

typedef struct { uint64_t s[4]; } xo256;

static inline uint64_t rotl64(uint64_t x, int k) { return (x << k) | (x >> (64 - k)); }

static inline uint64_t xo_next(xo256* g) {
    uint64_t* s = g->s;
    const uint64_t out = rotl64(s[1] * 5, 7) * 9;
    const uint64_t t = s[1] << 17;
    s[2] ^= s[0];
    s[3] ^= s[1];
    s[1] ^= s[2];
    s[0] ^= s[3];
    s[2] ^= t;
    s[3] = rotl64(s[3], 45);
    return out;
}

/* Stream key for (request r, stream index q): the base seed mixed with both
 * indices; the four state words are the first four splitmix64 outputs. */
uint64_t tg_stream_key(uint64_t seed, int64_t r, int64_t q) {
    return seed ^ ((uint64_t)(r + 1) * 0xD1B54A32D192ED03ull) ^ ((uint64_t)(q + 1) * 0xABC98388FB8FAC03ull);
}

static void xo_seed(xo256* g, uint64_t key) {
    for (int i = 0; i < 4; ++i) g->s[i] = sm64_at(key, (uint64_t)i);
}

/* uniform integer in [0, n): high 64 bits of the 128-bit product x*n. */
static inline uint64_t uniform_n(xo256* g, uint64_t n) {
    return (uint64_t)(((unsigned __int128)xo_next(g) * n) >> 64);
}

/* Bernoulli(p): the top 53 bits as a double in [0,1) compared with p. */
static inline int bernoulli(xo256* g, double p) {
    return (double)(xo_next(g) >> 11) * 0x1.0p-53 < p;
}

enum { TG_LOCALITY = 0, TG_UNIFORM = 1, TG_HITONLY = 2 };

typedef struct {
    int32_t* out;
    int steps, num_req, num_layers, group, k, mode, window;
    int64_t L;
    double p;
    uint64_t seed;
    int64_t n_streams, next;
    pthread_mutex_t mu;
    int err;
} trace_job;

static inline int bit_get(const uint64_t* bm, int64_t x) { return (int)((bm[x >> 6] >> (x & 63)) & 1u); }
static inline void bit_set(uint64_t* bm, int64_t x) { bm[x >> 6] |= 1ull << (x & 63); }
static inline void bit_clr(uint64_t* bm, int64_t x) { bm[x >> 6] &= ~(1ull << (x & 63)); }

/* One (request, stream) sequence over all steps, written to every layer of
 * its group. */
static void gen_stream(trace_job* J, int64_t sid, uint64_t* bm, int32_t* cur, int32_t* kept, uint8_t* keep) {
    const int ng = (J->num_layers + J->group - 1) / J->group;
    const int r = (int)(sid / ng), q = (int)(sid % ng);
    const int k = J->k;
    const int64_t L = J->L;
    xo256 g;
    xo_seed(&g, tg_stream_key(J->seed, r, q));
    for (int t = 0; t < J->steps; ++t) {
        if (t == 0 || J->mode == TG_UNIFORM) {
            if (t > 0)
                for (int j = 0; j < k; ++j) bit_clr(bm, cur[j]);
            for (int j = 0; j < k; ++j) {
                int64_t x;
                do { x = (int64_t)uniform_n(&g, (uint64_t)L); } while (bit_get(bm, x));
                bit_set(bm, x);
                cur[j] = (int32_t)x;
            }
        } else if (J->mode == TG_LOCALITY) {
            int nk = 0;
            for (int j = 0; j < k; ++j) keep[j] = (uint8_t)bernoulli(&g, J->p);
            for (int j = 0; j < k; ++j) {
                if (keep[j]) kept[nk++] = cur[j];
                else bit_clr(bm, cur[j]);
            }
            for (int j = 0; j < k; ++j) {
                if (keep[j]) continue;
                int64_t x;
                for (;;) {
                    const int heads = bernoulli(&g, 0.5);
                    if (heads || nk == 0) {
                        x = (int64_t)uniform_n(&g, (uint64_t)L);
                    } else {
                        const int64_t c = kept[uniform_n(&g, (uint64_t)nk)];
                        int64_t d = (int64_t)uniform_n(&g, (uint64_t)(2 * J->window));
                        d = d < J->window ? d - J->window : d - J->window + 1;
                        x = c + d;
                    }
                    if (x >= 0 && x < L && !bit_get(bm, x)) break;
                }
                bit_set(bm, x);
                cur[j] = (int32_t)x;
            }
        } /* TG_HITONLY: steps >= 1 repeat step 0 */
        for (int l = q * J->group; l < (q + 1) * J->group && l < J->num_layers; ++l) {
            int32_t* dst = J->out + (((int64_t)t * J->num_layers + l) * J->num_req + r) * (int64_t)k;
            memcpy(dst, cur, sizeof(int32_t) * (size_t)k);
        }
    }
}

static void* trace_worker(void* arg) {
    trace_job* J = (trace_job*)arg;
    uint64_t* bm = (uint64_t*)calloc((size_t)((J->L + 63) / 64), sizeof(uint64_t));
    int32_t* cur = (int32_t*)malloc(sizeof(int32_t) * (size_t)J->k);
    int32_t* kept = (int32_t*)malloc(sizeof(int32_t) * (size_t)J->k);
    uint8_t* keep = (uint8_t*)malloc((size_t)J->k);
    if (!bm || !cur || !kept || !keep) {
        pthread_mutex_lock(&J->mu); J->err = 1; pthread_mutex_unlock(&J->mu);
    } else {
        for (;;) {
            pthread_mutex_lock(&J->mu);
            const int64_t sid = J->next++;
            pthread_mutex_unlock(&J->mu);
            if (sid >= J->n_streams) break;
            memset(bm, 0, sizeof(uint64_t) * (size_t)((J->L + 63) / 64));
            gen_stream(J, sid, bm, cur, kept, keep);
        }
    }
    free(bm); free(cur); free(kept); free(keep);
    return NULL;
}

/* Fill out[steps][num_layers][num_req][k].  Returns 0, or -1 on bad
 * arguments / allocation failure. */
int tg_trace(int32_t* out, int steps, int num_req, int num_layers, int group, int k, int64_t L_ctx,
             double p_keep, int mode, int window, uint64_t seed, int nthreads) {
    if (!out || steps < 0 || num_req < 1 || num_layers < 1 || group < 1 || k < 1 || L_ctx < k ||
        L_ctx > (int64_t)INT32_MAX || window < 1 || mode < 0 || mode > 2 || !(p_keep >= 0.0 && p_keep <= 1.0))
        return -1;
    trace_job J;
    memset(&J, 0, sizeof J);
    J.out = out; J.steps = steps; J.num_req = num_req; J.num_layers = num_layers; J.group = group;
    J.k = k; J.L = L_ctx; J.p = p_keep; J.mode = mode; J.window = window; J.seed = seed;
    J.n_streams = (int64_t)num_req * ((num_layers + group - 1) / group);
    pthread_mutex_init(&J.mu, NULL);
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 64) nthreads = 64;
    if (nthreads > J.n_streams) nthreads = (int)J.n_streams;
    pthread_t th[64];
    int created[64] = {0};
    for (int i = 1; i < nthreads; ++i)
        created[i] = pthread_create(&th[i], NULL, trace_worker, &J) == 0;
    trace_worker(&J);
    for (int i = 1; i < nthreads; ++i)
        if (created[i]) pthread_join(th[i], NULL);
    pthread_mutex_destroy(&J.mu);
    return J.err ? -1 : 0;
}

/* ---- KV pool: seeded N(0,1) values rounded to bf16 ---------------------- */

/* fp32 -> bf16, round to nearest even (NaN cannot occur here). */
static inline uint16_t f32_to_bf16_rne(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

/* Element e of the pool: Box-Muller pair q = e/2 uses the splitmix64
 * outputs 2q and 2q+1 of the pool seed as u1 in (0,1] and u2 in [0,1);
 * even e takes the cosine branch, odd e the sine branch. */
static inline void pool_pair(uint64_t seed, uint64_t q, uint16_t* z0, uint16_t* z1) {
    const double u1 = (double)((sm64_at(seed, 2 * q) >> 11) + 1) * 0x1.0p-53;
    const double u2 = (double)(sm64_at(seed, 2 * q + 1) >> 11) * 0x1.0p-53;
    const double rr = sqrt(-2.0 * log(u1));
    const double a = 6.283185307179586476925286766559 * u2;
    *z0 = f32_to_bf16_rne((float)(rr * cos(a)));
    *z1 = f32_to_bf16_rne((float)(rr * sin(a)));
}

typedef struct { uint16_t* dst; uint64_t e0, n, seed; } pool_job;

static void* pool_worker(void* arg) {
    pool_job* P = (pool_job*)arg;
    uint64_t e = P->e0, end = P->e0 + P->n;
    uint16_t* d = P->dst;
    uint16_t a, b;
    if (e < end && (e & 1)) { pool_pair(P->seed, e >> 1, &a, &b); *d++ = b; ++e; }
    for (; e + 1 < end; e += 2) { pool_pair(P->seed, e >> 1, &a, &b); d[0] = a; d[1] = b; d += 2; }
    if (e < end) { pool_pair(P->seed, e >> 1, &a, &b); *d = a; }
    return NULL;
}

/* dst[i] = bf16 pool element (first_elem + i) for i < n_elems. */
void tg_pool_fill(uint16_t* dst, uint64_t first_elem, uint64_t n_elems, uint64_t seed, int nthreads) {
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 64) nthreads = 64;
    if (n_elems < (uint64_t)nthreads * 65536) nthreads = 1;
    pool_job jobs[64];
    pthread_t th[64];
    int created[64] = {0};
    const uint64_t per = ((n_elems / (uint64_t)nthreads) + 1) & ~1ull;
    for (int i = 0; i < nthreads; ++i) {
        const uint64_t a = (uint64_t)i * per;
        const uint64_t b = (i == nthreads - 1) ? n_elems : ((uint64_t)(i + 1) * per < n_elems ? (uint64_t)(i + 1) * per : n_elems);
        jobs[i].dst = dst + (a < n_elems ? a : n_elems);
        jobs[i].e0 = first_elem + (a < n_elems ? a : n_elems);
        jobs[i].n = b > a ? b - a : 0;
        jobs[i].seed = seed;
    }
    for (int i = 1; i < nthreads; ++i)
        created[i] = pthread_create(&th[i], NULL, pool_worker, &jobs[i]) == 0;
    pool_worker(&jobs[0]);
    for (int i = 1; i < nthreads; ++i) {
        if (created[i]) pthread_join(th[i], NULL);
        else pool_worker(&jobs[i]);
    }
}

/* Raw generator outputs, exposed so tests can pin them against the
 * published reference values of each generator. */
uint64_t tg_splitmix64_at(uint64_t seed, uint64_t i) { return sm64_at(seed, i); }
void tg_xoshiro_outputs(const uint64_t state[4], uint64_t* out, int n) {
    xo256 g;
    memcpy(g.s, state, sizeof g.s);
    for (int i = 0; i < n; ++i) out[i] = xo_next(&g);
}
