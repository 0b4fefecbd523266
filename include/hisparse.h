/*
 * hisparse.h -- C ABI of the MI355X (gfx950) RESOLVE library, libhisparse.so.
 *
 * The operation is the per-layer RESOLVE step of HiSparse ("HiSparse: Scaling
 * Sparse-Attention Decoding with Hierarchical KV Cache Management", arXiv
 * 2608.07009), as described by the blog "Inference Systems Infrastructure
 * Notes (6): HiSparse" (sections 2, 2.1, 3, 4) and by the pith.science review
 * of the paper ("What carries the argument", "Core claim"):
 *
 *   The full KV history of every request lives in a pinned host pool, the only
 *   authoritative copy.  Each (request, layer) pair owns a fixed GPU cache of
 *   B >= k record slots.  For each decode step and layer, RESOLVE takes the k
 *   logical positions chosen by the sparse indexer, builds a hash table over
 *   them, probes the cached positions to mark hits, chooses LRU victims for the
 *   misses (hits ranked above newly fetched misses), loads the missed records
 *   straight from host memory with wide GPU loads, and publishes the physical
 *   slot of every selected position.  Only placement changes; the records the
 *   consumer reads are byte-identical to the host rows.
 *
 * Conventions
 *   - Pointers named d_* are device pointers; all others are host pointers.
 *   - `stream` arguments are hipStream_t values passed as void*; NULL is the
 *     null stream.  Entry points marked "async" only enqueue work on the given
 *     stream: they never allocate, never synchronise and never read device
 *     memory on the host, so they may be captured into a HIP graph.
 *   - Every entry point returns HS_OK (0) or a negative HS_E_* code.  Argument
 *     and setup errors are reported synchronously and leave all state as it
 *     was.  Errors found in the data on the device (a position outside
 *     [0, length) of its history, a repeated position, a shared layer whose selection is not
 *     what its anchor installed) set a sticky device error word that
 *     hisparse_get_error() reads; the offending request publishes -1 in every
 *     slot_idx entry and its cache state is left unchanged.
 *   - A handle is not thread-safe.  Calls for one layer must be issued in
 *     decode-step order on one stream (or be ordered by the caller's events).
 *   - Graph capture: resolve and prefetch may be captured (the prefetch side
 *     stream must join the capture, e.g. by waiting on the capturing stream).
 *     Contract: a capture must begin after the library's earlier (eager) work
 *     has finished, e.g. after a device synchronise (torch.cuda.graph does one
 *     on entry).  Inside a capture the library cannot wait on, or query, its
 *     own events recorded before the capture began, so it drops those waits;
 *     a capture begun while an eager prefetch replay still runs would not be
 *     ordered after it.
 *
 * Layouts (all row-major, C order)
 *   host pool      rows of W_KV*s bytes; the history of (request r, layer l)
 *                  occupies L_ctx consecutive rows starting at
 *                  region_row[r*num_layers + l] (or (r*num_layers + l)*L_ctx
 *                  when region_row is NULL), i.e. a dense [req][layer][L_ctx][row].
 *   GPU cache      [layer][req][B][W_KV*s] bytes, library-owned; the identity
 *                  num_req*num_layers*B*W_KV*s of the blog's section 2 holds
 *                  exactly (hisparse_hbm_bytes).
 *   d_sel          int32 [num_req][k]; d_slot_idx int32 [num_req][k], each entry
 *                  a local slot in [0, B) of that (request, layer).
 */
#ifndef HISPARSE_H
#define HISPARSE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct hisparse_ctx* hisparse_t;

/* ---- return codes -------------------------------------------------------- */
#define HS_OK 0
#define HS_E_INVAL (-1)   /* bad argument (null pointer, negative size, ...) */
#define HS_E_HANDLE (-2)  /* null or destroyed handle */
#define HS_E_LAYER (-3)   /* layer index out of range */
#define HS_E_K (-4)       /* k < 1, k > B (B >= k, blog section 2) or k > HS_MAX_K */
#define HS_E_ALIGN (-5)   /* record bytes W_KV*s not a positive multiple of 16 */
#define HS_E_POOL (-6)    /* pool not device-accessible host memory, or a region outside it */
#define HS_E_NOMEM (-7)   /* device allocation failed */
#define HS_E_HIP (-8)     /* a HIP runtime call failed */
#define HS_E_DEVICE (-9)  /* the sticky device error word is set */
#define HS_E_ORDER (-10)  /* prefetch / shared-layer resolve issued out of order */
#define HS_E_SCRATCH (-11) /* the call needs more scratch than the fixed no-allocation area holds */

/* ---- device error codes (sticky word) -------------------------------------- */
#define HS_DEV_RANGE 1        /* a position outside [0, length) of its history (length <= L_ctx) */
#define HS_DEV_DUP 2          /* a position repeated within one request's selection */
#define HS_DEV_NOT_RESIDENT 3 /* shared layer: a selected position is not where the anchor's plan put it */
#define HS_DEV_DIVERGED 4     /* shared layer: its cache state no longer mirrors its anchor's, or its
                                 selection is not the anchor's (positions or order) */
#define HS_DEV_FULL 5         /* append: the history already holds L_ctx positions */

/* ---- limits --------------------------------------------------------------- */
#define HS_MAX_B 16384        /* slots per (request, layer) */
#define HS_MAX_K 4096         /* selections per (request, layer, step) */
#define HS_MAX_REQ 1024       /* requests per handle */
#define HS_MAX_HEADS 1024     /* query heads per hisparse_attend_mla call */

typedef enum { HS_BF16 = 0, HS_FP16 = 1, HS_FP8 = 2, HS_FP32 = 3 } hs_dtype; /* sets s only */

/* Host KV pool descriptor.  Caller-owned: `base` must be pinned host memory
 * that the device can read (e.g. from hisparse_host_alloc or hipHostMalloc);
 * it must outlive the handle and must not change while resolves that read it
 * are in flight (eviction never writes back: the host copy is authoritative,
 * blog section 2, item 1). */
typedef struct {
    const void* base;          /* first byte of row 0 */
    int64_t pool_rows;         /* number of rows of W_KV*s bytes at base */
    int64_t L_ctx;             /* logical positions per (request, layer) history */
    const int64_t* region_row; /* [num_req*num_layers] first row of each history, or NULL (dense) */
} hs_host_pool;

/* Create a handle: num_req x num_layers caches of B slots of W_KV elements of
 * `dtype`.  Allocates the cache (exactly num_req*num_layers*B*W_KV*s bytes),
 * slot map, stamps, page tables, clocks and plan buffers on the current
 * device, all empty.  Errors: HS_E_INVAL, HS_E_K (B < 1 or B > HS_MAX_B),
 * HS_E_ALIGN, HS_E_POOL, HS_E_NOMEM, HS_E_HIP.  (blog sections 2 and 2.1) */
int hisparse_create(int num_req, int num_layers, int B, int W_KV, int dtype, const hs_host_pool* host_pool,
                    hisparse_t* out);

/* RESOLVE one layer for all requests (async).  d_sel [num_req][k] holds the
 * positions S_t chosen for this layer; d_slot_idx [num_req][k] receives the
 * slot of each one after its record is resident.  Runs the five stages of the
 * pith review's "Core claim": hash build, cache probe, LRU victim choice,
 * host fetch of misses, publication (also writes the page table).
 * If `layer` was named as a shared layer in the last hisparse_prefetch call,
 * its plan has already been replayed and this call only verifies and
 * publishes.  Errors: HS_E_HANDLE, HS_E_LAYER, HS_E_K, HS_E_INVAL, HS_E_HIP. */
int hisparse_resolve(hisparse_t h, int layer, const int32_t* d_sel, int k, int32_t* d_slot_idx, void* stream);

/* RESOLVE several independent layers in one pair of launches (async).
 * d_sel_ptrs and d_slot_idx_ptrs are host arrays of n device pointers.  When
 * num_req * n exceeds 256 the metadata kernel copies each request-layer's
 * misses itself and no fetch launch follows (HS_OPT_FETCH_BLOCKS and
 * HS_OPT_FETCH_UNROLL then do not apply). */
int hisparse_resolve_layers(hisparse_t h, int n, const int* layers, const int32_t* const* d_sel_ptrs, int k,
                            int32_t* const* d_slot_idx_ptrs, void* stream);

/* Exact layer-wise prefetch (blog section 4, "Exact Layer-Wise Prefetching";
 * pith "Core claim"): must follow hisparse_resolve(anchor_layer) of the same
 * step.  The side stream waits for the anchor's plan, then a copy-only kernel
 * replays that plan into each shared layer (the same slots, records read from
 * the shared layer's own host rows) and mirrors the anchor's cache state into
 * it.  The next hisparse_resolve of each shared layer waits for the replay and
 * only publishes; its selection must equal the anchor's element by element
 * (same positions, same order), which that resolve checks against the
 * anchor's d_sel buffer -- so the anchor's selection buffer must stay
 * unchanged until the shared layers' resolves have run.  A shared layer whose
 * selection differs publishes -1 and sets HS_DEV_DIVERGED.  Async on both
 * streams.  Errors: HS_E_HANDLE, HS_E_LAYER, HS_E_INVAL, HS_E_ORDER, HS_E_HIP. */
int hisparse_prefetch(hisparse_t h, int anchor_layer, const int* shared_layers, int n_shared, void* side_stream);

/* Decode-time append (async).  d_rows [num_req][W_KV*s] holds the record of
 * each request's new token for `layer`; it is written to the next position
 * of that (request, layer) history in the host pool, the authoritative copy
 * (blog section 2, item 1: records go straight to pinned host memory), and
 * the history grows by one.  The record enters the GPU cache only when a
 * later selection names it.  A history already holding L_ctx positions is
 * left unchanged and sets HS_DEV_FULL.  Errors: HS_E_HANDLE, HS_E_LAYER,
 * HS_E_INVAL, HS_E_HIP. */
int hisparse_append(hisparse_t h, int layer, const void* d_rows, void* stream);

/* Set the number of positions already written in every history (e.g. the
 * prefill lengths): lengths [num_req*num_layers], index r*num_layers + l,
 * each in [0, L_ctx].  Selections must name positions below the length.
 * At create every history has length L_ctx.  A cached position at or past
 * its history's new length leaves the cache (its slot becomes empty, stamp 0,
 * the position host-only): a record appended there later is fetched from the
 * pool, the authoritative copy (blog section 2, item 1), never served from
 * the old copy.  Synchronises the device. */
int hisparse_set_lengths(hisparse_t h, const int64_t* lengths);
/* Read the history lengths into lengths [num_req*num_layers] (synchronises). */
int hisparse_get_lengths(hisparse_t h, int64_t* lengths);

/* Free everything the handle owns (synchronises the device first). */
int hisparse_destroy(hisparse_t h);

/* ---- support -------------------------------------------------------------- */

/* Footprint identity of blog section 2: num_req*num_layers*B*W_KV*s bytes.
 * Pure function; no GPU needed.  Returns 0 for invalid arguments. */
size_t hisparse_kv_bytes(int num_req, int num_layers, int B, int W_KV, int dtype);
/* Bytes of KV cache the handle holds on the device (equals hisparse_kv_bytes). */
size_t hisparse_hbm_bytes(hisparse_t h);
/* Bytes of metadata (slot map, stamps, page tables, clocks, plans) on the device. */
size_t hisparse_meta_bytes(hisparse_t h);

/* Device pointers to one layer's state, for inspection and verification. */
typedef struct {
    void* d_cache;          /* uint8 [num_req][B][row_bytes] */
    int32_t* d_slot_pos;    /* [num_req][B], -1 = empty */
    uint32_t* d_ts;         /* [num_req][B], 0 = never used */
    int32_t* d_page_table;  /* [num_req][L_ctx], -1 = host only */
    uint32_t* d_clock;      /* [num_req] resolves done */
    int32_t* d_plan;        /* [num_req][B][4] of the last resolve: {j, slot, evicted pos or -1, new pos} */
    int32_t* d_miss_count;  /* [num_req] of the last resolve */
    uint8_t* d_hit_mask;    /* [num_req][B], first k entries valid after the last resolve */
    int64_t row_bytes;
    int B, num_req;
    int64_t L_ctx;
} hs_layer_state;
int hisparse_layer_state(hisparse_t h, int layer, hs_layer_state* out);

/* Read the sticky device error word (synchronises the device).  code 0 = none. */
int hisparse_get_error(hisparse_t h, int* code, int* layer, int* req);
/* Clear the sticky device error word (synchronises the device). */
int hisparse_clear_error(hisparse_t h);

typedef struct {
    uint64_t hits, misses, miss_bytes, resolves;  /* resolves = (request, layer) resolutions */
} hs_stats;
/* Counters accumulated on the device since create/reset; layer = -1 sums all
 * layers.  Synchronises the device. */
int hisparse_stats(hisparse_t h, int layer, hs_stats* out);

/* Drop every cached record (all slots empty, page tables host-only, clocks 0,
 * counters 0).  The next step is all-miss and still exact because the host
 * pool is authoritative.  Synchronises the device. */
int hisparse_reset(hisparse_t h);

/* Tuning knobs. */
#define HS_OPT_FETCH_BLOCKS 1   /* workgroups of the fetch kernel (default 1024) */
#define HS_OPT_FETCH_UNROLL 2   /* 16-byte loads in flight per lane: 1, 2, 4 or 8 (default 4) */
#define HS_OPT_TIMING 3         /* 1: time every plan/fetch launch with HIP events */
#define HS_OPT_NT_LOADS 4       /* 1: non-temporal host loads and cache stores (default 1) */
#define HS_OPT_PHASE_TRACE 5    /* 1: the metadata kernel stamps the end of each of its phases */
#define HS_OPT_PROBE 6          /* how hits are found (same results either way):               */
#define HS_PROBE_PAGE_TABLE 0   /*   one page-table load per selected position                   */
#define HS_PROBE_SLOT_SCAN 1    /*   (default) every cached slot's position looked up in an LDS   */
                                /*   structure over the selection, as the pages describe (fewest  */
                                /*   HBM bytes): a bitmap over the history's positions with       */
                                /*   per-word ranks when it fits the LDS, else a hash             */
#define HS_PROBE_SLOT_SCAN_HASH 2 /* the slot scan with the LDS hash whatever the history length */
#define HS_OPT_ATTN_HEADS 7     /* heads per workgroup of hisparse_attend_mla: 32 or 64, or 0 to */
                                /* choose by shape (default)                                      */
#define HS_OPT_META_LANES 8     /* lanes a (request, layer) of the bitmap metadata kernel: 512 or */
                                /* 1024, or 0 to choose by launch size (default); 512 applies     */
                                /* only up to B = 4096 and k = 2048                               */
#define HS_OPT_META_WGS 9       /* workgroups per (request, layer) of a metadata launch over few  */
                                /* units (at most 256 request-layers), which all plan the unit    */
                                /* alike and copy its misses between them in the same launch, so  */
                                /* no fetch launch follows: G in 1..HS_MAX_META_WGS, 0 for one    */
                                /* workgroup and a separate fetch launch, -1 to choose by launch  */
                                /* size (default: split when the launch's misses cannot exceed    */
                                /* 64 MB, into about 64 workgroups; larger launches keep the      */
                                /* fetch launch, which balances the copy over all requests; so do */
                                /* layers that have been prefetch anchors, whose plan the shared  */
                                /* layers' replay then gets before the anchor's own copy).        */
                                /* Applies to the bitmap kernel at 1024 lanes                     */
                                /* with vector runs (k, B multiples of 4, 16-byte aligned arrays) */
                                /* and records up to 1 MB; other launches keep the fetch launch.  */
                                /* Same results either way.                                       */
#define HS_MAX_META_WGS 64
#define HS_OPT_MARKERS 10       /* 1: a roctx range ("hisparse_resolve layer 3", ...) around each */
                                /* call that enqueues work (resolve, resolve_layers, prefetch,    */
                                /* append, attend_mla and its no-allocation form), for host-side  */
                                /* traces (rocprofv3 --marker-trace); the ranges mark when a call */
                                /* enqueues, not when its kernels run.  HS_E_INVAL if the marker  */
                                /* library (librocprofiler-sdk-roctx) cannot be opened.           */
#define HS_OPT_PREFETCH_BLOCKS 11 /* workgroups of hisparse_prefetch's copy launch, which runs on  */
                                /* the side stream beside the main stream's work: 1..65536, or 0  */
                                /* (default) for the fetch kernel's HS_OPT_FETCH_BLOCKS.          */
int hisparse_set_option(hisparse_t h, int key, int64_t value);

/* Per-kernel times of launches issued while HS_OPT_TIMING was on, measured
 * with HIP events on the launch stream (launches captured into a graph are
 * not timed).  Synchronises the device.  `clear` non-zero restarts the
 * accumulation. */
typedef struct {
    double plan_ms, fetch_ms, replay_ms, publish_ms;
    int64_t plan_launches, fetch_launches, replay_launches, publish_launches;
    int64_t dropped;  /* launches not timed because the event ring was full */
} hs_timing;
int hisparse_timing(hisparse_t h, hs_timing* out, int clear);

/* Phase stamps of the last metadata launch of `layer` while HS_OPT_PHASE_TRACE
 * was on: out [num_req][16] raw ticks of the device's constant wall clock
 * (0 = phase not reached), ns_per_tick its period.  Synchronises the device. */
int hisparse_phase_trace(hisparse_t h, int layer, uint64_t* out, double* ns_per_tick);

/* Synchronous device-to-host copy (synchronises the device first), for
 * inspecting the state returned by hisparse_layer_state. */
int hisparse_memcpy_d2h(void* dst, const void* d_src, size_t bytes);

/* Pinned, device-readable host memory for a pool.  coherent = 1 asks for
 * fine-grained (coherent) memory, 0 for coarse-grained (non-coherent). */
int hisparse_host_alloc(size_t bytes, int coherent, void** out);
int hisparse_host_free(void* p);

/* Consumer stand-in: reads the k published records of each request of a
 * layer and reduces them to one 64-bit checksum per request (async):
 *   d_out[r] = sum over j, q of word(r, j, q) * (2*(j*Q + q) + 1)  mod 2^64,
 * where word(r, j, q) is the q-th little-endian 64-bit word of the record in
 * slot d_slot_idx[r][j] and Q = row_bytes / 8. */
int hisparse_gather_checksum(hisparse_t h, int layer, const int32_t* d_slot_idx, int k, uint64_t* d_out,
                             void* stream);

/* The consumer: sparse MLA decode attention over the k records each request
 * of `layer` published (async; blog section 5: attention reads exactly the
 * selected records and its math is unchanged).  Needs bf16 records of
 * W_KV = 576 elements (512 compressed-KV + 64 rotary-key elements).
 *   d_q     bf16 [num_req][num_heads][576], each head's query in record space
 *   d_out   fp32 [num_req][num_heads][512]:
 *           out[h] = sum_j softmax_j(scale * q[h] . rec_j) * rec_j[0:512]
 *   d_lse   fp32 [num_req][num_heads] log-sum-exp of the scaled scores, or NULL
 * A record whose slot is -1 (a rejected request) is left out; a request
 * with none gives zeros and lse = -inf.  num_heads must be a multiple of
 * 64, at most HS_MAX_HEADS; d_q and d_out must be 16-byte aligned (both are
 * moved 16 bytes a lane).  The first call for a larger shape allocates the handle's workspace
 * (make that call before capturing a graph).
 * Errors: HS_E_HANDLE, HS_E_LAYER, HS_E_INVAL, HS_E_K, HS_E_NOMEM, HS_E_HIP. */
int hisparse_attend_mla(hisparse_t h, int layer, const void* d_q, int num_heads, const int32_t* d_slot_idx, int k,
                        float scale, float* d_out, float* d_lse, void* stream);

/* hisparse_attend_mla without any allocation, for callers that cannot
 * allocate device memory (code under HIP graph capture, serving loops that
 * must not call hipMalloc, harnesses that forbid it).  Same arguments, same
 * kernels and the same results as hisparse_attend_mla; its split-k partials
 * (fp16 outputs, fp32 maxima and sums) go to a fixed device area of
 * HS_SCRATCH_BYTES that the library holds on each GPU until the process ends,
 * instead of the handle's workspace.  A call whose partials, num_req *
 * num_heads * chunks * 258 floats' worth, exceed that area is refused with
 * HS_E_SCRATCH (at k = 2048: above 256 requests at 128 heads, above 63
 * requests at 1024 heads).  The handle's device must be
 * current (else HS_E_INVAL).  All calls on one GPU share the area: calls that
 * overlap on one GPU (on different streams, or from different handles) race
 * and must be ordered by the caller.  Nothing in the area needs clearing
 * between calls.  Errors: those of hisparse_attend_mla, HS_E_SCRATCH. */
#define HS_SCRATCH_BYTES 67108864 /* 64 MiB */
int hisparse_attend_mla_noalloc(hisparse_t h, int layer, const void* d_q, int num_heads, const int32_t* d_slot_idx,
                                int k, float scale, float* d_out, float* d_lse, void* stream);

/* Peak probes (synchronous; time `iters` repetitions with HIP events):
 *   link_sdma  : hipMemcpyAsync host -> device (copy engines);
 *   link_kernel: a streaming kernel reading host memory with 16-byte loads;
 *   hbm        : a device-to-device streaming copy kernel (counts read + write). */
int hisparse_probe_link_sdma(const void* host_src, void* d_dst, size_t bytes, int iters, void* stream,
                             double* gbps);
int hisparse_probe_link_kernel(const void* host_src, void* d_dst, size_t bytes, int iters, void* stream,
                               double* gbps);
int hisparse_probe_hbm(const void* d_src, void* d_dst, size_t bytes, int iters, void* stream, double* gbps);

#ifdef __cplusplus
}
#endif
#endif /* HISPARSE_H */
