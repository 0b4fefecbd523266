// api.hip -- host side of libhisparse.so: the C ABI declared in include/hisparse.h.
//
// The handle owns every device array of the two-level hierarchy's GPU side
// (blog "Inference Systems Infrastructure Notes (6): HiSparse", section 2:
// GPU hot cache of B slots per request-layer and the metadata that maps
// positions to slots).  resolve() is two launches on the caller's stream --
// the metadata kernel (resolve.hip) and the fetch kernel (fetch.hip) -- and
// nothing else: no allocation, no synchronisation, no host read of device
// memory, so a decode step that calls it can be captured in a HIP graph.
#include <dlfcn.h>

#include <algorithm>
#include <climits>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <unordered_set>
#include <vector>

#include "hs_internal.h"

struct hisparse_ctx {
    int R = 0, NL = 0, B = 0, W_KV = 0, dtype = 0, elem = 0;
    int64_t row_bytes = 0, L_ctx = 0, pool_rows = 0;
    int device = 0;
    hs::StateBase s{};
    int64_t* d_region_row = nullptr;
    // tuning
    int fetch_blocks = 1024;
    int prefetch_blocks = 0;  // workgroups of the prefetch's copy launch: 0 = fetch_blocks
    int unroll = 4;
    bool nt = true;
    bool timing = false;
    int probe = HS_PROBE_SLOT_SCAN;
    int attn_heads = 0;  // heads per attention workgroup: 0 = by shape, 32 or 64
    int meta_lanes = 0;  // lanes a unit of the bitmap metadata kernel: 0 = by launch size, 512 or 1024
    int meta_wgs = -1;   // workgroups a unit that copies its own misses: -1 = by launch size, 0 = never, G
    bool markers = false;  // roctx range around each enqueueing entry point
    float* attn_ws = nullptr;       // consumer workspace (partials per chunk)
    size_t attn_ws_floats = 0;
    // ordering of resolve / prefetch (host-side bookkeeping only)
    std::vector<hipEvent_t> ev_plan, ev_join;
    std::vector<int> pending_anchor;   // shared layer -> anchor whose replay it must publish, or -1
    std::vector<char> join_outstanding;
    std::vector<char> anchor;  // the layer's plan has been replayed into shared layers
    std::vector<char> plan_in_capture, join_in_capture;  // event recorded while its stream was capturing
    std::vector<char> last_was_plan;
    std::vector<int64_t> steps;
    std::vector<int> last_k;
    std::vector<const int32_t*> last_sel;  // selection of each layer's last planned resolve
    // timing ring
    struct Timed { hipEvent_t a, b; int kind; };
    std::vector<Timed> ring;
    size_t ring_used = 0;
    int64_t dropped = 0;
    double acc_ms[4] = {0, 0, 0, 0};
    int64_t acc_n[4] = {0, 0, 0, 0};
};

// roctx ranges (HS_OPT_MARKERS): the profiler's marker library is opened on
// first use, so the library has no link-time dependency on it; with no tool
// attached its calls do nothing.
namespace {
struct RoctxApi {
    int (*push)(const char*) = nullptr;
    int (*pop)() = nullptr;
};
const RoctxApi* roctx_api() {
    static RoctxApi api;
    static std::once_flag once;
    std::call_once(once, [] {
        void* lib = dlopen("librocprofiler-sdk-roctx.so.1", RTLD_NOW | RTLD_LOCAL);
        if (!lib) lib = dlopen("librocprofiler-sdk-roctx.so", RTLD_NOW | RTLD_LOCAL);
        if (!lib) return;
        auto push = reinterpret_cast<int (*)(const char*)>(dlsym(lib, "roctxRangePushA"));
        auto pop = reinterpret_cast<int (*)()>(dlsym(lib, "roctxRangePop"));
        if (push && pop) {
            api.push = push;
            api.pop = pop;
        }
    });
    return api.push ? &api : nullptr;
}
// a range named after the entry point and its layer for the lifetime of the guard
class MarkRange {
   public:
    MarkRange(const hisparse_ctx* h, const char* what, int layer) {
        if (!h || !h->markers) return;
        api_ = roctx_api();
        if (!api_) return;
        char name[64];
        std::snprintf(name, sizeof name, "%s layer %d", what, layer);
        api_->push(name);
    }
    ~MarkRange() {
        if (api_) api_->pop();
    }
    MarkRange(const MarkRange&) = delete;
    MarkRange& operator=(const MarkRange&) = delete;

   private:
    const RoctxApi* api_ = nullptr;
};
}  // namespace

// Scratch area of the no-allocation attention entry point: the split-k
// partials of hisparse_attend_mla_noalloc (fp16 outputs, fp32 maxima and sums)
// live here instead of in a workspace the handle allocates.  Each GPU the library runs on holds its own copy
// until the process ends.  In host code `scratch` names a host-side stand-in,
// not the device copy: kernels and copies use the address that
// hipGetSymbolAddress returns for the current device (scratch_ptr below).
constexpr size_t kScratchFloats = static_cast<size_t>(16) << 20;  // 64 MiB
static __device__ __align__(256) float scratch[kScratchFloats];

namespace {

enum { K_PLAN = 0, K_FETCH = 1, K_REPLAY = 2, K_PUBLISH = 3 };

// Device address of `scratch` on each device, looked up once per device with
// that device current (at hisparse_create).
constexpr int kScratchDevices = 64;
std::mutex& scratch_mutex() {
    static std::mutex m;
    return m;
}
float* scratch_ptr[kScratchDevices] = {};

int lookup_scratch(int device) {
    if (device < 0 || device >= kScratchDevices) return HS_E_INVAL;
    std::lock_guard<std::mutex> g(scratch_mutex());
    if (scratch_ptr[device]) return HS_OK;
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
        (void)hipGetLastError();
        return HS_E_HIP;
    }
    scratch_ptr[device] = static_cast<float*>(p);
    return HS_OK;
}

float* device_scratch(int device) {
    if (device < 0 || device >= kScratchDevices) return nullptr;
    std::lock_guard<std::mutex> g(scratch_mutex());
    return scratch_ptr[device];
}
constexpr size_t kRingPairs = 8192;

#define HS_TRY(expr)                                      \
    do {                                                  \
        hipError_t e_ = (expr);                           \
        if (e_ != hipSuccess) return HS_E_HIP;            \
    } while (0)

int elem_bytes(int dtype) {
    switch (dtype) {
        case HS_BF16: return 2;
        case HS_FP16: return 2;
        case HS_FP8: return 1;
        case HS_FP32: return 4;
        default: return 0;
    }
}

int hash_bits_for(int k) {
    int bits = 4;
    while ((1 << bits) < 2 * k) ++bits;
    return bits;
}

void free_all(hisparse_ctx* h) {
    hs::StateBase& s = h->s;
    void* ptrs[] = {s.cache, s.slot_pos, s.ts, s.page_table, s.clock, s.plan, s.miss_count,
                    s.hit_mask, s.status, s.err, s.stats, s.phase, s.length, s.arrive, h->d_region_row};
    for (void* p : ptrs)
        if (p) (void)hipFree(p);
    for (hipEvent_t e : h->ev_plan)
        if (e) (void)hipEventDestroy(e);
    for (hipEvent_t e : h->ev_join)
        if (e) (void)hipEventDestroy(e);
    for (auto& t : h->ring) {
        (void)hipEventDestroy(t.a);
        (void)hipEventDestroy(t.b);
    }
    if (h->attn_ws) (void)hipFree(h->attn_ws);
}

int alloc_dev(void** p, size_t bytes) {
    if (hipMalloc(p, bytes ? bytes : 16) != hipSuccess) {
        *p = nullptr;
        (void)hipGetLastError();
        return HS_E_NOMEM;
    }
    return HS_OK;
}

int init_state(hisparse_ctx* h, hipStream_t st) {
    const hs::StateBase& s = h->s;
    const size_t nrl = static_cast<size_t>(h->R) * h->NL;
    HS_TRY(hipMemsetAsync(s.slot_pos, 0xFF, nrl * h->B * sizeof(int32_t), st));
    HS_TRY(hipMemsetAsync(s.ts, 0, nrl * h->B * sizeof(uint32_t), st));
    HS_TRY(hipMemsetAsync(s.page_table, 0xFF, nrl * static_cast<size_t>(h->L_ctx) * sizeof(int32_t), st));
    HS_TRY(hipMemsetAsync(s.clock, 0, nrl * sizeof(uint32_t), st));
    HS_TRY(hipMemsetAsync(s.plan, 0, nrl * h->B * sizeof(int4), st));
    HS_TRY(hipMemsetAsync(s.miss_count, 0, nrl * sizeof(int32_t), st));
    HS_TRY(hipMemsetAsync(s.hit_mask, 0, nrl * h->B, st));
    HS_TRY(hipMemsetAsync(s.status, 0, nrl * sizeof(int32_t), st));
    HS_TRY(hipMemsetAsync(s.err, 0, 4 * sizeof(int32_t), st));
    HS_TRY(hipMemsetAsync(s.stats, 0, nrl * 4 * sizeof(unsigned long long), st));
    HS_TRY(hipMemsetAsync(s.arrive, 0, nrl * sizeof(uint32_t), st));
    HS_TRY(hipStreamSynchronize(st));
    std::fill(h->pending_anchor.begin(), h->pending_anchor.end(), -1);
    std::fill(h->join_outstanding.begin(), h->join_outstanding.end(), 0);
    std::fill(h->last_was_plan.begin(), h->last_was_plan.end(), 0);
    std::fill(h->steps.begin(), h->steps.end(), 0);
    std::fill(h->last_k.begin(), h->last_k.end(), 0);
    return HS_OK;
}

// Live handles.  A destroyed handle is freed, so its pointer is checked
// against this set before anything reads through it: a call with a null or
// destroyed handle returns HS_E_HANDLE instead of touching freed memory.
std::mutex& handles_mutex() {
    static std::mutex m;
    return m;
}
std::unordered_set<const hisparse_ctx*>& live_handles() {
    static std::unordered_set<const hisparse_ctx*> set;
    return set;
}

bool valid(hisparse_t h) {
    if (h == nullptr) return false;
    std::lock_guard<std::mutex> g(handles_mutex());
    return live_handles().count(h) != 0 && h->s.cache != nullptr;
}

bool capturing(hipStream_t st) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(st, &cs) != hipSuccess) {
        (void)hipGetLastError();
        return false;
    }
    return cs == hipStreamCaptureStatusActive;
}

// Make `st` wait for `ev`.  Inside a graph capture, an event recorded before
// the capture began cannot be waited on, queried (a query invalidates a
// global-mode capture) or waited on as an external event (the runtime of this
// image crashes on it), so such a wait is dropped: the header makes it the
// caller's contract that a capture begins after the library's earlier work on
// the prefetch side stream has finished (a device synchronise, as
// torch.cuda.graph does on entry).
int wait_event(hipStream_t st, hipEvent_t ev, bool ev_in_capture) {
    if (capturing(st) && !ev_in_capture) return HS_OK;
    HS_TRY(hipStreamWaitEvent(st, ev, 0));
    return HS_OK;
}

// Launch `fn` bracketed by timing events when timing is on.  A launch being
// captured into a graph is not timed: its events would be graph nodes, never
// recorded on the stream, and could not be read back.
template <typename F>
int timed(hisparse_ctx* h, int kind, hipStream_t st, F fn) {
    if (!h->timing || capturing(st)) {
        return fn() == hipSuccess ? HS_OK : HS_E_HIP;
    }
    if (h->ring_used >= h->ring.size()) {
        ++h->dropped;
        return fn() == hipSuccess ? HS_OK : HS_E_HIP;
    }
    auto& t = h->ring[h->ring_used];
    t.kind = kind;
    HS_TRY(hipEventRecord(t.a, st));
    if (fn() != hipSuccess) return HS_E_HIP;  // the slot stays free: its stop event was never recorded
    HS_TRY(hipEventRecord(t.b, st));
    ++h->ring_used;
    return HS_OK;
}

int check_k(hisparse_ctx* h, int k) {
    if (k < 1 || k > h->B || k > HS_MAX_K) return HS_E_K;
    return HS_OK;
}

}  // namespace

extern "C" {

size_t hisparse_kv_bytes(int num_req, int num_layers, int B, int W_KV, int dtype) {
    const int s = elem_bytes(dtype);
    if (num_req < 1 || num_layers < 1 || B < 1 || W_KV < 1 || s == 0) return 0;
    return static_cast<size_t>(num_req) * num_layers * B * static_cast<size_t>(W_KV) * s;
}

int hisparse_create(int num_req, int num_layers, int B, int W_KV, int dtype, const hs_host_pool* pool,
                    hisparse_t* out) {
    if (!out || !pool) return HS_E_INVAL;
    *out = nullptr;
    if (num_req < 1 || num_req > HS_MAX_REQ || num_layers < 1 || W_KV < 1) return HS_E_INVAL;
    if (B < 1 || B > HS_MAX_B) return HS_E_K;
    const int es = elem_bytes(dtype);
    if (!es) return HS_E_INVAL;
    const int64_t row_bytes = static_cast<int64_t>(W_KV) * es;
    if (row_bytes % 16 != 0) return HS_E_ALIGN;
    if (!pool->base || pool->L_ctx < 1 || pool->L_ctx > INT32_MAX || pool->pool_rows < 1) return HS_E_POOL;
    const int64_t nrl = static_cast<int64_t>(num_req) * num_layers;
    std::vector<int64_t> region(static_cast<size_t>(nrl));
    for (int64_t i = 0; i < nrl; ++i) {
        region[i] = pool->region_row ? pool->region_row[i] : i * pool->L_ctx;
        if (region[i] < 0 || region[i] + pool->L_ctx > pool->pool_rows) return HS_E_POOL;
    }
    void* dpool = nullptr;
    if (hipHostGetDevicePointer(&dpool, const_cast<void*>(pool->base), 0) != hipSuccess || !dpool) {
        (void)hipGetLastError();
        return HS_E_POOL;
    }

    hisparse_ctx* h = new (std::nothrow) hisparse_ctx();
    if (!h) return HS_E_NOMEM;
    h->R = num_req;
    h->NL = num_layers;
    h->B = B;
    h->W_KV = W_KV;
    h->dtype = dtype;
    h->elem = es;
    h->row_bytes = row_bytes;
    h->L_ctx = pool->L_ctx;
    h->pool_rows = pool->pool_rows;
    if (hipGetDevice(&h->device) != hipSuccess) {
        delete h;
        return HS_E_HIP;
    }
    hs::StateBase& s = h->s;
    int rc = HS_OK;
    const size_t nB = static_cast<size_t>(nrl) * B;
    void* p;
    // the cache first, so that s.cache != nullptr marks a live handle
    if ((rc = alloc_dev(&p, nB * static_cast<size_t>(row_bytes))) != HS_OK) { delete h; return rc; }
    s.cache = static_cast<uint8_t*>(p);
#define HS_ALLOC(field, type, count)                                        \
    if ((rc = alloc_dev(&p, sizeof(type) * (count))) != HS_OK) {            \
        free_all(h);                                                        \
        delete h;                                                           \
        return rc;                                                          \
    }                                                                       \
    s.field = static_cast<type*>(p);
    HS_ALLOC(slot_pos, int32_t, nB)
    HS_ALLOC(ts, uint32_t, nB)
    HS_ALLOC(page_table, int32_t, static_cast<size_t>(nrl) * static_cast<size_t>(pool->L_ctx))
    HS_ALLOC(clock, uint32_t, static_cast<size_t>(nrl))
    HS_ALLOC(plan, int4, nB)
    HS_ALLOC(miss_count, int32_t, static_cast<size_t>(nrl))
    HS_ALLOC(hit_mask, uint8_t, nB)
    HS_ALLOC(status, int32_t, static_cast<size_t>(nrl))
    HS_ALLOC(err, int32_t, 4)
    HS_ALLOC(stats, unsigned long long, static_cast<size_t>(nrl) * 4)
    HS_ALLOC(length, int32_t, static_cast<size_t>(nrl))
    HS_ALLOC(arrive, uint32_t, static_cast<size_t>(nrl))
#undef HS_ALLOC
    if ((rc = alloc_dev(&p, sizeof(int64_t) * static_cast<size_t>(nrl))) != HS_OK) {
        free_all(h);
        delete h;
        return rc;
    }
    h->d_region_row = static_cast<int64_t*>(p);
    s.region_row = h->d_region_row;
    s.pool = static_cast<uint8_t*>(dpool);
    s.L_ctx = pool->L_ctx;
    s.row_bytes = row_bytes;
    s.R = num_req;
    s.NL = num_layers;
    s.B = B;
    h->ev_plan.assign(num_layers, nullptr);
    h->ev_join.assign(num_layers, nullptr);
    for (int l = 0; l < num_layers; ++l) {
        if (hipEventCreateWithFlags(&h->ev_plan[l], hipEventDisableTiming) != hipSuccess ||
            hipEventCreateWithFlags(&h->ev_join[l], hipEventDisableTiming) != hipSuccess) {
            free_all(h);
            delete h;
            return HS_E_HIP;
        }
    }
    h->pending_anchor.assign(num_layers, -1);
    h->join_outstanding.assign(num_layers, 0);
    h->anchor.assign(num_layers, 0);
    h->plan_in_capture.assign(num_layers, 0);
    h->join_in_capture.assign(num_layers, 0);
    h->last_was_plan.assign(num_layers, 0);
    h->steps.assign(num_layers, 0);
    h->last_k.assign(num_layers, 0);
    h->last_sel.assign(num_layers, nullptr);
    const std::vector<int32_t> full(static_cast<size_t>(nrl), static_cast<int32_t>(pool->L_ctx));
    if (hipMemcpy(h->d_region_row, region.data(), sizeof(int64_t) * region.size(), hipMemcpyHostToDevice) !=
            hipSuccess ||
        hipMemcpy(s.length, full.data(), sizeof(int32_t) * full.size(), hipMemcpyHostToDevice) != hipSuccess) {
        free_all(h);
        delete h;
        return HS_E_HIP;
    }
    if ((rc = lookup_scratch(h->device)) != HS_OK) {
        free_all(h);
        delete h;
        return rc;
    }
    hipStream_t st = nullptr;
    if ((rc = init_state(h, st)) != HS_OK) {
        free_all(h);
        delete h;
        return rc;
    }
    {
        std::lock_guard<std::mutex> g(handles_mutex());
        live_handles().insert(h);
    }
    *out = h;
    return HS_OK;
}

int hisparse_destroy(hisparse_t h) {
    if (!valid(h)) return HS_E_HANDLE;
    {
        std::lock_guard<std::mutex> g(handles_mutex());
        live_handles().erase(h);
    }
    (void)hipDeviceSynchronize();
    free_all(h);
    h->s.cache = nullptr;
    delete h;
    return HS_OK;
}

static int resolve_plan_path(hisparse_t h, int n, const int* layers, const int32_t* const* sel, int k,
                             int32_t* const* out, hipStream_t st) {
    hs::LayerBatch lb{};
    hs::FetchBatch fb{};
    lb.n = n;
    lb.k = k;
    lb.hash_bits = hash_bits_for(k);
    lb.probe = h->probe;
    lb.nt = h->nt;
    lb.lanes = h->meta_lanes;
    fb.n = n;
    for (int i = 0; i < n; ++i) {
        const int l = layers[i];
        if (h->join_outstanding[l]) {
            // this anchor's previous replay may still read its plan and state
            const int rc = wait_event(st, h->ev_join[l], h->join_in_capture[l]);
            if (rc != HS_OK) return rc;
            h->join_outstanding[l] = 0;
        }
        lb.sel[i] = sel[i];
        lb.out[i] = out[i];
        lb.layer[i] = l;
        fb.layer[i] = l;
    }
    // An anchor keeps one workgroup per unit and the fetch launch: its plan is
    // then ready for the shared layers' replay before its own rows are
    // copied, instead of after (a split launch copies inside the launch).
    bool any_anchor = false;
    for (int i = 0; i < n; ++i) any_anchor = any_anchor || h->anchor[layers[i]];
    lb.wgs = any_anchor ? 0 : hs::plan_wgs(h->s, lb, h->meta_wgs);
    int rc = timed(h, K_PLAN, st, [&] { return hs::launch_plan(h->s, lb, st); });
    if (rc != HS_OK) return rc;
    const bool cap = capturing(st);
    for (int i = 0; i < n; ++i) {
        HS_TRY(hipEventRecord(h->ev_plan[layers[i]], st));
        h->plan_in_capture[layers[i]] = cap;
    }
    if (!hs::plan_copies_misses(h->s, lb)) {
        rc = timed(h, K_FETCH, st, [&] { return hs::launch_fetch(h->s, fb, h->fetch_blocks, h->unroll, h->nt, st); });
        if (rc != HS_OK) return rc;
    }
    for (int i = 0; i < n; ++i) {
        const int l = layers[i];
        h->steps[l] += 1;
        h->last_was_plan[l] = 1;
        h->last_k[l] = k;
        h->last_sel[l] = sel[i];
    }
    return HS_OK;
}

int hisparse_resolve(hisparse_t h, int layer, const int32_t* d_sel, int k, int32_t* d_slot_idx, void* stream) {
    if (!valid(h)) return HS_E_HANDLE;
    MarkRange mark(h, "hisparse_resolve", layer);
    if (layer < 0 || layer >= h->NL) return HS_E_LAYER;
    if (!d_sel || !d_slot_idx) return HS_E_INVAL;
    int rc = check_k(h, k);
    if (rc != HS_OK) return rc;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int anchor = h->pending_anchor[layer];
    if (anchor >= 0) {
        if (k != h->last_k[anchor]) return HS_E_ORDER;
        rc = wait_event(st, h->ev_join[anchor], h->join_in_capture[anchor]);
        if (rc != HS_OK) return rc;
        hs::LayerBatch lb{};
        lb.n = 1;
        lb.k = k;
        lb.sel[0] = d_sel;
        lb.out[0] = d_slot_idx;
        lb.layer[0] = layer;
        lb.anchor_sel[0] = h->last_sel[anchor];
        rc = timed(h, K_PUBLISH, st, [&] { return hs::launch_publish(h->s, lb, st); });
        if (rc != HS_OK) return rc;
        h->pending_anchor[layer] = -1;
        h->steps[layer] += 1;
        h->last_was_plan[layer] = 0;
        h->last_k[layer] = k;
        return HS_OK;
    }
    const int32_t* sel[1] = {d_sel};
    int32_t* out[1] = {d_slot_idx};
    return resolve_plan_path(h, 1, &layer, sel, k, out, st);
}

int hisparse_resolve_layers(hisparse_t h, int n, const int* layers, const int32_t* const* d_sel_ptrs, int k,
                            int32_t* const* d_slot_idx_ptrs, void* stream) {
    if (!valid(h)) return HS_E_HANDLE;
    if (n < 1 || n > hs::kMaxBatch || !layers || !d_sel_ptrs || !d_slot_idx_ptrs) return HS_E_INVAL;
    MarkRange mark(h, "hisparse_resolve_layers", layers[0]);
    if (static_cast<int64_t>(n) * h->R > 8192) return HS_E_INVAL;
    int rc = check_k(h, k);
    if (rc != HS_OK) return rc;
    for (int i = 0; i < n; ++i) {
        if (layers[i] < 0 || layers[i] >= h->NL) return HS_E_LAYER;
        if (!d_sel_ptrs[i] || !d_slot_idx_ptrs[i]) return HS_E_INVAL;
        if (h->pending_anchor[layers[i]] >= 0) return HS_E_ORDER;
        for (int j = 0; j < i; ++j)
            if (layers[j] == layers[i]) return HS_E_INVAL;
    }
    return resolve_plan_path(h, n, layers, d_sel_ptrs, k, d_slot_idx_ptrs, static_cast<hipStream_t>(stream));
}

int hisparse_prefetch(hisparse_t h, int anchor, const int* shared, int n, void* side_stream) {
    if (!valid(h)) return HS_E_HANDLE;
    MarkRange mark(h, "hisparse_prefetch", anchor);
    if (anchor < 0 || anchor >= h->NL) return HS_E_LAYER;
    if (n < 1 || n > hs::kMaxBatch || !shared) return HS_E_INVAL;
    if (static_cast<int64_t>(n) * h->R > 8192) return HS_E_INVAL;
    if (!h->last_was_plan[anchor] || h->pending_anchor[anchor] >= 0) return HS_E_ORDER;
    for (int i = 0; i < n; ++i) {
        const int l = shared[i];
        if (l < 0 || l >= h->NL) return HS_E_LAYER;
        if (l == anchor) return HS_E_INVAL;
        for (int j = 0; j < i; ++j)
            if (shared[j] == l) return HS_E_INVAL;
        if (h->pending_anchor[l] >= 0 || h->steps[l] != h->steps[anchor] - 1) return HS_E_ORDER;
    }
    hipStream_t side = static_cast<hipStream_t>(side_stream);
    const int wrc = wait_event(side, h->ev_plan[anchor], h->plan_in_capture[anchor]);
    if (wrc != HS_OK) return wrc;
    hs::ReplayBatch rb{};
    hs::FetchBatch fb{};
    rb.anchor = anchor;
    rb.k = h->last_k[anchor];
    rb.n = n;
    fb.n = n;
    for (int i = 0; i < n; ++i) {
        rb.shared[i] = shared[i];
        fb.layer[i] = shared[i];
    }
    int rc = timed(h, K_REPLAY, side, [&] {
        hipError_t e = hs::launch_replay_meta(h->s, rb, side);
        if (e != hipSuccess) return e;
        return hs::launch_fetch(h->s, fb, h->prefetch_blocks ? h->prefetch_blocks : h->fetch_blocks, h->unroll,
                                h->nt, side);
    });
    if (rc != HS_OK) return rc;
    HS_TRY(hipEventRecord(h->ev_join[anchor], side));
    h->join_in_capture[anchor] = capturing(side);
    h->join_outstanding[anchor] = 1;
    h->anchor[anchor] = 1;
    for (int i = 0; i < n; ++i) h->pending_anchor[shared[i]] = anchor;
    return HS_OK;
}

int hisparse_append(hisparse_t h, int layer, const void* d_rows, void* stream) {
    if (!valid(h)) return HS_E_HANDLE;
    MarkRange mark(h, "hisparse_append", layer);
    if (layer < 0 || layer >= h->NL) return HS_E_LAYER;
    if (!d_rows) return HS_E_INVAL;
    return hs::launch_append(h->s, layer, static_cast<const uint8_t*>(d_rows), static_cast<hipStream_t>(stream)) ==
                   hipSuccess
               ? HS_OK
               : HS_E_HIP;
}

int hisparse_set_lengths(hisparse_t h, const int64_t* lengths) {
    if (!valid(h)) return HS_E_HANDLE;
    if (!lengths) return HS_E_INVAL;
    const size_t nrl = static_cast<size_t>(h->R) * h->NL;
    std::vector<int32_t> dev(nrl);
    for (int r = 0; r < h->R; ++r) {
        for (int l = 0; l < h->NL; ++l) {
            const int64_t v = lengths[static_cast<size_t>(r) * h->NL + l];
            if (v < 0 || v > h->L_ctx) return HS_E_INVAL;
            dev[static_cast<size_t>(l) * h->R + r] = static_cast<int32_t>(v);
        }
    }
    HS_TRY(hipDeviceSynchronize());
    HS_TRY(hipMemcpy(h->s.length, dev.data(), sizeof(int32_t) * nrl, hipMemcpyHostToDevice));
    // positions at or past a new length leave the cache (their records may be
    // rewritten by later appends)
    HS_TRY(hs::launch_trim(h->s, nullptr));
    HS_TRY(hipDeviceSynchronize());
    return HS_OK;
}

int hisparse_get_lengths(hisparse_t h, int64_t* lengths) {
    if (!valid(h)) return HS_E_HANDLE;
    if (!lengths) return HS_E_INVAL;
    const size_t nrl = static_cast<size_t>(h->R) * h->NL;
    std::vector<int32_t> dev(nrl);
    HS_TRY(hipDeviceSynchronize());
    HS_TRY(hipMemcpy(dev.data(), h->s.length, sizeof(int32_t) * nrl, hipMemcpyDeviceToHost));
    for (int r = 0; r < h->R; ++r)
        for (int l = 0; l < h->NL; ++l)
            lengths[static_cast<size_t>(r) * h->NL + l] = dev[static_cast<size_t>(l) * h->R + r];
    return HS_OK;
}

size_t hisparse_hbm_bytes(hisparse_t h) {
    if (!valid(h)) return 0;
    return static_cast<size_t>(h->R) * h->NL * h->B * static_cast<size_t>(h->row_bytes);
}

size_t hisparse_meta_bytes(hisparse_t h) {
    if (!valid(h)) return 0;
    const size_t nrl = static_cast<size_t>(h->R) * h->NL;
    return nrl * h->B * (sizeof(int32_t) + sizeof(uint32_t) + sizeof(int4) + 1) +
           nrl * static_cast<size_t>(h->L_ctx) * sizeof(int32_t) +
           nrl * (5 * sizeof(int32_t) + sizeof(int64_t)) +  // clock, miss count, status, length, arrival; region row
           nrl * 4 * sizeof(unsigned long long) + 4 * sizeof(int32_t);  // counters; error word
}

int hisparse_layer_state(hisparse_t h, int layer, hs_layer_state* out) {
    if (!valid(h)) return HS_E_HANDLE;
    if (layer < 0 || layer >= h->NL) return HS_E_LAYER;
    if (!out) return HS_E_INVAL;
    const hs::StateBase& s = h->s;
    const size_t rl = static_cast<size_t>(layer) * h->R;
    out->d_cache = s.cache + rl * h->B * static_cast<size_t>(h->row_bytes);
    out->d_slot_pos = s.slot_pos + rl * h->B;
    out->d_ts = s.ts + rl * h->B;
    out->d_page_table = s.page_table + rl * static_cast<size_t>(h->L_ctx);
    out->d_clock = s.clock + rl;
    out->d_plan = reinterpret_cast<int32_t*>(s.plan + rl * h->B);
    out->d_miss_count = s.miss_count + rl;
    out->d_hit_mask = s.hit_mask + rl * h->B;
    out->row_bytes = h->row_bytes;
    out->B = h->B;
    out->num_req = h->R;
    out->L_ctx = h->L_ctx;
    return HS_OK;
}

int hisparse_get_error(hisparse_t h, int* code, int* layer, int* req) {
    if (!valid(h)) return HS_E_HANDLE;
    int32_t w[4] = {0, 0, 0, 0};
    HS_TRY(hipDeviceSynchronize());
    HS_TRY(hipMemcpy(w, h->s.err, sizeof w, hipMemcpyDeviceToHost));
    if (code) *code = w[0];
    if (layer) *layer = w[1];
    if (req) *req = w[2];
    return HS_OK;
}

int hisparse_clear_error(hisparse_t h) {
    if (!valid(h)) return HS_E_HANDLE;
    HS_TRY(hipDeviceSynchronize());
    HS_TRY(hipMemset(h->s.err, 0, 4 * sizeof(int32_t)));
    HS_TRY(hipDeviceSynchronize());
    return HS_OK;
}

int hisparse_stats(hisparse_t h, int layer, hs_stats* out) {
    if (!valid(h)) return HS_E_HANDLE;
    if (!out || layer < -1 || layer >= h->NL) return layer >= h->NL ? HS_E_LAYER : HS_E_INVAL;
    std::vector<unsigned long long> st(static_cast<size_t>(h->NL) * h->R * 4);
    HS_TRY(hipDeviceSynchronize());
    HS_TRY(hipMemcpy(st.data(), h->s.stats, sizeof(unsigned long long) * st.size(), hipMemcpyDeviceToHost));
    std::memset(out, 0, sizeof *out);
    for (int l = 0; l < h->NL; ++l) {
        if (layer != -1 && l != layer) continue;
        for (int r = 0; r < h->R; ++r) {
            const unsigned long long* c = st.data() + 4 * (static_cast<size_t>(l) * h->R + r);
            out->hits += c[0];
            out->misses += c[1];
            out->miss_bytes += c[2];
            out->resolves += c[3];
        }
    }
    return HS_OK;
}

int hisparse_reset(hisparse_t h) {
    if (!valid(h)) return HS_E_HANDLE;
    HS_TRY(hipDeviceSynchronize());
    return init_state(h, nullptr);
}

int hisparse_set_option(hisparse_t h, int key, int64_t value) {
    if (!valid(h)) return HS_E_HANDLE;
    switch (key) {
        case HS_OPT_FETCH_BLOCKS:
            if (value < 1 || value > 65536) return HS_E_INVAL;
            h->fetch_blocks = static_cast<int>(value);
            return HS_OK;
        case HS_OPT_PREFETCH_BLOCKS:
            if (value < 0 || value > 65536) return HS_E_INVAL;
            h->prefetch_blocks = static_cast<int>(value);
            return HS_OK;
        case HS_OPT_FETCH_UNROLL:
            if (value != 1 && value != 2 && value != 4 && value != 8) return HS_E_INVAL;
            h->unroll = static_cast<int>(value);
            return HS_OK;
        case HS_OPT_PROBE:
            if (value != HS_PROBE_PAGE_TABLE && value != HS_PROBE_SLOT_SCAN && value != HS_PROBE_SLOT_SCAN_HASH)
                return HS_E_INVAL;
            h->probe = static_cast<int>(value);
            return HS_OK;
        case HS_OPT_NT_LOADS:
            h->nt = value != 0;
            return HS_OK;
        case HS_OPT_ATTN_HEADS:
            if (value != 0 && value != 32 && value != 64) return HS_E_INVAL;
            h->attn_heads = static_cast<int>(value);
            return HS_OK;
        case HS_OPT_META_LANES:
            if (value != 0 && value != 512 && value != 1024) return HS_E_INVAL;
            h->meta_lanes = static_cast<int>(value);
            return HS_OK;
        case HS_OPT_META_WGS:
            if (value < -1 || value > HS_MAX_META_WGS) return HS_E_INVAL;
            h->meta_wgs = static_cast<int>(value);
            return HS_OK;
        case HS_OPT_PHASE_TRACE:
            if (value && !h->s.phase) {
                const size_t n = static_cast<size_t>(h->R) * h->NL * hs::kPhaseSlots;
                void* p = nullptr;
                HS_TRY(hipDeviceSynchronize());
                if (alloc_dev(&p, n * sizeof(unsigned long long)) != HS_OK) return HS_E_NOMEM;
                HS_TRY(hipMemset(p, 0, n * sizeof(unsigned long long)));
                HS_TRY(hipDeviceSynchronize());
                h->s.phase = static_cast<unsigned long long*>(p);
            } else if (!value && h->s.phase) {
                HS_TRY(hipDeviceSynchronize());
                (void)hipFree(h->s.phase);
                h->s.phase = nullptr;
            }
            return HS_OK;
        case HS_OPT_MARKERS:
            if (value && !roctx_api()) return HS_E_INVAL;  // the marker library is not there
            h->markers = value != 0;
            return HS_OK;
        case HS_OPT_TIMING:
            if (value && h->ring.empty()) {
                h->ring.resize(kRingPairs);
                for (auto& t : h->ring) {
                    if (hipEventCreate(&t.a) != hipSuccess || hipEventCreate(&t.b) != hipSuccess) return HS_E_HIP;
                }
            }
            h->timing = value != 0;
            return HS_OK;
        default:
            return HS_E_INVAL;
    }
}

int hisparse_timing(hisparse_t h, hs_timing* out, int clear) {
    if (!valid(h)) return HS_E_HANDLE;
    if (!out) return HS_E_INVAL;
    HS_TRY(hipDeviceSynchronize());
    for (size_t i = 0; i < h->ring_used; ++i) {
        float ms = 0.f;
        HS_TRY(hipEventElapsedTime(&ms, h->ring[i].a, h->ring[i].b));
        h->acc_ms[h->ring[i].kind] += ms;
        h->acc_n[h->ring[i].kind] += 1;
    }
    h->ring_used = 0;
    out->plan_ms = h->acc_ms[K_PLAN];
    out->fetch_ms = h->acc_ms[K_FETCH];
    out->replay_ms = h->acc_ms[K_REPLAY];
    out->publish_ms = h->acc_ms[K_PUBLISH];
    out->plan_launches = h->acc_n[K_PLAN];
    out->fetch_launches = h->acc_n[K_FETCH];
    out->replay_launches = h->acc_n[K_REPLAY];
    out->publish_launches = h->acc_n[K_PUBLISH];
    out->dropped = h->dropped;
    if (clear) {
        for (int i = 0; i < 4; ++i) {
            h->acc_ms[i] = 0;
            h->acc_n[i] = 0;
        }
        h->dropped = 0;
    }
    return HS_OK;
}

int hisparse_host_alloc(size_t bytes, int coherent, void** out) {
    if (!out || bytes == 0) return HS_E_INVAL;
    *out = nullptr;
    const unsigned flags = hipHostMallocMapped | (coherent ? hipHostMallocCoherent : hipHostMallocNonCoherent);
    if (hipHostMalloc(out, bytes, flags) != hipSuccess) {
        (void)hipGetLastError();
        *out = nullptr;
        return HS_E_NOMEM;
    }
    return HS_OK;
}

int hisparse_phase_trace(hisparse_t h, int layer, uint64_t* out, double* ns_per_tick) {
    if (!valid(h)) return HS_E_HANDLE;
    if (layer < 0 || layer >= h->NL) return HS_E_LAYER;
    if (!out || !ns_per_tick || !h->s.phase) return HS_E_INVAL;
    int khz = 0;
    HS_TRY(hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, h->device));
    *ns_per_tick = khz > 0 ? 1e6 / khz : 0.0;
    HS_TRY(hipDeviceSynchronize());
    const size_t n = static_cast<size_t>(h->R) * hs::kPhaseSlots;
    HS_TRY(hipMemcpy(out, h->s.phase + static_cast<size_t>(layer) * n, n * sizeof(uint64_t), hipMemcpyDeviceToHost));
    return HS_OK;
}

int hisparse_memcpy_d2h(void* dst, const void* d_src, size_t bytes) {
    if (!dst || !d_src) return HS_E_INVAL;
    if (bytes == 0) return HS_OK;
    HS_TRY(hipDeviceSynchronize());
    HS_TRY(hipMemcpy(dst, d_src, bytes, hipMemcpyDeviceToHost));
    return HS_OK;
}

int hisparse_host_free(void* p) {
    if (!p) return HS_E_INVAL;
    return hipHostFree(p) == hipSuccess ? HS_OK : HS_E_HIP;
}

int hisparse_gather_checksum(hisparse_t h, int layer, const int32_t* d_slot_idx, int k, uint64_t* d_out,
                             void* stream) {
    if (!valid(h)) return HS_E_HANDLE;
    if (layer < 0 || layer >= h->NL) return HS_E_LAYER;
    if (!d_slot_idx || !d_out) return HS_E_INVAL;
    if (k < 1 || k > h->B) return HS_E_K;
    return hs::launch_gather_checksum(h->s, layer, d_slot_idx, k, d_out, static_cast<hipStream_t>(stream)) ==
                   hipSuccess
               ? HS_OK
               : HS_E_HIP;
}

// Argument checks and the launch shape shared by both attention entry points.
static int attend_shape(hisparse_t h, int layer, const void* d_q, int num_heads, const int32_t* d_slot_idx, int k,
                        float* d_out, int* ht, int* chunk, size_t* need) {
    if (!valid(h)) return HS_E_HANDLE;
    if (layer < 0 || layer >= h->NL) return HS_E_LAYER;
    if (!d_q || !d_slot_idx || !d_out || num_heads < 64 || num_heads % 64 != 0 || num_heads > HS_MAX_HEADS)
        return HS_E_INVAL;
    // queries are read and outputs written 16 bytes a lane
    if ((reinterpret_cast<uintptr_t>(d_q) | reinterpret_cast<uintptr_t>(d_out)) & 15u) return HS_E_INVAL;
    if (h->dtype != HS_BF16 || h->W_KV != 576) return HS_E_INVAL;
    if (k < 1 || k > h->B) return HS_E_K;
    *ht = h->attn_heads ? h->attn_heads / 16 : hs::attend_head_tiles(h->R, num_heads, k);
    *chunk = hs::attend_chunk(h->R, num_heads, k, *ht);
    const int nchunk = (k + *chunk - 1) / *chunk;
    *need = hs::attend_workspace_floats(h->R, num_heads, nchunk);
    return HS_OK;
}

int hisparse_attend_mla(hisparse_t h, int layer, const void* d_q, int num_heads, const int32_t* d_slot_idx, int k,
                        float scale, float* d_out, float* d_lse, void* stream) {
    int ht = 0, chunk = 0;
    size_t need = 0;
    const int rc = attend_shape(h, layer, d_q, num_heads, d_slot_idx, k, d_out, &ht, &chunk, &need);
    if (rc != HS_OK) return rc;
    MarkRange mark(h, "hisparse_attend_mla", layer);
    if (need > h->attn_ws_floats) {
        HS_TRY(hipDeviceSynchronize());
        if (h->attn_ws) (void)hipFree(h->attn_ws);
        h->attn_ws = nullptr;
        h->attn_ws_floats = 0;
        void* p = nullptr;
        if (alloc_dev(&p, need * sizeof(float)) != HS_OK) return HS_E_NOMEM;
        h->attn_ws = static_cast<float*>(p);
        h->attn_ws_floats = need;
    }
    return hs::launch_attend_mla(h->s, layer, static_cast<const uint16_t*>(d_q), num_heads, d_slot_idx, k, scale,
                                 d_out, d_lse, h->attn_ws, ht, chunk, static_cast<hipStream_t>(stream)) == hipSuccess
               ? HS_OK
               : HS_E_HIP;
}

int hisparse_attend_mla_noalloc(hisparse_t h, int layer, const void* d_q, int num_heads, const int32_t* d_slot_idx,
                                int k, float scale, float* d_out, float* d_lse, void* stream) {
    int ht = 0, chunk = 0;
    size_t need = 0;
    const int rc = attend_shape(h, layer, d_q, num_heads, d_slot_idx, k, d_out, &ht, &chunk, &need);
    if (rc != HS_OK) return rc;
    if (need > kScratchFloats) return HS_E_SCRATCH;
    MarkRange mark(h, "hisparse_attend_mla_noalloc", layer);
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev != h->device) {
        (void)hipGetLastError();
        return HS_E_INVAL;  // the handle's device must be current
    }
    float* ws = device_scratch(dev);
    if (!ws) return HS_E_HIP;
    return hs::launch_attend_mla(h->s, layer, static_cast<const uint16_t*>(d_q), num_heads, d_slot_idx, k, scale,
                                 d_out, d_lse, ws, ht, chunk, static_cast<hipStream_t>(stream)) == hipSuccess
               ? HS_OK
               : HS_E_HIP;
}

static int probe(int kind, const void* src, void* dst, size_t bytes, int iters, void* stream, double* gbps) {
    if (!src || !dst || !gbps || bytes < 16 || (bytes % 16) != 0 || iters < 1) return HS_E_INVAL;
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipEvent_t a = nullptr, b = nullptr;
    HS_TRY(hipEventCreate(&a));
    if (hipEventCreate(&b) != hipSuccess) {
        (void)hipEventDestroy(a);
        return HS_E_HIP;
    }
    auto one = [&]() -> hipError_t {
        if (kind == 0) return hipMemcpyAsync(dst, src, bytes, hipMemcpyHostToDevice, st);
        if (kind == 1) return hs::launch_link_read(src, dst, bytes, st);
        return hs::launch_hbm_copy(src, dst, bytes, st);
    };
    int rc = HS_OK;
    if (one() != hipSuccess) rc = HS_E_HIP;  // warm-up
    if (rc == HS_OK && hipEventRecord(a, st) != hipSuccess) rc = HS_E_HIP;
    for (int i = 0; rc == HS_OK && i < iters; ++i)
        if (one() != hipSuccess) rc = HS_E_HIP;
    if (rc == HS_OK && hipEventRecord(b, st) != hipSuccess) rc = HS_E_HIP;
    if (rc == HS_OK && hipEventSynchronize(b) != hipSuccess) rc = HS_E_HIP;
    float ms = 0.f;
    if (rc == HS_OK && hipEventElapsedTime(&ms, a, b) != hipSuccess) rc = HS_E_HIP;
    (void)hipEventDestroy(a);
    (void)hipEventDestroy(b);
    if (rc != HS_OK) return rc;
    const double moved = static_cast<double>(bytes) * iters * (kind == 2 ? 2.0 : 1.0);
    *gbps = moved / (static_cast<double>(ms) * 1e-3) / 1e9;
    return HS_OK;
}

int hisparse_probe_link_sdma(const void* host_src, void* d_dst, size_t bytes, int iters, void* stream,
                             double* gbps) {
    return probe(0, host_src, d_dst, bytes, iters, stream, gbps);
}

int hisparse_probe_link_kernel(const void* host_src, void* d_dst, size_t bytes, int iters, void* stream,
                               double* gbps) {
    void* dsrc = nullptr;
    if (!host_src || hipHostGetDevicePointer(&dsrc, const_cast<void*>(host_src), 0) != hipSuccess) {
        (void)hipGetLastError();
        return HS_E_POOL;
    }
    return probe(1, dsrc, d_dst, bytes, iters, stream, gbps);
}

int hisparse_probe_hbm(const void* d_src, void* d_dst, size_t bytes, int iters, void* stream, double* gbps) {
    return probe(2, d_src, d_dst, bytes, iters, stream, gbps);
}

}  // extern "C"
