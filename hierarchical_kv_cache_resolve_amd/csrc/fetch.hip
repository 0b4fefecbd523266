// fetch.hip -- the host-fetch half of RESOLVE on gfx950, plus the peak probes
// and the consumer stand-in.
//
// GPU-assisted IO (blog section 3 and the pith "Core claim": GPU threads load
// the missed records straight from pinned host memory with vectorised loads
// instead of a CPU-driven copy path).  Here every lane moves 16-byte pieces
// (global_load_dwordx4 on the host-mapped pool, global_store_dwordx4 into the
// HBM cache).  The misses of all requests of the launched layers form one
// flat index space of (row, 16-byte piece) pairs, so consecutive lanes of a
// wave read consecutive bytes of one record and the whole chip shares the
// transfer however unevenly the misses fall on requests.  Each lane takes U
// pieces a round; a piece's host address needs its plan entry and its
// history's first row, and the in-order vector-memory counter makes those
// loads wait for the previous piece's host load, so about one host load per
// lane is in flight -- with 262144 lanes, megabytes in flight, which is what
// hides the microsecond-scale latency of reads that cross the host link
// (keeping all U in flight per lane measured slower).
#include "hs_internal.h"

namespace hs {

namespace {

// Exclusive scan over the 256 lanes of a fetch workgroup.
__device__ inline int block256_excl_scan(int v, int* total, int* scratch) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int x = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
    }
    if (lane == 63) scratch[wave] = x;
    __syncthreads();
    int base = 0;
    for (int w = 0; w < wave; ++w) base += scratch[w];
    int tot = 0;
    for (int w = 0; w < kFetchThreads / 64; ++w) tot += scratch[w];
    *total = tot;
    __syncthreads();
    return base + x - v;
}

// Copy the rows named by each launched layer's plan from the host pool into
// that layer's cache slots.
template <int U, bool NT>
__global__ __launch_bounds__(kFetchThreads) void fetch_kernel(StateBase s, FetchBatch fb) {
    extern __shared__ int pref[];  // [units + 1] row prefix over (batch entry, request)
    __shared__ int scan_scratch[8];
    const int units = fb.n * s.R;
    const int per = (units + kFetchThreads - 1) / kFetchThreads;
    const int u0 = threadIdx.x * per;
    int mine = 0;
    for (int q = 0; q < per; ++q) {
        const int u = u0 + q;
        if (u < units) {
            const int b = u / s.R, r = u - b * s.R;
            mine += s.miss_count[static_cast<int64_t>(fb.layer[b]) * s.R + r];
        }
    }
    int rows;
    int run = block256_excl_scan(mine, &rows, scan_scratch);
    for (int q = 0; q < per; ++q) {
        const int u = u0 + q;
        if (u < units) {
            pref[u] = run;
            const int b = u / s.R, r = u - b * s.R;
            run += s.miss_count[static_cast<int64_t>(fb.layer[b]) * s.R + r];
        }
    }
    if (threadIdx.x == 0) pref[units] = rows;
    __syncthreads();

    const int row16 = static_cast<int>(s.row_bytes >> 4);
    const int64_t total = static_cast<int64_t>(rows) * row16;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kFetchThreads;
    for (int64_t c0 = static_cast<int64_t>(blockIdx.x) * kFetchThreads + threadIdx.x; c0 < total; c0 += stride * U) {
        u32x4 v[U];
        u32x4* dst[U];
#pragma unroll
        for (int x = 0; x < U; ++x) {
            const int64_t c = c0 + x * stride;
            dst[x] = nullptr;
            if (c < total) {
                const int g = static_cast<int>(c / row16);
                const int off = static_cast<int>(c - static_cast<int64_t>(g) * row16);
                int lo = 0, hi = units;  // pref[lo] <= g < pref[hi]
                while (hi - lo > 1) {
                    const int mid = (lo + hi) >> 1;
                    if (pref[mid] <= g) lo = mid;
                    else hi = mid;
                }
                const int b = lo / s.R, r = lo - b * s.R, layer = fb.layer[b];
                const int64_t rl = static_cast<int64_t>(layer) * s.R + r;
                const int4 e = s.plan[rl * s.B + (g - pref[lo])];
                const int64_t src_row = s.region_row[static_cast<int64_t>(r) * s.NL + layer] + e.w;
                const u32x4* src = reinterpret_cast<const u32x4*>(s.pool + src_row * s.row_bytes) + off;
                dst[x] = reinterpret_cast<u32x4*>(s.cache + (rl * s.B + e.y) * s.row_bytes) + off;
                v[x] = ld16<NT>(src);
            }
        }
#pragma unroll
        for (int x = 0; x < U; ++x)
            if (dst[x]) st16<NT>(dst[x], v[x]);
    }
}

// Decode-time append: the record of each request's new token goes to the
// next position of its history in the host pool, written by GPU lanes with
// 16-byte stores to host-mapped memory; the history grows by one.  A full
// history (length == L_ctx) is left as it is and reported.
__global__ __launch_bounds__(kFetchThreads) void append_kernel(StateBase s, int layer, const uint8_t* rows) {
    const int r = blockIdx.x;
    const int64_t rl = static_cast<int64_t>(layer) * s.R + r;
    const int pos = s.length[rl];
    if (pos >= s.L_ctx) {
        if (threadIdx.x == 0) record_error(s.err, HS_DEV_FULL, layer, r, pos);
        return;
    }
    const int row16 = static_cast<int>(s.row_bytes >> 4);
    const u32x4* src = reinterpret_cast<const u32x4*>(rows + static_cast<int64_t>(r) * s.row_bytes);
    u32x4* dst = reinterpret_cast<u32x4*>(
        s.pool + (s.region_row[static_cast<int64_t>(r) * s.NL + layer] + pos) * s.row_bytes);
    for (int c = threadIdx.x; c < row16; c += kFetchThreads) dst[c] = src[c];
    __syncthreads();
    if (threadIdx.x == 0) s.length[rl] = pos + 1;
}

// Link probe: stream `n16` 16-byte pieces from host memory into HBM.
template <int U>
__global__ __launch_bounds__(kFetchThreads) void link_read_kernel(const u32x4* src, u32x4* dst, int64_t n16) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kFetchThreads;
    for (int64_t c0 = static_cast<int64_t>(blockIdx.x) * kFetchThreads + threadIdx.x; c0 < n16; c0 += stride * U) {
        u32x4 v[U];
#pragma unroll
        for (int x = 0; x < U; ++x)
            if (c0 + x * stride < n16) v[x] = __builtin_nontemporal_load(src + c0 + x * stride);
#pragma unroll
        for (int x = 0; x < U; ++x)
            if (c0 + x * stride < n16) __builtin_nontemporal_store(v[x], dst + c0 + x * stride);
    }
}

// HBM probe: device-to-device streaming copy.
template <int U>
__global__ __launch_bounds__(kFetchThreads) void hbm_copy_kernel(const u32x4* src, u32x4* dst, int64_t n16) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kFetchThreads;
    for (int64_t c0 = static_cast<int64_t>(blockIdx.x) * kFetchThreads + threadIdx.x; c0 < n16; c0 += stride * U) {
        u32x4 v[U];
#pragma unroll
        for (int x = 0; x < U; ++x)
            if (c0 + x * stride < n16) v[x] = __builtin_nontemporal_load(src + c0 + x * stride);
#pragma unroll
        for (int x = 0; x < U; ++x)
            if (c0 + x * stride < n16) __builtin_nontemporal_store(v[x], dst + c0 + x * stride);
    }
}

// Consumer stand-in: reads the k published records of every request and
// reduces them to one checksum per request.  grid = (request, chunk of
// records); each workgroup adds its partial sum with a 64-bit atomic (the sum
// is modulo 2^64, so the order of the additions does not matter).
constexpr int kGatherRowsPerBlock = 32;

__global__ __launch_bounds__(kFetchThreads) void gather_zero_kernel(uint64_t* out, int n) {
    const int i = blockIdx.x * kFetchThreads + threadIdx.x;
    if (i < n) out[i] = 0ull;
}

__global__ __launch_bounds__(kFetchThreads) void gather_checksum_kernel(StateBase s, int layer,
                                                                        const int32_t* slot_idx, int k,
                                                                        uint64_t* out) {
    __shared__ uint64_t part[kFetchThreads / 64];
    const int r = blockIdx.x;
    const int64_t rl = static_cast<int64_t>(layer) * s.R + r;
    const int Q = static_cast<int>(s.row_bytes >> 3);
    const int j0 = blockIdx.y * kGatherRowsPerBlock;
    const int j1 = min(k, j0 + kGatherRowsPerBlock);
    const int64_t n = static_cast<int64_t>(j1 - j0) * Q;
    const int32_t* sidx = slot_idx + static_cast<int64_t>(r) * k;
    uint64_t acc = 0;
    for (int64_t i = threadIdx.x; i < n; i += kFetchThreads) {
        const int jj = static_cast<int>(i / Q), q = static_cast<int>(i - static_cast<int64_t>(jj) * Q);
        const int j = j0 + jj;
        const int slot = sidx[j];
        if (slot < 0 || slot >= s.B) continue;
        const uint64_t w = reinterpret_cast<const uint64_t*>(s.cache + (rl * s.B + slot) * s.row_bytes)[q];
        acc += w * (2ull * (static_cast<uint64_t>(j) * static_cast<uint64_t>(Q) + static_cast<uint64_t>(q)) + 1ull);
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint64_t t = 0;
        for (int w = 0; w < kFetchThreads / 64; ++w) t += part[w];
        atomicAdd(reinterpret_cast<unsigned long long*>(out + r), static_cast<unsigned long long>(t));
    }
}

}  // namespace

hipError_t launch_fetch(const StateBase& s, const FetchBatch& fb, int blocks, int unroll, bool nt, hipStream_t st) {
    const size_t lds = sizeof(int) * (static_cast<size_t>(fb.n) * s.R + 1);
    const dim3 grid(blocks), block(kFetchThreads);
#define HS_FETCH_CASE(UU)                                                                   \
    case UU:                                                                                \
        if (nt) hipLaunchKernelGGL((fetch_kernel<UU, true>), grid, block, lds, st, s, fb);  \
        else hipLaunchKernelGGL((fetch_kernel<UU, false>), grid, block, lds, st, s, fb);    \
        break;
    switch (unroll) {
        HS_FETCH_CASE(1)
        HS_FETCH_CASE(2)
        HS_FETCH_CASE(4)
        HS_FETCH_CASE(8)
        default:
            return hipErrorInvalidValue;
    }
#undef HS_FETCH_CASE
    return hipGetLastError();
}

hipError_t launch_gather_checksum(const StateBase& s, int layer, const int32_t* slot_idx, int k, uint64_t* out,
                                  hipStream_t st) {
    hipLaunchKernelGGL(gather_zero_kernel, dim3((s.R + kFetchThreads - 1) / kFetchThreads), dim3(kFetchThreads), 0,
                       st, out, s.R);
    const dim3 grid(s.R, (k + kGatherRowsPerBlock - 1) / kGatherRowsPerBlock);
    hipLaunchKernelGGL(gather_checksum_kernel, grid, dim3(kFetchThreads), 0, st, s, layer, slot_idx, k, out);
    return hipGetLastError();
}

hipError_t launch_append(const StateBase& s, int layer, const uint8_t* rows, hipStream_t st) {
    hipLaunchKernelGGL(append_kernel, dim3(s.R), dim3(kFetchThreads), 0, st, s, layer, rows);
    return hipGetLastError();
}

hipError_t launch_link_read(const void* src, void* dst, size_t bytes, hipStream_t st) {
    hipLaunchKernelGGL(link_read_kernel<4>, dim3(2048), dim3(kFetchThreads), 0, st,
                       static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), static_cast<int64_t>(bytes / 16));
    return hipGetLastError();
}

hipError_t launch_hbm_copy(const void* src, void* dst, size_t bytes, hipStream_t st) {
    // 65536 workgroups: measured on MI355X over 4 GiB, 5.2 TB/s against 4.7 TB/s with 4096
    // (and 4.6 TB/s for a device-to-device hipMemcpy), so the reported peak is not understated
    hipLaunchKernelGGL(hbm_copy_kernel<4>, dim3(65536), dim3(kFetchThreads), 0, st,
                       static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), static_cast<int64_t>(bytes / 16));
    return hipGetLastError();
}

}  // namespace hs
