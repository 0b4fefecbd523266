// attend.hip -- the consumer of RESOLVE: sparse MLA decode attention over the
// k records each request published, on gfx950 matrix cores.
//
// Sparse attention reads exactly the selected records and computes ordinary
// attention over them; placement does not change the math (blog "Inference
// Systems Infrastructure Notes (6): HiSparse", section 5 "Exact").  For an
// MLA-style latent record (576 bf16: a 512-element compressed KV followed by
// a 64-element rotary key) the absorbed decode form is used: the query of
// each head lives in the 576-element record space, scores are dot products
// with whole records and the values are the records' first 512 elements.
//
// Work split (flash-decoding): workgroup = (request, 64 heads, a chunk of
// records); 4 wave64s, one per 16 heads.  For each 64-record sub-chunk the
// records named by slot_idx are gathered from the HBM cache into LDS twice --
// row-major for S = Q K^T and transposed for O = P V -- so every MFMA operand
// is one 16-byte LDS read.  Scores use v_mfma_f32_16x16x32_bf16 with the
// query fragments held in registers; the softmax is online (running maximum
// and sum per head, in log2 units) and the probabilities go through LDS as
// bf16 to become the A operand of the value product.  A second kernel
// combines the chunks of each (request, head).
#include "hs_internal.h"

namespace hs {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kAttnThreads = 256;
constexpr int kHeadsPerWG = 64;
constexpr int kSub = 64;                 // records per LDS sub-chunk
constexpr int kDqk = 576, kDv = 512;
constexpr int kKcStride = kDqk + 8;      // bf16 per LDS record row (+16 B against bank conflicts)
constexpr int kVtStride = kSub + 8;      // bf16 per LDS transposed-value row
constexpr int kPwStride = kSub + 8;      // bf16 per LDS probability row
constexpr int kQSteps = kDqk / 32;       // 18 MFMA k-steps for the scores
constexpr int kDTiles = kDv / 16;        // 32 output tiles of 16 dimensions
constexpr size_t kAttnLds = sizeof(uint16_t) * (static_cast<size_t>(kSub) * kKcStride +
                                                static_cast<size_t>(kDv) * kVtStride +
                                                4 * 16 * static_cast<size_t>(kPwStride)) +
                            sizeof(int) * kSub;

__device__ inline uint16_t f32_to_bf16_bits(float f) {
    // round to nearest even (finite inputs: probabilities in [0, 1])
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

__global__ __launch_bounds__(kAttnThreads) void mla_partial_kernel(StateBase s, int layer, const uint16_t* q,
                                                                   int H, const int32_t* slot_idx, int k,
                                                                   int chunk, float scale_log2, float* part_o,
                                                                   float* part_ml) {
    extern __shared__ __align__(16) uint16_t attn_lds[];
    uint16_t* Kc = attn_lds;                                  // [kSub][kKcStride]
    uint16_t* Vt = Kc + kSub * kKcStride;                     // [kDv][kVtStride]
    uint16_t* Pw = Vt + kDv * kVtStride;                      // [4 waves][16][kPwStride]
    int* rvalid = reinterpret_cast<int*>(Pw + 4 * 16 * kPwStride);  // [kSub]

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int c = blockIdx.x, g = blockIdx.y, r = blockIdx.z;
    const int nchunk = gridDim.x;
    const int h0 = g * kHeadsPerWG + wave * 16;               // this wave's first head
    const int row = lane & 15, grp = lane >> 4;               // MFMA fragment coordinates
    const int j_begin = c * chunk, j_end = min(k, j_begin + chunk);
    const int64_t rl = static_cast<int64_t>(layer) * s.R + r;
    const uint8_t* cache = s.cache + rl * s.B * s.row_bytes;
    const int32_t* sidx = slot_idx + static_cast<int64_t>(r) * k;
    uint16_t* Pme = Pw + wave * 16 * kPwStride;

    // query fragments of this wave's 16 heads, held for the whole chunk
    bf16x8 aq[kQSteps];
    {
        const uint16_t* qrow = q + (static_cast<int64_t>(r) * H + h0 + row) * kDqk + 8 * grp;
#pragma unroll
        for (int st = 0; st < kQSteps; ++st) aq[st] = *reinterpret_cast<const bf16x8*>(qrow + 32 * st);
    }

    f32x4 acc_o[kDTiles];
#pragma unroll
    for (int t = 0; t < kDTiles; ++t) acc_o[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run[4], l_run[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        m_run[i] = -INFINITY;
        l_run[i] = 0.f;
    }

    for (int j0 = j_begin; j0 < j_end; j0 += kSub) {
        // gather the sub-chunk's records: row-major into Kc, values transposed into Vt
        if (tid < kSub) {
            const int j = j0 + tid;
            const int slot = j < j_end ? sidx[j] : -1;
            rvalid[tid] = (slot >= 0 && slot < s.B) ? slot : -1;
        }
        __syncthreads();
        constexpr int kPieces = kSub * (kDqk / 8);            // 16-byte pieces per sub-chunk
        for (int p = tid; p < kPieces; p += kAttnThreads) {
            const int rec = p / (kDqk / 8), off = p - rec * (kDqk / 8);
            const int slot = rvalid[rec];
            uint4 v = make_uint4(0u, 0u, 0u, 0u);
            if (slot >= 0) v = *reinterpret_cast<const uint4*>(cache + static_cast<int64_t>(slot) * s.row_bytes + 16 * off);
            *reinterpret_cast<uint4*>(Kc + rec * kKcStride + 8 * off) = v;
            if (off < kDv / 8) {
                const uint16_t e[8] = {static_cast<uint16_t>(v.x), static_cast<uint16_t>(v.x >> 16),
                                       static_cast<uint16_t>(v.y), static_cast<uint16_t>(v.y >> 16),
                                       static_cast<uint16_t>(v.z), static_cast<uint16_t>(v.z >> 16),
                                       static_cast<uint16_t>(v.w), static_cast<uint16_t>(v.w >> 16)};
#pragma unroll
                for (int i = 0; i < 8; ++i) Vt[(8 * off + i) * kVtStride + rec] = e[i];
            }
        }
        __syncthreads();

        // S = Q K^T for 16 heads x 64 records (4 tiles of 16 records)
        f32x4 sacc[4];
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
            sacc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
            const uint16_t* brow = Kc + (16 * nt + row) * kKcStride + 8 * grp;
#pragma unroll
            for (int st = 0; st < kQSteps; ++st) {
                const bf16x8 b = *reinterpret_cast<const bf16x8*>(brow + 32 * st);
                sacc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aq[st], b, sacc[nt], 0, 0, 0);
            }
        }
        // online softmax; this lane holds heads 4*grp + i and record 16*nt + row
        float mloc[4], alpha[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float mx = -INFINITY;
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) {
                const bool ok = rvalid[16 * nt + row] >= 0;
                const float v = ok ? sacc[nt][i] * scale_log2 : -INFINITY;
                sacc[nt][i] = v;
                mx = fmaxf(mx, v);
            }
#pragma unroll
            for (int off = 1; off < 16; off <<= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
            mloc[i] = mx;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float m_new = fmaxf(m_run[i], mloc[i]);
            alpha[i] = (m_new == -INFINITY) ? 1.f : exp2f(m_run[i] - m_new);
            float sum = 0.f;
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) {
                const float pr = (m_new == -INFINITY) ? 0.f : exp2f(sacc[nt][i] - m_new);
                sacc[nt][i] = pr;
                sum += pr;
            }
#pragma unroll
            for (int off = 1; off < 16; off <<= 1) sum += __shfl_xor(sum, off, 64);
            l_run[i] = l_run[i] * alpha[i] + sum;
            m_run[i] = m_new;
        }
#pragma unroll
        for (int t = 0; t < kDTiles; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc_o[t][i] *= alpha[i];
        // probabilities to LDS as bf16, [head][record], for the A operand
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
#pragma unroll
            for (int i = 0; i < 4; ++i) Pme[(4 * grp + i) * kPwStride + 16 * nt + row] = f32_to_bf16_bits(sacc[nt][i]);
        __syncthreads();

        // O += P V: 16 heads x 512 dims, k = 64 records in two steps of 32
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const bf16x8 a = *reinterpret_cast<const bf16x8*>(Pme + row * kPwStride + 32 * ks + 8 * grp);
#pragma unroll
            for (int t = 0; t < kDTiles; ++t) {
                const bf16x8 b = *reinterpret_cast<const bf16x8*>(Vt + (16 * t + row) * kVtStride + 32 * ks + 8 * grp);
                acc_o[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc_o[t], 0, 0, 0);
            }
        }
        __syncthreads();  // Kc, Vt and Pw are refilled by the next sub-chunk
    }

    // partials: unnormalised O, running maximum and sum (log2 units)
    const int64_t base = ((static_cast<int64_t>(r) * nchunk + c) * H);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int h = h0 + 4 * grp + i;
        float* orow = part_o + (base + h) * kDv;
#pragma unroll
        for (int t = 0; t < kDTiles; ++t) orow[16 * t + row] = acc_o[t][i];
        if (row == 0) {
            part_ml[(base + h) * 2 + 0] = m_run[i];
            part_ml[(base + h) * 2 + 1] = l_run[i];
        }
    }
}

// Combine the chunks of each (request, head): out = sum_c w_c O_c / sum_c w_c l_c
// with w_c = 2^(m_c - max_c m_c); lse in natural-log units.
__global__ __launch_bounds__(kAttnThreads) void mla_combine_kernel(const float* part_o, const float* part_ml, int H,
                                                                   int nchunk, float* out, float* lse) {
    const int h = blockIdx.x, r = blockIdx.y;
    float M = -INFINITY;
    for (int c = 0; c < nchunk; ++c) M = fmaxf(M, part_ml[((static_cast<int64_t>(r) * nchunk + c) * H + h) * 2]);
    float denom = 0.f;
    for (int c = 0; c < nchunk; ++c) {
        const float* ml = part_ml + ((static_cast<int64_t>(r) * nchunk + c) * H + h) * 2;
        if (ml[0] != -INFINITY) denom += exp2f(ml[0] - M) * ml[1];
    }
    float* orow = out + (static_cast<int64_t>(r) * H + h) * kDv;
    for (int d = threadIdx.x; d < kDv; d += kAttnThreads) {
        float acc = 0.f;
        for (int c = 0; c < nchunk; ++c) {
            const int64_t idx = (static_cast<int64_t>(r) * nchunk + c) * H + h;
            const float m = part_ml[idx * 2];
            if (m != -INFINITY) acc += exp2f(m - M) * part_o[idx * kDv + d];
        }
        orow[d] = denom > 0.f ? acc / denom : 0.f;
    }
    if (threadIdx.x == 0 && lse)
        lse[static_cast<int64_t>(r) * H + h] = denom > 0.f ? (M + log2f(denom)) * 0.69314718055994530942f : -INFINITY;
}

}  // namespace

size_t attend_workspace_floats(int R, int H, int nchunk) {
    return static_cast<size_t>(R) * nchunk * H * (kDv + 2);
}

int attend_chunk(int R, int H, int k) {
    // enough workgroups to cover the chip (about 256), in multiples of the sub-chunk
    const int64_t per = (static_cast<int64_t>(k) * R * (H / kHeadsPerWG) + 255) / 256;
    int chunk = static_cast<int>(((per + kSub - 1) / kSub) * kSub);
    if (chunk < kSub) chunk = kSub;
    if (chunk > k) chunk = ((k + kSub - 1) / kSub) * kSub;
    return chunk;
}

hipError_t launch_attend_mla(const StateBase& s, int layer, const uint16_t* q, int H, const int32_t* slot_idx, int k,
                             float scale, float* out, float* lse, float* workspace, int chunk, hipStream_t st) {
    const int nchunk = (k + chunk - 1) / chunk;
    float* part_o = workspace;
    float* part_ml = workspace + static_cast<size_t>(s.R) * nchunk * H * kDv;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&mla_partial_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(kAttnLds));
    if (e != hipSuccess) return e;
    const float scale_log2 = scale * 1.44269504088896340736f;
    hipLaunchKernelGGL(mla_partial_kernel, dim3(nchunk, H / kHeadsPerWG, s.R), dim3(kAttnThreads), kAttnLds, st, s,
                       layer, q, H, slot_idx, k, chunk, scale_log2, part_o, part_ml);
    hipLaunchKernelGGL(mla_combine_kernel, dim3(H, s.R), dim3(kAttnThreads), 0, st, part_o, part_ml, H, nchunk, out,
                       lse);
    return hipGetLastError();
}

}  // namespace hs
