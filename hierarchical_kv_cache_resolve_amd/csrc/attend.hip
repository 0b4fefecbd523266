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
// Work split (flash-decoding): workgroup = (request, 32 or 64 heads, a chunk
// of records); 4 wave64s at 32 heads, 8 at 64.  Records move HBM -> LDS with
// global_load_lds (16 bytes a lane, no registers), 64 records per sub-chunk
// into one of two LDS buffers, so the loads of sub-chunk i+1 are in flight
// while sub-chunk i is computed.
//
// LDS buffer layout: [9 lines][64 records][8 slots of 16 B]; line L of a
// record is its bytes 128L..128L+127 (one HBM cache line) and slot j holds
// piece 8L + (j ^ swz(rec)).  One global_load_lds moves whole lines of 8
// records (8 lanes a line, so every access is a full coalesced line), a lane
// loads the same record(s) for the whole sub-chunk, and the XOR swizzle
// keeps both operand reads below free of bank conflicts:
//   scores  wave w: S^T = K Q^T for one tile of 16 heads over 32 of the
//           sub-chunk's 64 records (two waves share a tile)
//           (v_mfma_f32_16x16x32_bf16, K from
//           LDS, Q fragments in registers); online softmax; the
//           probabilities go to LDS as bf16 MFMA fragments;
//   output  wave w: O^T = V^T P^T for output dimensions 512w/W.. (W waves) of all
//           the workgroup's heads; V^T comes from the gfx950 transposing LDS read
//           (ds_read_b64_tr_b16, the costliest LDS access here, so each wave
//           reads only its share of the values), P^T fragments from LDS.
// The record order inside each 32-wide k-step is permuted identically on
// both operands of O^T = V^T P^T, so the probability fragments are written
// exactly as the score registers hold them.  A lane of the score phase owns
// one head: running maximum and sum are per lane (log2 units) and reduce over
// the 4 lanes holding the same head (and, at 32 heads, over the two waves
// sharing the head, through LDS).  A chunk's output goes out normalised by
// its own sum, in fp16 (its values are weighted means of bf16 records, well
// inside fp16's range; rounding adds at most 2^-11 of sum_j p_j |v_j| to the
// error, next to 2^-9 from the bf16 probabilities), with its maximum and sum
// in fp32; a second kernel combines the chunks of each (request, head).
#include "hs_internal.h"

namespace hs {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int kMaxHeadTiles = 4;               // a workgroup takes 2 or 4 tiles of 16 heads
constexpr int kSub = 64;                       // records per LDS sub-chunk
constexpr int kDqk = 576, kDv = 512;
constexpr int kRecBytes = kDqk * 2;            // 1152
constexpr int kRecPieces = kRecBytes / 16;     // 72 pieces of 16 bytes
constexpr int kLines = kRecBytes / 128;        // 9 lines of 128 bytes a record
constexpr int kLineBlock = kSub * 128;         // 8 KB: one line of every record
constexpr int kBufBytes = kLines * kLineBlock; // 73728 per buffer
constexpr int kQSteps = kDqk / 32;             // 18 MFMA k-steps for the scores
constexpr int kPBytes = kMaxHeadTiles * 2 * 1024;   // P fragments: [head tile][k-step][64 lanes][16 B]
constexpr int kXBytes = 2 * 16 * kMaxHeadTiles * 4;  // [record half][head] partial maxima / sums
constexpr size_t kAttnLds =
    2 * static_cast<size_t>(kBufBytes) + kPBytes + 16 * kMaxHeadTiles * sizeof(float) + kXBytes;
// s_waitcnt immediate (gfx9 encoding) waiting for vmcnt == 0 only:
// vmcnt 0 (bits 3:0, 15:14), expcnt 7 (bits 6:4), lgkmcnt 15 (bits 11:8)
constexpr int kWaitVmcnt0 = 0x0F70;
constexpr float kRescaleSlack = 8.f;           // log2 units
constexpr int kSDepth = 2;                     // score k-steps read ahead
constexpr int kVDepth = 3;                     // value tiles read ahead

// a record of zeros: the source of every record left out (slot -1)
__device__ __align__(16) uint4 g_zero_record[kRecPieces];

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    // round to nearest even (finite inputs: probabilities in [0, 1])
    uint32_t ua = __float_as_uint(a), ub = __float_as_uint(b);
    ua += 0x7FFFu + ((ua >> 16) & 1u);
    ub += 0x7FFFu + ((ub >> 16) & 1u);
    return (ua >> 16) | (ub & 0xFFFF0000u);
}

// slot of piece p%8 inside line p/8 of LDS record rec is (p%8) ^ swz(rec).
// swz maps record bits {1,2,3} onto slot bits {1,2,0}: 16 consecutive
// records read at one piece, and 4 + 4 records read at two adjacent pieces,
// land on distinct 16-byte bank groups.
__device__ __forceinline__ int swz(int rec) { return (rec & 6) | ((rec >> 3) & 1); }

// This wave's share of one sub-chunk, HBM -> LDS: NR groups of 8 records
// (records 8NR·w .. 8NR·w + 8NR - 1; NR = 2 with 4 waves, 1 with 8), all 9
// lines (9·NR instructions of 1 KB).  src[h] points at this lane's piece of
// line 0 of record 8NR·w + 8h + lane/8.  The loads are issued as inline
// assembly on purpose: the compiler would otherwise guard the transposing LDS
// reads of the other buffer with a full vmcnt wait (it cannot tell the
// buffers apart), serialising loads and compute.  Their completion is waited
// for explicitly before the barrier that publishes a buffer.
template <int NR>
__device__ __forceinline__ void issue_records(uint8_t* buf, const uint8_t* const (&src)[NR], int wave) {
#pragma unroll
    for (int L = 0; L < kLines; ++L) {
#pragma unroll
        for (int h = 0; h < NR; ++h) {
            const uint8_t* dst = buf + L * kLineBlock + (NR * wave + h) * 1024;
            const uint32_t lds_addr = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void*)dst));
            // M0 carries the LDS destination; its previous value is restored
            uint32_t m0_saved;
            asm volatile(
                "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %2, off\n\ts_mov_b32 m0, %0"
                : "=&s"(m0_saved)
                : "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "v"(src[h] + 128 * L)
                : "memory");
        }
    }
}

// HT: head tiles of 16 per workgroup; W: waves per workgroup (4 or 8, one
// workgroup per CU either way).  The score phase spreads the HT tiles over
// the W waves: RS = W / HT waves share a tile, each taking 64 / RS of the
// sub-chunk's records (TPW score tiles of 16 records) and exchanging its
// partial maximum through LDS; the value phase gives each wave 512 / W output
// dimensions of every head.  HT = 2 halves the partial outputs per record
// read, which pays when the split over records is deep (few requests); HT = 4
// reads each record into fewer workgroups and runs 8 waves, so that two
// waves share each SIMD and hide each other's LDS and memory waits.
template <int HT, int W>
__global__ __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu(W / 4, W / 4)))
void mla_partial_kernel(StateBase s, int layer, const uint16_t* q, int H, const int32_t* slot_idx, int k, int chunk,
                        int nchunk, float scale_log2, _Float16* part_o, float* part_ml) {
    constexpr int HPW = 16 * HT;         // heads per workgroup
    constexpr int RS = W / HT;           // waves sharing a head tile in the score phase
    constexpr int TPW = 4 / RS;          // score tiles (of 16 records) per wave
    constexpr int NR = 8 / W;            // groups of 8 records each lane loads
    constexpr int kDimsPerWave = kDv / W;
    constexpr int kWaveDTiles = kDimsPerWave / 16;
    static_assert((W == 4 || W == 8) && TPW >= 2 && TPW % 2 == 0, "each wave owns whole k-steps of P");
    extern __shared__ __align__(16) uint8_t attn_lds[];
    uint8_t* pfrag = attn_lds + 2 * kBufBytes;                          // [HT][2][64][16 B]
    float* alpha_lds = reinterpret_cast<float*>(pfrag + kPBytes);       // [HPW] rescale of each head
    float* xchg = alpha_lds + 16 * kMaxHeadTiles;                       // [RS][HPW] per record share

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 15, grp = lane >> 4;                 // MFMA fragment coordinates
    // workgroup -> (chunk, head group, request); when the grid divides into the
    // 8 XCDs, consecutive tiles (the head groups of one chunk) share an XCD and
    // so its L2
    const int G = H / HPW;
    const int nwg = gridDim.x;
    int T = blockIdx.x;
    if ((nwg & 7) == 0) T = (T & 7) * (nwg >> 3) + (T >> 3);
    const int g = T % G, c = (T / G) % nchunk, r = T / (G * nchunk);
    // score phase: wave w takes head tile w % HT and record share w / HT of each
    // sub-chunk (score tiles rh*TPW .. rh*TPW + TPW - 1)
    const int hts = wave % HT, rh = wave / HT;
    const int h0 = g * HPW + hts * 16;                        // first head of this wave's scores
    const int j_begin = c * chunk, j_end = min(k, j_begin + chunk);
    const int nsub = (j_end - j_begin + kSub - 1) / kSub;
    const int64_t rl = static_cast<int64_t>(layer) * s.R + r;
    const uint8_t* cache = s.cache + rl * s.B * s.row_bytes;
    const int32_t* sidx = slot_idx + static_cast<int64_t>(r) * k;

    // slot of record i of sub-chunk `sub`: the raw load (index clamped into the
    // chunk, so it can be issued early and unconditionally), then the check
    auto raw_slot = [&](int sub, int i) -> int { return sidx[min(j_begin + sub * kSub + i, j_end - 1)]; };
    auto checked = [&](int sub, int i, int v) -> int {
        return (j_begin + sub * kSub + i < j_end && v >= 0 && v < s.B) ? v : -1;
    };
    // the two records this lane loads, and its piece slot inside each line
    int rec[NR], poff[NR];
#pragma unroll
    for (int h = 0; h < NR; ++h) {
        rec[h] = 8 * NR * wave + 8 * h + (lane >> 3);
        poff[h] = 16 * ((lane & 7) ^ swz(rec[h]));
    }
    auto record_src = [&](int slot, int piece_off) -> const uint8_t* {
        return (slot >= 0 ? cache + static_cast<int64_t>(slot) * kRecBytes
                          : reinterpret_cast<const uint8_t*>(g_zero_record)) + piece_off;
    };
    {
        const uint8_t* src[NR];
#pragma unroll
        for (int h = 0; h < NR; ++h) src[h] = record_src(checked(0, rec[h], raw_slot(0, rec[h])), poff[h]);
        issue_records<NR>(attn_lds, src, wave);
    }
    // slots are read one sub-chunk ahead of their use: `mk_*` names record
    // `lane` (validity mask), `la_*` / `lb_*` the records this lane loads
    int mk_cur = raw_slot(0, lane);
    int slot_nxt[NR];
#pragma unroll
    for (int h = 0; h < NR; ++h) slot_nxt[h] = raw_slot(1, rec[h]);
    int mk_nxt = raw_slot(1, lane);

    // query fragments of this wave's 16 heads (B operand of S^T = K Q^T)
    bf16x8 aq[kQSteps];
    {
        const uint16_t* qrow = q + (static_cast<int64_t>(r) * H + h0 + n) * kDqk + 8 * grp;
#pragma unroll
        for (int st = 0; st < kQSteps; ++st) aq[st] = *reinterpret_cast<const bf16x8*>(qrow + 32 * st);
    }
    // output accumulators: dimension tile dt (dims kDimsPerWave·w + 16dt ..) x head tile ht;
    // lane (grp, n) holds dims +4grp+i of head 16ht + n
    f32x4 acc_o[kWaveDTiles][HT];
#pragma unroll
    for (int dt = 0; dt < kWaveDTiles; ++dt)
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) acc_o[dt][ht] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;

    // per-lane LDS offsets of the two operand reads (the rest are immediates)
    //   score read: record 16nt + n, piece 4st + grp = line st/2, slot
    //   (4(st&1) + grp) ^ swz(n)
    const int s_even = 128 * n + 16 * (grp ^ swz(n));
    const int s_odd = 128 * n + 16 * ((4 + grp) ^ swz(n));
    //   transposing read: lane (grp, e, qq) points at dims 4qq..4qq+3 of record
    //   32ks + 16hi + 4grp + e, i.e. piece 2t + (qq >> 1) = line t/4, slot
    //   (2(t&3) + (qq>>1)) ^ swz = 2(t&3) ^ gv, half qq & 1
    const int e = n >> 2, qq = n & 3;
    const int gv = (qq >> 1) ^ swz(4 * grp + e);
    // (this wave's dimension tiles are t = kWaveDTiles·w + dt, so t & 3 = dt & 3)
    const int v_base = 128 * (4 * grp + e) + 8 * (qq & 1);
    const int v_off[4] = {v_base + 16 * (0 ^ gv), v_base + 16 * (2 ^ gv), v_base + 16 * (4 ^ gv),
                          v_base + 16 * (6 ^ gv)};

    for (int sub = 0; sub < nsub; ++sub) {
        uint8_t* buf = attn_lds + (sub & 1) * kBufBytes;
        // vmcnt(0): this wave's record loads (and everything else) have landed;
        // the builtin form lets the compiler know no load is outstanding
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
        __syncthreads();                          // sub-chunk `sub` is in LDS
        const uint64_t valid = __ballot(checked(sub, lane, mk_cur) >= 0);
        if (sub + 1 < nsub) {
            const uint8_t* src[NR];
#pragma unroll
            for (int h = 0; h < NR; ++h) src[h] = record_src(checked(sub + 1, rec[h], slot_nxt[h]), poff[h]);
            issue_records<NR>(attn_lds + ((sub + 1) & 1) * kBufBytes, src, wave);
        }
        mk_cur = mk_nxt;
#pragma unroll
        for (int h = 0; h < NR; ++h) slot_nxt[h] = raw_slot(sub + 2, rec[h]);
        mk_nxt = raw_slot(sub + 2, lane);

        // S^T = K Q^T: tile nt covers records 16nt..16nt+15; this lane ends with
        // head h0+n against records 16nt + 4grp + i
        // Software-pipelined: the fragments of step st + kSDepth are read while
        // step st multiplies; sched_barrier keeps the compiler from undoing it.
        auto k_frag = [&](int st, int nt) -> bf16x8 {
            return *reinterpret_cast<const bf16x8*>(buf + ((st & 1) ? s_odd : s_even) + (st >> 1) * kLineBlock +
                                                    2048 * nt);
        };
        f32x4 sacc[TPW];                          // tiles nt = rh*TPW + u
        bf16x8 kf[kSDepth + 1][TPW];
#pragma unroll
        for (int u = 0; u < TPW; ++u) sacc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int d = 0; d < kSDepth; ++d)
#pragma unroll
            for (int u = 0; u < TPW; ++u) kf[d][u] = k_frag(d, rh * TPW + u);
#pragma unroll
        for (int st = 0; st < kQSteps; ++st) {
            if (st + kSDepth < kQSteps) {
#pragma unroll
                for (int u = 0; u < TPW; ++u)
                    kf[(st + kSDepth) % (kSDepth + 1)][u] = k_frag(st + kSDepth, rh * TPW + u);
            }
#pragma unroll
            for (int u = 0; u < TPW; ++u)
                sacc[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[st % (kSDepth + 1)][u], aq[st], sacc[u], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
        // online softmax for head h0+n over the sub-chunk's 64 records, with a
        // lazily moved reference: probabilities are 2^(s - m_ref), and m_ref is
        // raised (rescaling the accumulators) only when some lane of the wave
        // sees a score above m_ref + kRescaleSlack.  Probabilities stay below
        // 2^kRescaleSlack, so nothing overflows; the final normalisation by the
        // running sum makes the result independent of m_ref.
        float mx = -INFINITY;
#pragma unroll
        for (int u = 0; u < TPW; ++u)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const bool ok = (valid >> (16 * (rh * TPW + u) + 4 * grp + i)) & 1ull;
                const float v = ok ? sacc[u][i] * scale_log2 : -INFINITY;
                sacc[u][i] = v;
                mx = fmaxf(mx, v);
            }
        mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        if constexpr (RS > 1) {
            // the waves of a head tile see different records: all take the
            // maximum over the 64, so all move the reference identically
            if (grp == 0) xchg[rh * HPW + hts * 16 + n] = mx;
            __syncthreads();
#pragma unroll
            for (int o = 0; o < RS; ++o)
                if (o != rh) mx = fmaxf(mx, xchg[o * HPW + hts * 16 + n]);
        }
        float alpha = 1.f;
        if (__builtin_amdgcn_read_exec() & __ballot(mx > m_run + kRescaleSlack)) {   // wave-uniform
            const float m_new = fmaxf(m_run, mx);
            alpha = (m_new == -INFINITY) ? 1.f : exp2f(m_run - m_new);
            l_run *= alpha;
            m_run = m_new;
        }
        float sum = 0.f;
#pragma unroll
        for (int u = 0; u < TPW; ++u)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float pr = (m_run == -INFINITY) ? 0.f : exp2f(sacc[u][i] - m_run);
                sacc[u][i] = pr;
                sum += pr;
            }
        sum += __shfl_xor(sum, 16, 64);
        sum += __shfl_xor(sum, 32, 64);
        l_run += sum;                             // this record share's part; the shares add at the end
        // publish: P fragments of this head tile for the k-steps its tiles cover
        // (k-step ks takes records 32ks + 4grp + i and 32ks + 16 + 4grp + i,
        // i < 4: the score registers of tiles 2ks and 2ks+1) and the rescale
        // factor of each head
#pragma unroll
        for (int kl = 0; kl < TPW / 2; ++kl) {
            const int ks = rh * (TPW / 2) + kl;
            const uint32_t w4[4] = {pack_bf16x2(sacc[2 * kl][0], sacc[2 * kl][1]),
                                    pack_bf16x2(sacc[2 * kl][2], sacc[2 * kl][3]),
                                    pack_bf16x2(sacc[2 * kl + 1][0], sacc[2 * kl + 1][1]),
                                    pack_bf16x2(sacc[2 * kl + 1][2], sacc[2 * kl + 1][3])};
            *reinterpret_cast<uint4*>(pfrag + ((hts * 2 + ks) * 64 + lane) * 16) =
                make_uint4(w4[0], w4[1], w4[2], w4[3]);
        }
        if (grp == 0 && rh == 0) alpha_lds[hts * 16 + n] = alpha;
        __syncthreads();                          // P and the rescale factors are visible

        // rescale this wave's accumulators where a score phase moved its reference
        float a_ht[HT];
        bool moved = false;
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) {
            a_ht[ht] = alpha_lds[ht * 16 + n];
            moved |= a_ht[ht] != 1.f;
        }
        if (sub > 0 && (__builtin_amdgcn_read_exec() & __ballot(moved))) {
#pragma unroll
            for (int dt = 0; dt < kWaveDTiles; ++dt)
#pragma unroll
                for (int ht = 0; ht < HT; ++ht) acc_o[dt][ht] *= a_ht[ht];
        }

        // O^T += V^T P^T for dims kDimsPerWave·w.. of the workgroup's heads
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            bf16x8 pf[HT];
#pragma unroll
            for (int ht = 0; ht < HT; ++ht)
                pf[ht] = *reinterpret_cast<const bf16x8*>(pfrag + ((ht * 2 + ks) * 64 + lane) * 16);
            const uint8_t* vb = buf + 4096 * ks + (wave * kWaveDTiles / 4) * kLineBlock;
            auto v_frag = [&](int dt) -> bf16x8 {
                const uint8_t* va = vb + v_off[dt & 3] + (dt >> 2) * kLineBlock;
                const s16x4 vv[2] = {__builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)va),
                                     __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(va + 2048))};
                return *reinterpret_cast<const bf16x8*>(vv);
            };
            bf16x8 vf[kVDepth + 1];
#pragma unroll
            for (int d = 0; d < kVDepth; ++d) vf[d] = v_frag(d);
#pragma unroll
            for (int dt = 0; dt < kWaveDTiles; ++dt) {
                if (dt + kVDepth < kWaveDTiles) vf[(dt + kVDepth) % (kVDepth + 1)] = v_frag(dt + kVDepth);
#pragma unroll
                for (int ht = 0; ht < HT; ++ht)
                    acc_o[dt][ht] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[dt % (kVDepth + 1)], pf[ht],
                                                                            acc_o[dt][ht], 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        // no barrier here: the next sub-chunk's first barrier (before any wave
        // issues loads into this buffer or rewrites P) orders it
    }

    // partials: O normalised by the chunk's sum (fp16), running maximum and
    // sum (log2 units, fp32).  The running sum of each head is split over its
    // record shares: the shares add first (this barrier also orders every
    // wave's last reads of the rescale factors before they are overwritten).
    float l_tot = l_run;
    if constexpr (RS > 1) {
        if (grp == 0 && rh > 0) xchg[(rh - 1) * HPW + hts * 16 + n] = l_run;
        __syncthreads();
#pragma unroll
        for (int o = 1; o < RS; ++o) l_tot += xchg[(o - 1) * HPW + hts * 16 + n];
    } else {
        __syncthreads();
    }
    const int64_t hbase = (static_cast<int64_t>(r) * nchunk + c) * H + g * HPW;
    if (grp == 0 && rh == 0) {
        part_ml[(hbase + hts * 16 + n) * 2 + 0] = m_run;
        part_ml[(hbase + hts * 16 + n) * 2 + 1] = l_tot;
        alpha_lds[hts * 16 + n] = l_tot;
    }
    __syncthreads();
    // lane (grp, n) holds dims kDimsPerWave·w + 16dt + 4grp + i of head 16ht + n
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
        const float l = alpha_lds[ht * 16 + n];
        const float inv = l > 0.f ? 1.f / l : 0.f;
        _Float16* orow = part_o + (hbase + ht * 16 + n) * kDv + wave * kDimsPerWave + 4 * grp;
#pragma unroll
        for (int dt = 0; dt < kWaveDTiles; ++dt)
            *reinterpret_cast<f16x4*>(orow + 16 * dt) = __builtin_convertvector(acc_o[dt][ht] * inv, f16x4);
    }
}

// Combine the chunks of each (request, head): out = sum_c w_c l_c o_c /
// sum_c w_c l_c with w_c = 2^(m_c - max_c m_c) and o_c the chunk's normalised
// output; lse in natural-log units.  128 lanes, four dimensions each; the
// partial loads of up to kCombineBatch chunks are all issued before any is
// used.
constexpr int kCombineThreads = kDv / 4;
constexpr int kCombineBatch = 8;

__global__ __launch_bounds__(kCombineThreads) void mla_combine_kernel(const _Float16* part_o, const float* part_ml,
                                                                      int H, int nchunk, float* out, float* lse) {
    const int h = blockIdx.x, r = blockIdx.y;
    const int64_t first = static_cast<int64_t>(r) * nchunk * H + h;   // chunk c at first + c * H
    float M = -INFINITY;
    for (int c = 0; c < nchunk; ++c) M = fmaxf(M, part_ml[(first + static_cast<int64_t>(c) * H) * 2]);
    float denom = 0.f;
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int c0 = 0; c0 < nchunk; c0 += kCombineBatch) {
        f16x4 o[kCombineBatch];
        float wgt[kCombineBatch];
#pragma unroll
        for (int u = 0; u < kCombineBatch; ++u) {
            const int c = min(c0 + u, nchunk - 1);
            const int64_t idx = first + static_cast<int64_t>(c) * H;
            o[u] = *reinterpret_cast<const f16x4*>(part_o + idx * kDv + 4 * threadIdx.x);
            const float m = part_ml[idx * 2];
            wgt[u] = (c0 + u < nchunk && m != -INFINITY) ? exp2f(m - M) * part_ml[idx * 2 + 1] : 0.f;
            denom += wgt[u];
        }
#pragma unroll
        for (int u = 0; u < kCombineBatch; ++u)
            if (wgt[u] != 0.f) acc += wgt[u] * __builtin_convertvector(o[u], f32x4);
    }
    const float inv = denom > 0.f ? 1.f / denom : 0.f;
    *reinterpret_cast<f32x4*>(out + (static_cast<int64_t>(r) * H + h) * kDv + 4 * threadIdx.x) = acc * inv;
    if (threadIdx.x == 0 && lse)
        lse[static_cast<int64_t>(r) * H + h] = denom > 0.f ? (M + log2f(denom)) * 0.69314718055994530942f : -INFINITY;
}

}  // namespace

size_t attend_workspace_floats(int R, int H, int nchunk) {
    // fp16 outputs (kDv halves) and fp32 maximum and sum per (request, chunk, head)
    return static_cast<size_t>(R) * nchunk * H * (kDv / 2 + 2);
}

int attend_chunk(int R, int H, int k, int ht) {
    // enough workgroups to cover the chip (about 256), in multiples of the sub-chunk
    const int64_t per = (static_cast<int64_t>(k) * R * (H / (16 * ht)) + 255) / 256;
    int chunk = static_cast<int>(((per + kSub - 1) / kSub) * kSub);
    if (chunk < kSub) chunk = kSub;
    if (chunk > k) chunk = ((k + kSub - 1) / kSub) * kSub;
    return chunk;
}

int attend_head_tiles(int R, int H, int k) {
    // 64 heads per workgroup read each record into the fewest workgroups; when
    // that leaves few records per workgroup, so that the split over records is
    // deep (sixteen chunks or more), the fp32 partials it writes and reads back
    // cost more than the extra record reads of 32 heads per workgroup
    const int c4 = attend_chunk(R, H, k, 4);
    return (k + c4 - 1) / c4 >= 16 ? 2 : 4;
}

hipError_t launch_attend_mla(const StateBase& s, int layer, const uint16_t* q, int H, const int32_t* slot_idx, int k,
                             float scale, float* out, float* lse, float* workspace, int ht, int chunk,
                             hipStream_t st) {
    if (ht != 2 && ht != 4) return hipErrorInvalidValue;
    const int nchunk = (k + chunk - 1) / chunk;
    _Float16* part_o = reinterpret_cast<_Float16*>(workspace);
    float* part_ml = workspace + static_cast<size_t>(s.R) * nchunk * H * (kDv / 2);
    const void* fn = ht == 2 ? reinterpret_cast<const void*>(&mla_partial_kernel<2, 4>)
                             : reinterpret_cast<const void*>(&mla_partial_kernel<4, 8>);
    static LdsGrants granted[2];  // one per kernel instance
    const hipError_t e = ensure_lds_limit(fn, kAttnLds, granted[ht / 4]);
    if (e != hipSuccess) return e;
    const float scale_log2 = scale * 1.44269504088896340736f;
    const int nwg = nchunk * (H / (16 * ht)) * s.R;
    if (ht == 2)
        hipLaunchKernelGGL((mla_partial_kernel<2, 4>), dim3(nwg), dim3(256), kAttnLds, st, s, layer, q, H, slot_idx, k,
                           chunk, nchunk, scale_log2, part_o, part_ml);
    else
        hipLaunchKernelGGL((mla_partial_kernel<4, 8>), dim3(nwg), dim3(512), kAttnLds, st, s, layer, q, H, slot_idx, k,
                           chunk, nchunk, scale_log2, part_o, part_ml);
    hipLaunchKernelGGL(mla_combine_kernel, dim3(H, s.R), dim3(kCombineThreads), 0, st, part_o, part_ml, H, nchunk, out,
                       lse);
    return hipGetLastError();
}

}  // namespace hs
