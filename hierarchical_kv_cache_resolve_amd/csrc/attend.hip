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
// into one of two LDS buffers; the loads of sub-chunk i+1 go out one line at
// a time between the score steps of sub-chunk i, so they are in flight while
// it is computed and no wave stalls on a burst of them.  The workgroup's
// queries come in once, through the second buffer, before the first
// sub-chunk is computed.
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
// the 4 lanes holding the same head with gfx950's row swaps (and over the two
// waves sharing the head, through LDS).  A chunk's output goes out normalised
// by its own sum, in fp16 (its values are weighted means of bf16 records, well
// inside fp16's range; rounding adds at most 2^-11 of sum_j p_j |v_j| to the
// error, next to 2^-9 from the bf16 probabilities), in whole 1 KB rows staged
// through LDS, with its maximum and sum in fp32; a second kernel combines the
// chunks of each (request, head).  (The combine cannot ride on the last chunk
// to finish: making one workgroup's stores visible to another inside a launch
// takes an agent-scope release, an L2 write-back that costs far more here than
// the second launch.)
#include "hs_internal.h"

namespace hs {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
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
constexpr int kMaxShares = 2;                  // waves sharing a head group in the score phase
constexpr int kXBytes = kMaxShares * 16 * kMaxHeadTiles * 4;  // [record share][head] partial maxima / sums
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

// slot of piece p%8 inside line p/8 of LDS record rec is (p%8) ^ swz(rec).
// swz takes record bits 0..2, so it depends only on the record's place in
// its tile of 16, which the precomputed read offsets below rely on.  Both
// operand reads are then free of bank conflicts (bank-conflict counter of a
// probe replaying their lane addresses: a 16-byte score read takes 4 LDS
// cycles a wave, a transposing 8-byte value read 2; with record bits 1..3 the
// value read took 4, with bits {1,2,3} onto slot bits {1,2,0} the score read
// took 8).  Partial kernel at 16 requests x 128 heads, five interleaved runs
// on one box: 20.1 us against 20.5 with bits 1..3 (and 21.9 with bits
// {1,2,3} onto slot bits {1,2,0}, 25.4 with none, in an earlier comparison).
__device__ __forceinline__ int swz(int rec) { return rec & 7; }

// This wave's share of line L of one sub-chunk, HBM -> LDS: NR groups of 8
// records (records 8NR·w .. 8NR·w + 8NR - 1; NR = 2 with 4 waves, 1 with 8),
// NR instructions of 1 KB.  src[h] points at this lane's piece of line 0 of
// record 8NR·w + 8h + lane/8.  The loads are issued as inline assembly on
// purpose: the compiler would otherwise guard the transposing LDS reads of
// the other buffer with a full vmcnt wait (it cannot tell the buffers apart),
// serialising loads and compute.  Their completion is waited for explicitly
// before the barrier that publishes a buffer.
template <int NR>
__device__ __forceinline__ void issue_line(uint8_t* buf, const uint8_t* const (&src)[NR], int wave, int L) {
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

// all 9 lines of this wave's share
template <int NR>
__device__ __forceinline__ void issue_records(uint8_t* buf, const uint8_t* const (&src)[NR], int wave) {
#pragma unroll
    for (int L = 0; L < kLines; ++L) issue_line<NR>(buf, src, wave, L);
}

// Reductions over the four 16-lane rows of a wave (lanes n, n+16, n+32, n+48
// hold one head's values): gfx950's row swaps pair rows 0-1 and 2-3, then the
// two halves, without a trip through LDS.  Every lane ends with the same
// value, summed in the same order.
__device__ __forceinline__ float rows_max(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float rows_sum(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// HT: head tiles of 16 per workgroup; W: waves per workgroup (4 or 8, one
// workgroup per CU either way); HPWS: head tiles each wave scores.  The score
// phase splits the workgroup's HT tiles into HG = HT / HPWS groups; RS = W / HG
// waves share a group, each taking 64 / RS of the sub-chunk's records (TPW
// score tiles of 16 records) and exchanging its partial maximum through LDS.
// A wave reads each K fragment once for all HPWS of its head tiles, so the
// LDS traffic of the scores falls as HPWS grows, at HPWS x 72 registers of
// query fragments.  The value phase gives each wave 512 / W output dimensions
// of every head.  HT = 2 halves the partial outputs per record read, which
// pays when the split over records is deep (few requests); HT = 4 reads each
// record into fewer workgroups.
template <int HT, int W, int HPWS>
__global__ __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu(W / 4, W / 4)))
void mla_partial_kernel(int H, int k, int chunk, int nchunk, int layer, float scale_log2, const uint16_t* q,
                        const int32_t* slot_idx, _Float16* part_o, float* part_ml, float* out, float* lse,
                        StateBase s) {
    // (scalar arguments first: the build preloads the first 16 argument dwords
    // into scalar registers, so the workgroup's tile and addresses need no
    // round trip to the argument block; 24.6 against 25.0 us a call at 16
    // requests x 128 heads over five interleaved runs)
    constexpr int HPW = 16 * HT;         // heads per workgroup
    constexpr int HG = HT / HPWS;        // head-tile groups of the score phase
    constexpr int RS = W / HG;           // waves sharing a group in the score phase
    constexpr int TPW = 4 / RS;          // score tiles (of 16 records) per wave
    constexpr int NR = 8 / W;            // groups of 8 records each lane loads
    constexpr int kDimsPerWave = kDv / W;
    constexpr int kWaveDTiles = kDimsPerWave / 16;
    static_assert((W == 4 || W == 8) && HT % HPWS == 0 && W % HG == 0, "whole tiles per wave");
    static_assert(TPW >= 2 && TPW % 2 == 0 && RS <= kMaxShares, "each wave owns whole k-steps of P");
    static_assert(kQSteps == 2 * kLines, "one line of the next sub-chunk every second score step");
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
    // score phase: wave w takes head tiles t0 .. t0 + HPWS - 1 and record share
    // rh of each sub-chunk (score tiles rh*TPW .. rh*TPW + TPW - 1)
    const int hts = wave % HG, rh = wave / HG;
    const int t0 = hts * HPWS;
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
    // the records (rows) this lane loads, and its piece slot inside each line
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
        // sub-chunk 0 -> buffer 0, then the queries of the workgroup's heads ->
        // buffer 1 in the records' layout (row i = head g*HPW + i; rows past
        // HPW read the zero record)
        const uint8_t* src[NR];
#pragma unroll
        for (int h = 0; h < NR; ++h) src[h] = record_src(checked(0, rec[h], raw_slot(0, rec[h])), poff[h]);
        issue_records<NR>(attn_lds, src, wave);
#pragma unroll
        for (int h = 0; h < NR; ++h)
            src[h] = (rec[h] < HPW ? reinterpret_cast<const uint8_t*>(q + (static_cast<int64_t>(r) * H + g * HPW +
                                                                          rec[h]) * kDqk)
                                   : reinterpret_cast<const uint8_t*>(g_zero_record)) + poff[h];
        issue_records<NR>(attn_lds + kBufBytes, src, wave);
    }
    // slots are read one sub-chunk ahead of their use: `mk_*` names record
    // `lane` (validity mask), `slot_nxt` the records this lane loads
    int mk_cur = raw_slot(0, lane);
    int slot_nxt[NR];
#pragma unroll
    for (int h = 0; h < NR; ++h) slot_nxt[h] = raw_slot(1, rec[h]);
    int mk_nxt = raw_slot(1, lane);

    // per-lane LDS offsets of the two operand reads (the rest are immediates)
    //   score read: row 16nt + n, piece 4st + grp = line st/2, slot
    //   (4(st&1) + grp) ^ swz(n)
    const int s_even = 128 * n + 16 * (grp ^ swz(n));
    const int s_odd = 128 * n + 16 * ((4 + grp) ^ swz(n));
    auto frag = [&](const uint8_t* buf, int st, int nt) -> bf16x8 {
        return *reinterpret_cast<const bf16x8*>(buf + ((st & 1) ? s_odd : s_even) + (st >> 1) * kLineBlock +
                                                2048 * nt);
    };
    //   transposing read: lane (grp, e, qq) points at dims 4qq..4qq+3 of record
    //   32ks + 16hi + 4grp + e, i.e. piece 2t + (qq >> 1) = line t/4, slot
    //   (2(t&3) + (qq>>1)) ^ swz = 2(t&3) ^ gv, half qq & 1
    const int e = n >> 2, qq = n & 3;
    const int gv = (qq >> 1) ^ swz(4 * grp + e);
    // (this wave's dimension tiles are t = kWaveDTiles·w + dt, so t & 3 = dt & 3)
    const int v_base = 128 * (4 * grp + e) + 8 * (qq & 1);
    const int v_off[4] = {v_base + 16 * (0 ^ gv), v_base + 16 * (2 ^ gv), v_base + 16 * (4 ^ gv),
                          v_base + 16 * (6 ^ gv)};

    // query fragments of this wave's head tiles (B operand of S^T = K Q^T),
    // read from buffer 1 once the first loads have landed; the second barrier
    // lets the next sub-chunk reuse the buffer
    bf16x8 aq[HPWS][kQSteps];
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
#pragma unroll
    for (int p = 0; p < HPWS; ++p)
#pragma unroll
        for (int st = 0; st < kQSteps; ++st) aq[p][st] = frag(attn_lds + kBufBytes, st, t0 + p);
    __syncthreads();

    // output accumulators: dimension tile dt (dims kDimsPerWave·w + 16dt ..) x head tile ht;
    // lane (grp, n) holds dims +4grp+i of head 16ht + n
    f32x4 acc_o[kWaveDTiles][HT];
#pragma unroll
    for (int dt = 0; dt < kWaveDTiles; ++dt)
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) acc_o[dt][ht] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run[HPWS], l_run[HPWS];
#pragma unroll
    for (int p = 0; p < HPWS; ++p) {
        m_run[p] = -INFINITY;
        l_run[p] = 0.f;
    }

    for (int sub = 0; sub < nsub; ++sub) {
        uint8_t* buf = attn_lds + (sub & 1) * kBufBytes;
        if (sub > 0) {
            // vmcnt(0): this wave's record loads (and everything else) have landed;
            // the builtin form lets the compiler know no load is outstanding
            __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
            __syncthreads();                      // sub-chunk `sub` is in LDS
        }
        const uint64_t valid = __ballot(checked(sub, lane, mk_cur) >= 0);
        // the next sub-chunk's loads go out one line every second score step,
        // so that no wave stalls on a burst of them at the address unit
        const bool more = sub + 1 < nsub;
        uint8_t* nbuf = attn_lds + ((sub + 1) & 1) * kBufBytes;
        const uint8_t* nsrc[NR];
#pragma unroll
        for (int h = 0; h < NR; ++h) nsrc[h] = record_src(checked(sub + 1, rec[h], slot_nxt[h]), poff[h]);
        mk_cur = mk_nxt;
#pragma unroll
        for (int h = 0; h < NR; ++h) slot_nxt[h] = raw_slot(sub + 2, rec[h]);
        mk_nxt = raw_slot(sub + 2, lane);

        // S^T = K Q^T: tile nt covers records 16nt..16nt+15; this lane ends with
        // head 16(t0+p)+n against records 16nt + 4grp + i.
        // Software-pipelined: the fragments of step st + kSDepth are read while
        // step st multiplies; sched_barrier keeps the compiler from undoing it.
        f32x4 sacc[HPWS][TPW];                    // tiles nt = rh*TPW + u
        bf16x8 kf[kSDepth + 1][TPW];
#pragma unroll
        for (int p = 0; p < HPWS; ++p)
#pragma unroll
            for (int u = 0; u < TPW; ++u) sacc[p][u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int d = 0; d < kSDepth; ++d)
#pragma unroll
            for (int u = 0; u < TPW; ++u) kf[d][u] = frag(buf, d, rh * TPW + u);
#pragma unroll
        for (int st = 0; st < kQSteps; ++st) {
            if (more && (st & 1) == 0) issue_line<NR>(nbuf, nsrc, wave, st >> 1);
            if (st + kSDepth < kQSteps) {
#pragma unroll
                for (int u = 0; u < TPW; ++u)
                    kf[(st + kSDepth) % (kSDepth + 1)][u] = frag(buf, st + kSDepth, rh * TPW + u);
            }
#pragma unroll
            for (int p = 0; p < HPWS; ++p)
#pragma unroll
                for (int u = 0; u < TPW; ++u)
                    sacc[p][u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[st % (kSDepth + 1)][u], aq[p][st],
                                                                         sacc[p][u], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
        // online softmax for each head over the sub-chunk's 64 records, with a
        // lazily moved reference: probabilities are 2^(s - m_ref), and m_ref is
        // raised (rescaling the accumulators) only when some lane of the wave
        // sees a score above m_ref + kRescaleSlack.  Probabilities stay below
        // 2^kRescaleSlack, so nothing overflows; the final normalisation by the
        // running sum makes the result independent of m_ref.  Records left out
        // score -inf; a sub-chunk without any (the usual case) skips the mask.
        float mx[HPWS];
#pragma unroll
        for (int p = 0; p < HPWS; ++p) {
            mx[p] = -INFINITY;
#pragma unroll
            for (int u = 0; u < TPW; ++u)
#pragma unroll
                for (int i = 0; i < 4; ++i) sacc[p][u][i] *= scale_log2;
        }
        if (valid != ~0ull) {
#pragma unroll
            for (int u = 0; u < TPW; ++u)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const bool ok = (valid >> (16 * (rh * TPW + u) + 4 * grp + i)) & 1ull;
#pragma unroll
                    for (int p = 0; p < HPWS; ++p) sacc[p][u][i] = ok ? sacc[p][u][i] : -INFINITY;
                }
        }
#pragma unroll
        for (int p = 0; p < HPWS; ++p) {
#pragma unroll
            for (int u = 0; u < TPW; ++u)
#pragma unroll
                for (int i = 0; i < 4; ++i) mx[p] = fmaxf(mx[p], sacc[p][u][i]);
            mx[p] = rows_max(mx[p]);
        }
        if constexpr (RS > 1) {
            // the waves of a head group see different records: all take the
            // maximum over the 64, so all move the reference identically
            if (grp == 0) {
#pragma unroll
                for (int p = 0; p < HPWS; ++p) xchg[rh * HPW + (t0 + p) * 16 + n] = mx[p];
            }
            __syncthreads();
#pragma unroll
            for (int o = 0; o < RS; ++o)
                if (o != rh) {
#pragma unroll
                    for (int p = 0; p < HPWS; ++p) mx[p] = fmaxf(mx[p], xchg[o * HPW + (t0 + p) * 16 + n]);
                }
        }
        float alpha[HPWS];
#pragma unroll
        for (int p = 0; p < HPWS; ++p) {
            alpha[p] = 1.f;
            if (__builtin_amdgcn_read_exec() & __ballot(mx[p] > m_run[p] + kRescaleSlack)) {   // wave-uniform
                const float m_new = fmaxf(m_run[p], mx[p]);
                alpha[p] = (m_new == -INFINITY) ? 1.f : exp2f(m_run[p] - m_new);
                l_run[p] *= alpha[p];
                m_run[p] = m_new;
            }
            // a head with no score yet keeps m_ref = -inf and all its scores are
            // -inf: exp2(-inf - 0) = 0
            const float m_use = (m_run[p] == -INFINITY) ? 0.f : m_run[p];
            float sum = 0.f;
#pragma unroll
            for (int u = 0; u < TPW; ++u)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float pr = exp2f(sacc[p][u][i] - m_use);
                    sacc[p][u][i] = pr;
                    sum += pr;
                }
            l_run[p] += rows_sum(sum);            // this record share's part; the shares add at the end
            // publish: P fragments of head tile t0+p for the k-steps its tiles
            // cover (k-step ks takes records 32ks + 4grp + i and 32ks + 16 +
            // 4grp + i, i < 4: the score registers of tiles 2ks and 2ks+1),
            // rounded to bf16 (nearest even) by the gfx950 pack
#pragma unroll
            for (int kl = 0; kl < TPW / 2; ++kl) {
                const int ks = rh * (TPW / 2) + kl;
                const bf16x2 w4[4] = {
                    __builtin_convertvector(f32x2{sacc[p][2 * kl][0], sacc[p][2 * kl][1]}, bf16x2),
                    __builtin_convertvector(f32x2{sacc[p][2 * kl][2], sacc[p][2 * kl][3]}, bf16x2),
                    __builtin_convertvector(f32x2{sacc[p][2 * kl + 1][0], sacc[p][2 * kl + 1][1]}, bf16x2),
                    __builtin_convertvector(f32x2{sacc[p][2 * kl + 1][2], sacc[p][2 * kl + 1][3]}, bf16x2)};
                *reinterpret_cast<uint4*>(pfrag + (((t0 + p) * 2 + ks) * 64 + lane) * 16) =
                    *reinterpret_cast<const uint4*>(w4);
            }
            if (grp == 0 && rh == 0) alpha_lds[(t0 + p) * 16 + n] = alpha[p];
        }
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
    float l_tot[HPWS];
#pragma unroll
    for (int p = 0; p < HPWS; ++p) l_tot[p] = l_run[p];
    if constexpr (RS > 1) {
        if (grp == 0 && rh > 0) {
#pragma unroll
            for (int p = 0; p < HPWS; ++p) xchg[(rh - 1) * HPW + (t0 + p) * 16 + n] = l_run[p];
        }
        __syncthreads();
#pragma unroll
        for (int o = 1; o < RS; ++o)
#pragma unroll
            for (int p = 0; p < HPWS; ++p) l_tot[p] += xchg[(o - 1) * HPW + (t0 + p) * 16 + n];
    } else {
        __syncthreads();
    }
    if (nchunk == 1) {
        // a single chunk: this workgroup's outputs are final -- fp32 rows
        // normalised by the sum and the log-sum-exp go straight out, and no
        // combine follows.  Rows of kDv floats (padded by 16 bytes) staged
        // through both record buffers, idle now, two 16-byte stores a lane a row.
        const int64_t obase = static_cast<int64_t>(r) * H + g * HPW;
        if (grp == 0 && rh == 0) {
#pragma unroll
            for (int p = 0; p < HPWS; ++p) {
                alpha_lds[(t0 + p) * 16 + n] = l_tot[p];
                if (lse)
                    lse[obase + (t0 + p) * 16 + n] =
                        l_tot[p] > 0.f ? (m_run[p] + log2f(l_tot[p])) * 0.69314718055994530942f : -INFINITY;
            }
        }
        __syncthreads();
        constexpr int kFRow = 4 * kDv + 16;
        static_assert(HPW * kFRow <= 2 * kBufBytes, "the fp32 outputs fit the two buffers");
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) {
            const float l = alpha_lds[ht * 16 + n];
            const float inv = l > 0.f ? 1.f / l : 0.f;
            uint8_t* orow = attn_lds + (ht * 16 + n) * kFRow + 4 * (wave * kDimsPerWave + 4 * grp);
#pragma unroll
            for (int dt = 0; dt < kWaveDTiles; ++dt) *reinterpret_cast<f32x4*>(orow + 64 * dt) = acc_o[dt][ht] * inv;
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < HPW / W; ++i) {
            const int row = wave * (HPW / W) + i;
            float* orow = out + (obase + row) * kDv;
#pragma unroll
            for (int half = 0; half < 2; ++half)
                *reinterpret_cast<uint4*>(orow + 4 * (lane + 64 * half)) =
                    *reinterpret_cast<const uint4*>(attn_lds + row * kFRow + 16 * (lane + 64 * half));
        }
        return;
    }
    const int64_t hbase = (static_cast<int64_t>(r) * nchunk + c) * H + g * HPW;
    if (grp == 0 && rh == 0) {
#pragma unroll
        for (int p = 0; p < HPWS; ++p) {
            part_ml[(hbase + (t0 + p) * 16 + n) * 2 + 0] = m_run[p];
            part_ml[(hbase + (t0 + p) * 16 + n) * 2 + 1] = l_tot[p];
            alpha_lds[(t0 + p) * 16 + n] = l_tot[p];
        }
    }
    __syncthreads();
    // The outputs go out through LDS (buffer 0, idle now: one row of kDv
    // halves per head, padded by 16 bytes against bank conflicts) so that each
    // store instruction writes one whole 1 KB row; stored straight from the
    // accumulators they would leave every cache line written in 32-byte pieces.
    // lane (grp, n) holds dims kDimsPerWave·w + 16dt + 4grp + i of head 16ht + n
    constexpr int kORow = 2 * kDv + 16;
    static_assert(HPW * kORow <= kBufBytes && HPW % W == 0, "the outputs fit one buffer, whole rows per wave");
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
        const float l = alpha_lds[ht * 16 + n];
        const float inv = l > 0.f ? 1.f / l : 0.f;
        uint8_t* orow = attn_lds + (ht * 16 + n) * kORow + 2 * (wave * kDimsPerWave + 4 * grp);
#pragma unroll
        for (int dt = 0; dt < kWaveDTiles; ++dt)
            *reinterpret_cast<f16x4*>(orow + 32 * dt) = __builtin_convertvector(acc_o[dt][ht] * inv, f16x4);
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < HPW / W; ++i) {
        const int row = wave * (HPW / W) + i;
        *reinterpret_cast<uint4*>(part_o + (hbase + row) * kDv + 8 * lane) =
            *reinterpret_cast<const uint4*>(attn_lds + row * kORow + 16 * lane);
    }
}

// Combine the chunks of each (request, head): out = sum_c w_c l_c o_c /
// sum_c w_c l_c with w_c = 2^(m_c - M) over the chunks' maxima M, and o_c the
// chunk's normalised output; lse in natural-log units.  One wave a head, eight
// dimensions a lane (one 16-byte load of each chunk's fp16 row), four heads a
// workgroup (3.8 us at 16 requests x 128 heads x 8 chunks, against 4.4 with
// 128 lanes of four dimensions a head; same results bit for bit).  The maxima,
// sums and outputs of up to kCombineBatch chunks are loaded together (one
// round trip to memory for the usual eight chunks or fewer); a later batch
// with a higher maximum rescales what came before.
constexpr int kCombineHeadsPerWg = 4;
constexpr int kCombineBatch = 8;
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

__global__ __launch_bounds__(64 * kCombineHeadsPerWg) void mla_combine_kernel(const _Float16* part_o,
                                                                            const float* part_ml, int H, int nchunk,
                                                                            float* out, float* lse) {
    const int lane = threadIdx.x & 63;
    const int h = blockIdx.x * kCombineHeadsPerWg + (threadIdx.x >> 6), r = blockIdx.y;
    if (h >= H) return;
    const int64_t first = static_cast<int64_t>(r) * nchunk * H + h;   // chunk c at first + c * H
    float M = -INFINITY, denom = 0.f;
    f32x4 acc_lo = f32x4{0.f, 0.f, 0.f, 0.f}, acc_hi = acc_lo;      // dimensions 8 lane + 0..3, + 4..7
    for (int c0 = 0; c0 < nchunk; c0 += kCombineBatch) {
        f16x8 o[kCombineBatch];
        float m[kCombineBatch], l[kCombineBatch];
#pragma unroll
        for (int u = 0; u < kCombineBatch; ++u) {
            const int64_t idx = first + static_cast<int64_t>(min(c0 + u, nchunk - 1)) * H;
            o[u] = *reinterpret_cast<const f16x8*>(part_o + idx * kDv + 8 * lane);
            m[u] = c0 + u < nchunk ? part_ml[idx * 2] : -INFINITY;
            l[u] = part_ml[idx * 2 + 1];
        }
        float Mb = M;
#pragma unroll
        for (int u = 0; u < kCombineBatch; ++u) Mb = fmaxf(Mb, m[u]);
        if (Mb > M) {
            // earlier batches were weighted against M; with M = -inf they hold nothing
            const float f = M == -INFINITY ? 0.f : exp2f(M - Mb);
            acc_lo *= f;
            acc_hi *= f;
            denom *= f;
            M = Mb;
        }
#pragma unroll
        for (int u = 0; u < kCombineBatch; ++u) {
            const float wgt = m[u] != -INFINITY ? exp2f(m[u] - M) * l[u] : 0.f;
            denom += wgt;
            if (wgt != 0.f) {
                acc_lo += wgt * __builtin_convertvector(__builtin_shufflevector(o[u], o[u], 0, 1, 2, 3), f32x4);
                acc_hi += wgt * __builtin_convertvector(__builtin_shufflevector(o[u], o[u], 4, 5, 6, 7), f32x4);
            }
        }
    }
    const float inv = denom > 0.f ? 1.f / denom : 0.f;
    float* orow = out + (static_cast<int64_t>(r) * H + h) * kDv + 8 * lane;
    *reinterpret_cast<f32x4*>(orow) = acc_lo * inv;
    *reinterpret_cast<f32x4*>(orow + 4) = acc_hi * inv;
    if (lane == 0 && lse)
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
    // deep (sixteen chunks or more), the partials it writes and reads back cost
    // more than the extra record reads of 32 heads per workgroup (8 requests x
    // 128 heads: 21.1 us with 32 heads and 8 chunks, 23.0 with 64 heads and 16)
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
    // 32 heads: 4 waves, 64 heads: 8 waves (two a SIMD, which hide each
    // other's LDS waits), each scoring one head tile
    const void* fn = ht == 2 ? reinterpret_cast<const void*>(&mla_partial_kernel<2, 4, 1>)
                             : reinterpret_cast<const void*>(&mla_partial_kernel<4, 8, 1>);
    static LdsGrants granted[2];  // one per kernel instance
    const hipError_t e = ensure_lds_limit(fn, kAttnLds, granted[ht / 4]);
    if (e != hipSuccess) return e;
    const float scale_log2 = scale * 1.44269504088896340736f;
    const int nwg = nchunk * (H / (16 * ht)) * s.R;
    if (ht == 2)
        hipLaunchKernelGGL((mla_partial_kernel<2, 4, 1>), dim3(nwg), dim3(256), kAttnLds, st, H, k, chunk, nchunk, layer,
                           scale_log2, q, slot_idx, part_o, part_ml, out, lse, s);
    else
        hipLaunchKernelGGL((mla_partial_kernel<4, 8, 1>), dim3(nwg), dim3(512), kAttnLds, st, H, k, chunk, nchunk, layer,
                           scale_log2, q, slot_idx, part_o, part_ml, out, lse, s);
    if (nchunk == 1) return hipGetLastError();  // the partial kernel wrote the final outputs
    hipLaunchKernelGGL(mla_combine_kernel, dim3((H + kCombineHeadsPerWg - 1) / kCombineHeadsPerWg, s.R),
                       dim3(64 * kCombineHeadsPerWg), 0, st, part_o, part_ml, H, nchunk, out,
                       lse);
    return hipGetLastError();
}

}  // namespace hs
