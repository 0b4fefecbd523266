// hs_device.h -- wave-level building blocks shared by the metadata kernels.
//
// Everything here works on 64-lane waves (gfx950): DPP row shifts and row
// broadcasts for scans, ballots for compaction, LDS atomics for histograms.
#pragma once

#include "hs_internal.h"

namespace hs {

__device__ inline unsigned long long lanemask_lt() {
    const int lane = threadIdx.x & 63;
    return lane ? (~0ull >> (64 - lane)) : 0ull;
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP: four row shifts
// scan each row of 16 lanes, then row broadcasts add lane 15's total into
// rows 1 and 3 and lane 31's into rows 2 and 3.
__device__ inline int wave_incl_scan(int x) {
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);  // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);  // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);  // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);  // row_shr:8
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31
    return x;
}

// Inclusive prefix sum within each row of 16 lanes (four DPP row shifts).
__device__ inline int row_incl_scan(int x) {
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);  // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);  // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);  // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);  // row_shr:8
    return x;
}

__device__ inline unsigned wave_min(unsigned v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v = min(v, static_cast<unsigned>(__shfl_xor(static_cast<int>(v), off, 64)));
    return v;
}

__device__ inline unsigned wave_max(unsigned v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v = max(v, static_cast<unsigned>(__shfl_xor(static_cast<int>(v), off, 64)));
    return v;
}

// Sum of words[0 .. n) (n <= 16) of a block scan's per-wave partials, for
// every lane: lane i < n of the wave reads word i (one LDS read), the first
// row of 16 lanes adds up with four DPP row shifts, and lane 15 holds the sum.
__device__ inline int sum_before(const int* words, int n) {
    const int lane = static_cast<int>(threadIdx.x) & 63;
    int v = lane < n ? words[lane & 15] : 0;
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);  // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);  // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);  // row_shr:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);  // row_shr:8
    return __builtin_amdgcn_readlane(v, 15);
}

// The workgroup's wave index as a wave-uniform (scalar) value.
__device__ inline int wave_id() { return __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6); }

// Block-wide OR of a small flag word: lanes holding a non-zero value OR it
// into one LDS word (the word must be zero before; read it after a barrier).
__device__ inline void block_or_into(int* word, int v) {
    if (__ballot(v != 0) != 0ull && v != 0) atomicOr(word, v);
}

// Histogram increment for this lane's bin (-1: none): one LDS atomic per
// lane.  Lanes of a wave that hit the same bin are serialised by the LDS,
// which costs less than detecting and merging them with ballots (the ages of
// a wave's candidate slots are spread over many bins).
__device__ inline void hist_add(int* hist, int bin) {
    if (bin >= 0) atomicAdd(&hist[bin], 1);
}

}  // namespace hs
