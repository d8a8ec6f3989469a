// bucket_dev.h -- the local experts' picks grouped by expert, as a
// workgroup-level device function (moe_bucket and moe_forward).
//
// Muse Spark K3 page, stage "route": from every token's top-8, the picks of
// this rank's experts; function "dn_loads": the table etab[u] of the active
// experts and their count nv. The result does not depend on thread timing: a
// pick's bucket row is its expert's offset plus the number of earlier tokens
// that picked the same expert, counted from a token bitmask in LDS.
#pragma once

#include "common.h"

namespace moeblk {

constexpr int kMaxTokens = 128;
constexpr int kMaskWords = kMaxTokens / 32;

struct BucketLds {
  uint32_t mask[32][kMaskWords];  // token bitmask of each local expert
  int32_t cnt[32];                // picks of each local expert
  int32_t off[33];                // bucket offsets (exclusive prefix sums)
  int32_t nv;                     // local experts with a pick
};

// All threads of the workgroup call this. Fills L; if rows_lds is given, the
// token of every bucket row; if `glob`, also the ABI outputs counts, offsets,
// rows (-1 past the last bucket row, up to R_max), pick_pos and active.
// A token's ids must be distinct.
__device__ __forceinline__ void bucket_block(const int32_t* __restrict__ ids, int S, int topk,
                                             int n_loc, int local_base, int R_max, BucketLds& L,
                                             int32_t* rows_lds, bool glob, int32_t* counts,
                                             int32_t* offsets, int32_t* rows, int32_t* pick_pos,
                                             int32_t* active) {
  const int tid = threadIdx.x;
  const int nth = blockDim.x;
  const int npick = S * topk;
  if (tid < 32 * kMaskWords) L.mask[tid / kMaskWords][tid % kMaskWords] = 0u;
  __syncthreads();
  for (int p = tid; p < npick; p += nth) {
    const int el = ids[p] - local_base;
    const int t = p / topk;
    if (el >= 0 && el < n_loc) atomicOr(&L.mask[el][t >> 5], 1u << (t & 31));
  }
  __syncthreads();

  // wave 0, lane e: expert e's count, its bucket offset (wave prefix sum) and
  // its slot in the active list (ballot of the experts with picks)
  if (tid < kWave) {
    const int e = tid;
    int c = 0;
    if (e < n_loc) {
#pragma unroll
      for (int w = 0; w < kMaskWords; ++w) c += __popc(L.mask[e][w]);
    }
    int incl = c;
#pragma unroll
    for (int m = 1; m < 32; m <<= 1) {
      const int o = __shfl_up(incl, m, kWave);
      if (e >= m) incl += o;
    }
    const uint64_t act = __ballot(e < n_loc && c > 0);
    const int nv = __popcll(act);
    if (e < n_loc) {
      L.cnt[e] = c;
      L.off[e] = incl - c;
    }
    if (e == n_loc - 1) L.off[n_loc] = incl;
    if (e == 0) L.nv = nv;
    if (glob) {
      if (e < n_loc) {
        counts[e] = c;
        offsets[e] = incl - c;
        if (c > 0) active[1 + __popcll(act & ((1ull << e) - 1ull))] = e;
        if (e >= nv) active[1 + e] = -1;
      }
      if (e == n_loc - 1) offsets[n_loc] = incl;
      if (e == 0) active[0] = nv;
    }
  }
  __syncthreads();

  for (int p = tid; p < npick; p += nth) {
    const int el = ids[p] - local_base;
    const int t = p / topk;
    int pos = -1;
    if (el >= 0 && el < n_loc) {
      int below = 0;
#pragma unroll
      for (int w = 0; w < kMaskWords; ++w) {
        const uint32_t bits = L.mask[el][w];
        if (w < (t >> 5)) below += __popc(bits);
        else if (w == (t >> 5)) below += __popc(bits & ((1u << (t & 31)) - 1u));
      }
      pos = L.off[el] + below;
      if (rows_lds) rows_lds[pos] = t;
      if (glob) rows[pos] = t;
    }
    if (glob) pick_pos[p] = pos;
  }
  if (glob)
    for (int r = L.off[n_loc] + tid; r < R_max; r += nth) rows[r] = -1;
  __syncthreads();
}

}  // namespace moeblk
