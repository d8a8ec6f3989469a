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
  int32_t off[33];                // bucket offsets (exclusive prefix sums)
};

// The steps, all threads of the workgroup calling each one:
//   bucket_clear(L); __syncthreads();
//   bucket_mark(L, el, t) for every local pick (any thread, any order);
//   __syncthreads(); bucket_finish(...).
__device__ __forceinline__ void bucket_clear(BucketLds& L) {
  if (threadIdx.x < 32 * kMaskWords) L.mask[threadIdx.x / kMaskWords][threadIdx.x % kMaskWords] = 0u;
}

// token t picked local expert el
__device__ __forceinline__ void bucket_mark(BucketLds& L, int el, int t) {
  atomicOr(&L.mask[el][t >> 5], 1u << (t & 31));
}

// a store that other workgroups of the same launch may read (kCoh: through to
// the coherence point, sc1), and the matching load
template <bool kCoh>
__device__ __forceinline__ void st_i32(int32_t* p, int32_t v) {
  if constexpr (kCoh) __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else *p = v;
}
template <bool kCoh>
__device__ __forceinline__ int32_t ld_i32(const int32_t* p) {  // one load: not batched
  if constexpr (kCoh) return __hip_atomic_load(const_cast<int32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else return *p;
}

struct NoMid {
  __device__ void operator()() const {}
};

// From the marks: counts, offsets, active (wave 0), then every pick's bucket
// row (rows, pick_pos; rows past the last bucket row are -1 up to R_max).
// A token's ids must be distinct (ids: global or LDS). The counts and the
// bucket rows are stored first; then mid() runs (all threads), then the rest.
// kCoh: counts and rows are read by other workgroups of the same launch once
// mid() has published them (stored through to the coherence point); the rest
// is read only after the launch.
template <bool kCoh = false, class Mid = NoMid>
__device__ __forceinline__ void bucket_finish(const int32_t* __restrict__ ids, int S, int topk,
                                              int n_loc, int local_base, int R_max, BucketLds& L,
                                              int32_t* counts, int32_t* offsets, int32_t* rows,
                                              int32_t* pick_pos, int32_t* active, Mid mid = Mid{}) {
  const int tid = threadIdx.x;
  const int nth = blockDim.x;
  const int npick = S * topk;
  // wave 0, lane e: expert e's count, its bucket offset (wave prefix sum) and
  // its slot in the active list (ballot of the experts with picks)
  int c = 0, incl = 0, nv = 0;
  uint64_t act = 0;
  const int e = tid;
  if (tid < kWave) {
    if (e < n_loc) {
#pragma unroll
      for (int w = 0; w < kMaskWords; ++w) c += __popc(L.mask[e][w]);
    }
    incl = c;
#pragma unroll
    for (int m = 1; m < 32; m <<= 1) {
      const int o = __shfl_up(incl, m, kWave);
      if (e >= m) incl += o;
    }
    act = __ballot(e < n_loc && c > 0);
    nv = __popcll(act);
    if (e < n_loc) {
      L.off[e] = incl - c;
      st_i32<kCoh>(&counts[e], c);
    }
    if (e == n_loc - 1) L.off[n_loc] = incl;
  }
  __syncthreads();

  // bucket row of pick p, -1 if not local
  auto pos_of = [&](int p) {
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
    }
    return pos;
  };
  for (int p = tid; p < npick; p += nth) {
    const int pos = pos_of(p);
    if (pos >= 0) st_i32<kCoh>(&rows[pos], p / topk);
  }
  mid();
  if (tid < kWave) {
    if (e < n_loc) {
      offsets[e] = incl - c;
      if (c > 0) active[1 + __popcll(act & ((1ull << e) - 1ull))] = e;
      if (e >= nv) active[1 + e] = -1;
    }
    if (e == n_loc - 1) offsets[n_loc] = incl;
    if (e == 0) active[0] = nv;
  }
  for (int p = tid; p < npick; p += nth) pick_pos[p] = pos_of(p);
  for (int r = L.off[n_loc] + tid; r < R_max; r += nth) rows[r] = -1;
}

// All of it from ids in memory (the moe_bucket kernel).
__device__ __forceinline__ void bucket_block(const int32_t* __restrict__ ids, int S, int topk,
                                             int n_loc, int local_base, int R_max, BucketLds& L,
                                             int32_t* counts, int32_t* offsets, int32_t* rows,
                                             int32_t* pick_pos, int32_t* active) {
  bucket_clear(L);
  __syncthreads();
  for (int p = threadIdx.x; p < S * topk; p += blockDim.x) {
    const int el = ids[p] - local_base;
    if (el >= 0 && el < n_loc) bucket_mark(L, el, p / topk);
  }
  __syncthreads();
  bucket_finish(ids, S, topk, n_loc, local_base, R_max, L, counts, offsets, rows, pick_pos, active);
}

}  // namespace moeblk
