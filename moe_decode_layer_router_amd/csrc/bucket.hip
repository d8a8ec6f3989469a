// bucket.hip -- the local experts' picks, grouped by expert.
//
// Muse Spark K3 page, stage "route": from every token's top-8, the picks of
// this rank's experts; function "dn_loads": the expert table etab[u] of the
// active experts and their count nv. One workgroup, one thread a pick. The
// result does not depend on thread timing: a pick's bucket row is the number
// of earlier tokens that picked the same expert, counted from a token bitmask.
#include "common.h"
#include "host.h"

namespace moeblk {
namespace {

constexpr int kMaxTokens = 128;
constexpr int kMaskWords = kMaxTokens / 32;

__global__ __launch_bounds__(1024) void bucket_kernel(const int32_t* __restrict__ ids,
                                                      int32_t* __restrict__ counts,
                                                      int32_t* __restrict__ offsets,
                                                      int32_t* __restrict__ rows,
                                                      int32_t* __restrict__ pick_pos,
                                                      int32_t* __restrict__ active, int S,
                                                      int topk, int n_loc, int local_base,
                                                      int R_max) {
  __shared__ uint32_t mask[32][kMaskWords];  // token bitmask a local expert
  __shared__ int32_t off[33];
  const int tid = threadIdx.x;
  if (tid < 32 * kMaskWords) mask[tid / kMaskWords][tid % kMaskWords] = 0u;
  __syncthreads();

  const int npick = S * topk;
  const int t = tid / topk;
  int el = -1;
  if (tid < npick) {
    el = ids[tid] - local_base;
    if (el < 0 || el >= n_loc) el = -1;
    else atomicOr(&mask[el][t >> 5], 1u << (t & 31));
  }
  __syncthreads();

  if (tid == 0) {
    int pos = 0, nv = 0;
    for (int e = 0; e < n_loc; ++e) {
      int c = 0;
#pragma unroll
      for (int w = 0; w < kMaskWords; ++w) c += __popc(mask[e][w]);
      off[e] = pos;
      counts[e] = c;
      offsets[e] = pos;
      pos += c;
      if (c > 0) active[1 + nv++] = e;
    }
    off[n_loc] = pos;
    offsets[n_loc] = pos;
    active[0] = nv;
    for (int u = nv; u < n_loc; ++u) active[1 + u] = -1;
  }
  __syncthreads();

  if (tid < npick) {
    int p = -1;
    if (el >= 0) {
      int below = 0;
#pragma unroll
      for (int w = 0; w < kMaskWords; ++w) {
        const uint32_t bits = mask[el][w];
        if (w < (t >> 5)) below += __popc(bits);
        else if (w == (t >> 5)) below += __popc(bits & ((1u << (t & 31)) - 1u));
      }
      p = off[el] + below;
      rows[p] = t;
    }
    pick_pos[tid] = p;
  }
  for (int r = off[n_loc] + tid; r < R_max; r += blockDim.x) rows[r] = -1;
}

}  // namespace
}  // namespace moeblk

using namespace moeblk;

extern "C" int moe_bucket(const moe_dims* dims, const int32_t* topk_ids, int32_t* counts,
                          int32_t* offsets, int32_t* rows, int32_t* pick_pos, int32_t* active,
                          hipStream_t stream) {
  const int rc = check_dims(dims);
  if (rc) return rc;
  MOE_REQUIRE(topk_ids && counts && offsets && rows && pick_pos && active, MOE_ERR_NULL);
  MOE_REQUIRE(aligned16(topk_ids) && aligned16(counts) && aligned16(offsets) && aligned16(rows) &&
                  aligned16(pick_pos) && aligned16(active),
              MOE_ERR_ALIGN);
  const moe_dims& m = *dims;
  hipLaunchKernelGGL(bucket_kernel, dim3(1), dim3(1024), 0, stream, topk_ids, counts, offsets,
                     rows, pick_pos, active, m.S, m.topk, m.n_local, m.local_base, r_max(m));
  return launch_status();
}
