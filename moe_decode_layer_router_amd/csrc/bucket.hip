// bucket.hip -- moe_bucket: one workgroup (bucket_dev.h).
#include "bucket_dev.h"
#include "host.h"
#include "launch.h"

namespace moeblk {
namespace {

__global__ __launch_bounds__(1024) void bucket_kernel(const int32_t* __restrict__ ids,
                                                      int32_t* __restrict__ counts,
                                                      int32_t* __restrict__ offsets,
                                                      int32_t* __restrict__ rows,
                                                      int32_t* __restrict__ pick_pos,
                                                      int32_t* __restrict__ active, int S,
                                                      int topk, int n_loc, int local_base,
                                                      int R_max) {
  __shared__ BucketLds L;
  bucket_block(ids, S, topk, n_loc, local_base, R_max, L, counts, offsets, rows, pick_pos, active);
}

}  // namespace

void launch_bucket(const moe_dims& m, const int32_t* ids, int32_t* counts, int32_t* offsets,
                   int32_t* rows, int32_t* pick_pos, int32_t* active, hipStream_t stream) {
  hipLaunchKernelGGL(bucket_kernel, dim3(1), dim3(1024), 0, stream, ids, counts, offsets, rows,
                     pick_pos, active, m.S, m.topk, m.n_local, m.local_base, r_max(m));
}

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
  launch_bucket(*dims, topk_ids, counts, offsets, rows, pick_pos, active, stream);
  return launch_status();
}
