// launch.h -- enqueue functions of the steps (arguments already checked),
// shared by the entry points.
#pragma once

#include "host.h"

namespace moeblk {

// The caller's bias goes to the router (bias_mode 0, part of the logit) or to
// the top-k (bias_mode 1, the selection only); these give each its share.
inline const float* logit_bias(const moe_dims& m, const float* bias) {
  return m.bias_mode == 0 ? bias : nullptr;
}
inline const float* select_bias(const moe_dims& m, const float* bias) {
  return m.bias_mode == 1 ? bias : nullptr;
}

// the router (applies logit_bias itself) and the top-k (select_bias)
void launch_router_logits(const moe_dims& m, const void* x, const float* wr, const float* bias,
                          float* logits, hipStream_t stream);
void launch_topk(const moe_dims& m, const float* logits, const float* bias, int32_t* ids, float* w,
                 hipStream_t stream);
void launch_bucket(const moe_dims& m, const int32_t* ids, int32_t* counts, int32_t* offsets,
                   int32_t* rows, int32_t* pick_pos, int32_t* active, hipStream_t stream);
// dense bf16 [N][K] -> the bf16 tile order (the down-projection row order)
void launch_pack_bf16(const uint16_t* w, void* packed, int N, int K, hipStream_t stream);
void launch_combine(const moe_dims& m, const void* y, const float* w, const int32_t* pick_pos,
                    const void* gamma, float* out, hipStream_t stream);

}  // namespace moeblk
