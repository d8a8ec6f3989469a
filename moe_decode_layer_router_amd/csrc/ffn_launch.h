// ffn_launch.h -- the expert-FFN launches shared by moe_expert_ffn and
// moe_forward: their argument block and workspace layout.
#pragma once

#include "common.h"
#include "host.h"

namespace moeblk {

constexpr int kSharedTTG = 2;  // shared expert: 32-token groups
constexpr int kSharedP = 2;

struct FfnArgs {
  const uint8_t* w13;  // packed MXFP4 gate_up of the local experts
  const uint8_t* w2;   // packed MXFP4 down
  const uint8_t* ws13; // packed bf16 shared gate_up (or NULL)
  const uint8_t* ws2;  // packed bf16 shared down (or NULL)
  const uint16_t* x;   // [S][d] bf16
  const int32_t* rows; // bucket row -> token
  const int32_t* counts;
  uint16_t* h;     // workspace: SwiGLU rows of the bucket rows [R_max][I]
  uint16_t* hs;    // workspace: the shared expert's SwiGLU rows [S][Is]
  uint16_t* y;     // [R_max (+ S)][d]
  int S, d, I, Is, n_loc, R_max, max_work;
};

struct FfnLayout {
  size_t h, hs, total;
  int max_work;
};

// bucket rows a routed work item holds: 16 while no expert can get more than
// 16 picks (S <= 16), else 32
inline int ffn_group(const moe_dims& m) { return m.S > 16 ? 32 : 16; }

FfnLayout ffn_layout(const moe_dims& m);

// enqueue the expert FFNs (after argument checks)
int launch_ffn(const moe_dims& m, const void* x, const void* w13, const void* w2, const void* ws13,
               const void* ws2, const int32_t* counts, const int32_t* rows, void* y,
               void* workspace, hipStream_t stream);

}  // namespace moeblk
