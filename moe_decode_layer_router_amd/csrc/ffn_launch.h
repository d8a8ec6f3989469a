// ffn_launch.h -- the expert-FFN launches shared by moe_expert_ffn and
// moe_forward: their argument block and workspace layout.
#pragma once

#include "common.h"
#include "host.h"

namespace moeblk {

constexpr int kSharedTTG = 2;  // shared expert: 32-token groups
#ifndef MOE_SHARED_P
#define MOE_SHARED_P 2
#endif
constexpr int kSharedP = MOE_SHARED_P;

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
  int32_t* prod;   // workspace: gate_up tasks done, a work item (single launch)
  int32_t* ready;  // workspace: a flag a down task: its item's SwiGLU rows are written
  int32_t* error;  // workspace: nonzero if a wait hit its bound
  int S, d, I, Is, n_loc, R_max, max_work;
};

// ints between two counters or flags (one 128-byte line each)
constexpr int kCtlStride = 32;

// workspace: SwiGLU rows h [R_max][I] and hs [S][Is] (bf16), then the
// counters prod (max_work lines), the ready flags (max_work * d / 64 lines)
// and the error word; these must start at zero and are left at zero
struct FfnLayout {
  size_t h, hs, prod, ready, error, total;
  int max_work;
};

// bucket rows a routed work item holds: 16, or 32 in the two launches with a
// shared expert at S > 16 (measured at S = 128: FFN 161.9 against 163.5 us
// with 16-row items there)
inline int ffn_group(const moe_dims& m) { return m.S > 16 && m.shared_I > 0 ? 32 : 16; }

// upper bound of the work items, sum over experts of ceil(count / G): with
// S <= G every expert with picks has one item
inline int max_work(const moe_dims& m) {
  const int R = r_max(m);
  const int G = ffn_group(m);
  const int experts = m.n_local < R ? m.n_local : R;
  return m.S <= G ? experts : experts + R / G;
}

FfnLayout ffn_layout(const moe_dims& m);

// enqueue the expert FFNs (after argument checks); error_word: where a wait
// that hits its bound records it (NULL: the workspace's own error word)
int launch_ffn(const moe_dims& m, const void* x, const void* w13, const void* w2, const void* ws13,
               const void* ws2, const int32_t* counts, const int32_t* rows, void* y,
               void* workspace, hipStream_t stream, int32_t* error_word = nullptr);

}  // namespace moeblk
