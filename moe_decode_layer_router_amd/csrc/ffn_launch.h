// ffn_launch.h -- the expert-FFN launches shared by moe_expert_ffn and
// moe_forward: their argument block and workspace layout.
#pragma once

#include "common.h"
#include "host.h"

namespace moeblk {

constexpr int kSharedTTG = 2;  // shared expert at S <= 16: 32-token groups
// shared expert at S > 16 (shared_rows_task in both launches): tokens a
// group in the gate_up launch and in the down launch. Measured at S = 128
// (d = 7168, I_s = 2048), kernel us with 32 / 64 tokens: gate_up 101.7 /
// 105.3, down 50.8 / 46.9 (the down tasks' weights, read once per group,
// come through L2 half as often).
#ifndef MOE_SG_TOK_GU
#define MOE_SG_TOK_GU 32
#endif
#ifndef MOE_SG_TOK_DN
#define MOE_SG_TOK_DN 64
#endif
constexpr int kSgTokGu = MOE_SG_TOK_GU;
constexpr int kSgTokDn = MOE_SG_TOK_DN;
#ifndef MOE_SHARED_P
#define MOE_SHARED_P 2
#endif
constexpr int kSharedP = MOE_SHARED_P;

// The routing front of moe_forward's expert-FFN launch: the top-k of every
// token (one workgroup a token) and the bucketing (one workgroup) run as the
// launch's first workgroups (K3 page, stage "route": the routing is computed
// inside the persistent launch that consumes it). A top-k workgroup sets its
// token's bit in the token mask of each local expert it picked and counts
// itself on the counter (kDoneCopies copies, one 128-byte line each, which
// spreads the tasks' polls). At S > kTopkLinesMinS it counts on line t mod
// kTopkLines instead (device-scope atomics on one address serialise: S adds
// on each copy cost about 13 ns each), and the bucketing workgroup waits for
// the lines to add up to S, then sets the copies to S (s128_shared steps,
// two boxes, two runs each: 162.5, 162.4 -> 159.8, 160.0 us and 161.6,
// 163.9 -> 161.0, 161.0 us). The expert tasks wait for the
// counter to reach S and take their expert counts and bucket rows from the
// masks (a bucket row's token is the rank-th set bit of its expert's mask, as
// the bucketing numbers them), so the bucketing, which writes the ABI's
// bucket outputs, is not on their path. The lines, the counter and the masks
// are zero when the launch starts: a call leaves them at zero for the next
// one (moe_forward's combine launch clears them).
//
// The whole block as one launch (moe_forward_one_launch: no shared expert,
// S <= 16, d <= 4096; K3 page, module docstring: the layer as one persistent
// launch): the router itself runs at the head of the front, as E workgroups
// of one router row each (summed exactly as the router launch sums it), and
// the combine as the launch's last S workgroups (one a token). The top-k
// workgroups wait for the router rows' count, kept on kRouterLines lines
// (router row b counts on line b mod kRouterLines: device-scope atomics on
// one address serialise, about 3.4 us for 256 of them, measured). Every
// workgroup that reads the routing counts itself on the kSeenLines lines once
// it has; the last combine workgroup waits for that count and clears the
// control block for the next call.
constexpr int kDoneCopies = 8;
constexpr int kMaskWordsAll = 32 * 4;  // 32 local experts x 128 tokens
constexpr int kRouterLines = 32;
constexpr int kSeenLines = 64;
constexpr int kTopkLines = 32;
constexpr int kTopkLinesMinS = 32;
// words of the front's control block: the counter copies, the masks, then
// (one launch) the router rows' lines, the seen lines and the combine count,
// then the top-k workgroups' lines
constexpr int kFrontMaskWord = kDoneCopies * 32;
constexpr int kFrontRouterWord = kFrontMaskWord + kMaskWordsAll;
constexpr int kFrontSeenWord = kFrontRouterWord + kRouterLines * 32;
constexpr int kFrontCombWord = kFrontSeenWord + kSeenLines * 32;
constexpr int kFrontTopkWord = kFrontCombWord + 32;
constexpr int kFrontWords = kFrontTopkWord + kTopkLines * 32;
struct RouteFront {
  const float* logits_in;  // no K parts: the router's logits
  const float* parts;      // else the router's K parts [KP][S][E]
  int KP;
  const float* lbias;      // K parts or router rows: the logit bias, or NULL
  const float* sel_bias;   // selection-only bias, or NULL
  float* logits_out;       // K parts: the summed logits; router rows: the logits
  const float* wr;         // router rows: the router weights [E][d]
  int n_router;            // workgroups of router rows (E), or 0
  int32_t* rdone;          // workspace: the router rows' lines
  int32_t* seen;           // workspace: the seen lines (one launch)
  int32_t* cdone;          // workspace: combine workgroups done (one launch)
  int32_t* ids;
  float* w;
  int32_t* offsets;
  int32_t* pick_pos;
  int32_t* active;
  int32_t* done;           // workspace: kDoneCopies counters of finished top-k workgroups
  int32_t* tkc;            // workspace: kTopkLines lines the top-k workgroups count on
  uint32_t* masks;         // workspace: [32][4] token masks of the local experts
  int E, topk, renorm, local_base;
};

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
  int front;       // workgroups of the routing front (router rows + S + 1), 0 without one
  RouteFront rf;
  // one launch: the combine as the last comb workgroups (S, or 0 without)
  int comb;
  int32_t* tokc;          // workspace: y rows written, a token (one line each)
  const uint16_t* gamma;  // post-expert norm weight [d] bf16, or NULL
  float* out;             // [S][d] fp32
  float eps;
};

// ints between two counters or flags (one 128-byte line each)
constexpr int kCtlStride = 32;

// workspace: SwiGLU rows h [R_max][I] and hs [S][Is] (bf16), then the
// counters prod (max_work lines), the ready flags (max_work * d / 64 lines),
// the token counters of the combine (S lines), the routing front's control
// block (kFrontWords words) and the error word; these must start at zero and
// are left at zero (the front's block is cleared by moe_forward's combine
// launch, or in one launch by its last combine workgroup)
struct FfnLayout {
  size_t h, hs, prod, ready, tokc, route, error, total;
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

// The routing inputs and outputs of moe_forward's front (launch_ffn with a
// front): the router's logits or K parts, the biases, and the outputs of
// moe_route and moe_bucket.
struct FrontIo {
  const float* logits_in;
  const float* parts;
  const float* wr;        // one launch: the router weights (the router rows), else NULL
  float* out;             // one launch: the combine's output [S][d], else NULL
  const uint16_t* gamma;  // one launch: the post-expert norm weight, or NULL
  const float* bias;  // the caller's bias (split by bias_mode)
  float* logits;
  int32_t* ids;
  float* w;
  int32_t* offsets;
  int32_t* pick_pos;
  int32_t* active;
};

// moe_forward_one_launch: the whole block as one launch (FrontIo.wr and
// .out), without a shared expert at S <= 16 and d <= 4096
inline bool one_launch(const moe_dims& m) { return m.shared_I == 0 && m.S <= 16 && m.d <= 4096; }

// the control block of the FFN launch's front (kFrontWords words), which the
// combine launch after it clears
int32_t* route_front_block(const moe_dims& m, void* workspace);

// enqueue the expert FFNs (after argument checks); error_word: where a wait
// that hits its bound records it (NULL: the workspace's own error word);
// front: run the top-k and the bucketing as the launch's first workgroups
// (counts and rows are then outputs)
int launch_ffn(const moe_dims& m, const void* x, const void* w13, const void* w2, const void* ws13,
               const void* ws2, const int32_t* counts, const int32_t* rows, void* y,
               void* workspace, hipStream_t stream, int32_t* error_word = nullptr,
               const FrontIo* front = nullptr);

}  // namespace moeblk
