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

// Router for S > kRouteSplitMinS with scratch: tiles of router_tile_tok(S)
// tokens x 64 router rows, K split into router_parts(m) parts (a power of two
// up to 32 that divides d / kRouteKB, so that the tiles times the parts stay within
// 256 workgroups); 0 parts below (no scratch). Router + top-k measured on
// MI355X, us, whole-K workgroups against split tiles: S = 32 10.2 / 10.7,
// S = 64 13.4 / 11.4, S = 96 18.7 / 14.9, S = 128 (d = 7168) 27.1 / 18.0.
constexpr int kRouteSplitMinS = 32;
#ifndef MOE_ROUTE_MAX_PARTS
#define MOE_ROUTE_MAX_PARTS 32
#endif
#ifndef MOE_ROUTE_MAX_WG
#define MOE_ROUTE_MAX_WG 256
#endif
constexpr int kMaxRouteParts = MOE_ROUTE_MAX_PARTS;  // K parts of the split router, at most
// K a lane a block of the split router (block = 4 KL = 32 K): the 8 K of a
// lane are one operand of the bf16 MFMA, and the lanes of one K group read
// whole 128-byte lines of the router rows
constexpr int kRouteKL = 8;
constexpr int kRouteKB = 4 * kRouteKL;  // K a block
inline int router_tile_tok(int S) { return S <= 64 ? 32 : 64; }
inline int router_parts(const moe_dims& m) {
  if (m.S <= kRouteSplitMinS) return 0;
  const int TT = router_tile_tok(m.S);
  const int tiles = ((m.S + TT - 1) / TT) * ((m.E + 63) / 64);
  int P = 1;
  while (P < kMaxRouteParts && tiles * P * 2 <= MOE_ROUTE_MAX_WG && (m.d / kRouteKB) % (2 * P) == 0)
    P *= 2;
  return P;
}
// scratch of the split router: parts [P][S][E] fp32
inline size_t router_parts_bytes(const moe_dims& m) {
  return round_up(static_cast<size_t>(router_parts(m)) * m.S * m.E * 4, 256);
}

// the router (applies logit_bias itself) and the top-k (select_bias). With
// `parts` (router_parts_bytes of scratch) and S > kRouteSplitMinS the router
// writes its K parts there and the top-k sums them into `logits_out`;
// otherwise the router writes `logits` itself.
void launch_router_logits(const moe_dims& m, const void* x, const float* wr, const float* bias,
                          float* logits, hipStream_t stream, float* parts = nullptr);
void launch_topk(const moe_dims& m, const float* logits, const float* bias, int32_t* ids, float* w,
                 hipStream_t stream, const float* parts = nullptr, float* logits_out = nullptr);
void launch_bucket(const moe_dims& m, const int32_t* ids, int32_t* counts, int32_t* offsets,
                   int32_t* rows, int32_t* pick_pos, int32_t* active, hipStream_t stream);
// dense bf16 [N][K] -> the bf16 tile order (the down-projection row order)
void launch_pack_bf16(const uint16_t* w, void* packed, int N, int K, hipStream_t stream);
// clear: n_clear words that workgroup 0 sets to zero (the control block of
// moe_forward's routing front, for its next call), or NULL
void launch_combine(const moe_dims& m, const void* y, const float* w, const int32_t* pick_pos,
                    const void* gamma, float* out, hipStream_t stream, int32_t* clear = nullptr,
                    int n_clear = 0);

}  // namespace moeblk
