// route.hip -- moe_route: router logits kernel + top-k kernel (route_dev.h).
#include "host.h"
#include "launch.h"
#include "route_dev.h"

namespace moeblk {
namespace {

// one workgroup an expert row: the row streams from HBM once, all of it in
// flight at once; every workgroup reads all of x (through L2)
template <int NW>
__global__ __launch_bounds__(kRouteThreads) void router_logits_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ wr, const float* __restrict__ bias,
    float* __restrict__ logits, int S, int d, int E) {
  __shared__ float red[kMaxRouteTiles][kRouteWaves][kTok];
  // NW = 4 (d > 8192): one tile buffer, for the register budget
  router_row<NW, (NW <= 2)>(x, wr, bias, logits, S, d, E, blockIdx.x, red);
}

// S > 16: kRouteBlockTok tokens x NE router rows a workgroup
template <int NW, int NE>
__global__ __launch_bounds__(kRouteThreads) void router_block_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ wr, const float* __restrict__ bias,
    float* __restrict__ logits, int S, int d, int E) {
  __shared__ float red[(kRouteBlockTok / kTok) * NE][kRouteWaves][kTok];
  router_block<NW, NE>(x, wr, bias, logits, S, d, E, NE * blockIdx.x, kRouteBlockTok * blockIdx.y,
                       red);
}

template <int NW, int NE>
void launch_block(const moe_dims& m, const uint16_t* x, const float* wr, const float* bias,
                  float* logits, hipStream_t stream) {
  hipLaunchKernelGGL((router_block_kernel<NW, NE>), dim3((m.E + NE - 1) / NE,
                     (m.S + kRouteBlockTok - 1) / kRouteBlockTok), dim3(kRouteThreads), 0, stream,
                     x, wr, bias, logits, m.S, m.d, m.E);
}

// NE: router rows a workgroup, so that about E * S / 16 / NE ~ E workgroups
// (at most 2 rows for d > 8192, for the register budget)
template <int NW>
void launch_blocks(const moe_dims& m, const uint16_t* x, const float* wr, const float* bias,
                   float* logits, hipStream_t stream) {
  if constexpr (NW >= 4) {
    launch_block<NW, 2>(m, x, wr, bias, logits, stream);
  } else {
    if (m.S <= 32) launch_block<NW, 2>(m, x, wr, bias, logits, stream);
    else if (m.S <= 64) launch_block<NW, 4>(m, x, wr, bias, logits, stream);
    else launch_block<NW, 8>(m, x, wr, bias, logits, stream);
  }
}

// S > kRouteSplitMinS with scratch: workgroup b = (tile (tt, et), K part p),
// tt fastest
template <int TT>
__global__ __launch_bounds__(4 * kWave) void router_split_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ wr, float* __restrict__ parts, int S,
    int d, int E, int Kp, int n_tt, int n_et) {
  int b = blockIdx.x;
  const int tt = b % n_tt;
  b /= n_tt;
  const int et = b % n_et;
  router_split_tile<TT>(x, wr, parts, S, d, E, Kp, tt, et, b / n_et);
}

template <int TT>
void launch_split(const moe_dims& m, const uint16_t* x, const float* wr, float* parts,
                  hipStream_t stream) {
  const int P = router_parts(m);
  const int n_tt = (m.S + TT - 1) / TT, n_et = (m.E + kRouteTileE - 1) / kRouteTileE;
  hipLaunchKernelGGL((router_split_kernel<TT>), dim3(n_tt * n_et * P), dim3(4 * kWave), 0, stream,
                     x, wr, parts, m.S, m.d, m.E, m.d / P, n_tt, n_et);
}

// one token a workgroup: the sum of its router parts (+ the logit bias) into
// logits, then its top-k
__global__ __launch_bounds__(4 * kWave) void topk_parts_kernel(
    const float* __restrict__ parts, int KP, const float* __restrict__ lbias,
    const float* __restrict__ sel_bias, float* __restrict__ logits, int32_t* __restrict__ ids,
    float* __restrict__ w, int S, int E, int topk, int renorm) {
  __shared__ float red[4][4][kWave];
  if (sel_bias)
    topk_parts_token<true>(parts, KP, lbias, sel_bias, logits, ids, w, S, E, topk, renorm,
                           blockIdx.x, red);
  else
    topk_parts_token<false>(parts, KP, lbias, nullptr, logits, ids, w, S, E, topk, renorm,
                            blockIdx.x, red);
}

// one wave per token
// (sel_bias: the selection-only bias, or NULL)
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ logits,
                                                   const float* __restrict__ sel_bias,
                                                   int32_t* __restrict__ ids,
                                                   float* __restrict__ w, int S, int E,
                                                   int topk, int renorm) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= S) return;
  if (sel_bias) topk_token<true>(logits, sel_bias, ids, w, nullptr, E, topk, renorm, t, NoMark{});
  else topk_token<false>(logits, nullptr, ids, w, nullptr, E, topk, renorm, t, NoMark{});
}

template <int NW>
void launch_router(const moe_dims& m, const uint16_t* x, const float* wr, const float* bias,
                   float* logits, hipStream_t stream) {
  hipLaunchKernelGGL(router_logits_kernel<NW>, dim3(m.E), dim3(kRouteThreads), 0, stream, x, wr,
                     bias, logits, m.S, m.d, m.E);
}

}  // namespace

void launch_router_logits(const moe_dims& m, const void* x, const float* wr, const float* bias,
                          float* logits, hipStream_t stream, float* parts) {
  bias = logit_bias(m, bias);
  const uint16_t* xx = static_cast<const uint16_t*>(x);
  if (parts && router_parts(m) > 0) {  // the top-k adds the bias
    if (router_tile_tok(m.S) == 32) launch_split<32>(m, xx, wr, parts, stream);
    else launch_split<64>(m, xx, wr, parts, stream);
    return;
  }
  if (m.S > kRouteBlockTok) {
    switch (router_nw(m.d)) {
      case 1: launch_blocks<1>(m, xx, wr, bias, logits, stream); break;
      case 2: launch_blocks<2>(m, xx, wr, bias, logits, stream); break;
      default: launch_blocks<4>(m, xx, wr, bias, logits, stream); break;
    }
    return;
  }
  switch (router_nw(m.d)) {
    case 1: launch_router<1>(m, xx, wr, bias, logits, stream); break;
    case 2: launch_router<2>(m, xx, wr, bias, logits, stream); break;
    default: launch_router<4>(m, xx, wr, bias, logits, stream); break;
  }
}

void launch_topk(const moe_dims& m, const float* logits, const float* bias, int32_t* ids, float* w,
                 hipStream_t stream, const float* parts, float* logits_out) {
  if (parts && router_parts(m) > 0) {
    hipLaunchKernelGGL(topk_parts_kernel, dim3(m.S), dim3(4 * kWave), 0, stream, parts,
                       router_parts(m), logit_bias(m, bias), select_bias(m, bias), logits_out, ids,
                       w, m.S, m.E, m.topk, m.renorm);
    return;
  }
  hipLaunchKernelGGL(topk_kernel, dim3((m.S + 3) / 4), dim3(256), 0, stream, logits,
                     select_bias(m, bias), ids, w, m.S, m.E, m.topk, m.renorm);
}

}  // namespace moeblk

using namespace moeblk;

extern "C" size_t moe_route_workspace_bytes(const moe_dims* dims) {
  if (check_dims(dims)) return 0;
  return router_parts_bytes(*dims);
}

extern "C" int moe_route(const moe_dims* dims, const void* x, const float* w_router,
                         const float* bias, float* logits, int32_t* topk_ids, float* topk_w,
                         void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const int rc = check_dims(dims);
  if (rc) return rc;
  const size_t need = router_parts_bytes(*dims);
  MOE_REQUIRE(x && w_router && logits && topk_ids && topk_w && (workspace || need == 0),
              MOE_ERR_NULL);
  MOE_REQUIRE(aligned16(x) && aligned16(w_router) && aligned16(logits) && aligned16(topk_ids) &&
                  aligned16(topk_w) && (!bias || aligned16(bias)) && aligned16(workspace),
              MOE_ERR_ALIGN);
  MOE_REQUIRE(workspace_bytes >= need, MOE_ERR_WORKSPACE);
  float* parts = need ? static_cast<float*>(workspace) : nullptr;
  launch_router_logits(*dims, x, w_router, bias, logits, stream, parts);
  launch_topk(*dims, logits, bias, topk_ids, topk_w, stream, parts, logits);
  return launch_status();
}
