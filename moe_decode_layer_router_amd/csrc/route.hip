// route.hip -- router logits (fp32) and sigmoid top-k.
//
// Muse Spark K3 page, stage "A": router logits in fp32; stage "route": every
// token's top-8 with identical results wherever it is computed. K5 page, HA
// routing tail: top-8 per token, then ids and weights handed to the expert
// launch. The bias is added to the logit before ranking (Kimi-K3 layer page,
// "k2_launch" takes the router weight and a bias).
#include "common.h"
#include "host.h"

namespace moeblk {
namespace {

constexpr int kTokTile = 16;  // tokens a wave accumulates at once

// 16 per-lane partial sums -> lane l (l % 4 == 0) holds the wave total of value
// index ((l >> 5) & 1) * 8 + ((l >> 4) & 1) * 4 + ((l >> 3) & 1) * 2 + ((l >> 2) & 1).
// Each step halves the values a lane keeps; the order of additions is fixed.
__device__ __forceinline__ float reduce16(float (&v)[16], int lane) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const bool hi = lane & 32;
    const float send = hi ? v[j] : v[8 + j];
    const float keep = hi ? v[8 + j] : v[j];
    v[j] = keep + __shfl_xor(send, 32, kWave);
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const bool hi = lane & 16;
    const float send = hi ? v[j] : v[4 + j];
    const float keep = hi ? v[4 + j] : v[j];
    v[j] = keep + __shfl_xor(send, 16, kWave);
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const bool hi = lane & 8;
    const float send = hi ? v[j] : v[2 + j];
    const float keep = hi ? v[2 + j] : v[j];
    v[j] = keep + __shfl_xor(send, 8, kWave);
  }
  {
    const bool hi = lane & 4;
    const float send = hi ? v[0] : v[1];
    const float keep = hi ? v[1] : v[0];
    v[0] = keep + __shfl_xor(send, 4, kWave);
  }
  float s = v[0];
  s += __shfl_xor(s, 2, kWave);
  s += __shfl_xor(s, 1, kWave);
  return s;
}

// One wave per (expert e, tile of up to 16 tokens); lanes split K, 8 elements
// a lane per step: the fp32 router row streams through 2 x dwordx4 per lane,
// the bf16 activations through one dwordx4 per token.
__global__ __launch_bounds__(256) void router_logits_kernel(const uint16_t* __restrict__ x,
                                                            const float* __restrict__ wr,
                                                            const float* __restrict__ bias,
                                                            float* __restrict__ logits, int S,
                                                            int d, int E) {
  const int lane = threadIdx.x & (kWave - 1);
  const int task = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int n_tt = (S + kTokTile - 1) / kTokTile;
  if (task >= E * n_tt) return;
  const int e = task % E;  // the block's waves share a token tile: x hits in L1
  const int t0 = (task / E) * kTokTile;
  const int nt = min(kTokTile, S - t0);

  float acc[16];
#pragma unroll
  for (int t = 0; t < 16; ++t) acc[t] = 0.0f;
  const float* wrow = wr + static_cast<size_t>(e) * d;
  const uint16_t* xt = x + static_cast<size_t>(t0) * d;
#pragma unroll 2
  for (int k = lane * 8; k < d; k += kWave * 8) {
    const float4 w0 = *reinterpret_cast<const float4*>(wrow + k);
    const float4 w1 = *reinterpret_cast<const float4*>(wrow + k + 4);
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      if (t < nt) {
        const uint4 xv = *reinterpret_cast<const uint4*>(xt + static_cast<size_t>(t) * d + k);
        float a = acc[t];
        a += bf16_lo(xv.x) * w0.x;
        a += bf16_hi(xv.x) * w0.y;
        a += bf16_lo(xv.y) * w0.z;
        a += bf16_hi(xv.y) * w0.w;
        a += bf16_lo(xv.z) * w1.x;
        a += bf16_hi(xv.z) * w1.y;
        a += bf16_lo(xv.w) * w1.z;
        a += bf16_hi(xv.w) * w1.w;
        acc[t] = a;
      }
    }
  }
  const float s = reduce16(acc, lane);
  const int tok = ((lane >> 5) & 1) * 8 + ((lane >> 4) & 1) * 4 + ((lane >> 3) & 1) * 2 +
                  ((lane >> 2) & 1);
  if ((lane & 3) == 0 && tok < nt)
    logits[static_cast<size_t>(t0 + tok) * E + e] = s + (bias ? bias[e] : 0.0f);
}

// A logit and its expert id as one unsigned key: larger logit first, and for
// equal logits the lower id first. -0 is folded into +0 so both compare equal.
__device__ __forceinline__ uint64_t rank_key(float l, int e) {
  l = l + 0.0f;
  const uint32_t u = __float_as_uint(l);
  const uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return (static_cast<uint64_t>(ord) << 32) | (0xffffffffu - static_cast<uint32_t>(e));
}
__device__ __forceinline__ float key_logit(uint64_t key) {
  const uint32_t ord = static_cast<uint32_t>(key >> 32);
  const uint32_t u = (ord & 0x80000000u) ? (ord & 0x7fffffffu) : ~ord;
  return __uint_as_float(u);
}
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const uint32_t lo = __shfl_xor(static_cast<uint32_t>(v), m, kWave);
    const uint32_t hi = __shfl_xor(static_cast<uint32_t>(v >> 32), m, kWave);
    const uint64_t o = (static_cast<uint64_t>(hi) << 32) | lo;
    v = o > v ? o : v;
  }
  return v;
}

// One wave per token: each lane holds experts lane, lane + 64, ..; k rounds of
// a wave-wide max of the rank keys. Then sigmoid scores and their renormalisation
// in slot order.
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ logits,
                                                   int32_t* __restrict__ ids,
                                                   float* __restrict__ w, int S, int E,
                                                   int topk, int renorm) {
  const int lane = threadIdx.x & (kWave - 1);
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= S) return;
  uint64_t key[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = lane + kWave * j;
    key[j] = e < E ? rank_key(logits[static_cast<size_t>(t) * E + e], e) : 0ull;
  }
  float lsel[8];
  int isel[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    lsel[s] = 0.0f;
    isel[s] = 0;
    if (s < topk) {
      uint64_t m = key[0];
#pragma unroll
      for (int j = 1; j < 4; ++j) m = key[j] > m ? key[j] : m;
      m = wave_max_u64(m);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (key[j] == m) key[j] = 0ull;  // ids are unique: only the owner matches
      isel[s] = static_cast<int>(0xffffffffu - static_cast<uint32_t>(m));
      lsel[s] = key_logit(m);
    }
  }
  float sc[8], sum = 0.0f;
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    sc[s] = s < topk ? 1.0f / (1.0f + expf(-lsel[s])) : 0.0f;
    sum += sc[s];
  }
#pragma unroll
  for (int s = 0; s < 8; ++s)
    if (s < topk && lane == s) {
      ids[static_cast<size_t>(t) * topk + s] = isel[s];
      w[static_cast<size_t>(t) * topk + s] = renorm ? sc[s] / sum : sc[s];
    }
}

}  // namespace
}  // namespace moeblk

using namespace moeblk;

extern "C" int moe_route(const moe_dims* dims, const void* x, const float* w_router,
                         const float* bias, float* logits, int32_t* topk_ids, float* topk_w,
                         hipStream_t stream) {
  const int rc = check_dims(dims);
  if (rc) return rc;
  MOE_REQUIRE(x && w_router && logits && topk_ids && topk_w, MOE_ERR_NULL);
  MOE_REQUIRE(aligned16(x) && aligned16(w_router) && aligned16(logits) && aligned16(topk_ids) &&
                  aligned16(topk_w) && (!bias || aligned16(bias)),
              MOE_ERR_ALIGN);
  const moe_dims& m = *dims;
  const int n_tt = (m.S + kTokTile - 1) / kTokTile;
  const int waves = m.E * n_tt;
  hipLaunchKernelGGL(router_logits_kernel, dim3((waves + 3) / 4), dim3(256), 0, stream,
                     static_cast<const uint16_t*>(x), w_router, bias, logits, m.S, m.d, m.E);
  hipLaunchKernelGGL(topk_kernel, dim3((m.S + 3) / 4), dim3(256), 0, stream, logits, topk_ids,
                     topk_w, m.S, m.E, m.topk, m.renorm);
  return launch_status();
}
