// route_dev.h -- router logits (fp32) and sigmoid top-k as device functions,
// used by the moe_route kernels and by moe_forward.
//
// Muse Spark K3 page, stage "A": router logits in fp32; stage "route": every
// token's top-8, identical wherever computed. K5 page, HA routing tail: top-8
// per token, ids and weights handed to the expert launch. The bias is added to
// the logit before ranking (Kimi-K3 layer page, "k2_launch": router weight and
// bias).
#pragma once

#include "common.h"

namespace moeblk {

constexpr int kTok = 8;  // tokens a wave sums at once

// 8 per-lane partial sums -> wave totals; lane l (l % 8 == 0) holds the total of
// value index ((l >> 5) & 1) * 4 + ((l >> 4) & 1) * 2 + ((l >> 3) & 1). Each step
// halves the values a lane keeps; the order of additions is fixed.
__device__ __forceinline__ float reduce8(float (&v)[kTok], int lane) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const bool hi = lane & 32;
    const float send = hi ? v[j] : v[4 + j];
    const float keep = hi ? v[4 + j] : v[j];
    v[j] = keep + __shfl_xor(send, 32, kWave);
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const bool hi = lane & 16;
    const float send = hi ? v[j] : v[2 + j];
    const float keep = hi ? v[2 + j] : v[j];
    v[j] = keep + __shfl_xor(send, 16, kWave);
  }
  {
    const bool hi = lane & 8;
    const float send = hi ? v[0] : v[1];
    const float keep = hi ? v[1] : v[0];
    v[0] = keep + __shfl_xor(send, 8, kWave);
  }
  float s = v[0];
  s += __shfl_xor(s, 4, kWave);
  s += __shfl_xor(s, 2, kWave);
  s += __shfl_xor(s, 1, kWave);
  return s;
}

__device__ __forceinline__ float dot4(uint2 xb, f32x4_t w, float a) {
  a += bf16_lo(xb.x) * w[0];
  a += bf16_hi(xb.x) * w[1];
  a += bf16_lo(xb.y) * w[2];
  a += bf16_hi(xb.y) * w[3];
  return a;
}

// float4s of one wave's K quarter a lane loads: the router kernels are
// instantiated for NW in {1, 2, 4, 8, 16}
inline int router_nw(int d) {
  const int nw = (d / 16 + kWave - 1) / kWave;
  return nw <= 1 ? 1 : nw <= 2 ? 2 : nw <= 4 ? 4 : nw <= 8 ? 8 : 16;
}

// Workgroup-level: logits of expert row e for all S tokens (256 threads). Its
// 4 waves split K into quarters; lane l takes the float4s l, l + 64, .. (NW of
// them) of its wave's quarter. The router row is loaded once, all of it in
// flight at once (non-temporal: it is read once); activations stream in tiles
// of 8 tokens (with DB, the next tile's loads issue before the current tile is
// summed). Loads past the quarter are clamped to its last float4 and not
// summed. Partial sums: a fixed shuffle tree, then the 4 quarters through LDS
// `red` [4][8] in wave order.
template <int NW, bool DB>
__device__ __forceinline__ void router_row(const uint16_t* __restrict__ x,
                                           const float* __restrict__ wr,
                                           const float* __restrict__ bias,
                                           float* __restrict__ logits, int S, int d, int E, int e,
                                           float (*red)[kTok]) {
  const int lane = threadIdx.x & (kWave - 1);
  const int w = threadIdx.x >> 6;
  const int kq = d / 4;   // K of one wave
  const int nf = kq / 4;  // its float4s
  const int k0 = w * kq;
  int f[NW];
  bool live[NW];
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    live[i] = lane + kWave * i < nf;
    f[i] = min(lane + kWave * i, nf - 1);
  }
  const float* wrow = wr + static_cast<size_t>(e) * d + k0;
  f32x4_t wv[NW];
#pragma unroll
  for (int i = 0; i < NW; ++i) wv[i] = ld_nt<f32x4_t>(wrow + 4 * f[i]);
  const float b = bias ? bias[e] : 0.0f;

  uint2 xa[kTok][NW], xb[kTok][DB ? NW : 1];
  auto load_tile = [&](auto& xv, int t0) {
#pragma unroll
    for (int t = 0; t < kTok; ++t) {
      const uint16_t* xr = x + static_cast<size_t>(min(t0 + t, S - 1)) * d + k0;
#pragma unroll
      for (int i = 0; i < NW; ++i) xv[t][i] = *reinterpret_cast<const uint2*>(xr + 4 * f[i]);
    }
  };
  auto sum_tile = [&](const auto& xv, int t0) {
    float acc[kTok];
#pragma unroll
    for (int t = 0; t < kTok; ++t) {
      acc[t] = 0.0f;
#pragma unroll
      for (int i = 0; i < NW; ++i)
        if (live[i]) acc[t] = dot4(xv[t][i], wv[i], acc[t]);
    }
    const float v = reduce8(acc, lane);
    const int tok = ((lane >> 5) & 1) * 4 + ((lane >> 4) & 1) * 2 + ((lane >> 3) & 1);
    __syncthreads();  // red of the previous tile consumed
    if ((lane & 7) == 0) red[w][tok] = v;
    __syncthreads();
    if (threadIdx.x < kTok && t0 + static_cast<int>(threadIdx.x) < S) {
      const int t = threadIdx.x;
      logits[static_cast<size_t>(t0 + t) * E + e] =
          ((red[0][t] + red[1][t]) + (red[2][t] + red[3][t])) + b;
    }
  };
  const int n_tiles = (S + kTok - 1) / kTok;
  if constexpr (!DB) {
    for (int tile = 0; tile < n_tiles; ++tile) {
      load_tile(xa, tile * kTok);
      sum_tile(xa, tile * kTok);
    }
  } else {
    load_tile(xa, 0);
    for (int tile = 0; tile < n_tiles; tile += 2) {
      if (tile + 1 < n_tiles) load_tile(xb, (tile + 1) * kTok);
      sum_tile(xa, tile * kTok);
      if (tile + 1 >= n_tiles) break;
      if (tile + 2 < n_tiles) load_tile(xa, (tile + 2) * kTok);
      sum_tile(xb, (tile + 1) * kTok);
    }
  }
}

// A logit as an unsigned key with the same order; -0 is folded into +0 so
// that both compare equal. Finite logits never map to 0.
__device__ __forceinline__ uint32_t order_key(float l) {
  const uint32_t u = __float_as_uint(l + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ int popc_ballot(bool p) { return __popcll(__ballot(p)); }

// Wave-level: the top-k of token t; lane l holds experts l, l + 64, l + 128,
// l + 192 (E <= 256).
// 1. Radix select on the order keys: the k-th largest key T (32 ballot steps).
// 2. Keys above T are in; keys equal to T are taken lowest id first.
// 3. A selected expert's slot is the number of selected ones ranking above it
//    (larger logit, or equal logit and lower id).
// 4. Sigmoid scores, renormalised by their sum in slot order.
// sl / se: this wave's 8-entry LDS scratch.
__device__ __forceinline__ void topk_token(const float* __restrict__ logits,
                                           int32_t* __restrict__ ids, float* __restrict__ w,
                                           int E, int topk, int renorm, int t, float* sl,
                                           int* se) {
  const int lane = threadIdx.x & (kWave - 1);
  float lg[4];
  uint32_t key[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = lane + kWave * j;
    lg[j] = e < E ? logits[static_cast<size_t>(t) * E + e] : 0.0f;
    key[j] = e < E ? order_key(lg[j]) : 0u;
  }
  uint32_t T = 0;
  for (int b = 31; b >= 0; --b) {
    const uint32_t c = T | (1u << b);
    int n = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) n += popc_ballot(key[j] >= c);
    if (n >= topk) T = c;
  }
  int gt = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) gt += popc_ballot(key[j] > T);
  const int need = topk - gt;  // ties at T still to take
  const uint64_t below = (1ull << lane) - 1ull;
  bool sel[4];
  int before = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint64_t eq = __ballot(key[j] == T);
    const int r = before + __popcll(eq & below);
    sel[j] = key[j] > T || (key[j] == T && r < need);
    before += __popcll(eq);
  }
  int slot[4] = {0, 0, 0, 0};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint64_t m = __ballot(sel[j]);
    while (m) {
      const int src = __builtin_ctzll(m);
      m &= m - 1ull;
      const uint32_t ks = __shfl(key[j], src, kWave);
      const int es = src + kWave * j;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int e = lane + kWave * jj;
        slot[jj] += (ks > key[jj] || (ks == key[jj] && es < e)) ? 1 : 0;
      }
    }
  }
#pragma unroll
  for (int j = 0; j < 4; ++j)
    if (sel[j]) {
      sl[slot[j]] = lg[j];
      se[slot[j]] = lane + kWave * j;
    }
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS writes done
  __builtin_amdgcn_wave_barrier();
  float sc[8], sum = 0.0f;
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    sc[s] = s < topk ? 1.0f / (1.0f + expf(-sl[s])) : 0.0f;
    sum += sc[s];
  }
  if (lane < topk) {
    float mine = 0.0f;
#pragma unroll
    for (int s = 0; s < 8; ++s)
      if (s == lane) mine = sc[s];
    ids[static_cast<size_t>(t) * topk + lane] = se[lane];
    w[static_cast<size_t>(t) * topk + lane] = renorm ? mine / sum : mine;
  }
  __builtin_amdgcn_wave_barrier();
}

}  // namespace moeblk
