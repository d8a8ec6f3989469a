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

constexpr int kTok = 8;  // tokens a router wave sums at once

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

// A router workgroup: 16 waves, each summing one sixteenth of K.
constexpr int kRouteWaves = 16;
constexpr int kRouteThreads = kRouteWaves * kWave;

// float4s of one wave's K slice a lane loads (d <= 16384): NW in {1, 2, 4}
inline int router_nw(int d) {
  const int nf = d / (4 * kRouteWaves);
  return nf <= kWave ? 1 : nf <= 2 * kWave ? 2 : 4;
}

// a logit store; kCoh: device-coherent (written through past this XCD's L2,
// for a reader on another XCD within the same launch)
template <bool kCoh>
__device__ __forceinline__ void store_logit(float* p, float v) {
  if constexpr (kCoh) __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else *p = v;
}

// Workgroup-level (kRouteThreads): logits of expert row e for all S tokens.
// Wave w sums K slice w; lane l takes the float4s l, l + 64, .. (NW of them)
// of the slice. The router row is loaded once, all of it in flight at once
// (non-temporal: it is read once); activations stream in tiles of 8 tokens
// (with DB, the next tile's loads issue before the current tile is summed).
// Loads past the slice are clamped to its last float4 and not summed. Partial
// sums: a fixed shuffle tree in the wave, then a fixed pairwise tree over the
// 16 slices through LDS `red`.
template <int NW, bool DB, bool kCoh>
__device__ __forceinline__ void router_row(const uint16_t* __restrict__ x,
                                           const float* __restrict__ wr,
                                           const float* __restrict__ bias,
                                           float* __restrict__ logits, int S, int d, int E, int e,
                                           float (*red)[kTok]) {
  const int lane = threadIdx.x & (kWave - 1);
  const int w = threadIdx.x >> 6;
  const int kq = d / kRouteWaves;  // K of one wave
  const int nf = kq / 4;           // its float4s
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
      float q[kRouteWaves / 2];
#pragma unroll
      for (int i = 0; i < kRouteWaves / 2; ++i) q[i] = red[2 * i][t] + red[2 * i + 1][t];
#pragma unroll
      for (int i = 0; i < kRouteWaves / 4; ++i) q[i] = q[2 * i] + q[2 * i + 1];
      const float sum = (q[0] + q[1]) + (q[2] + q[3]);
      store_logit<kCoh>(&logits[static_cast<size_t>(t0 + t) * E + e], sum + b);
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

// LDS scratch of one wave's top-k
struct TopkLds {
  uint32_t key[8];  // the selected experts, compacted: order keys,
  int32_t id[8];    // expert ids,
  float lg[8];      // logits
  float sl[8];      // the same in slot order
  int32_t se[8];
};

// Wave-level: the top-k of token t; lane l holds experts l, l + 64, l + 128,
// l + 192 (E <= 256).
// 1. Radix select on the order keys: the k-th largest key T (32 ballot steps).
// 2. Keys above T are in; keys equal to T are taken lowest id first.
// 3. The k selected are compacted into LDS; lane s < k ranks entry s against
//    the others (larger logit, or equal logit and lower id, ranks first): its
//    slot.
// 4. Sigmoid scores, renormalised by their sum in slot order.
// kCoh: the logits were written in the same launch by other workgroups (read
// past this XCD's L2). ids_lds: if not NULL, the ids are also written there
// ([t * topk + slot]).
template <bool kCoh>
__device__ __forceinline__ void topk_token(const float* __restrict__ logits,
                                           int32_t* __restrict__ ids, float* __restrict__ w,
                                           int32_t* ids_lds, int E, int topk, int renorm, int t,
                                           TopkLds& L) {
  const int lane = threadIdx.x & (kWave - 1);
  float lg[4];
  uint32_t key[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = lane + kWave * j;
    const float* p = logits + static_cast<size_t>(t) * E + e;
    if constexpr (kCoh)
      lg[j] = e < E ? __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0.0f;
    else
      lg[j] = e < E ? *p : 0.0f;
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
  int before = 0, nsel = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint64_t eq = __ballot(key[j] == T);
    const int r = before + __popcll(eq & below);
    const bool sel = key[j] > T || (key[j] == T && r < need);
    before += __popcll(eq);
    const uint64_t ms = __ballot(sel);
    if (sel) {
      const int pos = nsel + __popcll(ms & below);
      L.key[pos] = key[j];
      L.id[pos] = lane + kWave * j;
      L.lg[pos] = lg[j];
    }
    nsel += __popcll(ms);
  }
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS writes done
  __builtin_amdgcn_wave_barrier();
  if (lane < topk) {
    const uint32_t k = L.key[lane];
    const int id = L.id[lane];
    int slot = 0;
    for (int q = 0; q < topk; ++q) {
      const uint32_t kq = L.key[q];
      slot += (kq > k || (kq == k && L.id[q] < id)) ? 1 : 0;
    }
    L.sl[slot] = L.lg[lane];
    L.se[slot] = id;
  }
  __builtin_amdgcn_s_waitcnt(0xc07f);
  __builtin_amdgcn_wave_barrier();
  float sc[8], sum = 0.0f;
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    sc[s] = s < topk ? 1.0f / (1.0f + expf(-L.sl[s])) : 0.0f;
    sum += sc[s];
  }
  if (lane < topk) {
    float mine = 0.0f;
#pragma unroll
    for (int s = 0; s < 8; ++s)
      if (s == lane) mine = sc[s];
    const int id = L.se[lane];
    ids[static_cast<size_t>(t) * topk + lane] = id;
    if (ids_lds) ids_lds[t * topk + lane] = id;
    w[static_cast<size_t>(t) * topk + lane] = renorm ? mine / sum : mine;
  }
  __builtin_amdgcn_wave_barrier();
}

}  // namespace moeblk
