// route_dev.h -- router logits (fp32) and sigmoid top-k as device functions,
// used by the moe_route kernels and by moe_forward.
//
// Muse Spark K3 page, stage "A": router logits in fp32; stage "route": every
// token's top-8, identical wherever computed. K5 page, HA routing tail: top-8
// per token, ids and weights handed to the expert launch. The router bias
// (Kimi-K3 layer page, "k2_launch": router weight and bias) is either part of
// the logit, before ranking and sigmoid, or (selection-only) added to the
// ranking key alone while the sigmoid takes the unbiased logit: the K3 page's
// summary of "route_token" breaks off after "sigmoid +", which allows both.
#pragma once

#include "common.h"
#include "launch.h"

namespace moeblk {

constexpr int kTok = 8;  // tokens a router wave sums at once
constexpr int kMaxRouteTiles = 128 / kTok;  // S <= 128

// A DPP move of v within rows of 16 lanes (kCtrl: a dpp_ctrl value)
template <int kCtrl>
__device__ __forceinline__ float dpp_move(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xF, 0xF, false));
}

// 8 per-lane partial sums -> wave totals; lane l (l % 8 == 0) holds the total of
// value index ((l >> 5) & 1) * 4 + ((l >> 4) & 1) * 2 + ((l >> 3) & 1). Each step
// halves the values a lane keeps, adding a partner lane's: lane bit 5 through
// v_permlane32_swap (the swap of x's upper half with y's lower half leaves
// every lane the two addends of the half it keeps), bit 4 through
// v_permlane16_swap (odd rows with even rows), bit 3 through the DPP row
// mirror (lane i and 15 - i); then the 8 lanes of a group are summed with the
// half-row mirror and two quad permutations. No LDS; the order of additions
// is fixed.
__device__ __forceinline__ float reduce8(float (&v)[kTok], int lane) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[j]), __float_as_uint(v[4 + j]),
                                                    false, false);
    v[j] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v[j]), __float_as_uint(v[2 + j]),
                                                    false, false);
    v[j] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  const bool hi = lane & 8;
  const float send = hi ? v[0] : v[1];
  const float keep = hi ? v[1] : v[0];
  float s = keep + dpp_move<0x140>(send);  // row mirror: partner 15 - i
  s += dpp_move<0x141>(s);                 // half-row mirror: 7 - i within 8
  s += dpp_move<0x4E>(s);                  // quad [2, 3, 0, 1]
  s += dpp_move<0xB1>(s);                  // quad [1, 0, 3, 2]
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

// Sum of one token's NWV K-slice partials rt[slice][j], as a fixed pairwise
// tree: (0 + 1), (2 + 3), ..., then pairs of those, down to one value.
template <int NWV>
__device__ __forceinline__ float slice_tree(const float (*rt)[kTok], int j) {
  float q[NWV / 2];
#pragma unroll
  for (int i = 0; i < NWV / 2; ++i) q[i] = rt[2 * i][j] + rt[2 * i + 1][j];
#pragma unroll
  for (int n = NWV / 4; n >= 1; n >>= 1)
#pragma unroll
    for (int i = 0; i < n; ++i) q[i] = q[2 * i] + q[2 * i + 1];
  return q[0];
}

// Workgroup-level (NWV waves; kRouteThreads for the router launches): logits
// of expert row e for all S tokens. Wave w sums K slice w; lane l takes the float4s l, l + 64, .. (NW of them)
// of the slice. The router row is loaded once, all of it in flight at once
// (non-temporal: it is read once); activations stream in tiles of 8 tokens
// (with DB, the next tile's loads issue before the current tile is summed).
// Loads past the slice are clamped to its last float4 and not summed. Partial
// sums: a fixed shuffle tree in the wave into LDS `red` [tile][wave][token]
// (no barrier between tiles, so the waves stream their tiles independently),
// then, after one barrier, a fixed pairwise tree over the 16 slices.
template <int NW, bool DB, int NWV = kRouteWaves>
__device__ __forceinline__ void router_row(const uint16_t* __restrict__ x,
                                           const float* __restrict__ wr,
                                           const float* __restrict__ bias,
                                           float* __restrict__ logits, int S, int d, int E, int e,
                                           float (*red)[NWV][kTok]) {
  const int lane = threadIdx.x & (kWave - 1);
  const int w = threadIdx.x >> 6;
  const int kq = d / NWV;  // K of one wave
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
    if ((lane & 7) == 0) red[t0 / kTok][w][tok] = v;
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
  __syncthreads();
  for (int t = threadIdx.x; t < S; t += blockDim.x)
    logits[static_cast<size_t>(t) * E + e] = slice_tree<NWV>(red[t / kTok], t % kTok) + b;
}

// Larger S: kRouteBlockTok tokens x NE expert rows a workgroup. Every
// (token, expert) logit is summed exactly as router_row sums it (per-lane
// loop, shuffle tree, pairwise tree over the 16 K slices), so the two give
// the same bits; here each x tile a wave loads serves NE router rows, which
// cuts the x a workgroup reads from L2 to kRouteBlockTok / S of router_row's.
constexpr int kRouteBlockTok = 16;

template <int NW, int NE>
__device__ __forceinline__ void router_block(const uint16_t* __restrict__ x,
                                             const float* __restrict__ wr,
                                             const float* __restrict__ bias,
                                             float* __restrict__ logits, int S, int d, int E,
                                             int e0, int t0,
                                             float (*red)[kRouteWaves][kTok]) {
  const int lane = threadIdx.x & (kWave - 1);
  const int w = threadIdx.x >> 6;
  const int kq = d / kRouteWaves;
  const int nf = kq / 4;
  const int k0 = w * kq;
  const int tn = min(kRouteBlockTok, S - t0);
  int f[NW];
  bool live[NW];
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    live[i] = lane + kWave * i < nf;
    f[i] = min(lane + kWave * i, nf - 1);
  }
  f32x4_t wv[NE][NW];
#pragma unroll
  for (int j = 0; j < NE; ++j) {
    const float* wrow = wr + static_cast<size_t>(min(e0 + j, E - 1)) * d + k0;
#pragma unroll
    for (int i = 0; i < NW; ++i) wv[j][i] = ld_nt<f32x4_t>(wrow + 4 * f[i]);
  }
  const int tok = ((lane >> 5) & 1) * 4 + ((lane >> 4) & 1) * 2 + ((lane >> 3) & 1);
  for (int tile = 0; tile * kTok < tn; ++tile) {
    uint2 xv[kTok][NW];
#pragma unroll
    for (int t = 0; t < kTok; ++t) {
      const uint16_t* xr = x + static_cast<size_t>(min(t0 + tile * kTok + t, S - 1)) * d + k0;
#pragma unroll
      for (int i = 0; i < NW; ++i) xv[t][i] = *reinterpret_cast<const uint2*>(xr + 4 * f[i]);
    }
#pragma unroll
    for (int j = 0; j < NE; ++j) {
      float acc[kTok];
#pragma unroll
      for (int t = 0; t < kTok; ++t) {
        acc[t] = 0.0f;
#pragma unroll
        for (int i = 0; i < NW; ++i)
          if (live[i]) acc[t] = dot4(xv[t][i], wv[j][i], acc[t]);
      }
      const float v = reduce8(acc, lane);
      if ((lane & 7) == 0) red[tile * NE + j][w][tok] = v;
    }
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < tn * NE; idx += blockDim.x) {
    const int t = idx / NE, j = idx - t * NE;
    const int e = e0 + j;
    if (e >= E) continue;
    const float sum = slice_tree<kRouteWaves>(red[(t / kTok) * NE + j], t % kTok);
    logits[static_cast<size_t>(t0 + t) * E + e] = sum + (bias ? bias[e] : 0.0f);
  }
}

// router_row's logits of expert row e for all S tokens, bit for bit, from a
// workgroup of 4 waves (moe_forward's expert-FFN launch): wave w sums the K
// slices 4w .. 4w + 3 of the 16, each exactly as router_row's wave of that
// index sums it, with the activation tiles of SIF slices in flight at once;
// the same pairwise tree then adds the 16 slice sums. The logits are stored
// through to the coherence point, for other workgroups of the launch.
template <int NW, int SIF>
__device__ __forceinline__ void router_row_w4(const uint16_t* __restrict__ x,
                                              const float* __restrict__ wr,
                                              const float* __restrict__ bias,
                                              float* __restrict__ logits, int S, int d, int E,
                                              int e, float (*red)[kRouteWaves][kTok]) {
  constexpr int kVs = kRouteWaves / 4;  // slices a wave
  static_assert(kVs % SIF == 0, "slices in flight divide a wave's slices");
  const int lane = threadIdx.x & (kWave - 1);
  const int w = threadIdx.x >> 6;
  const int kq = d / kRouteWaves;
  const int nf = kq / 4;
  int f[NW];
  bool live[NW];
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    live[i] = lane + kWave * i < nf;
    f[i] = min(lane + kWave * i, nf - 1);
  }
  const float* wrow = wr + static_cast<size_t>(e) * d + kVs * w * kq;
  f32x4_t wv[kVs][NW];
#pragma unroll
  for (int s = 0; s < kVs; ++s)
#pragma unroll
    for (int i = 0; i < NW; ++i) wv[s][i] = ld_nt<f32x4_t>(wrow + s * kq + 4 * f[i]);
  const float b = bias ? bias[e] : 0.0f;
  const int tok = ((lane >> 5) & 1) * 4 + ((lane >> 4) & 1) * 2 + ((lane >> 3) & 1);
  const int n_tiles = (S + kTok - 1) / kTok;
  for (int tile = 0; tile < n_tiles; ++tile) {
#pragma unroll
    for (int s0 = 0; s0 < kVs; s0 += SIF) {
      uint2 xv[SIF][kTok][NW];
#pragma unroll
      for (int sl = 0; sl < SIF; ++sl)
#pragma unroll
        for (int t = 0; t < kTok; ++t) {
          const uint16_t* xr = x + static_cast<size_t>(min(tile * kTok + t, S - 1)) * d +
                               (kVs * w + s0 + sl) * kq;
#pragma unroll
          for (int i = 0; i < NW; ++i) xv[sl][t][i] = *reinterpret_cast<const uint2*>(xr + 4 * f[i]);
        }
#pragma unroll
      for (int sl = 0; sl < SIF; ++sl) {
        float acc[kTok];
#pragma unroll
        for (int t = 0; t < kTok; ++t) {
          acc[t] = 0.0f;
#pragma unroll
          for (int i = 0; i < NW; ++i)
            if (live[i]) acc[t] = dot4(xv[sl][t][i], wv[s0 + sl][i], acc[t]);
        }
        const float v = reduce8(acc, lane);
        if ((lane & 7) == 0) red[tile][kVs * w + s0 + sl][tok] = v;
      }
    }
  }
  __syncthreads();
  for (int t = threadIdx.x; t < S; t += blockDim.x)
    __hip_atomic_store(&logits[static_cast<size_t>(t) * E + e],
                       slice_tree<kRouteWaves>(red[t / kTok], t % kTok) + b, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}

// A logit as an unsigned key with the same order; -0 is folded into +0 so
// that both compare equal. Finite logits never map to 0.
__device__ __forceinline__ uint32_t order_key(float l) {
  const uint32_t u = __float_as_uint(l + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// the logit of an order key (-0 comes back as +0)
__device__ __forceinline__ float key_logit(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

__device__ __forceinline__ uint32_t umax32(uint32_t a, uint32_t b) { return a > b ? a : b; }

// maximum over the wave, in every lane: within each row of 16 lanes by DPP
// (pair swap, quad swap, half-row mirror, row mirror), then over the 4 rows
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = umax32(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0xB1, 0xF, 0xF, false)));
  v = umax32(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x4E, 0xF, 0xF, false)));
  v = umax32(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x141, 0xF, 0xF, false)));
  v = umax32(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x140, 0xF, 0xF, false)));
  const uint32_t r0 = __builtin_amdgcn_readlane(v, 15), r1 = __builtin_amdgcn_readlane(v, 31);
  const uint32_t r2 = __builtin_amdgcn_readlane(v, 47), r3 = __builtin_amdgcn_readlane(v, 63);
  return umax32(umax32(r0, r1), umax32(r2, r3));
}

// (ka, ia) ranks before (kb, ib): larger key, or equal key and lower id
struct NoMark {
  __device__ void operator()(int, int) const {}
};

__device__ __forceinline__ bool ranks_before(uint32_t ka, int ia, uint32_t kb, int ib) {
  return ka > kb || (ka == kb && ia < ib);
}

__device__ __forceinline__ void order2(uint32_t& ka, int& ia, uint32_t& kb, int& ib) {
  if (ranks_before(kb, ib, ka, ia)) {
    const uint32_t k = ka;
    const int i = ia;
    ka = kb;
    ia = ib;
    kb = k;
    ib = i;
  }
}

// order2 that also carries a value with each key
__device__ __forceinline__ void order2(uint32_t& ka, int& ia, float& la, uint32_t& kb, int& ib,
                                       float& lb) {
  if (ranks_before(kb, ib, ka, ia)) {
    const float l = la;
    la = lb;
    lb = l;
  }
  order2(ka, ia, kb, ib);
}

// Wave-level: the top-k of token t; lane l holds experts l, l + 64, l + 128,
// l + 192 (E <= 256).
// 1. Each lane orders its 4 experts (larger logit first, equal logits lower id
//    first): a 5-comparator network.
// 2. k rounds: the wave maximum of the lanes' first keys is the next slot;
//    among lanes tied at that key the lowest expert id wins; the winning lane
//    drops its first entry.
// 3. Lane s < k holds slot s: sigmoid score, renormalised by the sum of the k
//    scores in slot order.
// kSel (selection-only bias): the key is fl(logit + sel_bias[e]) and the
// sigmoid takes the unbiased logit, which travels with its key through the
// ordering.
// ids_lds: if not NULL, the ids are also written there ([t * topk + slot]);
// mark(id, t) runs for each of the token's ids (lanes < topk).
// topk_token_vals: the same with the token's logits already in registers
// (lane l: lv[j] = logit of expert l + 64 j, any value for ids >= E).
// kCohIds: the ids and weights are stored through to the coherence point
// (sc1), for other workgroups of the same launch to read.
template <bool kSel, class Mark, bool kCohIds = false>
__device__ __forceinline__ void topk_token_vals(const float (&lv)[4],
                                                const float* __restrict__ sel_bias,
                                                int32_t* __restrict__ ids, float* __restrict__ w,
                                                int32_t* ids_lds, int E, int topk, int renorm,
                                                int t, Mark mark) {
  const int lane = threadIdx.x & (kWave - 1);
  uint32_t k[4];
  int id[4];
  float lg[4];  // kSel: the unbiased logits
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = lane + kWave * j;
    lg[j] = e < E ? lv[j] : 0.0f;
    if constexpr (kSel) k[j] = e < E ? order_key(lg[j] + sel_bias[e]) : 0u;
    else k[j] = e < E ? order_key(lg[j]) : 0u;  // 0: below every expert
    id[j] = e;
  }
  if constexpr (kSel) {
    order2(k[0], id[0], lg[0], k[1], id[1], lg[1]);
    order2(k[2], id[2], lg[2], k[3], id[3], lg[3]);
    order2(k[0], id[0], lg[0], k[2], id[2], lg[2]);
    order2(k[1], id[1], lg[1], k[3], id[3], lg[3]);
    order2(k[1], id[1], lg[1], k[2], id[2], lg[2]);
  } else {
    order2(k[0], id[0], k[1], id[1]);
    order2(k[2], id[2], k[3], id[3]);
    order2(k[0], id[0], k[2], id[2]);
    order2(k[1], id[1], k[3], id[3]);
    order2(k[1], id[1], k[2], id[2]);
  }

  uint32_t my_key = 0;
  int my_id = 0;
  float my_lg = 0.0f;
  for (int r = 0; r < topk; ++r) {
    const uint32_t m = wave_max_u32(k[0]);
    const uint64_t tie = __ballot(k[0] == m);
    int wl = __builtin_ctzll(tie);
    int wid = __builtin_amdgcn_readlane(id[0], wl);
    if (__popcll(tie) > 1) {  // equal logits: the lowest expert id
      uint64_t rest = tie & (tie - 1ull);
      while (rest) {
        const int l = __builtin_ctzll(rest);
        rest &= rest - 1ull;
        const int il = __builtin_amdgcn_readlane(id[0], l);
        if (il < wid) {
          wid = il;
          wl = l;
        }
      }
    }
    if constexpr (kSel) {
      const float wlg = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(lg[0]), wl));
      if (lane == r) my_lg = wlg;
    }
    if (lane == r) {
      my_key = m;
      my_id = wid;
    }
    if (lane == wl) {
      k[0] = k[1];
      id[0] = id[1];
      k[1] = k[2];
      id[1] = id[2];
      k[2] = k[3];
      id[2] = id[3];
      k[3] = 0u;
      if constexpr (kSel) {
        lg[0] = lg[1];
        lg[1] = lg[2];
        lg[2] = lg[3];
      }
    }
  }
  const float l = kSel ? my_lg : key_logit(my_key);
  const float sc = 1.0f / (1.0f + expf(-l));
  float sum = 0.0f;
  for (int q = 0; q < topk; ++q)
    sum += __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(sc), q));
  if (lane < topk) {
    if constexpr (kCohIds)
      __hip_atomic_store(&ids[static_cast<size_t>(t) * topk + lane], my_id, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    else
      ids[static_cast<size_t>(t) * topk + lane] = my_id;
    if (ids_lds) ids_lds[t * topk + lane] = my_id;
    mark(my_id, t);
    const float wv = renorm ? sc / sum : sc;
    if constexpr (kCohIds)
      __hip_atomic_store(&w[static_cast<size_t>(t) * topk + lane], wv, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    else
      w[static_cast<size_t>(t) * topk + lane] = wv;
  }
}

template <bool kSel, class Mark, bool kCohIds = false>
__device__ __forceinline__ void topk_token(const float* __restrict__ logits,
                                           const float* __restrict__ sel_bias,
                                           int32_t* __restrict__ ids, float* __restrict__ w,
                                           int32_t* ids_lds, int E, int topk, int renorm, int t,
                                           Mark mark) {
  const int lane = threadIdx.x & (kWave - 1);
  float lv[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = lane + kWave * j;
    lv[j] = e < E ? logits[static_cast<size_t>(t) * E + e] : 0.0f;
  }
  topk_token_vals<kSel, Mark, kCohIds>(lv, sel_bias, ids, w, ids_lds, E, topk, renorm, t, mark);
}

// ---------------------------------------------------------------------------
// Router logits for S > 32 as a tiled product split over K, on bf16 MFMA
// (v_mfma_f32_16x16x32_bf16: A = 16 router rows x 32 K, B = 32 K x 16 tokens).
// The token rows are bf16 already; each fp32 router weight is split into three
// bf16 (split_bf16x3) whose sum is the weight exactly, and the three products
// with the bf16 token value are exact in fp32, so the three MFMAs a block add
// every exact product x w in fp32: the logit keeps fp32 accuracy (an
// accumulation order of its own) at 3 MFMAs of 16 cycles where the fp32
// 16 x 16 x 4 MFMA took 8 of 32 cycles.
//
// A workgroup of 4 waves owns TT tokens x 64 router rows over one K part of
// Kp: part p covers K [p Kp, (p + 1) Kp). It writes its tile unreduced to
// parts[p][t][e]; the top-k launch sums the parts in a fixed order. Tiles of
// TT x 64 load 2 / 64 + 4 / TT bytes per product, against 2 / NE + 4 / 16 for
// the 16-token x NE-row workgroups that take the whole K, and the K split
// keeps every CU busy.
//
// Wave w takes tokens (w & 1) TT / 2 .. + TT / 2 and rows (w >> 1) 32 .. + 32:
// NT = TT / 32 token tiles x 2 row tiles of 16 x 16. In a block of KB = 32 K a
// lane loads 8 consecutive K of one router row (32 bytes) and of one token row
// (8 bf16), K 8 (lane / 16) .. + 7 of the block: the MFMA's operand layout in
// both. The 16 lanes of one K group read whole 128-byte lines of 16 rows.
// Block b accumulates
// into set b % 4; the sets are added as (0 + 1) + (2 + 3), which keeps the
// sequential chains a quarter of the part. Rows past E and tokens past S
// repeat the last one and are not stored.
constexpr int kRouteTileE = 64;
#ifndef MOE_ROUTE_RING
#define MOE_ROUTE_RING 4
#endif
constexpr int kRouteRing = MOE_ROUTE_RING;  // blocks in flight a wave

template <int NT>
struct RouteBlk {
  f32x4_t w[2][kRouteKL / 4];     // 2 row tiles: KL K of this lane's row
  uint32_t x[NT][kRouteKL / 2];   // NT token tiles: KL bf16 of this lane's token
};

template <int NT>
__device__ __forceinline__ void route_blk_load(RouteBlk<NT>& b, const float* const (&wrow)[2],
                                               const uint16_t* const (&xrow)[NT], int blk) {
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int v = 0; v < kRouteKL / 4; ++v)
      b.w[i][v] = *reinterpret_cast<const f32x4_t*>(wrow[i] + kRouteKB * blk + 4 * v);
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    const uint4 u = *reinterpret_cast<const uint4*>(xrow[j] + kRouteKB * blk);
    b.x[j][0] = u.x; b.x[j][1] = u.y; b.x[j][2] = u.z; b.x[j][3] = u.w;
  }
}

// fp32 w as hi + mid + lo, three bf16 whose sum is w exactly: hi keeps the
// top 8 significant bits (truncated), mid the top 8 of the remainder, lo the
// rest (at most 8 bits); each subtraction is exact in fp32 (for |w| below
// about 2^-110 the remainders are subnormal and lo may drop low bits)
__device__ __forceinline__ void split_bf16x3(float w, uint32_t& hi, uint32_t& mid, uint32_t& lo) {
  const uint32_t wb = __float_as_uint(w);
  const uint32_t hb = wb & 0xffff0000u;
  const float r1 = w - __uint_as_float(hb);
  const uint32_t mb = __float_as_uint(r1) & 0xffff0000u;
  const float r2 = r1 - __uint_as_float(mb);
  hi = hb >> 16;
  mid = mb >> 16;
  lo = __float_as_uint(r2) >> 16;
}

template <int NT>
__device__ __forceinline__ void route_blk_mfma(const RouteBlk<NT>& b, f32x4_t (&acc)[2][NT]) {
  static_assert(kRouteKL == 8, "a lane's 8 K are the bf16 MFMA's operand");
  bf16x8_t xv[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j)
    xv[j] = __builtin_bit_cast(bf16x8_t, u32x4_t{b.x[j][0], b.x[j][1], b.x[j][2], b.x[j][3]});
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    uint32_t h[8], m[8], l[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) split_bf16x3(b.w[i][k / 4][k % 4], h[k], m[k], l[k]);
    u32x4_t hv, mv, lv;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      hv[q] = h[2 * q] | (h[2 * q + 1] << 16);
      mv[q] = m[2 * q] | (m[2 * q + 1] << 16);
      lv[q] = l[2 * q] | (l[2 * q + 1] << 16);
    }
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      acc[i][j] = mfma_bf16(__builtin_bit_cast(bf16x8_t, lv), xv[j], acc[i][j]);
      acc[i][j] = mfma_bf16(__builtin_bit_cast(bf16x8_t, mv), xv[j], acc[i][j]);
      acc[i][j] = mfma_bf16(__builtin_bit_cast(bf16x8_t, hv), xv[j], acc[i][j]);
    }
  }
}

// Workgroup (4 waves): tile (tt, et) of K part p.
template <int TT>
__device__ __forceinline__ void router_split_tile(const uint16_t* __restrict__ x,
                                                  const float* __restrict__ wr,
                                                  float* __restrict__ parts, int S, int d, int E,
                                                  int Kp, int tt, int et, int p) {
  constexpr int NT = TT / 32;
  constexpr int R = kRouteRing;
  const int lane = threadIdx.x & (kWave - 1);
  const int w = threadIdx.x >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int t0 = tt * TT + (w & 1) * (TT / 2);
  const int e0 = et * kRouteTileE + (w >> 1) * 32;
  const int k0 = p * Kp + kRouteKL * g;
  const float* wrow[2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
    wrow[i] = wr + static_cast<size_t>(min(e0 + 16 * i + c, E - 1)) * d + k0;
  const uint16_t* xrow[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j)
    xrow[j] = x + static_cast<size_t>(min(t0 + 16 * j + c, S - 1)) * d + k0;

  f32x4_t acc[4][2][NT];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < NT; ++j) acc[a][i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int nb = Kp / kRouteKB;
  RouteBlk<NT> ring[R];
#pragma unroll
  for (int i = 0; i < R; ++i) route_blk_load(ring[i], wrow, xrow, min(i, nb - 1));
  static_assert(R % 4 == 0, "block b goes to set b % 4");
  int b0 = 0;  // a multiple of R: block b0 + i goes to set i % 4
  for (; b0 + 2 * R <= nb; b0 += R) {
#pragma unroll
    for (int i = 0; i < R; ++i) {
      route_blk_mfma(ring[i], acc[i % 4]);
      route_blk_load(ring[i], wrow, xrow, b0 + i + R);
    }
  }
#pragma unroll
  for (int i = 0; i < R; ++i) {
    if (b0 + i < nb) {
      route_blk_mfma(ring[i], acc[i % 4]);
      if (b0 + i + R < nb) route_blk_load(ring[i], wrow, xrow, b0 + i + R);
    }
  }
#pragma unroll
  for (int i = 0; i < R; ++i)
    if (b0 + R + i < nb) route_blk_mfma(ring[i], acc[i % 4]);

  // lane holds rows e0 + 16 i + 4 g + r of token t0 + 16 j + c
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    const int t = t0 + 16 * j + c;
    if (t >= S) continue;
    float* prow = parts + (static_cast<size_t>(p) * S + t) * E;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const f32x4_t v = (acc[0][i][j] + acc[1][i][j]) + (acc[2][i][j] + acc[3][i][j]);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int e = e0 + 16 * i + 4 * g + r;
        if (e < E) prow[e] = v[r];
      }
    }
  }
}

// Workgroup (4 waves, kWave * 4 threads): logits of token t = the sum of its
// KP parts (wave w adds the parts w, w + 4, ... in order; then (0 + 1) +
// (2 + 3)) + bias, written to logits[t]; then wave 0 takes its top-k
// (kCohIds, mark: as topk_token_vals).
template <bool kSel, bool kCohIds = false, class Mark = NoMark>
__device__ __forceinline__ void topk_parts_token(const float* __restrict__ parts, int KP,
                                                 const float* __restrict__ lbias,
                                                 const float* __restrict__ sel_bias,
                                                 float* __restrict__ logits,
                                                 int32_t* __restrict__ ids, float* __restrict__ w,
                                                 int S, int E, int topk, int renorm, int t,
                                                 float (*red)[4][kWave], Mark mark = Mark{}) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = threadIdx.x >> 6;
  // every load of the wave's parts in flight at once, then the adds in order
  constexpr int kPartsAWave = kMaxRouteParts / 4;
  float v[kPartsAWave][4];
#pragma unroll
  for (int q = 0; q < kPartsAWave; ++q) {
    const int p = wv + 4 * q;
    const float* pr = parts + (static_cast<size_t>(min(p, KP - 1)) * S + t) * E;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = min(lane + kWave * j, E - 1);
      v[q][j] = pr[e];
    }
  }
  float s[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int q = 0; q < kPartsAWave; ++q)
    if (wv + 4 * q < KP)
#pragma unroll
      for (int j = 0; j < 4; ++j) s[j] += v[q][j];
#pragma unroll
  for (int j = 0; j < 4; ++j) red[wv][j][lane] = s[j];
  __syncthreads();
  if (wv != 0) return;
  float lv[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = lane + kWave * j;
    lv[j] = (red[0][j][lane] + red[1][j][lane]) + (red[2][j][lane] + red[3][j][lane]);
    if (e < E) {
      if (lbias) lv[j] += lbias[e];
      logits[static_cast<size_t>(t) * E + e] = lv[j];
    }
  }
  topk_token_vals<kSel, Mark, kCohIds>(lv, sel_bias, ids, w, nullptr, E, topk, renorm, t, mark);
}

}  // namespace moeblk
