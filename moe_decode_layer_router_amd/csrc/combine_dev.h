// combine_dev.h -- per-pick RMSNorm and the routing-weighted sum of one token,
// as a workgroup-level device function (moe_combine and moe_forward).
//
// Muse Spark K3 page, stage "E": each pick's expert output is normalised (the
// post-expert norm) and the picks are summed with their routing weights into
// the expert-parallel partial, which stays fp32 (K5 page, HB: HM's partial).
// The RMSNorm form y / sqrt(mean(y^2) + eps) * w is the one of the KDA page's
// "kda_norm" and "stage_mix". Slots are taken in order. The sum of squares and
// the inverse root are fp64 (a bf16 row can reach 3e38, whose square overflows
// fp32); the weighted sum is fp32.
#pragma once

#include "common.h"

namespace moeblk {

constexpr int kCombineThreads = 256;

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

// workgroup-wide sum (256 threads), every thread gets it; fixed order
__device__ __forceinline__ double block_sum(double v, double* red) {
  v = wave_sum_f64(v);
  const int w = threadIdx.x >> 6;
  __syncthreads();  // red is reused across calls
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  double s = red[0];
#pragma unroll
  for (int i = 1; i < kCombineThreads / kWave; ++i) s += red[i];
  return s;
}

// bf16x8 vectors a thread needs for a row of d: the kernels are instantiated
// for VPT in {1, 2, 4, 8}
inline int combine_vpt(int d) {
  const int nvec = d / 8;
  return nvec <= 256 ? 1 : nvec <= 512 ? 2 : nvec <= 1024 ? 4 : 8;
}

// token t: out[t] = sum over slots s with pick_pos >= 0 of
//   w[t][s] * y[p] / sqrt(mean(y[p]^2) + eps) * gamma  (+ y[shared_row0 + t])
template <int VPT>
__device__ __forceinline__ void combine_token(const uint16_t* __restrict__ y,
                                              const float* __restrict__ tw,
                                              const int32_t* __restrict__ pick_pos,
                                              const uint16_t* __restrict__ gamma,
                                              float* __restrict__ out, int d, int topk, float eps,
                                              long shared_row0, int t, double* red) {
  const int nvec = d / 8;
  float acc[VPT][8], gam[VPT][8];
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    const int v = threadIdx.x + kCombineThreads * i;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      acc[i][j] = 0.0f;
      gam[i][j] = 1.0f;
    }
    if (gamma && v < nvec) {
      const uint4 gv = *reinterpret_cast<const uint4*>(gamma + 8 * v);
      const uint32_t gw[4] = {gv.x, gv.y, gv.z, gv.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        gam[i][2 * j] = bf16_lo(gw[j]);
        gam[i][2 * j + 1] = bf16_hi(gw[j]);
      }
    }
  }
  const double inv_d = 1.0 / static_cast<double>(d);
  for (int s = 0; s < topk; ++s) {
    const int p = pick_pos[static_cast<size_t>(t) * topk + s];
    if (p < 0) continue;
    float yv[VPT][8];
    double ss = 0.0;
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int v = threadIdx.x + kCombineThreads * i;
#pragma unroll
      for (int j = 0; j < 8; ++j) yv[i][j] = 0.0f;
      if (v < nvec) {
        const uint4 q = *reinterpret_cast<const uint4*>(y + static_cast<size_t>(p) * d + 8 * v);
        const uint32_t qw[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          yv[i][2 * j] = bf16_lo(qw[j]);
          yv[i][2 * j + 1] = bf16_hi(qw[j]);
        }
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) ss += static_cast<double>(yv[i][j]) * yv[i][j];
    }
    ss = block_sum(ss, red);
    const double r = 1.0 / sqrt(ss * inv_d + static_cast<double>(eps));
    const float wt = tw[static_cast<size_t>(t) * topk + s];
#pragma unroll
    for (int i = 0; i < VPT; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j)
        acc[i][j] += wt * (static_cast<float>(yv[i][j] * r) * gam[i][j]);
  }
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    const int v = threadIdx.x + kCombineThreads * i;
    if (v >= nvec) continue;
    if (shared_row0 >= 0) {
      const uint4 q =
          *reinterpret_cast<const uint4*>(y + static_cast<size_t>(shared_row0 + t) * d + 8 * v);
      const uint32_t qw[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[i][2 * j] += bf16_lo(qw[j]);
        acc[i][2 * j + 1] += bf16_hi(qw[j]);
      }
    }
    float4* o = reinterpret_cast<float4*>(out + static_cast<size_t>(t) * d + 8 * v);
    o[0] = make_float4(acc[i][0], acc[i][1], acc[i][2], acc[i][3]);
    o[1] = make_float4(acc[i][4], acc[i][5], acc[i][6], acc[i][7]);
  }
}

}  // namespace moeblk
