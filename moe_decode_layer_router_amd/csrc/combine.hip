// combine.hip -- per-pick RMSNorm and the routing-weighted sum.
//
// Muse Spark K3 page, stage "E": each pick's expert output is normalised (the
// post-expert norm) and the picks are summed with their routing weights into
// the expert-parallel partial, which stays fp32 (K5 page, HB: HM's partial).
// The RMSNorm form y / sqrt(mean(y^2) + eps) * w is the one of the KDA page's
// "kda_norm" and "stage_mix". One workgroup a token; slots in order. The sum of
// squares and the inverse root are fp64 (a bf16 row can reach 3e38, whose
// square overflows fp32); the weighted sum is fp32.
#include "common.h"
#include "host.h"

namespace moeblk {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

// block-wide sum, every thread gets it; fixed order (deterministic)
__device__ __forceinline__ double block_sum(double v, double* red) {
  v = wave_sum_f64(v);
  const int w = threadIdx.x >> 6;
  __syncthreads();  // red is reused across calls
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  double s = red[0];
#pragma unroll
  for (int i = 1; i < kThreads / kWave; ++i) s += red[i];
  return s;
}

// VPT: 8-element vectors a thread (d / 8 <= 256 * VPT)
template <int VPT>
__global__ __launch_bounds__(kThreads) void combine_kernel(
    const uint16_t* __restrict__ y, const float* __restrict__ tw, const int32_t* __restrict__ pick_pos,
    const uint16_t* __restrict__ gamma, float* __restrict__ out, int d, int topk, float eps,
    long shared_row0) {
  __shared__ double red[kThreads / kWave];
  const int t = blockIdx.x;
  const int nvec = d / 8;
  float acc[VPT][8], gam[VPT][8];
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    const int v = threadIdx.x + kThreads * i;
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
    double ss = 0.0;  // fp64: bf16 rows reach 3e38, their squares overflow fp32
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int v = threadIdx.x + kThreads * i;
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
    const int v = threadIdx.x + kThreads * i;
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

template <int VPT>
void launch(const moe_dims& m, const uint16_t* y, const float* tw, const int32_t* pp,
            const uint16_t* gamma, float* out, hipStream_t stream) {
  const long shared_row0 = m.shared_I > 0 ? static_cast<long>(r_max(m)) : -1;
  hipLaunchKernelGGL(combine_kernel<VPT>, dim3(m.S), dim3(kThreads), 0, stream, y, tw, pp, gamma,
                     out, m.d, m.topk, m.eps, shared_row0);
}

}  // namespace
}  // namespace moeblk

using namespace moeblk;

extern "C" int moe_combine(const moe_dims* dims, const void* y, const float* topk_w,
                           const int32_t* pick_pos, const void* gamma, float* out,
                           hipStream_t stream) {
  const int rc = check_dims(dims);
  if (rc) return rc;
  MOE_REQUIRE(y && topk_w && pick_pos && out, MOE_ERR_NULL);
  MOE_REQUIRE(aligned16(y) && aligned16(topk_w) && aligned16(pick_pos) && aligned16(out) &&
                  (!gamma || aligned16(gamma)),
              MOE_ERR_ALIGN);
  const moe_dims& m = *dims;
  const uint16_t* yy = static_cast<const uint16_t*>(y);
  const uint16_t* gg = static_cast<const uint16_t*>(gamma);
  const int nvec = m.d / 8;
  if (nvec <= 256) launch<1>(m, yy, topk_w, pick_pos, gg, out, stream);
  else if (nvec <= 512) launch<2>(m, yy, topk_w, pick_pos, gg, out, stream);
  else if (nvec <= 1024) launch<4>(m, yy, topk_w, pick_pos, gg, out, stream);
  else launch<8>(m, yy, topk_w, pick_pos, gg, out, stream);
  return launch_status();
}
