// combine_dev.h -- per-pick RMSNorm and the routing-weighted sum of one token,
// as a workgroup-level device function (moe_combine and moe_forward).
//
// Muse Spark K3 page, stage "E": each pick's expert output is normalised (the
// post-expert norm) and the picks are summed with their routing weights into
// the expert-parallel partial, which stays fp32 (K5 page, HB: HM's partial).
// The RMSNorm form y / sqrt(mean(y^2) + eps) * w is the one of the KDA page's
// "kda_norm" and "stage_mix". Slots are taken in order. The sum of squares and
// the inverse root are fp64 (a bf16 row can reach 3e38, whose square overflows
// fp32); the weighted sum is fp32. For d <= 8192 a token's local picks are
// staged in LDS, four at a time, two waves a pick (combine_token_staged); for
// wider rows the slots' rows go through registers (combine_token_slots).
#pragma once

#include "common.h"

namespace moeblk {

// threads a token's workgroup: 8 waves, two a staged pick
#ifndef MOE_COMBINE_THREADS
#define MOE_COMBINE_THREADS 512
#endif
constexpr int kCombineThreads = MOE_COMBINE_THREADS;

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

// bf16x8 vectors a thread needs for a row of d: the kernels are instantiated
// for VPT in {1, 2, 4, 8}
inline int combine_vpt(int d) {
  const int nvec = d / 8;
  constexpr int T = kCombineThreads;
  return nvec <= T ? 1 : nvec <= 2 * T ? 2 : nvec <= 4 * T ? 4 : 8;
}

// 8 bf16 of y at element e (kCoh: written in the same launch by other
// workgroups, loaded from the coherence point)
template <bool kCoh>
__device__ __forceinline__ u32x4_t load_y8(const uint16_t* y, __amdgpu_buffer_rsrc_t yr, size_t e) {
  if constexpr (kCoh)
    return __builtin_amdgcn_raw_buffer_load_b128(yr, static_cast<uint32_t>(e * 2), 0, kCpolSc1);
  else
    return *reinterpret_cast<const u32x4_t*>(y + e);
}

// workgroup-wide sums of NB values at once (kCombineThreads, one barrier pair),
// every thread gets them; fixed order: the wave's butterfly, then the
// kCombineThreads / 64 waves in order
template <int NB>
__device__ __forceinline__ void block_sum_n(double (&v)[NB], double (*red)[kCombineThreads / kWave]) {
#pragma unroll
  for (int i = 0; i < NB; ++i) v[i] = wave_sum_f64(v[i]);
  const int w = threadIdx.x >> 6;
  __syncthreads();  // red is reused across calls
  if ((threadIdx.x & 63) == 0) {
#pragma unroll
    for (int i = 0; i < NB; ++i) red[i][w] = v[i];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    double s = red[i][0];
#pragma unroll
    for (int k = 1; k < kCombineThreads / kWave; ++k) s += red[i][k];
    v[i] = s;
  }
}

// slots of a token whose y rows are loaded together (measured: batching pays
// at d = 7168, not at d <= 4096)
template <int VPT>
constexpr int combine_batch() {
  return VPT * kCombineThreads == 1024 ? 2 : 1;
}

// combine_token_slots at 8 vectors a thread: the slots one at a time,
// their pick positions and weights read where they are used, gamma and the
// shared row read at use, so that the registers hold the accumulators and one
// y row. (Holding gamma, the shared row and the unrolled slots' state as well
// spilled 228 bytes a lane to scratch.) Same arithmetic, in the same order.
template <int VPT, bool kCoh>
__device__ __forceinline__ void combine_token_wide(const uint16_t* __restrict__ y,
                                                   const float* __restrict__ tw,
                                                   const int32_t* __restrict__ pick_pos,
                                                   const uint16_t* __restrict__ gamma,
                                                   float* __restrict__ out, int d, int topk,
                                                   float eps, long shared_row0, int t,
                                                   double (*red)[kCombineThreads / kWave]) {
  const int nvec = d / 8;
  float acc[VPT][8];
#pragma unroll
  for (int i = 0; i < VPT; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = 0.0f;
  __amdgpu_buffer_rsrc_t yr;
  if constexpr (kCoh)
    yr = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(y), 0, 0x7fffffff, 0x00020000);
  const double inv_d = 1.0 / static_cast<double>(d);
#pragma unroll 1
  for (int s = 0; s < topk; ++s) {
    const int p = pick_pos[static_cast<size_t>(t) * topk + s];  // the same in every thread
    if (p < 0) continue;
    const float wt = tw[static_cast<size_t>(t) * topk + s];
    u32x4_t q[VPT];
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int v = threadIdx.x + kCombineThreads * i;
      q[i] = u32x4_t{0u, 0u, 0u, 0u};
      if (v < nvec) {
        if constexpr (kCoh)
          q[i] = __builtin_amdgcn_raw_buffer_load_b128(
              yr, static_cast<uint32_t>((static_cast<size_t>(p) * d + 8 * v) * 2), 0, kCpolSc1);
        else
          q[i] = *reinterpret_cast<const u32x4_t*>(y + static_cast<size_t>(p) * d + 8 * v);
      }
    }
    double ss[1] = {0.0};
#pragma unroll
    for (int i = 0; i < VPT; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const double lo = bf16_lo(q[i][j]), hi = bf16_hi(q[i][j]);
        ss[0] += lo * lo;
        ss[0] += hi * hi;
      }
    block_sum_n<1>(ss, red);
    // the row's values are widened to fp64 again below instead of keeping
    // the widened copies of the sum of squares live (128 more registers)
#pragma unroll
    for (int i = 0; i < VPT; ++i) asm volatile("" : "+v"(q[i]));
    const double r = 1.0 / sqrt(ss[0] * inv_d + static_cast<double>(eps));
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int v = threadIdx.x + kCombineThreads * i;
      float g[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) g[j] = 1.0f;
      if (gamma && v < nvec) {
        const uint4 gv = *reinterpret_cast<const uint4*>(gamma + 8 * v);
        const uint32_t gw[4] = {gv.x, gv.y, gv.z, gv.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          g[2 * j] = bf16_lo(gw[j]);
          g[2 * j + 1] = bf16_hi(gw[j]);
        }
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[i][2 * j] += wt * (static_cast<float>(bf16_lo(q[i][j]) * r) * g[2 * j]);
        acc[i][2 * j + 1] += wt * (static_cast<float>(bf16_hi(q[i][j]) * r) * g[2 * j + 1]);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    const int v = threadIdx.x + kCombineThreads * i;
    if (v >= nvec) continue;
    if (shared_row0 >= 0) {
      const u32x4_t sh =
          *reinterpret_cast<const u32x4_t*>(y + static_cast<size_t>(shared_row0 + t) * d + 8 * v);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[i][2 * j] += bf16_lo(sh[j]);
        acc[i][2 * j + 1] += bf16_hi(sh[j]);
      }
    }
    float4* o = reinterpret_cast<float4*>(out + static_cast<size_t>(t) * d + 8 * v);
    o[0] = make_float4(acc[i][0], acc[i][1], acc[i][2], acc[i][3]);
    o[1] = make_float4(acc[i][4], acc[i][5], acc[i][6], acc[i][7]);
  }
}

// combine_token for d > 8192: the y rows of up to combine_batch() slots at
// once, whose norms share one block reduction (combine_token_wide at 8 vectors
// a thread); the weighted sum runs in slot order. red: LDS
// [8][kCombineThreads / kWave] doubles.
template <int VPT, bool kCoh = false>
__device__ __forceinline__ void combine_token_slots(const uint16_t* __restrict__ y,
                                                    const float* __restrict__ tw,
                                                    const int32_t* __restrict__ pick_pos,
                                                    const uint16_t* __restrict__ gamma,
                                                    float* __restrict__ out, int d, int topk,
                                                    float eps, long shared_row0, int t,
                                                    double (*red)[kCombineThreads / kWave]) {
  if constexpr (VPT >= 8) {
    combine_token_wide<VPT, kCoh>(y, tw, pick_pos, gamma, out, d, topk, eps, shared_row0, t, red);
    return;
  }
  constexpr int NB = combine_batch<VPT>();
  const int nvec = d / 8;
  int pp[8];
  float wt[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    pp[s] = s < topk ? pick_pos[static_cast<size_t>(t) * topk + s] : -1;
    wt[s] = s < topk ? tw[static_cast<size_t>(t) * topk + s] : 0.0f;
  }
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
  // the shared expert's row is loaded now, so that it arrives while the
  // routed picks are summed
  u32x4_t shq[VPT];
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    const int v = threadIdx.x + kCombineThreads * i;
    shq[i] = u32x4_t{0u, 0u, 0u, 0u};
    if (shared_row0 >= 0 && v < nvec)
      shq[i] = *reinterpret_cast<const u32x4_t*>(y + static_cast<size_t>(shared_row0 + t) * d + 8 * v);
  }
  __amdgpu_buffer_rsrc_t yr;
  if constexpr (kCoh)
    yr = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(y), 0, 0x7fffffff, 0x00020000);
  const double inv_d = 1.0 / static_cast<double>(d);
#pragma unroll
  for (int s0 = 0; s0 < 8; s0 += NB) {
    bool any = false;
#pragma unroll
    for (int b = 0; b < NB; ++b) any = any || pp[s0 + b] >= 0;
    if (!any) continue;  // uniform: every thread holds the same pick positions
    u32x4_t q[NB][VPT];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int i = 0; i < VPT; ++i) {
        const int v = threadIdx.x + kCombineThreads * i;
        const int p = pp[s0 + b];
        q[b][i] = u32x4_t{0u, 0u, 0u, 0u};
        if (p >= 0 && v < nvec) {
          if constexpr (kCoh)
            q[b][i] = __builtin_amdgcn_raw_buffer_load_b128(
                yr, static_cast<uint32_t>((static_cast<size_t>(p) * d + 8 * v) * 2), 0, kCpolSc1);
          else
            q[b][i] = *reinterpret_cast<const u32x4_t*>(y + static_cast<size_t>(p) * d + 8 * v);
        }
      }
    double ss[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      ss[b] = 0.0;
#pragma unroll
      for (int i = 0; i < VPT; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const double lo = bf16_lo(q[b][i][j]), hi = bf16_hi(q[b][i][j]);
          ss[b] += lo * lo;
          ss[b] += hi * hi;
        }
    }
    block_sum_n<NB>(ss, red);
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      if (pp[s0 + b] < 0) continue;
      const double r = 1.0 / sqrt(ss[b] * inv_d + static_cast<double>(eps));
#pragma unroll
      for (int i = 0; i < VPT; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc[i][2 * j] += wt[s0 + b] * (static_cast<float>(bf16_lo(q[b][i][j]) * r) * gam[i][2 * j]);
          acc[i][2 * j + 1] +=
              wt[s0 + b] * (static_cast<float>(bf16_hi(q[b][i][j]) * r) * gam[i][2 * j + 1]);
        }
    }
  }
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    const int v = threadIdx.x + kCombineThreads * i;
    if (v >= nvec) continue;
    if (shared_row0 >= 0) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[i][2 * j] += bf16_lo(shq[i][j]);
        acc[i][2 * j + 1] += bf16_hi(shq[i][j]);
      }
    }
    float4* o = reinterpret_cast<float4*>(out + static_cast<size_t>(t) * d + 8 * v);
    o[0] = make_float4(acc[i][0], acc[i][1], acc[i][2], acc[i][3]);
    o[1] = make_float4(acc[i][4], acc[i][5], acc[i][6], acc[i][7]);
  }
}

// local picks of a token staged at once (two waves each), and the LDS of a
// combine workgroup: kStagedPicks rows of up to MV vectors of 8 bf16
constexpr int kStagedPicks = 4;
constexpr int kMaxStagedVec = 1024;  // d <= 8192
template <int MV>
struct CombineLdsT {
  u32x4_t row[kStagedPicks][MV];
  double ss[kStagedPicks][2];  // the two halves' sums of squares
};
using CombineLds = CombineLdsT<kMaxStagedVec>;

// token t: out[t] = sum over slots s with pick_pos[s] >= 0 of
//   tw[s] * y[p] / sqrt(mean(y[p]^2) + eps) * gamma  (+ y[shared_row0 + t]),
// pick_pos and tw: the token's topk slots. The token's local picks are taken
// in slot order, kStagedPicks at a time: waves 2k and 2k + 1 load pick k's
// row once into LDS, each half of its vectors (wave 2k + h: vectors
// 64 (2i + h) + lane), and sum its squares in fp64 (a lane's vectors into 4
// sums by i mod 4, added as (0 + 1) + (2 + 3), then the wave's butterfly,
// then half 0 + half 1), so that all of the picks cost one round trip;
// r = 1 / sqrt(ss / d + eps). Then every thread adds the normalised rows in
// slot order from LDS, VPT vectors of 8 a thread, and the shared expert's row
// last. Those are the 8 waves of kCombineThreads threads; a workgroup of NT
// threads runs its wave w as waves w, w + NT / 64, ... and each thread takes
// VPT * kCombineThreads / NT vectors, so that every value is summed in the
// same order either way. A token's workgroup runs on one CU, whose loads
// stream at about 28 GB/s: a token moves (picks + 1) rows of d bf16 and its
// d fp32 outputs, the bound of the launch at S = 128. kCoh: the y rows were
// written in the same launch by other workgroups (sc1 loads).
// d <= 8 * VPT * kCombineThreads <= 8 * MV.
template <int VPT, bool kCoh = false, int NT = kCombineThreads, int MV = kMaxStagedVec>
__device__ __forceinline__ void combine_token_staged(const uint16_t* __restrict__ y,
                                                     const float* __restrict__ tw,
                                                     const int32_t* __restrict__ pick_pos,
                                                     const uint16_t* __restrict__ gamma,
                                                     float* __restrict__ out, int d, int topk,
                                                     float eps, long shared_row0, int t,
                                                     CombineLdsT<MV>& L) {
  constexpr int kVw = 2 * kStagedPicks;  // waves of the arithmetic
  static_assert(kCombineThreads / kWave == kVw, "two waves a staged pick");
  constexpr int PW = NT / kWave;         // waves of this workgroup
  static_assert(kVw % PW == 0, "each wave runs whole waves of the arithmetic");
  constexpr int kRuns = kVw / PW;
  constexpr int VT = VPT * kCombineThreads / NT;  // vectors a thread
  static_assert(VPT * kCombineThreads <= MV, "rows staged in LDS");
  const int nvec = d / 8;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & (kWave - 1);
  const __amdgpu_buffer_rsrc_t yr =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(y), 0, 0x7fffffff, 0x00020000);
  // the local picks in slot order (every thread holds the same)
  int lp[8] = {}, nl = 0;
  float lw[8] = {};
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const int p = s < topk ? pick_pos[s] : -1;
    const float wv = s < topk ? tw[s] : 0.0f;
#pragma unroll
    for (int b = 0; b <= s; ++b) {
      if (p >= 0 && b == nl) {
        lp[b] = p;
        lw[b] = wv;
      }
    }
    nl += p >= 0 ? 1 : 0;
  }
  // the shared expert's row is loaded now, so that it arrives while the
  // routed picks are summed
  u32x4_t shq[VT];
#pragma unroll
  for (int i = 0; i < VT; ++i) {
    const int v = threadIdx.x + NT * i;
    shq[i] = u32x4_t{0u, 0u, 0u, 0u};
    if (shared_row0 >= 0 && v < nvec)
      shq[i] = load_y8<kCoh>(y, yr, static_cast<size_t>(shared_row0 + t) * d + 8 * v);
  }
  float acc[VT][8], gam[VT][8];
#pragma unroll
  for (int i = 0; i < VT; ++i) {
    const int v = threadIdx.x + NT * i;
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
  constexpr int kPerLane = VPT * kCombineThreads / kWave / 2;  // a half row's vectors a lane
#pragma unroll
  for (int b0 = 0; b0 < 8; b0 += kStagedPicks) {
    if (b0 >= nl) break;  // uniform
    // waves 2k, 2k + 1: pick b0 + k into LDS, and its sum of squares
    u32x4_t q[kRuns][kPerLane];
#pragma unroll
    for (int m = 0; m < kRuns; ++m) {
      const int vw = w + PW * m, pk = vw >> 1, half = vw & 1;
      int p = 0;
#pragma unroll
      for (int k = 0; k < kStagedPicks; ++k)
        if (pk == k) p = lp[b0 + k];
      if (b0 + pk < nl) {
#pragma unroll
        for (int i = 0; i < kPerLane; ++i) {
          const int v = min(kWave * (2 * i + half) + lane, nvec - 1);
          q[m][i] = load_y8<kCoh>(y, yr, static_cast<size_t>(p) * d + 8 * v);
        }
      }
    }
#pragma unroll
    for (int m = 0; m < kRuns; ++m) {
      const int vw = w + PW * m, pk = vw >> 1, half = vw & 1;
      if (b0 + pk < nl) {
        double ss4[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
        for (int i = 0; i < kPerLane; ++i) {
          const int v = kWave * (2 * i + half) + lane;
          if (v >= nvec) continue;
          L.row[pk][v] = q[m][i];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const double lo = bf16_lo(q[m][i][j]), hi = bf16_hi(q[m][i][j]);
            ss4[i % 4] += lo * lo;
            ss4[i % 4] += hi * hi;
          }
        }
        const double ss = wave_sum_f64((ss4[0] + ss4[1]) + (ss4[2] + ss4[3]));
        if (lane == 0) L.ss[pk][half] = ss;
      }
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kStagedPicks; ++k) {
      if (b0 + k >= nl) break;  // uniform
      const double r =
          1.0 / sqrt((L.ss[k][0] + L.ss[k][1]) / static_cast<double>(d) + static_cast<double>(eps));
      float wt = 0.0f;
#pragma unroll
      for (int b = 0; b < 8; ++b)
        if (b == b0 + k) wt = lw[b];
#pragma unroll
      for (int i = 0; i < VT; ++i) {
        const int v = threadIdx.x + NT * i;
        if (v >= nvec) continue;
        const u32x4_t q = L.row[k][v];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc[i][2 * j] += wt * (static_cast<float>(bf16_lo(q[j]) * r) * gam[i][2 * j]);
          acc[i][2 * j + 1] += wt * (static_cast<float>(bf16_hi(q[j]) * r) * gam[i][2 * j + 1]);
        }
      }
    }
    __syncthreads();  // the staged rows are read before the next picks overwrite them
  }
#pragma unroll
  for (int i = 0; i < VT; ++i) {
    const int v = threadIdx.x + NT * i;
    if (v >= nvec) continue;
    if (shared_row0 >= 0) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[i][2 * j] += bf16_lo(shq[i][j]);
        acc[i][2 * j + 1] += bf16_hi(shq[i][j]);
      }
    }
    float4* o = reinterpret_cast<float4*>(out + static_cast<size_t>(t) * d + 8 * v);
    o[0] = make_float4(acc[i][0], acc[i][1], acc[i][2], acc[i][3]);
    o[1] = make_float4(acc[i][4], acc[i][5], acc[i][6], acc[i][7]);
  }
}

}  // namespace moeblk
