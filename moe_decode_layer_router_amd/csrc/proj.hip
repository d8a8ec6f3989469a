// proj.hip -- the steps around the block: the dense latent projections and
// the latent norm (moe_pre_expert, moe_latent_norm, moe_post_expert), the
// dense weight packing, and top-k from given logits (moe_topk).
//
// Muse Spark K5 page, HA routing tail: ffn_in feeds both the router (fp32)
// and pre_expert_proj (dense bf16, a rank's share of rows, K in 8 parts over
// 8-CTA groups); after the all-gather, h = pre_expert_norm(h_raw) is the
// experts' input. HB and the K3 page, stage "F": post_expert_proj (a rank's
// share of rows, K in 4 parts) of the summed expert partial. The Kimi-K3
// layer page's latent MoE ("k2_launch": w_ld, ln_w, w_up) is the same chain.
//
// The projection is a split-K bf16 GEMM built from the expert FFN's dense
// task (ffn_dev.h): a task is 64 weight rows x one group of 16 (S <= 16) or 32
// tokens x one K part; its 4 waves stream the part's packed tiles and
// accumulate with bf16 MFMA, and the task writes an fp32 partial. A second
// launch sums the parts of each output in part order (deterministic) and
// rounds once to bf16. The token groups of one (row block, K part) run on one
// XCD and share its L2 for the weights (group_task).
#include "combine_dev.h"
#include "ffn_dev.h"
#include "host.h"
#include "launch.h"

namespace moeblk {

namespace {

constexpr int kProjP = 2;  // chunks in flight a wave

// tokens a task: 16 while S <= 16, else 32
inline int proj_ttg(const moe_proj_dims& m) { return m.S > 16 ? 2 : 1; }

// K parts: enough tasks to spread the weights over the chip, at least one
// 128-K chunk a wave in every part
inline int proj_parts(const moe_proj_dims& m) {
  const int NC = m.K / kChunkK;
  const int G = 16 * proj_ttg(m);
  const int tasks = (m.N / kRowsPerBlock) * ((m.S + G - 1) / G);
  for (int kp = 16; kp > 1; kp >>= 1)
    if (NC % kp == 0 && NC / kp >= kSplit && tasks * kp <= 2048) return kp;
  return 1;
}

struct ProjLayout {
  size_t part, in16, total;  // fp32 partials [KP][S][N]; bf16 input [S][K] (post)
  int kp;
};

ProjLayout proj_layout(const moe_proj_dims& m) {
  ProjLayout l;
  l.kp = proj_parts(m);
  l.part = 0;
  l.in16 = round_up(static_cast<size_t>(l.kp) * m.S * m.N * 4, 256);
  l.total = l.in16 + round_up(static_cast<size_t>(m.S) * m.K * 2, 256);
  return l;
}

// task = (row block, K part) x token group; the fp32 partial of part kp is
// part + kp * S * N, row-major [S][N]
template <int TTG>
__global__ __launch_bounds__(kSplit * kWave, 2) void proj_kernel(const uint8_t* __restrict__ w,
                                                                 const uint16_t* __restrict__ in,
                                                                 float* __restrict__ part, int S,
                                                                 int K, int N, int KP) {
  __shared__ f32x4_t red[kSplit][TTG][4][kWave];
  constexpr int G = 16 * TTG;
  const int NC = K / kChunkK, NCp = NC / KP;
  const int ng = (S + G - 1) / G;
  int u, grp;
  group_task(blockIdx.x, ng, (N / kRowsPerBlock) * KP, u, grp);
  const int rb = u / KP, kp = u - rb * KP;
  const int row0 = grp * G, ntok = min(G, S - row0);
  const uint8_t* tiles = w + (static_cast<size_t>(rb) * NC + static_cast<size_t>(kp) * NCp) * kBfTileBytes;
  float* out = part + static_cast<size_t>(kp) * S * N;
  ffn_task<false, TTG, kProjP, false, false, true>(
      tiles, NCp, in + static_cast<size_t>(kp) * NCp * kChunkK, K, row0, ntok, rb,
      reinterpret_cast<uint16_t*>(out), N, [](int r) { return r; }, NoWait{}, red);
}

// out[i] = bf16(sum over the K parts, in part order), 4 outputs a thread
__global__ __launch_bounds__(256) void proj_finish_kernel(const float* __restrict__ part,
                                                          uint16_t* __restrict__ out, int SN,
                                                          int KP) {
  const int i = (blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= SN) return;
  f32x4_t v = *reinterpret_cast<const f32x4_t*>(part + i);
  for (int kp = 1; kp < KP; ++kp) v += *reinterpret_cast<const f32x4_t*>(part + static_cast<size_t>(kp) * SN + i);
  *reinterpret_cast<u32x2_t*>(out + i) = u32x2_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
}

// the fp32 partial handed to the bf16 GEMM: round to bf16, 4 values a thread
__global__ __launch_bounds__(256) void to_bf16_kernel(const float* __restrict__ in,
                                                      uint16_t* __restrict__ out, int n) {
  const int i = (blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= n) return;
  const f32x4_t v = *reinterpret_cast<const f32x4_t*>(in + i);
  *reinterpret_cast<u32x2_t*>(out + i) = u32x2_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
}

// pre_expert_norm, one workgroup a token: the sum of squares in fp64 (each
// thread's vectors in order, then the wave tree, then the 4 waves in order),
// r = (ss / L + eps)^-1/2, h = bf16(h_raw * r * gamma) evaluated in fp64
constexpr int kNormThreads = 256;
constexpr int kNormMaxVec = 8;  // bf16x8 vectors a thread: L <= 16384

__global__ __launch_bounds__(kNormThreads) void latent_norm_kernel(const uint16_t* __restrict__ h_raw,
                                                                   const uint16_t* __restrict__ gamma,
                                                                   uint16_t* __restrict__ h, int L,
                                                                   float eps) {
  __shared__ double red[kNormThreads / kWave];
  const int t = blockIdx.x;
  const int nvec = L / 8;
  const u32x4_t* src = reinterpret_cast<const u32x4_t*>(h_raw + static_cast<size_t>(t) * L);
  u32x4_t v[kNormMaxVec];
  double ss = 0.0;
#pragma unroll
  for (int i = 0; i < kNormMaxVec; ++i) {
    const int j = threadIdx.x + kNormThreads * i;
    if (j < nvec) {
      v[i] = src[j];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const double a = bf16_lo(v[i][q]), b = bf16_hi(v[i][q]);
        ss += a * a;
        ss += b * b;
      }
    }
  }
  ss = wave_sum_f64(ss);
  if ((threadIdx.x & (kWave - 1)) == 0) red[threadIdx.x / kWave] = ss;
  __syncthreads();
  double tot = red[0];
#pragma unroll
  for (int k = 1; k < kNormThreads / kWave; ++k) tot += red[k];
  const double r = 1.0 / sqrt(tot / L + static_cast<double>(eps));
  u32x4_t* dst = reinterpret_cast<u32x4_t*>(h + static_cast<size_t>(t) * L);
  const u32x4_t* gv = reinterpret_cast<const u32x4_t*>(gamma);
#pragma unroll
  for (int i = 0; i < kNormMaxVec; ++i) {
    const int j = threadIdx.x + kNormThreads * i;
    if (j < nvec) {
      const u32x4_t g = gamma ? gv[j] : u32x4_t{0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u};
      u32x4_t o;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t lo = f64_to_bf16_bits(static_cast<double>(bf16_lo(v[i][q])) * r * bf16_lo(g[q]));
        const uint32_t hi = f64_to_bf16_bits(static_cast<double>(bf16_hi(v[i][q])) * r * bf16_hi(g[q]));
        o[q] = lo | (hi << 16);
      }
      dst[j] = o;
    }
  }
}

// the projection of in [S][K] bf16 through packed w into out [S][N] bf16
int launch_proj(const moe_proj_dims& m, const uint16_t* in, const void* w_packed, uint16_t* out,
                void* workspace, hipStream_t stream) {
  const ProjLayout l = proj_layout(m);
  float* part = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + l.part);
  const int ttg = proj_ttg(m);
  const int ng = (m.S + 16 * ttg - 1) / (16 * ttg);
  const int grid = (m.N / kRowsPerBlock) * l.kp * ng;
  const uint8_t* w = static_cast<const uint8_t*>(w_packed);
  if (ttg == 1)
    hipLaunchKernelGGL(proj_kernel<1>, dim3(grid), dim3(kSplit * kWave), 0, stream, w, in, part, m.S,
                       m.K, m.N, l.kp);
  else
    hipLaunchKernelGGL(proj_kernel<2>, dim3(grid), dim3(kSplit * kWave), 0, stream, w, in, part, m.S,
                       m.K, m.N, l.kp);
  const int SN = m.S * m.N;
  hipLaunchKernelGGL(proj_finish_kernel, dim3((SN / 4 + 255) / 256), dim3(256), 0, stream, part, out,
                     SN, l.kp);
  return launch_status();
}

}  // namespace
}  // namespace moeblk

using namespace moeblk;

extern "C" int moe_check_proj_dims(const moe_proj_dims* dims) { return check_proj_dims(dims); }

extern "C" size_t moe_packed_dense_bytes(const moe_proj_dims* dims) {
  if (check_proj_dims(dims)) return 0;
  return static_cast<size_t>(dims->N) * dims->K * 2;
}

extern "C" int moe_pack_dense(const moe_proj_dims* dims, const void* w, void* packed,
                              hipStream_t stream) {
  const int rc = check_proj_dims(dims);
  if (rc) return rc;
  MOE_REQUIRE(w && packed, MOE_ERR_NULL);
  MOE_REQUIRE(aligned16(w) && aligned16(packed), MOE_ERR_ALIGN);
  launch_pack_bf16(static_cast<const uint16_t*>(w), packed, dims->N, dims->K, stream);
  return launch_status();
}

extern "C" size_t moe_proj_workspace_bytes(const moe_proj_dims* dims) {
  if (check_proj_dims(dims)) return 0;
  return proj_layout(*dims).total;
}

extern "C" int moe_pre_expert(const moe_proj_dims* dims, const void* ffn_in, const void* w_packed,
                              const float* w_router, const float* bias, float* logits, void* h_raw,
                              void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const int rc = check_proj_dims(dims);
  if (rc) return rc;
  const moe_proj_dims& m = *dims;
  MOE_REQUIRE(ffn_in && w_packed && h_raw && workspace, MOE_ERR_NULL);
  MOE_REQUIRE(m.E == 0 || (w_router && logits), MOE_ERR_NULL);
  MOE_REQUIRE(aligned16(ffn_in) && aligned16(w_packed) && aligned16(h_raw) && aligned16(workspace) &&
                  (!w_router || aligned16(w_router)) && (!logits || aligned16(logits)) &&
                  (!bias || aligned16(bias)),
              MOE_ERR_ALIGN);
  MOE_REQUIRE(workspace_bytes >= moe_proj_workspace_bytes(dims), MOE_ERR_WORKSPACE);
  if (m.E > 0) {
    moe_dims r{};
    r.S = m.S;
    r.d = m.K;
    r.E = m.E;
    r.bias_mode = m.bias_mode;
    launch_router_logits(r, ffn_in, w_router, bias, logits, stream);
  }
  return launch_proj(m, static_cast<const uint16_t*>(ffn_in), w_packed, static_cast<uint16_t*>(h_raw),
                     workspace, stream);
}

extern "C" int moe_latent_norm(const moe_proj_dims* dims, const void* h_raw, const void* gamma,
                               void* h, hipStream_t stream) {
  const int rc = check_proj_dims(dims);
  if (rc) return rc;
  MOE_REQUIRE(h_raw && h, MOE_ERR_NULL);
  MOE_REQUIRE(aligned16(h_raw) && aligned16(h) && (!gamma || aligned16(gamma)), MOE_ERR_ALIGN);
  hipLaunchKernelGGL(latent_norm_kernel, dim3(dims->S), dim3(kNormThreads), 0, stream,
                     static_cast<const uint16_t*>(h_raw), static_cast<const uint16_t*>(gamma),
                     static_cast<uint16_t*>(h), dims->N, dims->eps);
  return launch_status();
}

extern "C" int moe_post_expert(const moe_proj_dims* dims, const float* partial, const void* w_packed,
                               void* out, void* workspace, size_t workspace_bytes,
                               hipStream_t stream) {
  const int rc = check_proj_dims(dims);
  if (rc) return rc;
  const moe_proj_dims& m = *dims;
  MOE_REQUIRE(partial && w_packed && out && workspace, MOE_ERR_NULL);
  MOE_REQUIRE(aligned16(partial) && aligned16(w_packed) && aligned16(out) && aligned16(workspace),
              MOE_ERR_ALIGN);
  MOE_REQUIRE(workspace_bytes >= moe_proj_workspace_bytes(dims), MOE_ERR_WORKSPACE);
  const ProjLayout l = proj_layout(m);
  uint16_t* in16 = reinterpret_cast<uint16_t*>(static_cast<uint8_t*>(workspace) + l.in16);
  const int n = m.S * m.K;
  hipLaunchKernelGGL(to_bf16_kernel, dim3((n / 4 + 255) / 256), dim3(256), 0, stream, partial, in16, n);
  return launch_proj(m, in16, w_packed, static_cast<uint16_t*>(out), workspace, stream);
}

extern "C" int moe_topk(const moe_dims* dims, const float* logits, const float* bias,
                        int32_t* topk_ids, float* topk_w, hipStream_t stream) {
  const int rc = check_dims(dims);
  if (rc) return rc;
  MOE_REQUIRE(logits && topk_ids && topk_w, MOE_ERR_NULL);
  MOE_REQUIRE(aligned16(logits) && aligned16(topk_ids) && aligned16(topk_w) && (!bias || aligned16(bias)),
              MOE_ERR_ALIGN);
  launch_topk(*dims, logits, bias, topk_ids, topk_w, stream);
  return launch_status();
}
