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
// The projection is one launch, a split-K bf16 GEMM built from the expert
// FFN's dense task (ffn_dev.h): a task is 64 weight rows x one
// group of 16 (S <= 16) or 32 tokens x one K part; its 4 waves stream the
// part's packed tiles and accumulate with bf16 MFMA, and the task writes an
// fp32 partial. The task that completes a (row block, token group) sums its
// parts in part order (deterministic) and rounds once to bf16. The token
// groups of one (row block, K part) run on one XCD and share its L2 for the
// weights (group_task). In moe_pre_expert the router rows on the same input
// are extra workgroups of the same launch (the K5 page's "router and
// pre_expert_proj" on ffn_in). The post step's 16-token tasks (S <= 16) read
// its fp32 input directly and round each value to bf16 where they use it;
// above, one small launch rounds the input first.
#include "combine_dev.h"
#include "ffn_dev.h"
#include "host.h"
#include "launch.h"
#include "route_dev.h"

namespace moeblk {
namespace {

constexpr int kProjP = 2;  // chunks in flight a wave

// tokens a task: 16 while S <= 16, else 32
inline int proj_ttg(const moe_proj_dims& m) { return m.S > 16 ? 2 : 1; }

// K parts: at least one 128-K chunk a wave in every part, and at most
// max(128, 2 S) tasks. The task that completes a (row block, token group)
// reads all of its parts, on one CU (about 28 GB/s), so more parts than that
// cost more in the sum than they gain in the spread. Measured, us, at the
// K5 page's shapes (pre: 512 rows, K = 8192 + 32 router rows; post: 1024
// rows, K = 4096), tasks at most 2048 / 256 / 128: S = 128 pre 24.8 / 14.1 /
// 16.4, post 17.8 / 13.4 / 15.0; S = 64 pre 13.9 / 13.9 / 10.7, post 12.9 /
// 13.2 / 12.2; S <= 16 unchanged.
#ifndef MOE_PROJ_MAX_PARTS
#define MOE_PROJ_MAX_PARTS 16
#endif
inline int proj_parts(const moe_proj_dims& m) {
  const int NC = m.K / kChunkK;
  const int G = 16 * proj_ttg(m);
  const int tasks = (m.N / kRowsPerBlock) * ((m.S + G - 1) / G);
  const int max_tasks = m.S * 2 > 128 ? m.S * 2 : 128;
  for (int kp = MOE_PROJ_MAX_PARTS; kp > 1; kp >>= 1)
    if (NC % kp == 0 && NC / kp >= kSplit && tasks * kp <= max_tasks) return kp;
  return 1;
}

// workspace: fp32 partials [KP][S][N], the counters [N / 64][token groups]
// (zero between calls), then at S > 16 the post step's bf16 input [S][K]
struct ProjLayout {
  size_t part, ctr, in16, total;
  int kp;
};

ProjLayout proj_layout(const moe_proj_dims& m) {
  ProjLayout l;
  l.kp = proj_parts(m);
  const int G = 16 * proj_ttg(m);
  l.part = 0;
  l.ctr = round_up(static_cast<size_t>(l.kp) * m.S * m.N * 4, 256);
  l.in16 = l.ctr + round_up(static_cast<size_t>(m.N / kRowsPerBlock) * ((m.S + G - 1) / G) * 4, 256);
  l.total = l.in16 + (proj_ttg(m) > 1 ? round_up(static_cast<size_t>(m.S) * m.K * 2, 256) : 0);
  return l;
}

struct ProjArgs {
  const uint8_t* w;   // packed dense weight [N][K]
  const uint16_t* in; // [S][K] bf16, or NULL with in32
  const float* in32;  // [S][K] fp32 (rounded to bf16 as the tasks use it), or NULL
  float* part;        // workspace: fp32 partials
  int32_t* ctr;       // workspace: parts done a (row block, token group)
  uint16_t* out;      // [S][N] bf16
  const float* wr;    // router rows [E][K] fp32
  const float* bias;  // [E] or NULL (added to the logit)
  float* logits;      // [S][E]
  int S, K, N, KP, E;
};

// float4s a lane of a router row split over the 4 waves: K <= 8192
inline int proj_router_nw(int K) { return K <= 1024 ? 1 : K <= 2048 ? 2 : K <= 4096 ? 4 : 8; }

constexpr int kRouterTok = 16;  // tokens a router workgroup

// Workgroups [0, E * ceil(S / 16)) (RNW > 0): one router row for 16 tokens
// each, its K split over the 4 waves (router_row). Then the projection tasks: task = (row
// block, K part) x token group; each writes its fp32 partial through to the
// coherence point and counts itself for its (row block, token group); the
// task that completes the count sums the KP partials in part order with
// coherent loads, rounds to bf16, writes the output and resets the count. No
// workgroup waits for another.
template <int TTG, int RNW, bool kF32In = false>
__global__ __launch_bounds__(kSplit * kWave, 2) void proj_kernel(ProjArgs a) {
  static_assert(!kF32In || RNW == 0, "router rows read bf16 rows");
  __shared__ f32x4_t red[kSplit][TTG][4][kWave];
  __shared__ int last;
  int t = blockIdx.x;
  if constexpr (RNW > 0) {
    // router workgroup t: row t % E for the 16 tokens of group t / E (the
    // groups of one row are E ids apart: the same XCD when E % 8 == 0)
    static_assert(sizeof(red) >= sizeof(float) * kMaxRouteTiles * kSplit * kTok, "router LDS");
    const int n_router = a.E * ((a.S + kRouterTok - 1) / kRouterTok);
    if (t < n_router) {
      const int e = t % a.E, t0 = (t / a.E) * kRouterTok;
      router_row<RNW, false, kSplit>(a.in + static_cast<size_t>(t0) * a.K, a.wr, a.bias,
                                     a.logits + static_cast<size_t>(t0) * a.E, min(kRouterTok, a.S - t0),
                                     a.K, a.E, e, reinterpret_cast<float(*)[kSplit][kTok]>(&red[0][0][0][0]));
      return;
    }
    t -= n_router;
  }
  constexpr int G = 16 * TTG;
  const int NC = a.K / kChunkK, NCp = NC / a.KP;
  const int ng = (a.S + G - 1) / G;
  int u, grp;
  group_task(t, ng, (a.N / kRowsPerBlock) * a.KP, u, grp);
  const int rb = u / a.KP, kp = u - rb * a.KP;
  const int row0 = grp * G, ntok = min(G, a.S - row0);
  const uint8_t* tiles =
      a.w + (static_cast<size_t>(rb) * NC + static_cast<size_t>(kp) * NCp) * kBfTileBytes;
  const size_t SN = static_cast<size_t>(a.S) * a.N;
  const size_t k0 = static_cast<size_t>(kp) * NCp * kChunkK;
  const uint16_t* bsrc =
      kF32In ? reinterpret_cast<const uint16_t*>(a.in32 + k0) : a.in + k0;
  static_assert(!kF32In || TTG == 1, "fp32 rows: 16-token tasks");
  ffn_task<false, TTG, kProjP, false, false, true, 0, false, kF32In>(
      tiles, NCp, bsrc, a.K, row0, ntok, rb, reinterpret_cast<uint16_t*>(a.part + kp * SN), a.N,
      [](int r) { return r; }, NoWait{}, red);

  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): this thread's partial stores are done
  __syncthreads();
  if (a.KP > 1) {
    int32_t* ctr = &a.ctr[rb * ng + grp];
    if (threadIdx.x == 0)
      last = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == a.KP - 1;
    __syncthreads();
    if (!last) return;
    if (threadIdx.x == 0) __hip_atomic_store(ctr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  // 4 outputs a thread: (token, 4 consecutive rows) of this row block
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(a.part, 0, 0x7fffffff, 0x00020000);
  constexpr int kQuads = kRowsPerBlock / 4;
  for (int i = threadIdx.x; i < ntok * kQuads; i += blockDim.x) {
    const int tok = row0 + i / kQuads;
    const int n = rb * kRowsPerBlock + 4 * (i % kQuads);
    const uint32_t off = static_cast<uint32_t>((static_cast<size_t>(tok) * a.N + n) * 4);
    f32x4_t pv[MOE_PROJ_MAX_PARTS];  // every part's load in flight, then the sum in part order
#pragma unroll
    for (int p = 0; p < MOE_PROJ_MAX_PARTS; ++p)
      if (p < a.KP)
        pv[p] = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                                rs, off + static_cast<uint32_t>(p * SN * 4), 0, kCpolSc1));
    f32x4_t v = pv[0];
#pragma unroll
    for (int p = 1; p < MOE_PROJ_MAX_PARTS; ++p)
      if (p < a.KP) v += pv[p];
    *reinterpret_cast<u32x2_t*>(a.out + static_cast<size_t>(tok) * a.N + n) =
        u32x2_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
  }
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

// the fp32 partial handed to the bf16 GEMM at S > 16: rounded to bf16 by a
// launch of its own, 4 values a thread (32-token tasks have no registers
// left for fp32 rows)
__global__ __launch_bounds__(256) void to_bf16_kernel(const float* __restrict__ in,
                                                      uint16_t* __restrict__ out, int n) {
  const int i = (blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= n) return;
  const f32x4_t v = *reinterpret_cast<const f32x4_t*>(in + i);
  *reinterpret_cast<u32x2_t*>(out + i) = u32x2_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
}

template <int TTG, int RNW>
void launch_proj_t(const ProjArgs& a, int grid, hipStream_t stream) {
  hipLaunchKernelGGL((proj_kernel<TTG, RNW>), dim3(grid), dim3(kSplit * kWave), 0, stream, a);
}

template <int TTG>
void launch_proj_r(const ProjArgs& a, int grid, hipStream_t stream) {
  if constexpr (TTG == 1) {
    if (a.in32) {
      hipLaunchKernelGGL((proj_kernel<1, 0, true>), dim3(grid), dim3(kSplit * kWave), 0, stream, a);
      return;
    }
  }
  if (a.E == 0) return launch_proj_t<TTG, 0>(a, grid, stream);
  switch (proj_router_nw(a.K)) {
    case 1: return launch_proj_t<TTG, 1>(a, grid, stream);
    case 2: return launch_proj_t<TTG, 2>(a, grid, stream);
    case 4: return launch_proj_t<TTG, 4>(a, grid, stream);
    default: return launch_proj_t<TTG, 8>(a, grid, stream);
  }
}

// The projection of in [S][K] bf16 (or in32 [S][K] fp32, each value rounded
// to bf16) through packed w into out [S][N] bf16, with E router rows of the
// same bf16 input in the same launch (E = 0: none)
void launch_proj(const moe_proj_dims& m, const uint16_t* in, const void* w_packed,
                 uint16_t* out, const float* wr, const float* bias, float* logits, int E,
                 void* workspace, hipStream_t stream, const float* in32 = nullptr) {
  const ProjLayout l = proj_layout(m);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  ProjArgs a{};
  a.w = static_cast<const uint8_t*>(w_packed);
  a.in = in;
  a.in32 = in32;
  a.part = reinterpret_cast<float*>(ws + l.part);
  a.ctr = reinterpret_cast<int32_t*>(ws + l.ctr);
  a.out = out;
  a.wr = wr;
  a.bias = bias;
  a.logits = logits;
  a.S = m.S;
  a.K = m.K;
  a.N = m.N;
  a.KP = l.kp;
  a.E = E;
  const int ttg = proj_ttg(m);
  const int ng = (m.S + 16 * ttg - 1) / (16 * ttg);
  const int grid = E * ((m.S + kRouterTok - 1) / kRouterTok) + (m.N / kRowsPerBlock) * l.kp * ng;
  ttg == 1 ? launch_proj_r<1>(a, grid, stream) : launch_proj_r<2>(a, grid, stream);
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
  const float* lbias = m.bias_mode == 0 ? bias : nullptr;  // else the top-k adds it to its key
  int fused_E = m.E;
  if (m.E > 0 && m.K > 8192) {  // wider rows: the router's own launch
    moe_dims r{};
    r.S = m.S;
    r.d = m.K;
    r.E = m.E;
    r.bias_mode = m.bias_mode;
    launch_router_logits(r, ffn_in, w_router, bias, logits, stream);
    fused_E = 0;
  }
  launch_proj(m, static_cast<const uint16_t*>(ffn_in), w_packed, static_cast<uint16_t*>(h_raw),
              w_router, lbias, logits, fused_E, workspace, stream);
  return launch_status();
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
  if (proj_ttg(m) == 1) {  // 16-token tasks round the fp32 rows as they use them
    launch_proj(m, nullptr, w_packed, static_cast<uint16_t*>(out), nullptr, nullptr, nullptr, 0,
                workspace, stream, partial);
  } else {
    uint16_t* in16 =
        reinterpret_cast<uint16_t*>(static_cast<uint8_t*>(workspace) + proj_layout(m).in16);
    const int n = m.S * m.K;
    hipLaunchKernelGGL(to_bf16_kernel, dim3((n / 4 + 255) / 256), dim3(256), 0, stream, partial,
                       in16, n);
    launch_proj(m, in16, w_packed, static_cast<uint16_t*>(out), nullptr, nullptr, nullptr, 0,
                workspace, stream);
  }
  return launch_status();
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
