// ffn.hip -- the local experts' gate_up -> SwiGLU -> down.
//
// Muse Spark K3 page, stages "C, D": gate_up and down of the local experts with
// MXFP4 weights decoded in registers and fed to bf16 MFMA; functions "mx_chunk"
// and "fp4_mma": a 16-row MXFP4 group is processed in 256-K chunks of 8 MFMA
// steps with one e8m0 scale per 32 K. K5 page: every row tile is 16 tokens (the
// MFMA N dimension). The shared expert of the Kimi-K3 layer page ("k2_launch":
// w_sgu, w_sd) runs the same chain on dense bf16 weights.
//
// Work split. A workgroup of 4 waves owns one task: 64 weight rows (4 MFMA row
// tiles) of one expert against one group of up to 16 * TTG bucket rows. The
// four waves split K: wave w takes chunks c = w, w + 4, ... of 128 K, so the
// workgroup streams the task's packed tiles front to back. Each wave keeps P
// chunks of loads in flight (weights non-temporal, activations through the
// cache), decodes MXFP4 with the scaled fp4 -> bf16 converts and accumulates
// with v_mfma_f32_16x16x32_bf16. The four partial tiles are summed through LDS
// in wave order (deterministic), then the epilogue rounds to bf16 and, for
// gate_up, applies SwiGLU in registers: the packed row order gives each lane
// matching gate and up rows.
#include <type_traits>

#include "common.h"
#include "host.h"

namespace moeblk {
namespace {

constexpr int kSplit = 4;  // waves a workgroup, = row tiles a task

struct FfnArgs {
  const uint8_t* wp;        // packed weights
  const uint16_t* bsrc;     // B rows (x or h), row length K
  const int32_t* rows;      // bucket row -> B row (token); NULL: B row = bucket row
  const int32_t* counts;    // bucket sizes; NULL: one "expert" holding n_fixed rows
  uint16_t* out;            // output rows, indexed by bucket row
  int K, NC, RB;            // K, chunks (K / 128), row blocks (N / 64)
  int out_ld;               // output row length
  int n_fixed;              // rows of the single expert when counts == NULL
  int n_loc;                // local experts (entries of counts), <= 32
};

// Locate this workgroup's (expert, row group). Work items enumerate, for the
// local experts in order, their groups of 16 * TTG bucket rows (an expert
// without picks has none). Lane u reads expert u's count; wave prefix sums of
// the group counts and of the counts give the item's expert and its first
// bucket row (the bucket offsets are the exclusive prefix sums of the counts),
// so the lookup costs a single load.
template <int TTG>
__device__ __forceinline__ bool find_task(const FfnArgs& a, int wi, int lane, int& el, int& row0,
                                          int& ntok) {
  constexpr int G = 16 * TTG;
  if (!a.counts) {
    el = 0;
    row0 = wi * G;
    ntok = min(G, a.n_fixed - row0);
    return ntok > 0;
  }
  const int cnt = lane < a.n_loc ? a.counts[lane] : 0;
  const int ng = (cnt + G - 1) / G;
  int incl_ng = ng, incl_cnt = cnt;  // inclusive scans over lanes 0..31
#pragma unroll
  for (int m = 1; m < 32; m <<= 1) {
    const int o1 = __shfl_up(incl_ng, m, kWave);
    const int o2 = __shfl_up(incl_cnt, m, kWave);
    if (lane >= m) {
      incl_ng += o1;
      incl_cnt += o2;
    }
  }
  const uint64_t hit = __ballot(lane < a.n_loc && wi < incl_ng);
  if (hit == 0) return false;
  const int u = __builtin_ctzll(hit);
  const int g = wi - (__shfl(incl_ng, u, kWave) - __shfl(ng, u, kWave));
  const int c = __shfl(cnt, u, kWave);
  el = u;
  row0 = __shfl(incl_cnt, u, kWave) - c + g * G;
  ntok = min(G, c - g * G);
  return true;
}

template <int TTG>
struct MxChunk {
  u32x4_t w[4];         // 4 row tiles x 32 e2m1 codes a lane
  uint32_t s;           // the 4 row tiles' e8m0 bytes
  u32x4_t b[TTG][4];    // activations: 32 bf16 a lane a token tile
};

template <int TTG>
struct BfChunk {
  u32x4_t w[4][4];      // 4 row tiles x 4 MFMA steps x 8 bf16
  u32x4_t b[TTG][4];
};

// Loads are unconditional (every token tile, clamped chunk indices): the
// waitcnt insertion then sees one fixed issue order and keeps the ring in flight.
template <int TTG>
__device__ __forceinline__ void load_b(u32x4_t (&b)[TTG][4], const uint16_t* const (&bp)[TTG],
                                       int c) {
#pragma unroll
  for (int tt = 0; tt < TTG; ++tt) {
    const u32x4_t* p = reinterpret_cast<const u32x4_t*>(bp[tt] + c * kChunkK);
#pragma unroll
    for (int q = 0; q < 4; ++q) b[tt][q] = p[q];
  }
}

template <int TTG>
__device__ __forceinline__ void load_w(MxChunk<TTG>& ch, const uint8_t* wlane, const uint8_t* slane,
                                       int c) {
  const uint8_t* t = wlane + static_cast<size_t>(c) * kMxTileBytes;
#pragma unroll
  for (int r = 0; r < 4; ++r) ch.w[r] = ld_nt<u32x4_t>(t + r * 1024);
  ch.s = ld_nt<uint32_t>(slane + static_cast<size_t>(c) * kMxTileBytes);
}

template <int TTG>
__device__ __forceinline__ void load_w(BfChunk<TTG>& ch, const uint8_t* wlane, const uint8_t*,
                                       int c) {
  const uint8_t* t = wlane + static_cast<size_t>(c) * kBfTileBytes;
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int q = 0; q < 4; ++q) ch.w[r][q] = ld_nt<u32x4_t>(t + r * 4096 + q * 1024);
}

template <int TTG>
__device__ __forceinline__ void compute_chunk(const MxChunk<TTG>& ch, f32x4_t (&acc)[TTG][4],
                                              int n_tt) {
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float sc = e8m0_scale((ch.s >> (8 * r)) & 0xffu);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const bf16x8_t av = decode_fp4x8(ch.w[r][q], sc);
#pragma unroll
      for (int tt = 0; tt < TTG; ++tt)
        if (tt < n_tt)
          acc[tt][r] = mfma_bf16(av, __builtin_bit_cast(bf16x8_t, ch.b[tt][q]), acc[tt][r]);
    }
  }
}

template <int TTG>
__device__ __forceinline__ void compute_chunk(const BfChunk<TTG>& ch, f32x4_t (&acc)[TTG][4],
                                              int n_tt) {
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const bf16x8_t av = __builtin_bit_cast(bf16x8_t, ch.w[r][q]);
#pragma unroll
      for (int tt = 0; tt < TTG; ++tt)
        if (tt < n_tt)
          acc[tt][r] = mfma_bf16(av, __builtin_bit_cast(bf16x8_t, ch.b[tt][q]), acc[tt][r]);
    }
}

template <bool kMx, int TTG, int P, bool kGateUp>
__global__ __launch_bounds__(kSplit * kWave) void ffn_kernel(FfnArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int w = threadIdx.x >> 6;
  const int g = lane >> 4;
  const int col = lane & 15;

  const int wi = blockIdx.x / a.RB;
  const int rb = blockIdx.x - wi * a.RB;
  int el, row0, ntok;
  if (!find_task<TTG>(a, wi, lane, el, row0, ntok)) return;
  const int n_tt = (ntok + 15) / 16;

  constexpr int kTile = kMx ? kMxTileBytes : kBfTileBytes;
  const uint8_t* tiles =
      a.wp + (static_cast<size_t>(el) * a.RB + rb) * static_cast<size_t>(a.NC) * kTile;
  const uint8_t* wlane = tiles + lane * 16;
  const uint8_t* slane = tiles + 4096 + lane * 4;

  // this lane's B rows (token tile tt, column col); columns past the group's
  // rows repeat its last row and are never stored. The token lookup is issued
  // before the weights so that waiting for it leaves them in flight.
  int src[TTG];
#pragma unroll
  for (int tt = 0; tt < TTG; ++tt) {
    const int r = row0 + min(tt * 16 + col, ntok - 1);
    src[tt] = a.rows ? a.rows[r] : r;
  }

  using Chunk = typename std::conditional<kMx, MxChunk<TTG>, BfChunk<TTG>>::type;
  const int my_n = (a.NC - w + kSplit - 1) / kSplit;  // this wave's chunks: w, w + 4, ...
  Chunk ring[P];
#pragma unroll
  for (int i = 0; i < P; ++i) load_w<TTG>(ring[i], wlane, slane, min(w + kSplit * i, a.NC - 1));

  const uint16_t* bp[TTG];
#pragma unroll
  for (int tt = 0; tt < TTG; ++tt) bp[tt] = a.bsrc + static_cast<size_t>(src[tt]) * a.K + 32 * g;
#pragma unroll
  for (int i = 0; i < P; ++i) load_b<TTG>(ring[i].b, bp, min(w + kSplit * i, a.NC - 1));

  f32x4_t acc[TTG][4];
#pragma unroll
  for (int tt = 0; tt < TTG; ++tt)
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[tt][r] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  int j0 = 0;
  for (; j0 + 2 * P <= my_n; j0 += P) {  // steady state: every refill is needed
#pragma unroll
    for (int i = 0; i < P; ++i) {
      compute_chunk<TTG>(ring[i], acc, n_tt);
      const int c = w + kSplit * (j0 + i + P);
      load_w<TTG>(ring[i], wlane, slane, c);
      load_b<TTG>(ring[i].b, bp, c);
    }
  }
#pragma unroll
  for (int i = 0; i < P; ++i) {  // fewer than 2P chunks left
    if (j0 + i < my_n) {
      compute_chunk<TTG>(ring[i], acc, n_tt);
      if (j0 + i + P < my_n) {
        const int c = w + kSplit * (j0 + i + P);
        load_w<TTG>(ring[i], wlane, slane, c);
        load_b<TTG>(ring[i].b, bp, c);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < P; ++i)
    if (j0 + P + i < my_n) compute_chunk<TTG>(ring[i], acc, n_tt);

  // sum the 4 waves' partial tiles in wave order
  __shared__ f32x4_t red[kSplit][TTG][4][kWave];
#pragma unroll
  for (int tt = 0; tt < TTG; ++tt)
#pragma unroll
    for (int r = 0; r < 4; ++r) red[w][tt][r][lane] = acc[tt][r];
  __syncthreads();

  const int r = w;  // this thread finishes row tile r, MFMA lane `lane`
#pragma unroll
  for (int tt = 0; tt < TTG; ++tt) {
    if (tt >= n_tt) break;
    f32x4_t s = red[0][tt][r][lane];
#pragma unroll
    for (int ww = 1; ww < kSplit; ++ww) s += red[ww][tt][r][lane];
    const int c = tt * 16 + col;
    if (c >= ntok) continue;
    uint16_t* orow = a.out + static_cast<size_t>(row0 + c) * a.out_ld;
    if constexpr (kGateUp) {
      // rows 4g..4g+3 of tile r: gate i, gate i+1, up i, up i+1
      const float g0 = round_bf16(s[0]), g1 = round_bf16(s[1]);
      const float u0 = round_bf16(s[2]), u1 = round_bf16(s[3]);
      const int i0 = 32 * rb + 8 * r + 2 * g;
      *reinterpret_cast<uint32_t*>(orow + i0) = pack_bf16x2(silu(g0) * u0, silu(g1) * u1);
    } else {
      const int n0 = kRowsPerBlock * rb + 16 * r + 4 * g;
      *reinterpret_cast<u32x2_t*>(orow + n0) =
          u32x2_t{pack_bf16x2(s[0], s[1]), pack_bf16x2(s[2], s[3])};
    }
  }
}

template <bool kMx, int TTG, int P, bool kGateUp>
void launch(const FfnArgs& a, int n_work, hipStream_t stream) {
  hipLaunchKernelGGL((ffn_kernel<kMx, TTG, P, kGateUp>), dim3(n_work * a.RB), dim3(kSplit * kWave),
                     0, stream, a);
}

// upper bound of the work items: sum over experts of ceil(count / G)
int max_work(const moe_dims& m, int G) {
  const int R = r_max(m);
  const int experts = m.n_local < R ? m.n_local : R;
  return experts + R / G;
}

}  // namespace
}  // namespace moeblk

using namespace moeblk;

extern "C" size_t moe_ffn_workspace_bytes(const moe_dims* dims) {
  if (check_dims(dims)) return 0;
  const moe_dims& m = *dims;
  size_t b = round_up(static_cast<size_t>(r_max(m)) * m.I * 2, 256);
  b += round_up(static_cast<size_t>(m.S) * m.shared_I * 2, 256);
  return b;
}

extern "C" int moe_expert_ffn(const moe_dims* dims, const void* x, const void* w13_packed,
                              const void* w2_packed, const int32_t* counts,
                              const int32_t* offsets, const int32_t* rows,
                              const int32_t* active, const void* ws13_packed,
                              const void* ws2_packed, void* y, void* workspace,
                              size_t workspace_bytes, hipStream_t stream) {
  const int rc = check_dims(dims);
  if (rc) return rc;
  const moe_dims& m = *dims;
  MOE_REQUIRE(x && w13_packed && w2_packed && counts && offsets && rows && active && y && workspace,
              MOE_ERR_NULL);
  MOE_REQUIRE(m.shared_I == 0 || (ws13_packed && ws2_packed), MOE_ERR_NULL);
  MOE_REQUIRE(aligned16(x) && aligned16(w13_packed) && aligned16(w2_packed) && aligned16(counts) &&
                  aligned16(offsets) && aligned16(rows) && aligned16(active) && aligned16(y) &&
                  aligned16(workspace) && (!ws13_packed || aligned16(ws13_packed)) &&
                  (!ws2_packed || aligned16(ws2_packed)),
              MOE_ERR_ALIGN);
  MOE_REQUIRE(workspace_bytes >= moe_ffn_workspace_bytes(dims), MOE_ERR_WORKSPACE);

  const int R = r_max(m);
  uint16_t* h = static_cast<uint16_t*>(workspace);
  uint16_t* hs = reinterpret_cast<uint16_t*>(static_cast<uint8_t*>(workspace) +
                                             round_up(static_cast<size_t>(R) * m.I * 2, 256));
  uint16_t* yo = static_cast<uint16_t*>(y);
  const bool big = m.S > 16;  // expert buckets can exceed one 16-row tile

  FfnArgs gu{};
  gu.wp = static_cast<const uint8_t*>(w13_packed);
  gu.bsrc = static_cast<const uint16_t*>(x);
  gu.rows = rows;
  gu.counts = counts;
  gu.n_loc = m.n_local;
  gu.out = h;
  gu.K = m.d;
  gu.NC = m.d / kChunkK;
  gu.RB = 2 * m.I / kRowsPerBlock;
  gu.out_ld = m.I;

  FfnArgs dn = gu;
  dn.wp = static_cast<const uint8_t*>(w2_packed);
  dn.bsrc = h;
  dn.rows = nullptr;
  dn.out = yo;
  dn.K = m.I;
  dn.NC = m.I / kChunkK;
  dn.RB = m.d / kRowsPerBlock;
  dn.out_ld = m.d;

  if (!big) {
    launch<true, 1, 4, true>(gu, max_work(m, 16), stream);
    launch<true, 1, 4, false>(dn, max_work(m, 16), stream);
  } else {
    launch<true, 2, 3, true>(gu, max_work(m, 32), stream);
    launch<true, 2, 3, false>(dn, max_work(m, 32), stream);
  }

  if (m.shared_I > 0) {
    FfnArgs sg{};
    sg.wp = static_cast<const uint8_t*>(ws13_packed);
    sg.bsrc = static_cast<const uint16_t*>(x);
    sg.rows = nullptr;
    sg.counts = nullptr;
    sg.out = hs;
    sg.K = m.d;
    sg.NC = m.d / kChunkK;
    sg.RB = 2 * m.shared_I / kRowsPerBlock;
    sg.out_ld = m.shared_I;
    sg.n_fixed = m.S;
    FfnArgs sd = sg;
    sd.wp = static_cast<const uint8_t*>(ws2_packed);
    sd.bsrc = hs;
    sd.out = yo + static_cast<size_t>(R) * m.d;
    sd.K = m.shared_I;
    sd.NC = m.shared_I / kChunkK;
    sd.RB = m.d / kRowsPerBlock;
    sd.out_ld = m.d;
    const int groups = (m.S + 31) / 32;
    launch<false, 2, 2, true>(sg, groups, stream);
    launch<false, 2, 2, false>(sd, groups, stream);
  }
  return launch_status();
}
