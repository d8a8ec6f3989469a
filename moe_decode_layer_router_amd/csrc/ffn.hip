// ffn.hip -- moe_expert_ffn: the expert FFNs of one step as two launches,
// gate_up + SwiGLU, then down (tasks in ffn_dev.h).
//
// Muse Spark K3 page, stages "C, D": down needs every SwiGLU row of its expert,
// a dependency across all workgroups of the gate_up stage. Here the kernel
// boundary carries it. (Measured on MI355X: a dependent launch costs about
// 2.5 us; a barrier across a resident grid, or per-item counters polled by
// waiting workgroups, cost more than that at these sizes.)
//
// Grid of each launch: the shared expert's tasks first, then the routed work
// items in order (item-major, row block minor), then workgroups past the last
// item, which leave at once. The host does not know the bucket sizes, so the
// grid covers the largest possible number of items.
#include "ffn_dev.h"
#include "ffn_launch.h"
#include "host.h"

namespace moeblk {

namespace {

template <int TTG, int P, bool kShared>
__global__ __launch_bounds__(kSplit * kWave, 2) void gate_up_kernel(FfnArgs a) {
  __shared__ f32x4_t red[kSplit][kSharedTTG > TTG ? kSharedTTG : TTG][4][kWave];
  const int NC = a.d / kChunkK;
  int t = blockIdx.x;
  if constexpr (kShared) {
    constexpr int GS = 16 * kSharedTTG;
    const int RBs = 2 * a.Is / kRowsPerBlock;
    const int n_sg = (a.S + GS - 1) / GS;
    if (t < n_sg * RBs) {
      const int grp = t / RBs, rb = t - grp * RBs;
      const int row0 = grp * GS, ntok = min(GS, a.S - row0);
      const uint8_t* tiles = a.ws13 + static_cast<size_t>(rb) * NC * kBfTileBytes;
      ffn_task<false, kSharedTTG, kSharedP, true>(
          tiles, NC, a.x, a.d, row0, ntok, rb, a.hs, a.Is, [](int r) { return r; },
          reinterpret_cast<f32x4_t(*)[kSharedTTG][4][kWave]>(&red[0][0][0][0]));
      return;
    }
    t -= n_sg * RBs;
  }
  const int RB = 2 * a.I / kRowsPerBlock;
  const int wi = t / RB, rb = t - wi * RB;
  const int lane = threadIdx.x & (kWave - 1);
  const int cnt = lane < a.n_loc ? a.counts[lane] : 0;
  int el, row0, ntok;
  if (!find_task<TTG>(cnt, wi, el, row0, ntok)) return;
  const uint8_t* tiles = a.w13 + (static_cast<size_t>(el) * RB + rb) * NC * kMxTileBytes;
  const int32_t* rows = a.rows;
  ffn_task<true, TTG, P, true>(tiles, NC, a.x, a.d, row0, ntok, rb, a.h, a.I,
                               [rows](int r) { return rows[r]; },
                               reinterpret_cast<f32x4_t(*)[TTG][4][kWave]>(&red[0][0][0][0]));
}

template <int TTG, int P, bool kShared>
__global__ __launch_bounds__(kSplit * kWave, 2) void down_kernel(FfnArgs a) {
  __shared__ f32x4_t red[kSplit][kSharedTTG > TTG ? kSharedTTG : TTG][4][kWave];
  const int RB = a.d / kRowsPerBlock;
  auto same = [](int r) { return r; };
  int t = blockIdx.x;
  if constexpr (kShared) {
    constexpr int GS = 16 * kSharedTTG;
    const int n_sg = (a.S + GS - 1) / GS;
    if (t < n_sg * RB) {
      const int NCs = a.Is / kChunkK;
      const int grp = t / RB, rb = t - grp * RB;
      const int row0 = grp * GS, ntok = min(GS, a.S - row0);
      const uint8_t* tiles = a.ws2 + static_cast<size_t>(rb) * NCs * kBfTileBytes;
      ffn_task<false, kSharedTTG, kSharedP, false>(
          tiles, NCs, a.hs, a.Is, row0, ntok, rb, a.y + static_cast<size_t>(a.R_max) * a.d, a.d,
          same, reinterpret_cast<f32x4_t(*)[kSharedTTG][4][kWave]>(&red[0][0][0][0]));
      return;
    }
    t -= n_sg * RB;
  }
  const int NC = a.I / kChunkK;
  const int wi = t / RB, rb = t - wi * RB;
  const int lane = threadIdx.x & (kWave - 1);
  const int cnt = lane < a.n_loc ? a.counts[lane] : 0;
  int el, row0, ntok;
  if (!find_task<TTG>(cnt, wi, el, row0, ntok)) return;
  const uint8_t* tiles = a.w2 + (static_cast<size_t>(el) * RB + rb) * NC * kMxTileBytes;
  ffn_task<true, TTG, P, false>(tiles, NC, a.h, a.I, row0, ntok, rb, a.y, a.d, same,
                                reinterpret_cast<f32x4_t(*)[TTG][4][kWave]>(&red[0][0][0][0]));
}

// PG / PD: chunks in flight a wave in gate_up / down
template <int TTG, int PG, int PD, bool kShared>
void launch_pair(const FfnArgs& a, hipStream_t stream) {
  constexpr int GS = 16 * kSharedTTG;
  const int n_sg = kShared ? (a.S + GS - 1) / GS : 0;
  const int g1 = n_sg * (2 * a.Is / kRowsPerBlock) + a.max_work * (2 * a.I / kRowsPerBlock);
  const int g2 = (n_sg + a.max_work) * (a.d / kRowsPerBlock);
  hipLaunchKernelGGL((gate_up_kernel<TTG, PG, kShared>), dim3(g1), dim3(kSplit * kWave), 0, stream,
                     a);
  hipLaunchKernelGGL((down_kernel<TTG, PD, kShared>), dim3(g2), dim3(kSplit * kWave), 0, stream, a);
}

}  // namespace

FfnLayout ffn_layout(const moe_dims& m) {
  const int R = r_max(m);
  FfnLayout l;
  l.max_work = max_work(R, m.n_local, ffn_group(m));
  l.h = 0;
  l.hs = round_up(static_cast<size_t>(R) * m.I * 2, 256);
  l.total = l.hs + round_up(static_cast<size_t>(m.S) * m.shared_I * 2, 256);
  return l;
}

int launch_ffn(const moe_dims& m, const void* x, const void* w13, const void* w2, const void* ws13,
               const void* ws2, const int32_t* counts, const int32_t* rows, void* y,
               void* workspace, hipStream_t stream) {
  const FfnLayout l = ffn_layout(m);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  FfnArgs a{};
  a.w13 = static_cast<const uint8_t*>(w13);
  a.w2 = static_cast<const uint8_t*>(w2);
  a.ws13 = static_cast<const uint8_t*>(ws13);
  a.ws2 = static_cast<const uint8_t*>(ws2);
  a.x = static_cast<const uint16_t*>(x);
  a.rows = rows;
  a.counts = counts;
  a.h = reinterpret_cast<uint16_t*>(ws + l.h);
  a.hs = reinterpret_cast<uint16_t*>(ws + l.hs);
  a.y = static_cast<uint16_t*>(y);
  a.S = m.S;
  a.d = m.d;
  a.I = m.I;
  a.Is = m.shared_I;
  a.n_loc = m.n_local;
  a.R_max = r_max(m);
  a.max_work = l.max_work;
  const bool big = ffn_group(m) > 16;
  if (m.shared_I) big ? launch_pair<2, 2, 2, true>(a, stream) : launch_pair<1, 2, 4, true>(a, stream);
  else big ? launch_pair<2, 2, 2, false>(a, stream) : launch_pair<1, 2, 4, false>(a, stream);
  return launch_status();
}

}  // namespace moeblk

using namespace moeblk;

extern "C" size_t moe_ffn_workspace_bytes(const moe_dims* dims) {
  if (check_dims(dims)) return 0;
  return ffn_layout(*dims).total;
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
  return launch_ffn(m, x, w13_packed, w2_packed, ws13_packed, ws2_packed, counts, rows, y,
                    workspace, stream);
}
