// ffn.hip -- moe_expert_ffn: the expert FFNs of one step in one launch (tasks
// in ffn_dev.h).
//
// Workgroup ids are laid out so that every gate_up task (routed experts, then
// the shared expert) comes before every down task. A gate_up task writes its
// SwiGLU rows through to the coherence point and counts itself in
// prod[work item] once the stores are done; a down task first issues its weight
// prefetch, then waits until prod[work item] reaches the item's number of
// gate_up tasks, then loads the SwiGLU rows with coherent loads. The
// Kimi-K3 layer page's module docstring states the same order of work for its
// launch: weights are issued before the first wait, so they stream while the
// earlier stage settles.
//
// Forward progress: the launch holds no more workgroups than the device keeps
// resident at once, each workgroup runs all of its gate_up tasks before its
// first down task, and gate_up tasks wait for nothing. A wait that exceeds its
// bound (which a correct run never reaches; a device shared with other work
// could delay it) sets the error word and stops waiting.
//
// The counters return to zero within the launch: each down task counts itself
// in cons[work item] once past its wait, and the last one resets both words.
// They must therefore be zero before the first launch on a workspace.
#include "ffn_dev.h"
#include "ffn_launch.h"
#include "host.h"

namespace moeblk {

namespace {

constexpr long long kWaitCycles = 1ll << 31;  // wait bound, about a second

// thread 0 waits until *ctr >= target (bounded). The SwiGLU rows the counted
// tasks wrote are then read with coherent loads, so no cache invalidation is
// needed (a device-scope acquire fence would invalidate this XCD's whole L2).
struct WaitCount {
  const int32_t* ctr;
  int target;
  int32_t* error;
  __device__ void operator()() const {
    if (threadIdx.x == 0) {
      const long long t0 = clock64();
      while (__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
        __builtin_amdgcn_s_sleep(4);
        if (clock64() - t0 > kWaitCycles) {
          __hip_atomic_store(error, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          break;
        }
      }
    }
    __syncthreads();
  }
};

// The task's SwiGLU rows were written through (sc1 stores): once every thread
// has seen its stores complete, one count publishes them. (A device-scope
// release fence would write back this XCD's whole L2.)
__device__ __forceinline__ void publish(int32_t* ctr) {
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): this thread's stores are done
  __syncthreads();
  if (threadIdx.x == 0) __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// a down task is past its wait: the last of the item's n resets both counters
__device__ __forceinline__ void consume(int32_t* prod, int32_t* cons, int n) {
  if (threadIdx.x == 0) {
    const int old = __hip_atomic_fetch_add(cons, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (old == n - 1) {
      __hip_atomic_store(prod, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(cons, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// Persistent: the grid is the number of workgroups the device holds at once,
// and workgroup b runs tasks b, b + G, ... of the list [routed gate_up | shared
// gate_up | routed down | shared down]. Every gate_up task precedes every down
// task in the list, so a workgroup waits only after its own gate_up tasks are
// done, and those wait for nothing: all waits end.
// PG / PD: chunks in flight a wave in gate_up / down tasks
template <int TTG, int PG, int PD, bool kShared>
__global__ __launch_bounds__(kSplit * kWave, 2) void ffn_kernel(FfnArgs a) {
  __shared__ f32x4_t red[kSplit][2][4][kWave];
  auto red_r = reinterpret_cast<f32x4_t(*)[TTG][4][kWave]>(&red[0][0][0][0]);
  auto red_s = reinterpret_cast<f32x4_t(*)[kSharedTTG][4][kWave]>(&red[0][0][0][0]);
  constexpr int GS = 16 * kSharedTTG;
  const int lane = threadIdx.x & (kWave - 1);
  const int cnt = lane < a.n_loc ? a.counts[lane] : 0;  // this lane's expert's picks
  const int n_work = count_work<TTG>(cnt);
  const int RB13 = 2 * a.I / kRowsPerBlock, NC13 = a.d / kChunkK;
  const int RB2 = a.d / kRowsPerBlock, NC2 = a.I / kChunkK;
  const int RBs13 = kShared ? 2 * a.Is / kRowsPerBlock : 0, NCs2 = kShared ? a.Is / kChunkK : 1;
  const int n_sg = kShared ? (a.S + GS - 1) / GS : 0;
  const int A = n_work * RB13;  // routed gate_up
  const int B = n_sg * RBs13;   // shared gate_up
  const int C = n_work * RB2;   // routed down
  const int D = n_sg * RB2;     // shared down
  const int32_t* rows = a.rows;
  auto tok_of = [rows](int r) { return rows[r]; };
  auto same = [](int r) { return r; };

  for (int t = blockIdx.x; t < A + B + C + D; t += gridDim.x) {
    int id = t;
    if (id < A) {  // routed gate_up + SwiGLU
      const int wi = id / RB13, rb = id - wi * RB13;
      int el, row0, ntok;
      find_task<TTG>(cnt, wi, el, row0, ntok);
      const uint8_t* tiles = a.w13 + (static_cast<size_t>(el) * RB13 + rb) * NC13 * kMxTileBytes;
      ffn_task<true, TTG, PG, true>(tiles, NC13, a.x, a.d, row0, ntok, rb, a.h, a.I, tok_of,
                                    NoWait{}, red_r);
      publish(&a.prod[wi]);
      continue;
    }
    id -= A;
    if constexpr (kShared) {
      if (id < B) {  // shared gate_up + SwiGLU
        const int grp = id / RBs13, rb = id - grp * RBs13;
        const int row0 = grp * GS, ntok = min(GS, a.S - row0);
        const uint8_t* tiles = a.ws13 + static_cast<size_t>(rb) * NC13 * kBfTileBytes;
        ffn_task<false, kSharedTTG, kSharedP, true>(tiles, NC13, a.x, a.d, row0, ntok, rb, a.hs,
                                                    a.Is, same, NoWait{}, red_s);
        publish(&a.prod[a.max_work + grp]);
        continue;
      }
      id -= B;
    }
    if (id < C) {  // routed down
      const int wi = id / RB2, rb = id - wi * RB2;
      int el, row0, ntok;
      find_task<TTG>(cnt, wi, el, row0, ntok);
      const uint8_t* tiles = a.w2 + (static_cast<size_t>(el) * RB2 + rb) * NC2 * kMxTileBytes;
      ffn_task<true, TTG, PD, false>(tiles, NC2, a.h, a.I, row0, ntok, rb, a.y, a.d, same,
                                     WaitCount{&a.prod[wi], RB13, a.error}, red_r);
      consume(&a.prod[wi], &a.cons[wi], RB2);
      continue;
    }
    id -= C;
    if constexpr (kShared) {  // shared down
      const int grp = id / RB2, rb = id - grp * RB2;
      const int row0 = grp * GS, ntok = min(GS, a.S - row0);
      const uint8_t* tiles = a.ws2 + static_cast<size_t>(rb) * NCs2 * kBfTileBytes;
      int32_t* pc = &a.prod[a.max_work + grp];
      ffn_task<false, kSharedTTG, kSharedP, false>(
          tiles, NCs2, a.hs, a.Is, row0, ntok, rb, a.y + static_cast<size_t>(a.R_max) * a.d, a.d,
          same, WaitCount{pc, RBs13, a.error}, red_s);
      consume(pc, &a.cons[a.max_work + grp], RB2);
    }
  }
}

// workgroups of ffn_kernel<...> the device holds at once (cached per device)
template <int TTG, int PG, int PD, bool kShared>
int resident_grid() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (cache[dev] == 0) {
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &per_cu, reinterpret_cast<const void*>(&ffn_kernel<TTG, PG, PD, kShared>), kSplit * kWave,
            0) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return 0;
    cache[dev] = per_cu > 0 && cus > 0 ? per_cu * cus : 0;
  }
  return cache[dev];
}

template <int TTG, int PG, int PD, bool kShared>
int launch_k(const FfnArgs& a, hipStream_t stream) {
  const int grid = resident_grid<TTG, PG, PD, kShared>();
  if (grid <= 0) return MOE_ERR_HIP;
  hipLaunchKernelGGL((ffn_kernel<TTG, PG, PD, kShared>), dim3(grid), dim3(kSplit * kWave), 0,
                     stream, a);
  return MOE_OK;
}

}  // namespace

FfnLayout ffn_layout(const moe_dims& m) {
  const int R = r_max(m);
  const int mw = max_work(R, m.n_local, ffn_group(m));
  const int n_sg = m.shared_I ? (m.S + 16 * kSharedTTG - 1) / (16 * kSharedTTG) : 0;
  FfnLayout l;
  l.max_work = mw;
  l.h = 0;
  l.hs = round_up(static_cast<size_t>(R) * m.I * 2, 256);
  l.prod = l.hs + round_up(static_cast<size_t>(m.S) * m.shared_I * 2, 256);
  l.cons = l.prod + round_up(static_cast<size_t>(mw + n_sg) * 4, 256);
  l.error = l.cons + round_up(static_cast<size_t>(mw + n_sg) * 4, 256);
  l.total = l.error + 256;
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
  a.prod = reinterpret_cast<int32_t*>(ws + l.prod);
  a.cons = reinterpret_cast<int32_t*>(ws + l.cons);
  a.error = reinterpret_cast<int32_t*>(ws + l.error);
  a.S = m.S;
  a.d = m.d;
  a.I = m.I;
  a.Is = m.shared_I;
  a.n_loc = m.n_local;
  a.R_max = r_max(m);
  a.max_work = l.max_work;
  const bool big = ffn_group(m) > 16;
  int rc;
  if (m.shared_I) rc = big ? launch_k<2, 2, 2, true>(a, stream) : launch_k<1, 2, 4, true>(a, stream);
  else rc = big ? launch_k<2, 2, 2, false>(a, stream) : launch_k<1, 2, 4, false>(a, stream);
  return rc ? rc : launch_status();
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
