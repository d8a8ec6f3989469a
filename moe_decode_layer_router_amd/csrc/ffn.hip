// ffn.hip -- moe_expert_ffn: the expert FFNs of one step (tasks in ffn_dev.h).
//
// Muse Spark K3 page, stages "C, D": down needs every SwiGLU row of its expert,
// a dependency across all workgroups of the gate_up stage. Two shapes:
//
// * Without a shared expert: ONE launch. Workgroup ids run over the gate_up
//   tasks, then the down tasks (item-major, row block minor), then workgroups
//   past the last item, which leave at once. Every workgroup reads the 32
//   bucket counts first, so the ids of real tasks are dense. A gate_up task
//   writes its SwiGLU rows through to the coherence point (sc1) and counts
//   itself in prod[item] once its stores are done; the last one of the item
//   sets a ready flag for each of the item's down tasks. A down task issues
//   its first weight loads, then waits for its flag, then reads the SwiGLU
//   rows with coherent loads: its weights stream while gate_up finishes. At
//   S > 32 each wave also stages two more weight chunks in LDS before it
//   waits.
// * With a shared expert: gate_up + SwiGLU, then down; the kernel boundary
//   carries the dependency. Grid of each: the shared expert's tasks first,
//   then the routed items, then workgroups past the last item. With 32-row
//   items (S > 16) the shared expert's tasks give each wave a row tile
//   (shared_rows_task), which lets the launches hold 3 (gate_up) and 4 (down)
//   workgroups a CU.
//
// Work items hold 16 bucket rows, or 32 with a shared expert at S > 16.
//
// The host does not know the bucket sizes, so a grid covers the largest
// possible number of items.
#include "bucket_dev.h"
#include "combine_dev.h"
#include "ffn_dev.h"
#include "ffn_launch.h"
#include "host.h"
#include "launch.h"
#include "route_dev.h"

namespace moeblk {

namespace {

constexpr long long kWaitCycles = 1ll << 31;  // wait bound, about a second

// thread 0 waits until its flag is set (bounded), then clears it for the next
// call. The SwiGLU rows the flag covers are then read with coherent loads, so
// no cache invalidation is needed (a device-scope acquire fence would
// invalidate this XCD's whole L2). Every down task polls its own 128-byte line:
// hundreds of workgroups polling one line would load a single memory channel.
struct WaitFlag {
  int32_t* flag;
  int32_t* error;
  __device__ void operator()() const {
    if (threadIdx.x == 0) {
      const long long t0 = clock64();
      while (__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0) {
        __builtin_amdgcn_s_sleep(8);
        if (clock64() - t0 > kWaitCycles) {
          __hip_atomic_store(error, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          break;
        }
      }
      __hip_atomic_store(flag, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
  }
};

// A gate_up task of a work item is done. Its SwiGLU rows were written through
// (sc1 stores): once every thread has seen its own stores complete, one count
// publishes them. (A device-scope release fence would write back this XCD's
// whole L2.) The task that brings the count to n resets it and sets the ready
// flag of each of the item's nd down tasks.
__device__ __forceinline__ void publish(int32_t* ctr, int n, int32_t* flags, int nd) {
  __shared__ int last;
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): this thread's stores are done
  __syncthreads();
  if (threadIdx.x == 0)
    last = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == n - 1;
  __syncthreads();
  if (!last) return;
  if (threadIdx.x == 0) __hip_atomic_store(ctr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  for (int i = threadIdx.x; i < nd; i += blockDim.x)
    __hip_atomic_store(&flags[i * kCtlStride], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// a workgroup that has read the routing counts itself on a seen line (one
// launch: the control block is cleared once every reader has)
__device__ __forceinline__ void count_seen(const FfnArgs& a) {
  if (threadIdx.x == 0)
    __hip_atomic_fetch_add(&a.rf.seen[(blockIdx.x % kSeenLines) * kCtlStride], 1, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}

// The routing front (moe_forward). With router rows (RNW > 0), workgroup
// b < E first computes expert row b's logits for every token (stored
// through) and counts itself on its router line; the rest of the front
// follows with b - E. Workgroup b < S takes token b's top-k (from the
// router's logits, or summing its K parts), sets the token's bit in the mask
// of each local expert it picked, and, once its stores are done, counts
// itself in every copy of the counter. Workgroup S waits for all S and
// writes the bucket outputs (ids stored through by the top-k workgroups, read
// back in one batch). smem: at least sizeof(BucketLds) + 4 KiB. kOne: the
// whole block is one launch (the bucketing counts itself as a reader).
template <int RNW, bool kOne>
__device__ __forceinline__ void route_front(const FfnArgs& a, int b, uint8_t* smem) {
  const RouteFront& f = a.rf;
  if constexpr (RNW > 0) {
    if (b < f.n_router) {
      router_row_w4<RNW, 4 / RNW>(a.x, f.wr, f.lbias, f.logits_out, a.S, a.d, f.E, b,
                                  reinterpret_cast<float(*)[kRouteWaves][kTok]>(smem));
      __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): this thread's logit stores are done
      __syncthreads();
      if (threadIdx.x == 0)
        __hip_atomic_fetch_add(&f.rdone[(b % kRouterLines) * kCtlStride], 1, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
      return;
    }
    b -= f.n_router;
  }
  if (b < a.S) {
    auto mark = [&](int id, int t) {
      const int el = id - f.local_base;
      if (el >= 0 && el < a.n_loc)
        __hip_atomic_fetch_or(&f.masks[el * 4 + (t >> 5)], 1u << (t & 31), __ATOMIC_RELAXED,
                              __HIP_MEMORY_SCOPE_AGENT);
    };
    if (f.parts) {
      auto red = reinterpret_cast<float(*)[4][kWave]>(smem);
      if (f.sel_bias)
        topk_parts_token<true, true>(f.parts, f.KP, f.lbias, f.sel_bias, f.logits_out, f.ids, f.w,
                                     a.S, f.E, f.topk, f.renorm, b, red, mark);
      else
        topk_parts_token<false, true>(f.parts, f.KP, f.lbias, nullptr, f.logits_out, f.ids, f.w,
                                      a.S, f.E, f.topk, f.renorm, b, red, mark);
    } else if (RNW > 0) {  // the router rows' logits, written in this launch
      if (threadIdx.x < kWave) {
        // lane l < kRouterLines watches line l until it holds its count of
        // router rows (bounded)
        const int lane = threadIdx.x;
        const int l = min(lane, kRouterLines - 1);
        const int need = (f.n_router - l + kRouterLines - 1) / kRouterLines;
        const long long t0 = clock64();
        while (!__all(__hip_atomic_load(&f.rdone[l * kCtlStride], __ATOMIC_RELAXED,
                                        __HIP_MEMORY_SCOPE_AGENT) >= need)) {
          __builtin_amdgcn_s_sleep(4);
          if (clock64() - t0 > kWaitCycles) {
            if (lane == 0) __hip_atomic_store(a.error, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            break;
          }
        }
        const __amdgpu_buffer_rsrc_t lr =
            __builtin_amdgcn_make_buffer_rsrc(f.logits_out, 0, 0x7fffffff, 0x00020000);
        float lv[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int e = min(lane + kWave * j, f.E - 1);
          lv[j] = __builtin_bit_cast(
              float, __builtin_amdgcn_raw_buffer_load_b32(
                         lr, static_cast<uint32_t>(b * f.E + e) * 4u, 0, kCpolSc1));
        }
        if (f.sel_bias)
          topk_token_vals<true, decltype(mark), true>(lv, f.sel_bias, f.ids, f.w, nullptr, f.E,
                                                      f.topk, f.renorm, b, mark);
        else
          topk_token_vals<false, decltype(mark), true>(lv, nullptr, f.ids, f.w, nullptr, f.E,
                                                       f.topk, f.renorm, b, mark);
      }
    } else if (threadIdx.x < kWave) {
      if (f.sel_bias)
        topk_token<true, decltype(mark), true>(f.logits_in, f.sel_bias, f.ids, f.w, nullptr, f.E,
                                               f.topk, f.renorm, b, mark);
      else
        topk_token<false, decltype(mark), true>(f.logits_in, nullptr, f.ids, f.w, nullptr, f.E,
                                                f.topk, f.renorm, b, mark);
    }
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): this thread's stores and atomics are done
    __syncthreads();
    if (a.S > kTopkLinesMinS) {
      if (threadIdx.x == 0)
        __hip_atomic_fetch_add(&f.tkc[(b % kTopkLines) * kCtlStride], 1, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    } else if (threadIdx.x < kDoneCopies) {
      __hip_atomic_fetch_add(&f.done[threadIdx.x * kCtlStride], 1, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
    }
    return;
  }
  if (a.S <= kTopkLinesMinS) {
    if (threadIdx.x == 0) {
      const long long t0 = clock64();
      while (__hip_atomic_load(f.done, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < a.S) {
        __builtin_amdgcn_s_sleep(4);
        if (clock64() - t0 > kWaitCycles) {
          __hip_atomic_store(a.error, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          break;
        }
      }
    }
  } else if (threadIdx.x < kWave) {
    // lane l < kTopkLines watches line l until it holds its count of top-k
    // workgroups (bounded), then the counter's copies are set to S
    const int lane = threadIdx.x;
    const int l = min(lane, kTopkLines - 1);
    const int need = (a.S - l + kTopkLines - 1) / kTopkLines;
    const long long t0 = clock64();
    while (!__all(__hip_atomic_load(&f.tkc[l * kCtlStride], __ATOMIC_RELAXED,
                                    __HIP_MEMORY_SCOPE_AGENT) >= need)) {
      __builtin_amdgcn_s_sleep(4);
      if (clock64() - t0 > kWaitCycles) {
        if (lane == 0) __hip_atomic_store(a.error, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
    }
    if (lane < kDoneCopies)
      __hip_atomic_store(&f.done[lane * kCtlStride], a.S, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if constexpr (kOne) count_seen(a);
  BucketLds& L = *reinterpret_cast<BucketLds*>(smem);
  int32_t* ids_l = reinterpret_cast<int32_t*>(smem + sizeof(BucketLds));
  bucket_clear(L);
  __syncthreads();
  // every token's ids into LDS, all loads in flight at once (coherent loads:
  // the top-k workgroups stored them in this launch)
  const int npick = a.S * f.topk;
  constexpr int kPer = kMaxTokens * 8 / (kSplit * kWave);
  const __amdgpu_buffer_rsrc_t ir =
      __builtin_amdgcn_make_buffer_rsrc(f.ids, 0, 0x7fffffff, 0x00020000);
  int32_t v[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int p = min(i * kSplit * kWave + static_cast<int>(threadIdx.x), npick - 1);
    v[i] = __builtin_amdgcn_raw_buffer_load_b32(ir, static_cast<uint32_t>(p) * 4u, 0, kCpolSc1);
  }
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int p = i * kSplit * kWave + threadIdx.x;
    if (p < npick) {
      ids_l[p] = v[i];
      const int el = v[i] - f.local_base;
      if (el >= 0 && el < a.n_loc) bucket_mark(L, el, p / f.topk);
    }
  }
  __syncthreads();
  bucket_finish(ids_l, a.S, f.topk, a.n_loc, f.local_base, a.R_max, L,
                const_cast<int32_t*>(a.counts), f.offsets, const_cast<int32_t*>(a.rows),
                f.pick_pos, f.active);
}

// A workgroup that needs the routing (j: its index among them) waits for its
// copy of the counter to reach S; then each wave's lane e < n_loc loads local
// expert e's token mask (coherent load) and returns its pick count.
__device__ __forceinline__ int wait_route(const FfnArgs& a, int j, uint32_t (&mk)[4]) {
  if (threadIdx.x == 0) {
    const int32_t* c = &a.rf.done[(j % kDoneCopies) * kCtlStride];
    const long long t0 = clock64();
    while (__hip_atomic_load(const_cast<int32_t*>(c), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT) < a.S) {
      __builtin_amdgcn_s_sleep(4);
      if (clock64() - t0 > kWaitCycles) {
        __hip_atomic_store(a.error, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
    }
  }
  __syncthreads();
  const int lane = threadIdx.x & (kWave - 1);
  const __amdgpu_buffer_rsrc_t mr =
      __builtin_amdgcn_make_buffer_rsrc(a.rf.masks, 0, 0x7fffffff, 0x00020000);
  const u32x4_t m = __builtin_amdgcn_raw_buffer_load_b128(
      mr, static_cast<uint32_t>(min(lane, 31)) * 16u, 0, kCpolSc1);
  int cnt = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    mk[w] = lane < a.n_loc ? m[w] : 0u;
    cnt += __popc(mk[w]);
  }
  return cnt;
}

// The tokens of bucket rows first .. first + ntok - 1 of local expert el (the
// rank-th set bit of its mask is its bucket row offset + rank) into list[]:
// wave 0 writes them, then the workgroup syncs. mk: the lanes' masks.
__device__ __forceinline__ void front_rows(const uint32_t (&mk)[4], int el, int first, int ntok,
                                           int32_t* list) {
  if (threadIdx.x < kWave) {
    const int lane = threadIdx.x;
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = __builtin_amdgcn_readlane(mk[i], el);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int t = lane + kWave * h;  // tokens t and t + 64
      const int wi = t >> 5;
      const uint32_t below = w[wi] & ((1u << (t & 31)) - 1u);
      int rank = __popc(below);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (i < wi) rank += __popc(w[i]);
      if (((w[wi] >> (t & 31)) & 1u) && rank >= first && rank < first + ntok) list[rank - first] = t;
    }
  }
  __syncthreads();
}

// One launch: a down task's y rows are stored through to the coherence point
// (sc1); once every thread's stores are done, the task counts each of its rows
// in its token's counter (tokc), d / 64 counts a local pick.
__device__ __forceinline__ void count_rows(const FfnArgs& a, const uint32_t (&mk)[4], int el,
                                           int first, int ntok, uint8_t* smem) {
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): this thread's y stores are done
  __syncthreads();                     // ... every thread's, and the task's LDS is free
  int32_t* list = reinterpret_cast<int32_t*>(smem);
  front_rows(mk, el, first, ntok, list);
  if (static_cast<int>(threadIdx.x) < ntok)
    __hip_atomic_fetch_add(&a.tokc[list[threadIdx.x] * kCtlStride], 1, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}

constexpr int kOneMaxVec = 512;  // d <= 4096 in one launch
struct OneCombineLds {
  int32_t pp[8];
  float wt[8];
  CombineLdsT<kOneMaxVec> c;
};

// One launch: token t's combine (K3 page, stage "E"), as the launch's last S
// workgroups. Its pick positions come from the masks, as the bucketing
// numbers them (expert el's bucket starts at the sum of the counts below el;
// the token's row in it is the rank of its bit in el's mask), its ids and
// weights from the top-k workgroups' stores (coherent loads); cnt / mk:
// wait_route's counts and masks. It waits until its d / 64 rows a local pick
// are counted (then resets its counter), sums them as moe_combine does, and
// counts itself; the last combine workgroup waits until every reader of the
// routing has counted itself and clears the front's control block for the
// next call.
__device__ __forceinline__ void combine_one(const FfnArgs& a, int t, int cnt,
                                            const uint32_t (&mk)[4], int n_readers,
                                            uint8_t* smem) {
  OneCombineLds& L = *reinterpret_cast<OneCombineLds*>(smem);
  const RouteFront& f = a.rf;
  const int lane = threadIdx.x & (kWave - 1);
  if (threadIdx.x < kWave) {
    int incl = cnt;
#pragma unroll
    for (int m = 1; m < 32; m <<= 1) {
      const int o = __shfl_up(incl, m, kWave);
      if (lane >= m) incl += o;
    }
    const int off = incl - cnt;
    int id = -1;
    float w = 0.0f;
    if (lane < f.topk) {
      const size_t i = static_cast<size_t>(t) * f.topk + lane;
      id = __hip_atomic_load(&f.ids[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      w = __hip_atomic_load(&f.w[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    const int el = id - f.local_base;
    const bool local = lane < f.topk && el >= 0 && el < a.n_loc;
    const int src = local ? el : 0;
    int rank = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t bits = __shfl(mk[i], src, kWave);
      if (i < (t >> 5)) rank += __popc(bits);
      else if (i == (t >> 5)) rank += __popc(bits & ((1u << (t & 31)) - 1u));
    }
    const int base = __shfl(off, src, kWave);
    const int n = __popcll(__ballot(local));
    if (lane < 8) {
      L.pp[lane] = local ? base + rank : -1;
      L.wt[lane] = w;
    }
    if (lane == 0) {  // this token's y rows
      int32_t* c = &a.tokc[t * kCtlStride];
      const int need = (a.d / kRowsPerBlock) * n;
      const long long t0 = clock64();
      while (__hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < need) {
        __builtin_amdgcn_s_sleep(4);
        if (clock64() - t0 > kWaitCycles) {
          __hip_atomic_store(a.error, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          break;
        }
      }
      __hip_atomic_store(c, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);  // for the next call
    }
  }
  __syncthreads();
  combine_token_staged<1, true, kSplit * kWave, kOneMaxVec>(a.y, L.wt, L.pp, a.gamma, a.out, a.d,
                                                            f.topk, a.eps, -1, t, L.c);
  // the last combine workgroup clears the control block once every reader
  // of the routing has counted itself
  __shared__ int last;
  if (threadIdx.x == 0)
    last = __hip_atomic_fetch_add(f.cdone, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
           a.comb - 1;
  __syncthreads();
  if (!last) return;
  if (threadIdx.x < kWave) {
    const long long t0 = clock64();
    for (;;) {
      int v = __hip_atomic_load(&f.seen[lane * kCtlStride], __ATOMIC_RELAXED,
                                __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
      if (v >= n_readers) break;
      __builtin_amdgcn_s_sleep(4);
      if (clock64() - t0 > kWaitCycles) {
        if (lane == 0) __hip_atomic_store(a.error, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
    }
  }
  __syncthreads();
  int32_t* blk = f.done;  // the front's control block starts with the counter copies
  for (int i = threadIdx.x; i < kFrontWords; i += blockDim.x)
    __hip_atomic_store(&blk[i], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The single launch (no shared expert), items of 16 bucket rows at every S;
// PG / PD: chunks in flight a wave in gate_up / down tasks. Forward progress:
// every gate_up workgroup id is below every down workgroup id, and workgroups
// are dispatched in id order, so when a down task waits, every gate_up task
// has been dispatched; gate_up tasks wait for nothing. A wait is bounded
// (about a second) and sets the error word if it ever hits the bound.
//
// 16-row items at S > 16 too: a popular expert's weights are then read once
// per 16 picks rather than per 32, but the kernel holds 4 workgroups a CU
// (116 VGPRs) instead of 3 (168 for 32-row tiles). Measured steps, us, 16-row
// items against 32-row items (those with their rows staged in LDS): S = 32
// 58.8 / 60.2, S = 64 Zipf 50.2 / 51.4, S = 96 87.5 / 88.2.
#ifndef MOE_SINGLE_PD
#define MOE_SINGLE_PD 2  // down chunks in flight a wave (issued before the wait)
#endif
#ifndef MOE_SINGLE_OCC
#define MOE_SINGLE_OCC 4  // workgroups a CU
#endif
// PL: down chunks a wave staged in LDS before the wait (besides PD in
// registers), 2 at S > 32 and none below. Measured FFN us without / with:
// S = 8 22.15 / 22.50, S = 16 46.95 / 47.49, S = 32 40.97 / 41.43,
// S = 64 (Zipf) 31.54 / 30.62, S = 96 64.12 / 62.79. The extra bytes in
// flight pay once the tasks outnumber the resident workgroups; below that
// they compete with the gate_up tasks' weight stream.
#ifndef MOE_SINGLE_PL_LARGE_S
#define MOE_SINGLE_PL_LARGE_S 2
#endif
// kFront: the routing front runs as the first a.front workgroups, and every
// other workgroup waits for it. kOne (with kFront): the whole block as one
// launch, the front starting with the router rows (router_row_w4 with RNW
// float4s a lane a K slice) and the combine as the last a.comb workgroups.
template <int PG, int PD, int PL, bool kFront, int RNW = 0, bool kOne = false>
__global__ __launch_bounds__(kSplit * kWave, MOE_SINGLE_OCC) void ffn_single_kernel(FfnArgs a) {
  constexpr int TTG = 1;
  constexpr int kRed = static_cast<int>(sizeof(f32x4_t)) * kSplit * TTG * 4 * kWave;
  constexpr int kStage = kSplit * PL * kMxTileBytes;
  constexpr int kTask = kRed > kStage ? kRed : kStage;
  constexpr int kComb = kOne ? static_cast<int>(sizeof(OneCombineLds)) : 0;
  __shared__ __attribute__((aligned(16))) uint8_t smem[kTask > kComb ? kTask : kComb];
  static_assert(!kOne || (kFront && RNW > 0 && PL == 0), "one launch: front, router rows");
  auto red = reinterpret_cast<f32x4_t(*)[TTG][4][kWave]>(smem);
  const int lane = threadIdx.x & (kWave - 1);
  int t = blockIdx.x;
  uint32_t mk[4];
  int cnt;
  const int RB13 = 2 * a.I / kRowsPerBlock, NC13 = a.d / kChunkK;
  const int RB2 = a.d / kRowsPerBlock, NC2 = a.I / kChunkK;
  if constexpr (kFront) {
    if (t < a.front) {
      route_front<RNW, kOne>(a, t, smem);
      return;
    }
    t -= a.front;
    cnt = wait_route(a, t, mk);
    if constexpr (kOne) {
      const int n_tasks = a.max_work * (RB13 + RB2);
      if (t >= n_tasks) {  // past every task: the combine
        if (t - n_tasks < a.comb) combine_one(a, t - n_tasks, cnt, mk, n_tasks + 1, smem);
        return;
      }
      count_seen(a);
    }
  } else {
    cnt = lane < a.n_loc ? a.counts[lane] : 0;
  }
  const int n_work = count_work<TTG>(cnt);
  int el, row0, ntok, first;
  if (t < n_work * RB13) {
    const int wi = t / RB13, rb = t - wi * RB13;
    find_task<TTG>(cnt, wi, el, row0, ntok, &first);
    const uint8_t* tiles = a.w13 + (static_cast<size_t>(el) * RB13 + rb) * NC13 * kMxTileBytes;
    if constexpr (kFront) {  // the item's tokens from the masks, in LDS (read before red is)
      int32_t* list = reinterpret_cast<int32_t*>(smem);
      front_rows(mk, el, first, ntok, list);
      ffn_task<true, TTG, PG, true, true>(tiles, NC13, a.x, a.d, row0, ntok, rb, a.h, a.I,
                                          [list, row0](int r) { return list[r - row0]; }, NoWait{},
                                          red);
    } else {
      const int32_t* rows = a.rows;
      ffn_task<true, TTG, PG, true, true>(tiles, NC13, a.x, a.d, row0, ntok, rb, a.h, a.I,
                                          [rows](int r) { return rows[r]; }, NoWait{}, red);
    }
    publish(&a.prod[wi * kCtlStride], RB13, &a.ready[wi * RB2 * kCtlStride], RB2);
    return;
  }
  t -= n_work * RB13;
  if (t >= n_work * RB2) return;
  const int wi = t / RB2, rb = t - wi * RB2;
  find_task<TTG>(cnt, wi, el, row0, ntok, &first);
  const uint8_t* tiles = a.w2 + (static_cast<size_t>(el) * RB2 + rb) * NC2 * kMxTileBytes;
  ffn_task<true, TTG, PD, false, true, false, PL, kOne>(tiles, NC2, a.h, a.I, row0, ntok, rb, a.y,
                                                        a.d, [](int r) { return r; },
                                                        WaitFlag{&a.ready[t * kCtlStride], a.error},
                                                        red);
  if constexpr (kOne) count_rows(a, mk, el, first, ntok, smem);
}

// chunks in flight a wave of the routed tasks in the two launches for
// 32-token groups (measured at S = 128 with the shared expert, FFN us:
// 1/1 176.0, 1/2 177.4, 1/3 179.1, 2/2 181.5)
#ifndef MOE_PAIR_PG
#define MOE_PAIR_PG 1
#endif
#ifndef MOE_PAIR_PD
#define MOE_PAIR_PD 1
#endif

// Routed tasks of the two launches whose bucket rows fit in kPairLdsB bytes of
// LDS stage them there (ffn_task_ldsb) and keep this many weight chunks in
// flight a wave (gate_up / down); the row copy goes out after the first chunk
// (measured at S = 128 with the shared expert, FFN us: first chunk 162.6,
// all 6 chunks 168.7; 4 / 6 / 8 chunks 161.8 / 162.6 / 164.3)
constexpr int kPairLdsB = 65536;
#ifndef MOE_PAIR_LDSB_PG
#define MOE_PAIR_LDSB_PG 4
#endif
#ifndef MOE_PAIR_LDSB_PD
#define MOE_PAIR_LDSB_PD 4
#endif
// chunks in flight a wave of the routed tasks of 32-row items that hold at
// most 16 rows but do not fit the LDS budget (one token tile, register ring;
// at S = 128 with the shared expert items of 5 to 8 rows at d = 7168: FFN
// 159.0 us against 161.8 us with two token tiles; 3 chunks 159.1 us)
#ifndef MOE_PAIR_TT1_P
#define MOE_PAIR_TT1_P 2
#endif

// LDS of the two launches: the partial tiles of the reduction, the B rows of
// a routed task that stages them, or the shared task's staged rows of SG
// tokens (0: none)
template <int TTG, int kLdsB = kPairLdsB, int SG = 0>
constexpr int pair_smem() {
  constexpr int red = static_cast<int>(sizeof(f32x4_t)) * kSplit *
                      (kSharedTTG > TTG ? kSharedTTG : TTG) * 4 * kWave;
  constexpr int m = red > ldsb_smem<kLdsB>() ? red : ldsb_smem<kLdsB>();
  return SG > 0 && sd_smem<SG>() > m ? sd_smem<SG>() : m;
}

// With 32-row items (S > 16) the down launch runs the shared expert's tasks as
// shared_rows_task (waves own row tiles, the group's rows staged in LDS: 128
// VGPRs instead of the bf16 ring's 243) and stages routed rows of at most
// MOE_DOWN_LDSB bytes in LDS, so it holds MOE_DOWN_OCC workgroups a CU
// instead of 2. Measured at S = 128 (d = 7168, I = 2048), down step: 49.1 us,
// against 60.6 us as one launch at 2 workgroups a CU and 41.0 + 15.7 us as
// two launches (routed tasks alone at 4 a CU, then the old shared tasks);
// steps 176.3 / 177.0 against 184.5 / 185.3 us for the two launches. A ring of
// 2 chunks in the shared task: 49.9 us.
// The gate_up launch at S > 16 likewise runs the shared tasks as
// shared_rows_task (154 VGPRs instead of 243) and stages routed rows of at
// most MOE_GU_LDSB bytes (3 rows at d = 7168) at MOE_GU_OCC workgroups a CU.
// Measured at S = 128, gate_up launch: 94.9 us against 101.1 us (bf16 ring,
// 64 KiB, 2 a CU); 95.9 us at 4 a CU with 32 KiB, 103.6 us at 2 a CU with
// 64 KiB; steps 170.8 / 171.6 against 177.1 / 177.1 us.
#ifndef MOE_GU_OCC
#define MOE_GU_OCC 3
#endif
#ifndef MOE_GU_LDSB
#define MOE_GU_LDSB 49152
#endif
#ifndef MOE_DOWN_OCC
#define MOE_DOWN_OCC 4
#endif
#ifndef MOE_DOWN_LDSB
#define MOE_DOWN_LDSB 32768
#endif

#ifndef MOE_SG_PW
#define MOE_SG_PW 4  // weight chunks in flight a wave, shared gate_up tasks
#endif
// kFront: the routing front runs as the first a.front workgroups; the routed
// tasks wait for it (the shared expert's tasks do not need it).
template <int TTG, int P, bool kShared, int OCC = 2, int kLdsB = kPairLdsB, bool kSgRows = false,
          bool kFront = false>
__global__ __launch_bounds__(kSplit * kWave, OCC) void gate_up_kernel(FfnArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[pair_smem<TTG, kLdsB, kSgRows ? kSgTokGu : 0>()];
  static_assert(pair_smem<TTG, kLdsB>() >= sizeof(BucketLds) + 4 * kMaxTokens * 8,
                "LDS of the routing front");
  auto red = reinterpret_cast<f32x4_t(*)[kSharedTTG > TTG ? kSharedTTG : TTG][4][kWave]>(smem);
  const int NC = a.d / kChunkK;
  int t = blockIdx.x;
  if constexpr (kFront) {
    if (t < a.front) {
      route_front<0, false>(a, t, smem);
      return;
    }
    t -= a.front;
  }
  if constexpr (kShared) {
    constexpr int GS = kSgRows ? kSgTokGu : 16 * kSharedTTG;
    const int RBs = 2 * a.Is / kRowsPerBlock;
    const int n_sg = (a.S + GS - 1) / GS;
    if (t < n_sg * RBs) {
      int rb, grp;
      group_task(t, n_sg, RBs, rb, grp);
      const int row0 = grp * GS, ntok = min(GS, a.S - row0);
      const uint8_t* tiles = a.ws13 + static_cast<size_t>(rb) * NC * kBfTileBytes;
      if constexpr (kSgRows) {
        shared_rows_task<MOE_SG_PW, true, kSgTokGu>(tiles, NC, a.x, a.d, row0, ntok, rb, a.hs, a.Is,
                                                    smem);
      } else {
        ffn_task<false, kSharedTTG, kSharedP, true, false>(
            tiles, NC, a.x, a.d, row0, ntok, rb, a.hs, a.Is, [](int r) { return r; }, NoWait{},
            reinterpret_cast<f32x4_t(*)[kSharedTTG][4][kWave]>(&red[0][0][0][0]));
      }
      return;
    }
    t -= n_sg * RBs;
  }
  const int lane = threadIdx.x & (kWave - 1);
  uint32_t mk[4];
  int cnt;
  if constexpr (kFront) cnt = wait_route(a, t, mk);
  else cnt = lane < a.n_loc ? a.counts[lane] : 0;
  const int RB = 2 * a.I / kRowsPerBlock;
  const int wi = t / RB, rb = t - wi * RB;
  int el, row0, ntok, first;
  if (!find_task<TTG>(cnt, wi, el, row0, ntok, &first)) return;
  el = __builtin_amdgcn_readfirstlane(el);
  row0 = __builtin_amdgcn_readfirstlane(row0);
  ntok = __builtin_amdgcn_readfirstlane(ntok);
  first = __builtin_amdgcn_readfirstlane(first);
  const uint8_t* tiles = a.w13 + (static_cast<size_t>(el) * RB + rb) * NC * kMxTileBytes;
  // the item's tokens: the bucket rows, or (front) from the masks into LDS,
  // read before the task writes its LDS
  int32_t* list = reinterpret_cast<int32_t*>(smem);
  if constexpr (kFront) front_rows(mk, el, first, ntok, list);
  const int32_t* rows = a.rows;
  auto src_of = [rows, list, row0](int r) { return kFront ? list[r - row0] : rows[r]; };
  if (ntok <= 16 && ntok * a.d * 2 <= kLdsB) {
    ffn_task_ldsb<MOE_PAIR_LDSB_PG, 1, kLdsB, true, false>(
        tiles, NC, a.x, a.d, row0, ntok, rb, a.h, a.I, src_of, NoWait{}, smem);
    return;
  }
  if (TTG > 1 && ntok <= 16) {  // one token tile: half the MFMAs and activation loads
    ffn_task<true, 1, MOE_PAIR_TT1_P, true, false>(
        tiles, NC, a.x, a.d, row0, ntok, rb, a.h, a.I, src_of, NoWait{},
        reinterpret_cast<f32x4_t(*)[1][4][kWave]>(smem));
    return;
  }
  ffn_task<true, TTG, P, true, false>(tiles, NC, a.x, a.d, row0, ntok, rb, a.h, a.I, src_of,
                                      NoWait{},
                                      reinterpret_cast<f32x4_t(*)[TTG][4][kWave]>(&red[0][0][0][0]));
}

// Grid: the shared expert's tasks (kShared), then the routed items. OCC
// workgroups a CU; routed tasks with rows of at most kLdsB bytes stage them in
// LDS; kSgRows: the shared tasks run as shared_rows_task.
#ifndef MOE_SD_PW
#define MOE_SD_PW (MOE_SG_TOK_DN > 32 ? 2 : 4)  // weight chunks in flight a wave, shared down tasks
#endif
template <int TTG, int P, bool kShared, int OCC = 2, int kLdsB = kPairLdsB, bool kSgRows = false>
__global__ __launch_bounds__(kSplit * kWave, OCC) void down_kernel(FfnArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[pair_smem<TTG, kLdsB, kSgRows ? kSgTokDn : 0>()];
  auto red = reinterpret_cast<f32x4_t(*)[kSharedTTG > TTG ? kSharedTTG : TTG][4][kWave]>(smem);
  const int RB = a.d / kRowsPerBlock;
  auto same = [](int r) { return r; };
  int t = blockIdx.x;
  if constexpr (kShared) {
    constexpr int GS = kSgRows ? kSgTokDn : 16 * kSharedTTG;
    const int n_sg = (a.S + GS - 1) / GS;
    if (t < n_sg * RB) {
      const int NCs = a.Is / kChunkK;
      int rb, grp;
      group_task(t, n_sg, RB, rb, grp);
      const int row0 = grp * GS, ntok = min(GS, a.S - row0);
      const uint8_t* tiles = a.ws2 + static_cast<size_t>(rb) * NCs * kBfTileBytes;
      uint16_t* ys = a.y + static_cast<size_t>(a.R_max) * a.d;
      if constexpr (kSgRows) {
        shared_rows_task<MOE_SD_PW, false, kSgTokDn>(tiles, NCs, a.hs, a.Is, row0, ntok, rb, ys,
                                                     a.d, smem);
      } else {
        ffn_task<false, kSharedTTG, kSharedP, false, false>(
            tiles, NCs, a.hs, a.Is, row0, ntok, rb, ys, a.d, same, NoWait{},
            reinterpret_cast<f32x4_t(*)[kSharedTTG][4][kWave]>(&red[0][0][0][0]));
      }
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
  el = __builtin_amdgcn_readfirstlane(el);
  row0 = __builtin_amdgcn_readfirstlane(row0);
  ntok = __builtin_amdgcn_readfirstlane(ntok);
  const uint8_t* tiles = a.w2 + (static_cast<size_t>(el) * RB + rb) * NC * kMxTileBytes;
  if (ntok <= 16 && ntok * a.I * 2 <= kLdsB) {
    ffn_task_ldsb<MOE_PAIR_LDSB_PD, 1, kLdsB, false, false>(tiles, NC, a.h, a.I, row0, ntok, rb,
                                                            a.y, a.d, same, NoWait{}, smem);
    return;
  }
  if (TTG > 1 && ntok <= 16) {
    ffn_task<true, 1, MOE_PAIR_TT1_P, false, false>(
        tiles, NC, a.h, a.I, row0, ntok, rb, a.y, a.d, same, NoWait{},
        reinterpret_cast<f32x4_t(*)[1][4][kWave]>(smem));
    return;
  }
  ffn_task<true, TTG, P, false, false>(tiles, NC, a.h, a.I, row0, ntok, rb, a.y, a.d, same,
                                       NoWait{}, reinterpret_cast<f32x4_t(*)[TTG][4][kWave]>(&red[0][0][0][0]));
}

// PG / PD: chunks in flight a wave in gate_up / down; kLean: the shared tasks
// as shared_rows_task, the launches at MOE_GU_OCC / MOE_DOWN_OCC workgroups a
// CU; a.front: the routing front ahead of the gate_up launch's tasks
template <int TTG, int PG, int PD, bool kShared, bool kLean>
void launch_pair(const FfnArgs& a, hipStream_t stream) {
  constexpr int GSG = kLean ? kSgTokGu : 16 * kSharedTTG;  // token groups of the shared tasks
  constexpr int GSD = kLean ? kSgTokDn : 16 * kSharedTTG;
  const int n_sgg = kShared ? (a.S + GSG - 1) / GSG : 0;
  const int n_sgd = kShared ? (a.S + GSD - 1) / GSD : 0;
  const int g1 = a.front + n_sgg * (2 * a.Is / kRowsPerBlock) + a.max_work * (2 * a.I / kRowsPerBlock);
  const int g2 = (n_sgd + a.max_work) * (a.d / kRowsPerBlock);
  if (a.front) {
    if constexpr (kLean)
      hipLaunchKernelGGL((gate_up_kernel<TTG, PG, kShared, MOE_GU_OCC, MOE_GU_LDSB, true, true>),
                         dim3(g1), dim3(kSplit * kWave), 0, stream, a);
    else
      hipLaunchKernelGGL((gate_up_kernel<TTG, PG, kShared, 2, kPairLdsB, false, true>), dim3(g1),
                         dim3(kSplit * kWave), 0, stream, a);
  } else if constexpr (kLean)
    hipLaunchKernelGGL((gate_up_kernel<TTG, PG, kShared, MOE_GU_OCC, MOE_GU_LDSB, true>), dim3(g1),
                       dim3(kSplit * kWave), 0, stream, a);
  else
    hipLaunchKernelGGL((gate_up_kernel<TTG, PG, kShared>), dim3(g1), dim3(kSplit * kWave), 0,
                       stream, a);
  if constexpr (kLean)
    hipLaunchKernelGGL((down_kernel<TTG, PD, kShared, MOE_DOWN_OCC, MOE_DOWN_LDSB, true>), dim3(g2),
                       dim3(kSplit * kWave), 0, stream, a);
  else
    hipLaunchKernelGGL((down_kernel<TTG, PD, kShared>), dim3(g2), dim3(kSplit * kWave), 0, stream,
                       a);
}

bool single_launch(const moe_dims& m) { return m.shared_I == 0; }

}  // namespace

FfnLayout ffn_layout(const moe_dims& m) {
  const int R = r_max(m);
  FfnLayout l;
  l.max_work = max_work(m);
  l.h = 0;
  l.hs = round_up(static_cast<size_t>(R) * m.I * 2, 256);
  l.prod = l.hs + round_up(static_cast<size_t>(m.S) * m.shared_I * 2, 256);
  l.ready = l.prod + static_cast<size_t>(l.max_work) * kCtlStride * 4;
  l.tokc = l.ready + static_cast<size_t>(l.max_work) * (m.d / kRowsPerBlock) * kCtlStride * 4;
  l.route = l.tokc + static_cast<size_t>(m.S) * kCtlStride * 4;
  l.error = l.route + round_up(static_cast<size_t>(kFrontWords) * 4, 256);
  l.total = l.error + 256;
  return l;
}

int32_t* route_front_block(const moe_dims& m, void* workspace) {
  return reinterpret_cast<int32_t*>(static_cast<uint8_t*>(workspace) + ffn_layout(m).route);
}

int launch_ffn(const moe_dims& m, const void* x, const void* w13, const void* w2, const void* ws13,
               const void* ws2, const int32_t* counts, const int32_t* rows, void* y,
               void* workspace, hipStream_t stream, int32_t* error_word, const FrontIo* front) {
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
  a.prod = reinterpret_cast<int32_t*>(ws + l.prod);
  a.ready = reinterpret_cast<int32_t*>(ws + l.ready);
  a.error = error_word ? error_word : reinterpret_cast<int32_t*>(ws + l.error);
  a.y = static_cast<uint16_t*>(y);
  a.S = m.S;
  a.d = m.d;
  a.I = m.I;
  a.Is = m.shared_I;
  a.n_loc = m.n_local;
  a.R_max = r_max(m);
  a.max_work = l.max_work;
  a.front = 0;
  if (front) {  // the routing front: S top-k workgroups and the bucketing
    RouteFront& f = a.rf;
    f.logits_in = front->logits_in;
    f.parts = front->parts;
    f.KP = front->parts ? router_parts(m) : 0;
    f.lbias = front->parts || front->wr ? logit_bias(m, front->bias) : nullptr;
    f.sel_bias = select_bias(m, front->bias);
    f.logits_out = front->logits;
    f.ids = front->ids;
    f.w = front->w;
    f.offsets = front->offsets;
    f.pick_pos = front->pick_pos;
    f.active = front->active;
    f.done = reinterpret_cast<int32_t*>(ws + l.route);
    int32_t* blk = reinterpret_cast<int32_t*>(ws + l.route);
    f.masks = reinterpret_cast<uint32_t*>(blk + kFrontMaskWord);
    f.rdone = blk + kFrontRouterWord;
    f.seen = blk + kFrontSeenWord;
    f.cdone = blk + kFrontCombWord;
    f.tkc = blk + kFrontTopkWord;
    f.E = m.E;
    f.topk = m.topk;
    f.renorm = m.renorm;
    f.local_base = m.local_base;
    a.front = m.S + 1;
    if (front->wr && front->out && one_launch(m)) {  // the whole block as one launch
      f.wr = front->wr;
      f.n_router = m.E;
      a.front += m.E;
      a.comb = m.S;
      a.tokc = reinterpret_cast<int32_t*>(ws + l.tokc);
      a.gamma = front->gamma;
      a.out = front->out;
      a.eps = m.eps;
    }
  }
  if (single_launch(m)) {
    const int tasks = l.max_work * (2 * m.I + m.d) / kRowsPerBlock;
    const int grid = a.front + tasks + a.comb;
    if (a.comb) {
      hipLaunchKernelGGL((ffn_single_kernel<2, MOE_SINGLE_PD, 0, true, 1, true>), dim3(grid),
                         dim3(kSplit * kWave), 0, stream, a);
    } else if (a.front) {
      if (m.S > 32)
        hipLaunchKernelGGL((ffn_single_kernel<2, MOE_SINGLE_PD, MOE_SINGLE_PL_LARGE_S, true>),
                           dim3(grid), dim3(kSplit * kWave), 0, stream, a);
      else
        hipLaunchKernelGGL((ffn_single_kernel<2, MOE_SINGLE_PD, 0, true>), dim3(grid),
                           dim3(kSplit * kWave), 0, stream, a);
    } else if (m.S > 32)
      hipLaunchKernelGGL((ffn_single_kernel<2, MOE_SINGLE_PD, MOE_SINGLE_PL_LARGE_S, false>),
                         dim3(grid), dim3(kSplit * kWave), 0, stream, a);
    else
      hipLaunchKernelGGL((ffn_single_kernel<2, MOE_SINGLE_PD, 0, false>), dim3(grid),
                         dim3(kSplit * kWave), 0, stream, a);
  } else if (ffn_group(m) > 16) {  // a shared expert, 32-row items
    launch_pair<2, MOE_PAIR_PG, MOE_PAIR_PD, true, true>(a, stream);
  } else {  // 16-row items: at MOE_DOWN_OCC a CU their ring of 4 chunks would spill
    launch_pair<1, 2, 4, true, false>(a, stream);
  }
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
