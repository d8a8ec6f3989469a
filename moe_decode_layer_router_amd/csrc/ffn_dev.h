// ffn_dev.h -- one task of the expert GEMMs (gate_up + SwiGLU, or down) as a
// workgroup-level device function, used by the moe_expert_ffn kernels.
//
// Muse Spark K3 page, stages "C, D": gate_up and down of the local experts with
// MXFP4 weights decoded in registers and fed to bf16 MFMA; functions "mx_chunk"
// and "fp4_mma": a 16-row MXFP4 group is processed in 256-K chunks of 8 MFMA
// steps with one e8m0 scale per 32 K; "task_ring": compute one task while the
// next ones' loads are in flight. K5 page: every row tile is 16 tokens (the
// MFMA N dimension). The Kimi-K3 layer page's shared expert ("k2_launch": w_sgu,
// w_sd) runs the same chain on dense bf16 weights.
//
// A task: 64 weight rows (4 MFMA row tiles) of one expert against one group of
// up to 16 * TTG bucket rows, over the full K. The workgroup's 4 waves split K:
// wave w takes chunks c = w, w + 4, ... of 128 K, so together they stream the
// task's packed tiles front to back. Each wave keeps P chunks of loads in
// flight (weights non-temporal, activations through the cache), decodes MXFP4
// with the scaled fp4 -> bf16 converts and accumulates with
// v_mfma_f32_16x16x32_bf16. The four partial tiles are summed through LDS in
// wave order (deterministic); the epilogue rounds to bf16 and, for gate_up,
// applies SwiGLU in registers (the packed row order gives each lane matching
// gate and up rows).
#pragma once

#include <type_traits>

#include "common.h"

namespace moeblk {

constexpr int kSplit = 4;  // waves a workgroup, = row tiles a task

// Work items enumerate, for the local experts in order, their groups of
// G = 16 * TTG bucket rows (an expert without picks has none). Wave-level:
// lane u holds expert u's count `cnt` (0 for u >= n_loc); wave prefix sums of
// the group counts and of the counts give the item's expert and its first
// bucket row (the bucket offsets are the exclusive prefix sums of the counts).
// Returns false past the last item.
template <int TTG>
__device__ __forceinline__ bool find_task(int cnt, int wi, int& el, int& row0, int& ntok,
                                          int* first = nullptr) {
  constexpr int G = 16 * TTG;
  const int lane = threadIdx.x & (kWave - 1);
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
  const uint64_t hit = __ballot(lane < 32 && wi < incl_ng);
  if (hit == 0) return false;
  const int u = __builtin_ctzll(hit);
  const int g = wi - (__shfl(incl_ng, u, kWave) - __shfl(ng, u, kWave));
  const int c = __shfl(cnt, u, kWave);
  el = u;
  row0 = __shfl(incl_cnt, u, kWave) - c + g * G;
  ntok = min(G, c - g * G);
  if (first) *first = g * G;  // the item's first row within its expert's bucket
  return true;
}

// Work items of all local experts (wave-level, every lane gets it).
template <int TTG>
__device__ __forceinline__ int count_work(int cnt) {
  constexpr int G = 16 * TTG;
  int ng = (cnt + G - 1) / G;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) ng += __shfl_xor(ng, m, kWave);
  return ng;
}

// Dense weights read by several token groups: task t of n_g token groups x
// RB weight blocks -> (block, group). Workgroups go to the 8 XCDs round-robin
// by id, so the groups of one block get ids that are equal mod 8 and adjacent
// in that XCD's order: they run together on one XCD and share its L2 for the
// block's weights.
__device__ __forceinline__ void group_task(int t, int n_g, int RB, int& rb, int& grp) {
  constexpr int kXcd = 8;
  if (RB % kXcd == 0) {
    const int slot = t / kXcd;
    grp = slot % n_g;
    rb = (slot / n_g) * kXcd + t % kXcd;
  } else {
    rb = t / n_g;
    grp = t - rb * n_g;
  }
}

template <int TTG>
struct MxChunk {
  u32x4_t w[4];       // 4 row tiles x 32 e2m1 codes a lane
  uint32_t s;         // the 4 row tiles' e8m0 bytes
  u32x4_t b[TTG][4];  // activations: 32 bf16 a lane a token tile
};

template <int TTG>
struct BfChunk {
  u32x4_t w[4][4];  // 4 row tiles x 4 MFMA steps x 8 bf16
  u32x4_t b[TTG][4];
};

// Activation (B) rows of a task. Loads are unconditional (every token tile,
// clamped chunk indices): the waitcnt insertion then sees one fixed issue order
// and keeps the ring in flight. With kCoh the loads carry the device-scope
// coherence bit (sc1): rows written earlier in the same launch by another XCD
// are read from the coherence point, not from a stale line of this XCD's L2.
template <int TTG, bool kCoh>
struct BRows {
  const uint16_t* bp[TTG];      // !kCoh: this lane's row pointers (+ its K group)
  __amdgpu_buffer_rsrc_t rsrc;  // kCoh: buffer over the B rows
  uint32_t boff[TTG];           // kCoh: this lane's byte offsets

  __device__ __forceinline__ void init(const uint16_t* bsrc, int K, const int (&src)[TTG], int g) {
    if constexpr (kCoh) {
      rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(bsrc), 0, 0x7fffffff,
                                               0x00020000);
#pragma unroll
      for (int tt = 0; tt < TTG; ++tt) boff[tt] = (static_cast<uint32_t>(src[tt]) * K + 32 * g) * 2u;
    } else {
#pragma unroll
      for (int tt = 0; tt < TTG; ++tt) bp[tt] = bsrc + static_cast<size_t>(src[tt]) * K + 32 * g;
    }
  }

  __device__ __forceinline__ void load(u32x4_t (&b)[TTG][4], int c) const {
#pragma unroll
    for (int tt = 0; tt < TTG; ++tt) {
      if constexpr (kCoh) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          b[tt][q] = __builtin_amdgcn_raw_buffer_load_b128(
              rsrc, boff[tt] + static_cast<uint32_t>(c * kChunkK + 8 * q) * 2u, 0, kCpolSc1);
      } else {
        const u32x4_t* p = reinterpret_cast<const u32x4_t*>(bp[tt] + c * kChunkK);
#pragma unroll
        for (int q = 0; q < 4; ++q) b[tt][q] = p[q];
      }
    }
  }
};

// fp32 B rows (kF32In: the post-expert projection's summed partial), each
// value rounded to bf16 where the chunk is used, as one rounding launch
// before the GEMM would: the lane's K 32 g + 8 q .. + 7 as two float4s a step
template <int TTG>
struct BfChunkF32 {
  u32x4_t w[4][4];
  u32x4_t b[TTG][8];  // step q: floats 8 q .. 8 q + 3, then 8 q + 4 .. 8 q + 7
};

template <int TTG>
struct BRowsF32 {
  const float* bp[TTG];

  // bsrc: the fp32 rows (K floats each), passed as the byte-compatible pointer
  __device__ __forceinline__ void init(const uint16_t* bsrc, int K, const int (&src)[TTG], int g) {
    const float* f = reinterpret_cast<const float*>(bsrc);
#pragma unroll
    for (int tt = 0; tt < TTG; ++tt) bp[tt] = f + static_cast<size_t>(src[tt]) * K + 32 * g;
  }

  __device__ __forceinline__ void load(u32x4_t (&b)[TTG][8], int c) const {
#pragma unroll
    for (int tt = 0; tt < TTG; ++tt) {
      const u32x4_t* p = reinterpret_cast<const u32x4_t*>(bp[tt] + c * kChunkK);
#pragma unroll
      for (int i = 0; i < 8; ++i) b[tt][i] = p[i];
    }
  }
};

template <int TTG>
__device__ __forceinline__ void load_w(MxChunk<TTG>& ch, const uint8_t* wlane, const uint8_t* slane,
                                       int c) {
  const uint8_t* t = wlane + static_cast<size_t>(c) * kMxTileBytes;
#pragma unroll
  for (int r = 0; r < 4; ++r) ch.w[r] = ld_nt<u32x4_t>(t + r * 1024);
  ch.s = ld_nt<uint32_t>(slane + static_cast<size_t>(c) * kMxTileBytes);
}

// Dense bf16 tiles (the shared expert, the latent projections) are read once
// per token group, by tasks placed on one XCD (group_task): plain loads, so
// the groups after the first find them in that XCD's L2.
__device__ __forceinline__ void load_bf_w(u32x4_t (&w)[4][4], const uint8_t* wlane, int c) {
  const uint8_t* t = wlane + static_cast<size_t>(c) * kBfTileBytes;
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int q = 0; q < 4; ++q)
      w[r][q] = *reinterpret_cast<const u32x4_t*>(t + r * 4096 + q * 1024);
}
template <int TTG>
__device__ __forceinline__ void load_w(BfChunk<TTG>& ch, const uint8_t* wlane, const uint8_t*,
                                       int c) {
  load_bf_w(ch.w, wlane, c);
}
template <int TTG>
__device__ __forceinline__ void load_w(BfChunkF32<TTG>& ch, const uint8_t* wlane, const uint8_t*,
                                       int c) {
  load_bf_w(ch.w, wlane, c);
}

// One MXFP4 chunk tile (kMxTileBytes: 4 row tiles of 64 lanes x 16 bytes, then
// 64 lanes x 4 scale bytes) of chunk c copied to LDS at dst by the wave, with
// loads that write LDS directly (lane l's piece lands at dst + l x size).
__device__ __forceinline__ void stage_mx_lds(uint8_t* dst, const uint8_t* tiles, int c) {
  typedef const __attribute__((address_space(1))) void* gptr_t;
  typedef __attribute__((address_space(3))) void* lptr_t;
  const int lane = threadIdx.x & (kWave - 1);
  const uint8_t* src = tiles + static_cast<size_t>(c) * kMxTileBytes;
#pragma unroll
  for (int r = 0; r < 4; ++r)
    __builtin_amdgcn_global_load_lds((gptr_t)(src + r * 1024 + lane * 16), (lptr_t)(dst + r * 1024),
                                     16, 0, 0);
  __builtin_amdgcn_global_load_lds((gptr_t)(src + 4096 + lane * 4), (lptr_t)(dst + 4096), 4, 0, 0);
}

// The weights of an MXFP4 chunk from a tile staged by stage_mx_lds. The
// compiler does not order LDS reads after these direct LDS loads, so the wave
// first waits for all of its vector loads (the "memory" clobber keeps the
// reads below the wait).
template <int TTG>
__device__ __forceinline__ void lds_mx_chunk(MxChunk<TTG>& ch, const uint8_t* src) {
  const int lane = threadIdx.x & (kWave - 1);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
  for (int r = 0; r < 4; ++r) ch.w[r] = *reinterpret_cast<const u32x4_t*>(src + r * 1024 + lane * 16);
  ch.s = *reinterpret_cast<const uint32_t*>(src + 4096 + lane * 4);
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
__device__ __forceinline__ void compute_chunk(const BfChunkF32<TTG>& ch, f32x4_t (&acc)[TTG][4],
                                              int n_tt) {
  // step q of every (token tile, row tile): each accumulator still takes the
  // steps in order, as in the bf16 chunk
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int tt = 0; tt < TTG; ++tt) {
      if (tt >= n_tt) continue;
      const f32x4_t l = __builtin_bit_cast(f32x4_t, ch.b[tt][2 * q]);
      const f32x4_t h = __builtin_bit_cast(f32x4_t, ch.b[tt][2 * q + 1]);
      const u32x4_t bq{pack_bf16x2(l[0], l[1]), pack_bf16x2(l[2], l[3]), pack_bf16x2(h[0], h[1]),
                       pack_bf16x2(h[2], h[3])};
#pragma unroll
      for (int r = 0; r < 4; ++r)
        acc[tt][r] = mfma_bf16(__builtin_bit_cast(bf16x8_t, ch.w[r][q]),
                               __builtin_bit_cast(bf16x8_t, bq), acc[tt][r]);
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

// Sum of the 4 waves' partial tiles of a task in wave order, then the
// epilogue: gate_up rounds gate and up to bf16 and writes SwiGLU rows; down
// writes bf16 rows (kOutCoh: through to the coherence point, for a combine
// in the same launch); kF32Out writes unrounded fp32 rows. Workgroup-level.
template <int TTG, bool kGateUp, bool kCoh, bool kF32Out, bool kOutCoh = false>
__device__ __forceinline__ void task_epilogue(const f32x4_t (&acc)[TTG][4], int n_tt, int ntok,
                                              int row0, int rb, uint16_t* __restrict__ out,
                                              int out_ld, f32x4_t (*red)[TTG][4][kWave]) {
  const int lane = threadIdx.x & (kWave - 1);
  const int w = threadIdx.x >> 6;
  const int g = lane >> 4;
  const int col = lane & 15;
  // sum the 4 waves' partial tiles in wave order
  __syncthreads();  // the previous task's epilogue has read red
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
    uint16_t* orow = out + static_cast<size_t>(row0 + c) * out_ld;
    if constexpr (kGateUp) {
      // rows 4g..4g+3 of tile r: gate i, gate i+1, up i, up i+1
      const float g0 = round_bf16(s[0]), g1 = round_bf16(s[1]);
      const float u0 = round_bf16(s[2]), u1 = round_bf16(s[3]);
      const int i0 = 32 * rb + 8 * r + 2 * g;
      const uint32_t hv = swiglu_bf16_bits(g0, u0) | (swiglu_bf16_bits(g1, u1) << 16);
      uint32_t* hp = reinterpret_cast<uint32_t*>(orow + i0);
      if constexpr (kCoh) __hip_atomic_store(hp, hv, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      else *hp = hv;
    } else if constexpr (kF32Out) {
      const int n0 = kRowsPerBlock * rb + 16 * r + 4 * g;
      float* frow = reinterpret_cast<float*>(out) + static_cast<size_t>(row0 + c) * out_ld + n0;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        __hip_atomic_store(frow + i, s[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
      const int n0 = kRowsPerBlock * rb + 16 * r + 4 * g;
      const u32x2_t v{pack_bf16x2(s[0], s[1]), pack_bf16x2(s[2], s[3])};
      if constexpr (kOutCoh)
        __hip_atomic_store(reinterpret_cast<uint64_t*>(orow + n0), __builtin_bit_cast(uint64_t, v),
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      else
        *reinterpret_cast<u32x2_t*>(orow + n0) = v;
    }
  }
}

struct NoWait {
  __device__ void operator()() const {}
};

// Workgroup-level (4 waves). tiles: the packed tiles of (expert, row block rb);
// B rows: src_of(r) for bucket rows r = row0 .. row0 + ntok - 1 (row length K;
// gate_up: token rows of x; down: SwiGLU rows); out: output rows indexed by
// bucket row (row length out_ld); before_b() runs after the weight prefetch and
// before the first activation load; red: LDS. kCoh: the SwiGLU rows pass
// between workgroups of one launch (gate_up writes them through to the
// coherence point, down reads them from there). kF32Out (not gate_up): out
// holds fp32 rows (a split-K partial), written unrounded through to the
// coherence point, for another workgroup to sum.
// PL > 0 (MXFP4 only): the wave's chunks P .. P + PL - 1 go to LDS (red, PL
// chunk tiles a wave) before before_b(), by loads that write LDS directly, and
// are read from there when the ring takes them: a task that waits (a down task
// of the single launch) then has P + PL chunks in flight at the register cost
// of P. The LDS is read only after every vector load of the wave has arrived.
// kOutCoh (down): the output rows go through to the coherence point.
// kF32In (dense): bsrc holds fp32 rows (K floats each), rounded to bf16 as
// they are used.
template <bool kMx, int TTG, int P, bool kGateUp, bool kCoh, bool kF32Out = false, int PL = 0,
          bool kOutCoh = false, bool kF32In = false, class SrcOf, class BeforeB>
__device__ __forceinline__ void ffn_task(const uint8_t* __restrict__ tiles, int NC,
                                         const uint16_t* __restrict__ bsrc, int K, int row0,
                                         int ntok, int rb, uint16_t* __restrict__ out, int out_ld,
                                         SrcOf src_of, BeforeB before_b,
                                         f32x4_t (*red)[TTG][4][kWave]) {
  const int lane = threadIdx.x & (kWave - 1);
  const int w = threadIdx.x >> 6;
  const int g = lane >> 4;
  const int col = lane & 15;
  const int n_tt = (ntok + 15) / 16;
  const uint8_t* wlane = tiles + lane * 16;
  const uint8_t* slane = tiles + 4096 + lane * 4;

  // this lane's B rows (token tile tt, column col); columns past the group's
  // rows repeat its last row and are never stored. The row lookup is issued
  // before the weights so that waiting for it leaves them in flight.
  int src[TTG];
#pragma unroll
  for (int tt = 0; tt < TTG; ++tt) src[tt] = src_of(row0 + min(tt * 16 + col, ntok - 1));

  using Chunk = typename std::conditional<
      kMx, MxChunk<TTG>,
      typename std::conditional<kF32In, BfChunkF32<TTG>, BfChunk<TTG>>::type>::type;
  static_assert(PL == 0 || kMx, "LDS-staged chunks are MXFP4 tiles");
  static_assert(!kF32In || (!kMx && !kCoh), "fp32 B rows: dense tiles, plain loads");
  const int my_n = (NC - w + kSplit - 1) / kSplit;  // this wave's chunks: w, w + 4, ...
  Chunk ring[P];
#pragma unroll
  for (int i = 0; i < P; ++i) load_w<TTG>(ring[i], wlane, slane, min(w + kSplit * i, NC - 1));

  uint8_t* lw = reinterpret_cast<uint8_t*>(red) + w * (PL * kMxTileBytes);  // this wave's LDS chunks
  if constexpr (PL > 0) {
#pragma unroll
    for (int l = 0; l < PL; ++l)
      if (P + l < my_n) stage_mx_lds(lw + l * kMxTileBytes, tiles, w + kSplit * (P + l));
  }
  // the ring takes the wave's chunk j (chunk w + 4 j)
  auto refill = [&](Chunk& ch, int j) {
    if constexpr (PL > 0) {
      if (j < P + PL) {
        lds_mx_chunk<TTG>(ch, lw + (j - P) * kMxTileBytes);
        return;
      }
    }
    load_w<TTG>(ch, wlane, slane, w + kSplit * j);
  };

  before_b();

  typename std::conditional<kF32In, BRowsF32<TTG>, BRows<TTG, kCoh && !kGateUp>>::type bp;
  bp.init(bsrc, K, src, g);
#pragma unroll
  for (int i = 0; i < P; ++i) bp.load(ring[i].b, min(w + kSplit * i, NC - 1));

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
      refill(ring[i], j0 + i + P);
      bp.load(ring[i].b, c);
    }
  }
#pragma unroll
  for (int i = 0; i < P; ++i) {  // fewer than 2P chunks left
    if (j0 + i < my_n) {
      compute_chunk<TTG>(ring[i], acc, n_tt);
      if (j0 + i + P < my_n) {
        const int c = w + kSplit * (j0 + i + P);
        refill(ring[i], j0 + i + P);
        bp.load(ring[i].b, c);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < P; ++i)
    if (j0 + P + i < my_n) compute_chunk<TTG>(ring[i], acc, n_tt);

  task_epilogue<TTG, kGateUp, kCoh, kF32Out, kOutCoh>(acc, n_tt, ntok, row0, rb, out, out_ld, red);
}

// ---------------------------------------------------------------------------
// A routed MXFP4 task whose few bucket rows fit in LDS (ntok * K * 2 bytes at
// most kLdsB): the rows are copied into LDS once, and every MFMA step
// reads its B operand from there. The register ring then holds weights only
// (17 VGPRs a chunk instead of 33), so a wave keeps PW weight chunks in flight
// at the register cost of about PW / 2 chunks of the ring with activations,
// and the LDS reads wait on their own counter, not behind the weight loads.
// The routed items of the two launches with a shared expert (32 rows at
// S > 16) often hold only a few picks: the task then runs one token tile
// instead of two.
// Columns past the task's rows read its last row (an LDS broadcast) and are
// never stored. After the main loop the same LDS holds the partial tiles of
// the wave-order reduction (task_epilogue).

// LDS of a task that stages its B rows: kLdsB bytes of rows + their sources
// (32 ints)
template <int kLdsB>
constexpr int ldsb_smem() { return kLdsB + 128; }

struct MxW {
  u32x4_t w[4];  // 4 row tiles x 32 e2m1 codes a lane
  uint32_t s;    // the 4 row tiles' e8m0 bytes
};

__device__ __forceinline__ void load_w(MxW& ch, const uint8_t* wlane, const uint8_t* slane, int c) {
  const uint8_t* t = wlane + static_cast<size_t>(c) * kMxTileBytes;
#pragma unroll
  for (int r = 0; r < 4; ++r) ch.w[r] = ld_nt<u32x4_t>(t + r * 1024);
  ch.s = ld_nt<uint32_t>(slane + static_cast<size_t>(c) * kMxTileBytes);
}

// lb: this lane's B row in LDS (its token column, + its K group 32 g)
__device__ __forceinline__ void compute_chunk_ldsb(const MxW& ch, const uint16_t* lb, int c,
                                                   f32x4_t (&acc)[4]) {
  u32x4_t b[4];
  const u32x4_t* p = reinterpret_cast<const u32x4_t*>(lb + c * kChunkK);
#pragma unroll
  for (int q = 0; q < 4; ++q) b[q] = p[q];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float sc = e8m0_scale((ch.s >> (8 * r)) & 0xffu);
#pragma unroll
    for (int q = 0; q < 4; ++q)
      acc[r] = mfma_bf16(decode_fp4x8(ch.w[r][q], sc), __builtin_bit_cast(bf16x8_t, b[q]), acc[r]);
  }
}

// Workgroup-level, same contract as ffn_task<true, TTG, ., kGateUp, kCoh> for
// ntok <= 16 and ntok * K * 2 <= kLdsB; smem: ldsb_smem<kLdsB>() bytes of LDS.
// The first kPre weight chunks of a wave are issued before before_b() and the
// row copy, the rest after the copy's loads: vector loads complete in issue
// order, so the copy then waits for kPre chunks only (a down task that waits
// for its flag issues all PW chunks first).
template <int PW, int kPre, int kLdsB, bool kGateUp, bool kCoh, class SrcOf, class BeforeB>
__device__ __forceinline__ void ffn_task_ldsb(const uint8_t* __restrict__ tiles, int NC,
                                              const uint16_t* __restrict__ bsrc, int K, int row0,
                                              int ntok, int rb, uint16_t* __restrict__ out,
                                              int out_ld, SrcOf src_of, BeforeB before_b,
                                              uint8_t* smem) {
  constexpr int kThreads = kSplit * kWave;
  constexpr int kPer = kLdsB / 16 / kThreads;  // 16-byte pieces a thread copies, at most
  const int lane = threadIdx.x & (kWave - 1);
  const int w = threadIdx.x >> 6;
  const int g = lane >> 4;
  const int col = lane & 15;
  uint16_t* lds_b = reinterpret_cast<uint16_t*>(smem);
  int* srow = reinterpret_cast<int*>(smem + kLdsB);

  // the rows' sources first: waiting for them leaves the weights in flight
  int src = 0;
  if (threadIdx.x < ntok) src = src_of(row0 + threadIdx.x);

  const uint8_t* wlane = tiles + lane * 16;
  const uint8_t* slane = tiles + 4096 + lane * 4;
  const int my_n = (NC - w + kSplit - 1) / kSplit;  // this wave's chunks: w, w + 4, ...
  static_assert(kPre >= 1 && kPre <= PW, "chunks issued before the row copy");
  MxW ring[PW];
#pragma unroll
  for (int i = 0; i < kPre; ++i) load_w(ring[i], wlane, slane, min(w + kSplit * i, NC - 1));

  if (threadIdx.x < ntok) srow[threadIdx.x] = src;
  before_b();
  __syncthreads();

  // copy the ntok rows (K bf16 each) into LDS, row r at r * K
  const int pieces = K / 8;
  const int total = ntok * pieces;
  constexpr bool kCohB = kCoh && !kGateUp;  // SwiGLU rows of this launch
  u32x4_t v[kPer];
  __amdgpu_buffer_rsrc_t rsrc;
  if constexpr (kCohB)
    rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(bsrc), 0, 0x7fffffff, 0x00020000);
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int q = i * kThreads + threadIdx.x;
    if (q < total) {
      const int r = q / pieces, p = q - r * pieces;
      const uint32_t e = static_cast<uint32_t>(srow[r]) * K + 8 * p;  // element offset
      if constexpr (kCohB)
        v[i] = __builtin_amdgcn_raw_buffer_load_b128(rsrc, e * 2u, 0, kCpolSc1);
      else
        v[i] = *reinterpret_cast<const u32x4_t*>(bsrc + e);
    }
  }
  __builtin_amdgcn_sched_barrier(0);  // the row loads go out before the later chunks
#pragma unroll
  for (int i = kPre; i < PW; ++i) load_w(ring[i], wlane, slane, min(w + kSplit * i, NC - 1));
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int q = i * kThreads + threadIdx.x;
    if (q < total) *reinterpret_cast<u32x4_t*>(lds_b + 8 * q) = v[i];
  }
  __syncthreads();

  const uint16_t* lb = lds_b + min(col, ntok - 1) * K + 32 * g;
  f32x4_t acc[1][4];
#pragma unroll
  for (int r = 0; r < 4; ++r) acc[0][r] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  int j0 = 0;
  for (; j0 + 2 * PW <= my_n; j0 += PW) {  // steady state: every refill is needed
#pragma unroll
    for (int i = 0; i < PW; ++i) {
      compute_chunk_ldsb(ring[i], lb, w + kSplit * (j0 + i), acc[0]);
      load_w(ring[i], wlane, slane, w + kSplit * (j0 + i + PW));
      // keep each refill right after its chunk: the scheduler would otherwise
      // sink all PW refills to the end of the iteration and drain the ring
      __builtin_amdgcn_sched_barrier(0);
    }
  }
#pragma unroll
  for (int i = 0; i < PW; ++i) {  // fewer than 2 PW chunks left
    if (j0 + i < my_n) {
      compute_chunk_ldsb(ring[i], lb, w + kSplit * (j0 + i), acc[0]);
      if (j0 + i + PW < my_n) load_w(ring[i], wlane, slane, w + kSplit * (j0 + i + PW));
    }
  }
#pragma unroll
  for (int i = 0; i < PW; ++i)
    if (j0 + PW + i < my_n) compute_chunk_ldsb(ring[i], lb, w + kSplit * (j0 + PW + i), acc[0]);

  // the barrier at the start of the epilogue ends every wave's B reads before
  // the partial tiles overwrite them
  task_epilogue<1, kGateUp, kCoh, false>(acc, 1, ntok, row0, rb, out, out_ld,
                                         reinterpret_cast<f32x4_t(*)[1][4][kWave]>(smem));
}

// ---------------------------------------------------------------------------
// The shared expert for one 64-row block and one group of up to TOK tokens
// (Kimi-K3 layer page, "k2_launch": w_sgu and w_sd, the always-on expert's
// gate_up and down), with waves owning row tiles instead of K quarters: wave w
// streams row tile w over all NC chunks through a ring of PW chunks (16 VGPRs
// a chunk) and needs no reduction across waves. The chunk's B rows (TOK x 128
// bf16: token rows of x for gate_up, SwiGLU rows for down) are staged in LDS
// once for the 4 waves, two chunks ahead through registers, in two buffers
// whose rows are padded to 272 bytes so that the 16 rows one ds_read_b128
// touches fall on distinct banks. Workgroup-level; smem: sd_smem<TOK>() bytes.
// Output rows row0 .. row0 + ntok - 1 of out (row length out_ld): gate_up
// rounds gate and up to bf16 and writes SwiGLU rows, down writes bf16 rows.
constexpr int kSdPitch = 136;  // bf16 a staged row (128 + 8 pad)
template <int TOK>
constexpr int sd_buf() { return TOK * kSdPitch; }  // bf16 a buffer of TOK rows
template <int TOK>
constexpr int sd_smem() { return 2 * sd_buf<TOK>() * 2; }  // bytes (two buffers)

// TOK: tokens of the group (32 or 64)
template <int PW, bool kGateUp, int TOK>
__device__ __forceinline__ void shared_rows_task(const uint8_t* __restrict__ tiles, int NC,
                                                 const uint16_t* __restrict__ bsrc, int K, int row0,
                                                 int ntok, int rb, uint16_t* __restrict__ out,
                                                 int out_ld, uint8_t* smem) {
  static_assert(PW % 2 == 0, "the stage registers alternate with the chunk's parity");
  static_assert(TOK % 16 == 0 && TOK <= 64, "token tiles of 16");
  constexpr int kThreads = kSplit * kWave;
  constexpr int kSdBuf = sd_buf<TOK>();
  constexpr int kPer = TOK * 16 / kThreads;  // 16-byte pieces a thread stages a chunk
  constexpr int NTT = TOK / 16;
  const int lane = threadIdx.x & (kWave - 1);
  const int w = threadIdx.x >> 6;
  const int g = lane >> 4, col = lane & 15;
  const int ntt = (ntok + 15) / 16;
  uint16_t* lx = reinterpret_cast<uint16_t*>(smem);

  // weights: row tile w of chunk c at tiles + c kBfTileBytes + w 4096 + q 1024
  const uint8_t* wl = tiles + w * 4096 + lane * 16;
  u32x4_t ring[PW][4];
  auto load_wc = [&](u32x4_t (&r)[4], int c) {
    const uint8_t* t = wl + static_cast<size_t>(c) * kBfTileBytes;
#pragma unroll
    for (int q = 0; q < 4; ++q) r[q] = *reinterpret_cast<const u32x4_t*>(t + q * 1024);
  };
  // token rows of chunk c: piece i * kThreads + tid = (token, 16-byte piece);
  // tokens past the group's repeat its last row and are never stored
  u32x4_t xs[2][kPer];
  auto load_x = [&](u32x4_t (&v)[kPer], int c) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int q = i * kThreads + threadIdx.x;
      const int t = row0 + min(q >> 4, ntok - 1);
      v[i] = *reinterpret_cast<const u32x4_t*>(bsrc + static_cast<size_t>(t) * K + c * kChunkK +
                                               8 * (q & 15));
    }
  };
  auto store_x = [&](const u32x4_t (&v)[kPer], int buf) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int q = i * kThreads + threadIdx.x;
      *reinterpret_cast<u32x4_t*>(lx + buf * kSdBuf + (q >> 4) * kSdPitch + 8 * (q & 15)) = v[i];
    }
  };

  f32x4_t acc[NTT];
#pragma unroll
  for (int tt = 0; tt < NTT; ++tt) acc[tt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  load_x(xs[0], 0);
#pragma unroll
  for (int i = 0; i < PW; ++i) load_wc(ring[i], min(i, NC - 1));
  load_x(xs[1], min(1, NC - 1));
  store_x(xs[0], 0);
  if (NC > 2) load_x(xs[0], 2);

  // chunk c: ring slot c % PW, staged rows in buffer c % 2; the stage
  // registers xs[(c + 1) % 2] hold chunk c + 1, then receive chunk c + 3
  for (int cb = 0; cb < NC; cb += PW) {
#pragma unroll
    for (int i = 0; i < PW; ++i) {
      const int c = cb + i;
      if (c < NC) {
        __syncthreads();  // buffer c % 2 holds chunk c; buffer (c + 1) % 2 is free
        const uint16_t* lb = lx + (c & 1) * kSdBuf + col * kSdPitch + 32 * g;
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt) {
          if (tt < ntt) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const u32x4_t b = *reinterpret_cast<const u32x4_t*>(lb + tt * 16 * kSdPitch + 8 * q);
              acc[tt] = mfma_bf16(__builtin_bit_cast(bf16x8_t, ring[i][q]),
                                  __builtin_bit_cast(bf16x8_t, b), acc[tt]);
            }
          }
        }
        if (c + PW < NC) load_wc(ring[i], c + PW);
        if (c + 1 < NC) {
          store_x(xs[(i + 1) & 1], (c + 1) & 1);  // PW is even: c + 1 and i + 1 agree mod 2
          if (c + 3 < NC) load_x(xs[(i + 1) & 1], c + 3);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }

  // rows 4g .. 4g + 3 of row tile w, token tt * 16 + col
#pragma unroll
  for (int tt = 0; tt < NTT; ++tt) {
    const int c = tt * 16 + col;
    if (tt >= ntt || c >= ntok) continue;
    uint16_t* orow = out + static_cast<size_t>(row0 + c) * out_ld;
    const f32x4_t v = acc[tt];
    if constexpr (kGateUp) {  // gate i, gate i + 1, up i, up i + 1
      const float g0 = round_bf16(v[0]), g1 = round_bf16(v[1]);
      const float u0 = round_bf16(v[2]), u1 = round_bf16(v[3]);
      *reinterpret_cast<uint32_t*>(orow + 32 * rb + 8 * w + 2 * g) =
          swiglu_bf16_bits(g0, u0) | (swiglu_bf16_bits(g1, u1) << 16);
    } else {
      *reinterpret_cast<u32x2_t*>(orow + kRowsPerBlock * rb + 16 * w + 4 * g) =
          u32x2_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
    }
  }
}

}  // namespace moeblk
