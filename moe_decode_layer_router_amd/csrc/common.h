// common.h -- device helpers and the packed weight layout shared by the
// kernels of libmoeblk (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moeblk.h"

namespace moeblk {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// ---------------------------------------------------------------- layout
//
// Packed MXFP4 weight, per expert an N x K matrix (N % 64 == 0, K % 128 == 0):
// row blocks of 64 rows (4 MFMA row tiles of 16) x chunks of 128 K. One tile
// (expert e, row block rb, chunk c) is 4352 contiguous bytes:
//   [r * 1024 + lane * 16, +16)  row tile r, lane: the 32 e2m1 codes of row
//                                m = lane % 16 at K = 128 c + 32 (lane / 16) .. + 32
//                                (canonical bytes, low nibble = even K);
//   [4096 + lane * 4 + r]        the e8m0 byte of those 32 elements.
// Tiles are ordered (e, rb, c). A wave streaming its chunks of one row block
// reads 4 x 1 KiB + 256 B contiguous per chunk.
//
// Packed bf16 weight (shared expert), one N x K matrix: tile (rb, c) is 16 KiB,
//   [r * 4096 + q * 1024 + lane * 16, +16)  8 bf16 of row m = lane % 16 of row
//                                tile r at K = 128 c + 32 (lane / 16) + 8 q .. + 8.
//
// Row order inside a row block. Down (MOE_W2): row 64 rb + 16 r + m. Gate_up
// (MOE_W13): the 64 rows of block rb hold the gate and up rows of intermediates
// i = 32 rb .. 32 rb + 31, interleaved so that one MFMA lane owns matching
// gate / up outputs: row m of tile r is, with i = 32 rb + 8 r + 2 (m / 4) + (m % 2),
// gate row i for m % 4 < 2 and up row I + i otherwise. The MFMA output lane with
// k-group g = lane / 16 holds rows 4 g .. 4 g + 3 = (gate i, gate i+1, up i, up i+1).
constexpr int kRowsPerBlock = 64;
constexpr int kChunkK = 128;
constexpr int kMxTileBytes = 4352;  // 4 * 1024 + 256
constexpr int kBfTileBytes = 16384;

__host__ __device__ inline int packed_row(int which, int half_n, int rb, int r, int m) {
  if (which == MOE_W2) return kRowsPerBlock * rb + 16 * r + m;
  const int i = 32 * rb + 8 * r + 2 * (m >> 2) + (m & 1);
  return (m & 2) ? half_n + i : i;
}

// ---------------------------------------------------------------- bf16

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp32 -> bf16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}
__device__ __forceinline__ float round_bf16(float f) {
  return __uint_as_float(f32_to_bf16_bits(f) << 16);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

// ---------------------------------------------------------------- MXFP4

// e8m0 byte -> the fp32 scale operand of the scaled fp4 converts: the byte
// in the exponent field, zero mantissa. The converts read only that field as
// an e8m0 scale (measured on MI355X for every byte and code, through an MFMA
// read-back): byte 0 scales by 2^-127 (0.5 decodes to the bf16 subnormal
// 2^-128), 255 makes every element NaN, and at bytes 253 and 254 a decoded
// magnitude of 2^128 or more becomes +-inf (bf16 has fp32's exponent range).
__device__ __forceinline__ float e8m0_scale(uint32_t x) { return __uint_as_float(x << 23); }

// 8 e2m1 codes (one dword, low nibble first) times `scale` -> 8 bf16, in K order.
// Feeding MFMA operands, this compiles to four converts with the four byte
// selects. (A probe that stored the 8 results to memory one by one compiled
// to a single convert whose first element was copied to all 8; such uses need
// their assembly checked.)
__device__ __forceinline__ bf16x8_t decode_fp4x8(uint32_t w, float scale) {
  const bf16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 0);
  const bf16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 1);
  const bf16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 2);
  const bf16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 3);
  return bf16x8_t{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// D[16x16] += A[16x32] B[32x16], bf16 in, fp32 accumulate. Lane l holds A row
// l % 16 and B column l % 16, 8 K values each; D rows 4 (l / 16) .. + 3 of column l % 16.
__device__ __forceinline__ f32x4_t mfma_bf16(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// cache-policy operand of the buffer intrinsics: sc1 = device-scope coherent
constexpr int kCpolSc1 = 16;

template <typename T>
__device__ __forceinline__ T ld_nt(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const T*>(p));
}

// fp64 -> bf16 bits, round to nearest even, without double rounding: the
// value is first rounded to fp32 "to odd" (an inexact result gets its last
// significand bit set), which keeps enough information for the final rounding.
__device__ __forceinline__ uint32_t f64_to_bf16_bits(double v) {
  if (v != v) return 0x7fc0u;
  const float f = static_cast<float>(v);  // nearest fp32
  uint32_t u = __float_as_uint(f);
  if (static_cast<double>(f) != v && (u & 0x7f800000u) != 0x7f800000u) {
    if (f == 0.0f) {
      u |= 1u;  // below the smallest subnormal: an odd neighbour of zero
    } else if ((u & 1u) == 0u) {
      const bool away = (v > static_cast<double>(f)) == (f > 0.0f);  // toward v = larger magnitude?
      u = away ? u + 1u : u - 1u;
    }
  }
  return f32_to_bf16_bits(__uint_as_float(u));
}

// SwiGLU of one gate / up pair of bf16 values, evaluated in fp64 and rounded
// once to bf16: silu(g) * u with silu(g) = g / (1 + exp(-g)). In fp32, 1 + exp(-g)
// is exactly 1 above g ~ 17 and exp(-g) overflows below g ~ -88, which would move
// results across bf16 rounding boundaries; fp64 keeps the elementwise rounding
// of the exact product.
__device__ __forceinline__ uint32_t swiglu_bf16_bits(float g, float u) {
  const double gd = g;
  return f64_to_bf16_bits(gd / (1.0 + exp(-gd)) * static_cast<double>(u));
}

// wave-wide sum, every lane gets the total; fixed butterfly order
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

}  // namespace moeblk
