// pack.hip -- one-time repacking of canonical weights into the kernels' tile
// order (common.h, "layout"). The Muse Spark K3 page's stages "C, D" read MXFP4
// weights in pre-shuffled layouts; this is the same idea for this library's
// own tiles: the bytes are only permuted, never changed.
#include "common.h"
#include "host.h"

namespace moeblk {
namespace {

// one workgroup a tile (e, rb, c); thread = (row tile r, lane)
__global__ __launch_bounds__(256) void pack_mxfp4_kernel(const uint8_t* __restrict__ q,
                                                         const uint8_t* __restrict__ sc,
                                                         uint8_t* __restrict__ out, int which,
                                                         int N, int K, int RB, int NC) {
  const int tile = blockIdx.x;
  const int c = tile % NC;
  const int rb = (tile / NC) % RB;
  const int e = tile / (NC * RB);
  const int r = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int m = lane & 15, g = lane >> 4;
  const int n = packed_row(which, N / 2, rb, r, m);
  const size_t row = static_cast<size_t>(e) * N + n;
  const int k0 = kChunkK * c + 32 * g;
  const uint4 v = *reinterpret_cast<const uint4*>(q + row * (K / 2) + k0 / 2);
  uint8_t* t = out + static_cast<size_t>(tile) * kMxTileBytes;
  *reinterpret_cast<uint4*>(t + r * 1024 + lane * 16) = v;
  t[4096 + lane * 4 + r] = sc[row * (K / 32) + k0 / 32];
}

__global__ __launch_bounds__(256) void pack_bf16_kernel(const uint16_t* __restrict__ w,
                                                        uint8_t* __restrict__ out, int which,
                                                        int N, int K, int NC) {
  const int tile = blockIdx.x;
  const int c = tile % NC;
  const int rb = tile / NC;
  const int r = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int m = lane & 15, g = lane >> 4;
  const int n = packed_row(which, N / 2, rb, r, m);
  uint8_t* t = out + static_cast<size_t>(tile) * kBfTileBytes + r * 4096 + lane * 16;
#pragma unroll
  for (int qq = 0; qq < 4; ++qq) {
    const int k0 = kChunkK * c + 32 * g + 8 * qq;
    *reinterpret_cast<uint4*>(t + qq * 1024) =
        *reinterpret_cast<const uint4*>(w + static_cast<size_t>(n) * K + k0);
  }
}

bool weight_shape(const moe_dims& m, int which, bool shared, int& N, int& K) {
  const int I = shared ? m.shared_I : m.I;
  if (which == MOE_W13) {
    N = 2 * I;
    K = m.d;
  } else if (which == MOE_W2) {
    N = m.d;
    K = I;
  } else {
    return false;
  }
  return true;
}

}  // namespace

void launch_pack_bf16(const uint16_t* w, void* packed, int N, int K, hipStream_t stream) {
  const int RB = N / kRowsPerBlock, NC = K / kChunkK;
  hipLaunchKernelGGL(pack_bf16_kernel, dim3(RB * NC), dim3(256), 0, stream, w,
                     static_cast<uint8_t*>(packed), static_cast<int>(MOE_W2), N, K, NC);
}

}  // namespace moeblk

using namespace moeblk;

extern "C" size_t moe_packed_mxfp4_bytes(const moe_dims* dims, int which) {
  int N, K;
  if (check_dims(dims) || !weight_shape(*dims, which, false, N, K)) return 0;
  return static_cast<size_t>(dims->n_local) * (N / kRowsPerBlock) * (K / kChunkK) * kMxTileBytes;
}

extern "C" int moe_pack_mxfp4(const moe_dims* dims, int which, const void* q, const void* scales,
                              void* packed, hipStream_t stream) {
  const int rc = check_dims(dims);
  if (rc) return rc;
  int N, K;
  MOE_REQUIRE(weight_shape(*dims, which, false, N, K), MOE_ERR_UNSUPPORTED);
  MOE_REQUIRE(q && scales && packed, MOE_ERR_NULL);
  MOE_REQUIRE(aligned16(q) && aligned16(packed), MOE_ERR_ALIGN);
  const int RB = N / kRowsPerBlock, NC = K / kChunkK;
  hipLaunchKernelGGL(pack_mxfp4_kernel, dim3(dims->n_local * RB * NC), dim3(256), 0, stream,
                     static_cast<const uint8_t*>(q), static_cast<const uint8_t*>(scales),
                     static_cast<uint8_t*>(packed), which, N, K, RB, NC);
  return launch_status();
}

extern "C" size_t moe_packed_bf16_bytes(const moe_dims* dims, int which) {
  int N, K;
  if (check_dims(dims) || dims->shared_I == 0 || !weight_shape(*dims, which, true, N, K)) return 0;
  return static_cast<size_t>(N) * K * 2;
}

extern "C" int moe_pack_bf16(const moe_dims* dims, int which, const void* w, void* packed,
                             hipStream_t stream) {
  const int rc = check_dims(dims);
  if (rc) return rc;
  MOE_REQUIRE(dims->shared_I > 0, MOE_ERR_UNSUPPORTED);
  int N, K;
  MOE_REQUIRE(weight_shape(*dims, which, true, N, K), MOE_ERR_UNSUPPORTED);
  MOE_REQUIRE(w && packed, MOE_ERR_NULL);
  MOE_REQUIRE(aligned16(w) && aligned16(packed), MOE_ERR_ALIGN);
  if (which == MOE_W2) {
    launch_pack_bf16(static_cast<const uint16_t*>(w), packed, N, K, stream);
  } else {
    const int RB = N / kRowsPerBlock, NC = K / kChunkK;
    hipLaunchKernelGGL(pack_bf16_kernel, dim3(RB * NC), dim3(256), 0, stream,
                       static_cast<const uint16_t*>(w), static_cast<uint8_t*>(packed), which, N, K,
                       NC);
  }
  return launch_status();
}
