// combine.hip -- moe_combine: one workgroup a token (combine_dev.h).
#include "combine_dev.h"
#include "host.h"
#include "launch.h"

namespace moeblk {
namespace {

template <int VPT>
__global__ __launch_bounds__(kCombineThreads) void combine_kernel(
    const uint16_t* __restrict__ y, const float* __restrict__ tw, const int32_t* __restrict__ pick_pos,
    const uint16_t* __restrict__ gamma, float* __restrict__ out, int d, int topk, float eps,
    long shared_row0, int32_t* __restrict__ clear, int n_clear) {
  // words the next call's launches need at zero (moe_forward's routing
  // front): plain stores, which the launch boundary publishes
  if (clear && blockIdx.x == 0)
    for (int i = threadIdx.x; i < n_clear; i += blockDim.x) clear[i] = 0;
  if constexpr (VPT <= 2) {  // d <= 8192: the picks' rows staged in LDS
    __shared__ CombineLds L;
    const size_t s0 = static_cast<size_t>(blockIdx.x) * topk;
    combine_token_staged<VPT>(y, tw + s0, pick_pos + s0, gamma, out, d, topk, eps, shared_row0,
                              blockIdx.x, L);
  } else {
    __shared__ double red[8][kCombineThreads / kWave];
    combine_token_slots<VPT>(y, tw, pick_pos, gamma, out, d, topk, eps, shared_row0, blockIdx.x,
                             red);
  }
}

template <int VPT>
void launch(const moe_dims& m, const uint16_t* y, const float* tw, const int32_t* pp,
            const uint16_t* gamma, float* out, hipStream_t stream, int32_t* clear, int n_clear) {
  const long shared_row0 = m.shared_I > 0 ? static_cast<long>(r_max(m)) : -1;
  hipLaunchKernelGGL(combine_kernel<VPT>, dim3(m.S), dim3(kCombineThreads), 0, stream, y, tw, pp,
                     gamma, out, m.d, m.topk, m.eps, shared_row0, clear, n_clear);
}

}  // namespace

void launch_combine(const moe_dims& m, const void* y, const float* w, const int32_t* pick_pos,
                    const void* gamma, float* out, hipStream_t stream, int32_t* clear,
                    int n_clear) {
  const uint16_t* yy = static_cast<const uint16_t*>(y);
  const uint16_t* gg = static_cast<const uint16_t*>(gamma);
  switch (combine_vpt(m.d)) {
    case 1: launch<1>(m, yy, w, pick_pos, gg, out, stream, clear, n_clear); break;
    case 2: launch<2>(m, yy, w, pick_pos, gg, out, stream, clear, n_clear); break;
    case 4: launch<4>(m, yy, w, pick_pos, gg, out, stream, clear, n_clear); break;
    default: launch<8>(m, yy, w, pick_pos, gg, out, stream, clear, n_clear); break;
  }
}

}  // namespace moeblk

using namespace moeblk;

extern "C" int moe_combine(const moe_dims* dims, const void* y, const float* topk_w,
                           const int32_t* pick_pos, const void* gamma, float* out,
                           hipStream_t stream) {
  const int rc = check_dims(dims);
  if (rc) return rc;
  MOE_REQUIRE(y && topk_w && pick_pos && out, MOE_ERR_NULL);
  MOE_REQUIRE(aligned16(y) && aligned16(topk_w) && aligned16(pick_pos) && aligned16(out) &&
                  (!gamma || aligned16(gamma)),
              MOE_ERR_ALIGN);
  launch_combine(*dims, y, topk_w, pick_pos, gamma, out, stream);
  return launch_status();
}
