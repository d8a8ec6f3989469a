// forward.hip -- moe_forward: the whole block as a chain of launches on one
// stream.
//
//   1  router logits (S <= 16: one workgroup an expert row; S <= 32: 16
//      tokens x a few rows a workgroup; beyond: tiles split over K, their
//      parts in the workspace)
//   2  the expert FFNs (ffn.hip: one launch, or two with a shared expert),
//      whose first S + 1 workgroups take every token's top-k (summing the
//      router's K parts beyond S = 32) and the bucketing; the expert tasks
//      wait for them on flags in the workspace, the shared expert's tasks do
//      not (K3 page, stage "route": the routing runs inside the persistent
//      launch that consumes it)
//   3  per-pick RMSNorm and the weighted sum (one workgroup a token), whose
//      workgroup 0 leaves the front's control block at zero for the next call
//
// moe_forward_one_launch runs all of it as one launch (S <= 16, d <= 4096, no
// shared expert): the router rows at the head of the front, the combine as
// the launch's last workgroups.
//
// The outputs are those of moe_route, moe_bucket, moe_expert_ffn and
// moe_combine, bit for bit: the same device code computes every value.
#include <mutex>

#include "bucket_dev.h"
#include "ffn_launch.h"
#include "host.h"
#include "launch.h"
#include "route_dev.h"

// The scratch of moe_forward_static, one copy a device for the life of the
// process. In host code `scratch` names a host-side stand-in, not device
// memory: the device address comes from hipGetSymbolAddress (below).
static __device__ __align__(256) uint8_t scratch[MOE_STATIC_SCRATCH_BYTES];

namespace moeblk {
namespace {

// zero n16 16-byte words at p, and *word if given (the control words of the
// FFN launch and a caller's error word): a kernel, not hipMemsetAsync, so
// that a captured graph replays it as a kernel node
__global__ void clear_kernel(uint4* __restrict__ p, size_t n16, int32_t* __restrict__ word) {
  for (size_t i = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x; i < n16;
       i += static_cast<size_t>(gridDim.x) * blockDim.x)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
  if (word && blockIdx.x == 0 && threadIdx.x == 0) *word = 0;
}

// the device address of `scratch` on the current device, looked up once per
// device with that device current
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};

int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
      (void)hipGetLastError();
      return MOE_ERR_HIP;
    }
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return MOE_OK;
}

// moe_forward runs the top-k and the bucketing as the routing front of the
// expert-FFN launch with a shared expert (its tasks stream during the front)
// or at S <= 64; without one at S > 64, where the front sums the router's K
// parts for every token before any task starts, the separate top-k and
// bucketing launches measured faster (S = 96 step: 86.2 against 84.7 us).
bool routing_front(const moe_dims& m) { return m.shared_I > 0 || m.S <= 64; }

// the block on one stream, after the argument checks; the workspace holds the
// router's K parts (S > 32), then the FFN's layout
int forward_enqueue(const moe_dims& m, const void* x, const float* w_router, const float* bias,
                    const void* w13_packed, const void* w2_packed, const void* ws13_packed,
                    const void* ws2_packed, const void* gamma, float* logits, int32_t* topk_ids,
                    float* topk_w, int32_t* counts, int32_t* offsets, int32_t* rows,
                    int32_t* pick_pos, int32_t* active, void* y, float* out, void* workspace,
                    hipStream_t stream, int32_t* error_word, bool one = false) {
  const size_t parts_bytes = router_parts_bytes(m);
  float* parts = parts_bytes ? static_cast<float*>(workspace) : nullptr;
  void* ffn_ws = static_cast<uint8_t*>(workspace) + parts_bytes;
  int frc;
  if (one) {
    // the whole block in the expert-FFN launch: router rows, top-k and
    // bucketing at its head, the combine at its tail; its last combine
    // workgroup leaves the front's control block at zero for the next call
    const FrontIo fio{nullptr, nullptr, w_router, out, static_cast<const uint16_t*>(gamma), bias,
                      logits, topk_ids, topk_w, offsets, pick_pos, active};
    frc = launch_ffn(m, x, w13_packed, w2_packed, ws13_packed, ws2_packed, counts, rows, y, ffn_ws,
                     stream, error_word, &fio);
    return frc ? frc : launch_status();
  }
  int32_t* front_block = nullptr;
  if (routing_front(m)) {
    launch_router_logits(m, x, w_router, bias, logits, stream, parts);
    // the top-k and the bucketing run at the head of the expert-FFN launch;
    // its control block is zero at the start of the call and the combine
    // launch leaves it at zero again
    const FrontIo fio{parts ? nullptr : logits, parts, nullptr, nullptr, nullptr, bias, logits,
                      topk_ids, topk_w, offsets, pick_pos, active};
    frc = launch_ffn(m, x, w13_packed, w2_packed, ws13_packed, ws2_packed, counts, rows, y, ffn_ws,
                     stream, error_word, &fio);
    front_block = route_front_block(m, ffn_ws);
  } else {  // the four calls' launches
    launch_router_logits(m, x, w_router, bias, logits, stream, parts);
    launch_topk(m, logits, bias, topk_ids, topk_w, stream, parts, logits);
    launch_bucket(m, topk_ids, counts, offsets, rows, pick_pos, active, stream);
    frc = launch_ffn(m, x, w13_packed, w2_packed, ws13_packed, ws2_packed, counts, rows, y, ffn_ws,
                     stream, error_word);
  }
  if (frc) return frc;
  launch_combine(m, y, topk_w, pick_pos, gamma, out, stream, front_block,
                 front_block ? kFrontWords : 0);
  return launch_status();
}

int check_forward_args(const moe_dims* dims, const void* x, const float* w_router,
                       const float* bias, const void* w13_packed, const void* w2_packed,
                       const void* ws13_packed, const void* ws2_packed, const void* gamma,
                       float* logits, int32_t* topk_ids, float* topk_w, int32_t* counts,
                       int32_t* offsets, int32_t* rows, int32_t* pick_pos, int32_t* active,
                       void* y, float* out) {
  const int rc = check_dims(dims);
  if (rc) return rc;
  const moe_dims& m = *dims;
  MOE_REQUIRE(x && w_router && w13_packed && w2_packed && logits && topk_ids && topk_w && counts &&
                  offsets && rows && pick_pos && active && y && out,
              MOE_ERR_NULL);
  MOE_REQUIRE(m.shared_I == 0 || (ws13_packed && ws2_packed), MOE_ERR_NULL);
  MOE_REQUIRE(aligned16(x) && aligned16(w_router) && (!bias || aligned16(bias)) &&
                  aligned16(w13_packed) && aligned16(w2_packed) &&
                  (!ws13_packed || aligned16(ws13_packed)) && (!ws2_packed || aligned16(ws2_packed)) &&
                  (!gamma || aligned16(gamma)) && aligned16(logits) && aligned16(topk_ids) &&
                  aligned16(topk_w) && aligned16(counts) && aligned16(offsets) && aligned16(rows) &&
                  aligned16(pick_pos) && aligned16(active) && aligned16(y) && aligned16(out),
              MOE_ERR_ALIGN);
  return MOE_OK;
}

}  // namespace
}  // namespace moeblk

using namespace moeblk;

// workspace: the router's K parts (S > 32), then the FFN's layout (its error
// word stays last)
extern "C" size_t moe_forward_workspace_bytes(const moe_dims* dims) {
  if (check_dims(dims)) return 0;
  return router_parts_bytes(*dims) + ffn_layout(*dims).total;
}

extern "C" int moe_forward(const moe_dims* dims, const void* x, const float* w_router,
                           const float* bias, const void* w13_packed, const void* w2_packed,
                           const void* ws13_packed, const void* ws2_packed, const void* gamma,
                           float* logits, int32_t* topk_ids, float* topk_w, int32_t* counts,
                           int32_t* offsets, int32_t* rows, int32_t* pick_pos, int32_t* active,
                           void* y, float* out, void* workspace, size_t workspace_bytes,
                           hipStream_t stream) {
  const int rc = check_forward_args(dims, x, w_router, bias, w13_packed, w2_packed, ws13_packed,
                                    ws2_packed, gamma, logits, topk_ids, topk_w, counts, offsets,
                                    rows, pick_pos, active, y, out);
  if (rc) return rc;
  MOE_REQUIRE(workspace, MOE_ERR_NULL);
  MOE_REQUIRE(aligned16(workspace), MOE_ERR_ALIGN);
  MOE_REQUIRE(workspace_bytes >= moe_forward_workspace_bytes(dims), MOE_ERR_WORKSPACE);
  return forward_enqueue(*dims, x, w_router, bias, w13_packed, w2_packed, ws13_packed, ws2_packed,
                         gamma, logits, topk_ids, topk_w, counts, offsets, rows, pick_pos, active,
                         y, out, workspace, stream, nullptr);
}

extern "C" int moe_forward_one_launch(const moe_dims* dims, const void* x, const float* w_router,
                                      const float* bias, const void* w13_packed,
                                      const void* w2_packed, const void* gamma, float* logits,
                                      int32_t* topk_ids, float* topk_w, int32_t* counts,
                                      int32_t* offsets, int32_t* rows, int32_t* pick_pos,
                                      int32_t* active, void* y, float* out, void* workspace,
                                      size_t workspace_bytes, hipStream_t stream) {
  const int dc = check_dims(dims);
  if (dc) return dc;
  MOE_REQUIRE(one_launch(*dims), MOE_ERR_UNSUPPORTED);
  const int rc = check_forward_args(dims, x, w_router, bias, w13_packed, w2_packed, nullptr, nullptr,
                                    gamma, logits, topk_ids, topk_w, counts, offsets, rows,
                                    pick_pos, active, y, out);
  if (rc) return rc;
  MOE_REQUIRE(workspace, MOE_ERR_NULL);
  MOE_REQUIRE(aligned16(workspace), MOE_ERR_ALIGN);
  MOE_REQUIRE(workspace_bytes >= moe_forward_workspace_bytes(dims), MOE_ERR_WORKSPACE);
  return forward_enqueue(*dims, x, w_router, bias, w13_packed, w2_packed, nullptr, nullptr, gamma,
                         logits, topk_ids, topk_w, counts, offsets, rows, pick_pos, active, y, out,
                         workspace, stream, nullptr, true);
}

extern "C" int moe_forward_static(const moe_dims* dims, const void* x, const float* w_router,
                                  const float* bias, const void* w13_packed, const void* w2_packed,
                                  const void* ws13_packed, const void* ws2_packed,
                                  const void* gamma, float* logits, int32_t* topk_ids,
                                  float* topk_w, int32_t* counts, int32_t* offsets, int32_t* rows,
                                  int32_t* pick_pos, int32_t* active, void* y, float* out,
                                  int32_t* wait_error, hipStream_t stream) {
  const int rc = check_forward_args(dims, x, w_router, bias, w13_packed, w2_packed, ws13_packed,
                                    ws2_packed, gamma, logits, topk_ids, topk_w, counts, offsets,
                                    rows, pick_pos, active, y, out);
  if (rc) return rc;
  const size_t need = moe_forward_workspace_bytes(dims);
  MOE_REQUIRE(need <= MOE_STATIC_SCRATCH_BYTES, MOE_ERR_WORKSPACE);
  void* base = nullptr;
  const int src = scratch_address(&base);
  if (src) return src;
  // the FFN's control words (counters, ready flags, error word) must start at
  // zero; the rest of the layout is written before it is read
  const moe_dims& m = *dims;
  const size_t ctl = router_parts_bytes(m) + ffn_layout(m).prod;
  const size_t n16 = (need - ctl) / 16;
  const int blocks = static_cast<int>(n16 / 256 + 1 < 256 ? n16 / 256 + 1 : 256);
  hipLaunchKernelGGL(clear_kernel, dim3(blocks), dim3(256), 0, stream,
                     reinterpret_cast<uint4*>(static_cast<uint8_t*>(base) + ctl), n16, wait_error);
  return forward_enqueue(m, x, w_router, bias, w13_packed, w2_packed, ws13_packed, ws2_packed, gamma,
                         logits, topk_ids, topk_w, counts, offsets, rows, pick_pos, active, y, out,
                         base, stream, wait_error);
}
