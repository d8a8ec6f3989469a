// abi.hip -- version, status strings and the dims checks (host only).
#include <math.h>

#include "host.h"

namespace moeblk {

int check_dims(const moe_dims* d) {
  MOE_REQUIRE(d != nullptr, MOE_ERR_NULL);
  MOE_REQUIRE(d->S >= 1 && d->S <= 128, MOE_ERR_SHAPE);
  MOE_REQUIRE(d->d >= 128 && d->d <= 16384 && d->d % 128 == 0, MOE_ERR_SHAPE);
  MOE_REQUIRE(d->E >= 1 && d->E <= 256, MOE_ERR_SHAPE);
  MOE_REQUIRE(d->topk >= 1 && d->topk <= 8 && d->topk <= d->E, MOE_ERR_SHAPE);
  MOE_REQUIRE(d->n_local >= 1 && d->n_local <= 32, MOE_ERR_SHAPE);
  MOE_REQUIRE(d->local_base >= 0 && d->local_base + d->n_local <= d->E, MOE_ERR_SHAPE);
  MOE_REQUIRE(d->I >= 128 && d->I <= 8192 && d->I % 128 == 0, MOE_ERR_SHAPE);
  MOE_REQUIRE(d->shared_I == 0 ||
                  (d->shared_I >= 128 && d->shared_I <= 8192 && d->shared_I % 128 == 0),
              MOE_ERR_SHAPE);
  MOE_REQUIRE(d->renorm == 0 || d->renorm == 1, MOE_ERR_UNSUPPORTED);
  MOE_REQUIRE(d->bias_mode == 0 || d->bias_mode == 1, MOE_ERR_UNSUPPORTED);
  MOE_REQUIRE(isfinite(d->eps) && d->eps >= 0.0f, MOE_ERR_UNSUPPORTED);
  return MOE_OK;
}

int check_proj_dims(const moe_proj_dims* d) {
  MOE_REQUIRE(d != nullptr, MOE_ERR_NULL);
  MOE_REQUIRE(d->S >= 1 && d->S <= 128, MOE_ERR_SHAPE);
  MOE_REQUIRE(d->K >= 128 && d->K <= 16384 && d->K % 128 == 0, MOE_ERR_SHAPE);
  MOE_REQUIRE(d->N >= 64 && d->N <= 16384 && d->N % 64 == 0, MOE_ERR_SHAPE);
  MOE_REQUIRE(d->E >= 0 && d->E <= 256, MOE_ERR_SHAPE);
  MOE_REQUIRE(d->bias_mode == 0 || d->bias_mode == 1, MOE_ERR_UNSUPPORTED);
  MOE_REQUIRE(isfinite(d->eps) && d->eps >= 0.0f, MOE_ERR_UNSUPPORTED);
  return MOE_OK;
}

int launch_status() { return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

}  // namespace moeblk

extern "C" {

int moe_abi_version(void) { return MOEBLK_ABI_VERSION; }

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_NULL: return "a required pointer is NULL";
    case MOE_ERR_SHAPE: return "a size is out of the supported range or inconsistent";
    case MOE_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case MOE_ERR_UNSUPPORTED: return "unsupported parameter value";
    case MOE_ERR_WORKSPACE: return "workspace too small";
    case MOE_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

int moe_check_dims(const moe_dims* dims) { return moeblk::check_dims(dims); }

}  // extern "C"
