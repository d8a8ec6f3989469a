// host.h -- host-side argument checks shared by the entry points.
#pragma once

#include <stdint.h>

#include "moeblk.h"

namespace moeblk {

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline int r_max(const moe_dims& d) { return d.S * (d.topk < d.n_local ? d.topk : d.n_local); }

int check_dims(const moe_dims* d);  // MOE_OK or an error code
int check_proj_dims(const moe_proj_dims* d);

inline size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

int launch_status();  // MOE_OK, or MOE_ERR_HIP if the last launch failed

}  // namespace moeblk

#define MOE_REQUIRE(cond, code) \
  do {                          \
    if (!(cond)) return (code); \
  } while (0)
