// Host-side validation of the MoE layer library's arguments: plain C++ (no
// HIP), shared by the host entry points (host.cpp) and the device entry
// points (api.hip).  Not installed.
#pragma once

#include <stdint.h>

#include "moe.h"

namespace moe {

// Shape and format of a layer descriptor: MOE_OK or the status to return.
int check_shape(const moe_layer_desc* d);
// expert_stride: at least one blob, a multiple of 256 bytes.
int check_stride(const moe_layer_desc* d);
// A required pointer: non-null and aligned to `align` bytes.
int check_ptr(const void* p, uintptr_t align = 16);
// An optional pointer: null, or aligned to `align` bytes.
int check_opt_ptr(const void* p, uintptr_t align = 16);

}  // namespace moe

#define MOE_TRY(expr)              \
  do {                             \
    const int _st = (expr);        \
    if (_st != MOE_OK) return _st; \
  } while (0)
