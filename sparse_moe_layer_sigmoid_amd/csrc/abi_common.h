// Host-side helpers for the C ABI: status reporting and argument checks.
#pragma once

#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>

#include "moe.h"

namespace moe {

void set_error(const char* fmt, ...) __attribute__((format(printf, 1, 2)));
void clear_error();

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Report a launch error (if any) of the kernels just enqueued.
moe_status check_launch(const char* what);

}  // namespace moe

#define MOE_REQUIRE(cond, code, ...)   \
  do {                                 \
    if (!(cond)) {                     \
      ::moe::set_error(__VA_ARGS__);   \
      return (code);                   \
    }                                  \
  } while (0)
