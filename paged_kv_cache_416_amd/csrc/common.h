// Shared host-side helpers of the pkv library: status codes, thread-local error text.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdint>

#include "pkv.h"

namespace pkv {

// Record a formatted message as this thread's last error and return `code`.
int fail(int code, const char *fmt, ...) __attribute__((format(printf, 2, 3)));

// PKV_OK if e == hipSuccess, else PKV_EHIP with the runtime's message.
int hip_status(hipError_t e, const char *what);

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline int elt_bytes(int32_t dtype) { return dtype == PKV_F32 ? 4 : 2; }

inline bool valid_dtype(int32_t dtype) { return dtype == PKV_F32 || dtype == PKV_F16 || dtype == PKV_BF16; }

}  // namespace pkv
