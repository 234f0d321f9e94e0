// Internal helpers shared by the library's translation units (not installed).
#pragma once

#include <cstdarg>
#include <cstdint>

#include "../../include/pagedkv.h"

namespace pkv {

// Records a formatted message as this thread's last error and returns `s`.
pkv_status fail(pkv_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

// Clears this thread's last error (called on entry of every ABI function that can fail).
void clear_error();

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline int dtype_bytes(int32_t dt) {
  switch (dt) {
    case PKV_F32: return 4;
    case PKV_F16: return 2;
    case PKV_BF16: return 2;
    default: return 0;
  }
}

}  // namespace pkv
