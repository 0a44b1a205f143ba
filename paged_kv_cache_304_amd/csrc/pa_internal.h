// Host-side helpers shared by the C-ABI entry points (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pagedkv.h"

namespace pa {

// Records a formatted message for pa_last_error() and returns `status`.
pa_status fail(pa_status status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

// Maps a pending launch error to PA_EHIP (with `what` in the message).
pa_status after_launch(const char* what);

// Clears the calling thread's error text.
void clear_error();

inline bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

inline int dtype_bytes(pa_dtype t) {
  switch (t) {
    case PA_BF16: return 2;
    case PA_F32: return 4;
    case PA_FP8_E4M3FN: return 1;
    default: return 0;
  }
}

inline const char* dtype_name(pa_dtype t) {
  switch (t) {
    case PA_BF16: return "bf16";
    case PA_F32: return "f32";
    case PA_FP8_E4M3FN: return "fp8_e4m3fn";
    default: return "unknown";
  }
}

}  // namespace pa
