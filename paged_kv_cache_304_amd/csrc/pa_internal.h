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

// PA_CHECK=1 in the environment: the entry points copy their device-resident
// metadata to the host and validate it before launching (synchronising the
// stream; a test and debugging aid, not for graph capture). Each check returns
// PA_EINVAL with a message naming the first violation.
bool checks_on();
// Kept tokens' final slots (after the SWA table, if any) inside the pool and unique.
pa_status check_slots(const char* fn, hipStream_t st, const int64_t* slot_mapping, int64_t num_tokens,
                      const int64_t* swa, int64_t swa_len, int64_t num_blocks, int32_t block_size);
// Context lengths within the table and every entry they use inside the pool.
pa_status check_tables(const char* fn, hipStream_t st, const int32_t* block_tables, int32_t num_seqs, int32_t W,
                       const int32_t* context_lens, int64_t num_blocks, int32_t block_size);
// Packed query offsets non-decreasing, within the tokens, each chunk no longer than its context.
pa_status check_chunks(const char* fn, hipStream_t st, const int32_t* cu_seqlens_q, int32_t num_seqs,
                       int64_t num_tokens, const int32_t* context_lens);

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
