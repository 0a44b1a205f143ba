// Optional host validation of the device-resident metadata of a call
// (PA_CHECK=1 in the environment; a test and debugging aid, never for graph
// capture or timing: it synchronises the stream and copies the metadata to
// the host before the launch).
//
// Without it the kernels treat out-of-range metadata as defined skips: a slot
// outside the SWA table or the pool skips its token, a table entry outside the
// pool removes its positions from the softmax, a length past the table is
// clamped. With it those become PA_EINVAL, and so do the preconditions the
// kernels cannot detect at all: two kept tokens resolving to the same final
// slot (their writes would race), and a prefill chunk longer than its context
// or packed query offsets that go backwards.
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <utility>
#include <vector>

#include "pa_internal.h"

namespace pa {

bool checks_on() {
  const char* v = getenv("PA_CHECK");
  return v != nullptr && strcmp(v, "1") == 0;
}

namespace {

// n elements of device (or host-visible) memory at src into out, after
// everything queued on the stream has run.
template <typename T>
pa_status fetch(const char* fn, hipStream_t st, const T* src, int64_t n, std::vector<T>& out) {
  out.assign((size_t)(n > 0 ? n : 0), T{});
  if (n <= 0) return PA_OK;
  if (hipStreamSynchronize(st) != hipSuccess)
    return fail(PA_EHIP, "%s: PA_CHECK: stream synchronisation failed", fn);
  if (hipMemcpy(out.data(), src, (size_t)n * sizeof(T), hipMemcpyDefault) != hipSuccess)
    return fail(PA_EHIP, "%s: PA_CHECK: copying the metadata to the host failed", fn);
  return PA_OK;
}

}  // namespace

pa_status check_slots(const char* fn, hipStream_t st, const int64_t* slot_mapping, int64_t num_tokens,
                      const int64_t* swa, int64_t swa_len, int64_t num_blocks, int32_t block_size) {
  std::vector<int64_t> slots, table;
  pa_status s = fetch(fn, st, slot_mapping, num_tokens, slots);
  if (s != PA_OK) return s;
  if (swa && (s = fetch(fn, st, swa, swa_len, table)) != PA_OK) return s;
  const int64_t pool = num_blocks * (int64_t)block_size;
  std::vector<std::pair<int64_t, int64_t>> kept;  // (final slot, token)
  for (int64_t t = 0; t < num_tokens; ++t) {
    int64_t v = slots[(size_t)t];
    if (v < 0) continue;
    if (swa) {
      if (v >= swa_len)
        return fail(PA_EINVAL, "%s: PA_CHECK: token %lld: slot %lld is past the SWA table (%lld entries)", fn,
                    (long long)t, (long long)v, (long long)swa_len);
      v = table[(size_t)v];
      if (v < 0) continue;
    }
    if (v >= pool)
      return fail(PA_EINVAL, "%s: PA_CHECK: token %lld: slot %lld is past the pool (%lld slots)", fn, (long long)t,
                  (long long)v, (long long)pool);
    kept.emplace_back(v, t);
  }
  std::sort(kept.begin(), kept.end());
  for (size_t i = 1; i < kept.size(); ++i)
    if (kept[i].first == kept[i - 1].first)
      return fail(PA_EINVAL, "%s: PA_CHECK: tokens %lld and %lld both write slot %lld", fn,
                  (long long)kept[i - 1].second, (long long)kept[i].second, (long long)kept[i].first);
  return PA_OK;
}

pa_status check_tables(const char* fn, hipStream_t st, const int32_t* block_tables, int32_t num_seqs, int32_t W,
                       const int32_t* context_lens, int64_t num_blocks, int32_t block_size) {
  std::vector<int32_t> bt, ctx;
  pa_status s = fetch(fn, st, context_lens, num_seqs, ctx);
  if (s != PA_OK) return s;
  if ((s = fetch(fn, st, block_tables, (int64_t)num_seqs * W, bt)) != PA_OK) return s;
  const int64_t cap = (int64_t)W * block_size;
  for (int32_t b = 0; b < num_seqs; ++b) {
    const int64_t c = ctx[(size_t)b];
    if (c < 0 || c > cap)
      return fail(PA_EINVAL, "%s: PA_CHECK: sequence %d: context length %lld outside [0, %lld]", fn, b, (long long)c,
                  (long long)cap);
    const int64_t nb = (c + block_size - 1) / block_size;
    for (int64_t j = 0; j < nb; ++j) {
      const int64_t e = bt[(size_t)((int64_t)b * W + j)];
      if (e < 0 || e >= num_blocks)
        return fail(PA_EINVAL, "%s: PA_CHECK: sequence %d: table entry %lld = %lld is outside the pool (%lld blocks)",
                    fn, b, (long long)j, (long long)e, (long long)num_blocks);
    }
  }
  return PA_OK;
}

pa_status check_chunks(const char* fn, hipStream_t st, const int32_t* cu_seqlens_q, int32_t num_seqs,
                       int64_t num_tokens, const int32_t* context_lens) {
  std::vector<int32_t> cu, ctx;
  pa_status s = fetch(fn, st, cu_seqlens_q, (int64_t)num_seqs + 1, cu);
  if (s != PA_OK) return s;
  if ((s = fetch(fn, st, context_lens, num_seqs, ctx)) != PA_OK) return s;
  if (cu[0] < 0) return fail(PA_EINVAL, "%s: PA_CHECK: cu_seqlens_q[0] = %d < 0", fn, cu[0]);
  for (int32_t b = 0; b < num_seqs; ++b) {
    const int64_t n = (int64_t)cu[(size_t)b + 1] - cu[(size_t)b];
    if (n < 0)
      return fail(PA_EINVAL, "%s: PA_CHECK: cu_seqlens_q decreases at sequence %d (%d -> %d)", fn, b, cu[(size_t)b],
                  cu[(size_t)b + 1]);
    if (n > ctx[(size_t)b])
      return fail(PA_EINVAL, "%s: PA_CHECK: sequence %d: chunk of %lld tokens is longer than its context (%d)", fn, b,
                  (long long)n, ctx[(size_t)b]);
  }
  if (cu[(size_t)num_seqs] > num_tokens)
    return fail(PA_EINVAL, "%s: PA_CHECK: cu_seqlens_q ends at %d, past the %lld packed tokens", fn,
                cu[(size_t)num_seqs], (long long)num_tokens);
  return PA_OK;
}

}  // namespace pa
