// Host block manager: allocation of paged KV blocks in block_size units and
// the per-step metadata the cache kernels read (slot_mapping, block_tables,
// context_lens, cu_seqlens_q), staged in one host blob and uploaded with one
// copy.
//
// Follows the "PagedAttention principle" page, paged attention principle
// section: a request of n tokens holds ceil(n / block_size) blocks (less than
// one block wasted), its blocks need not be adjacent and a table keeps their
// order, and the host copies that table to the device before the kernel runs.
// Slots are the Qwen3-0.6B engine walkthrough page's (section 2.6)
// block * block_size + offset.
//
// State is plain arrays sized at creation: a free stack, and per sequence its
// length, block count and a max_blocks_per_seq row of block ids. Planning a
// step is O(new blocks + new tokens + listed table rows); nothing allocates
// after creation.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <climits>
#include <cstring>
#include <new>
#include <vector>

#include "pa_internal.h"
#include "pagedkv.h"

struct pa_block_manager {
  int64_t num_blocks;
  int32_t block_size, max_seqs, W, max_step_seqs;
  int64_t max_step_tokens;
  pa_bm_layout layout;
  std::vector<int32_t> free_stack;  // top = back()
  std::vector<int64_t> len;         // per sequence
  std::vector<int32_t> nblk;        // per sequence
  std::vector<int32_t> table;       // [max_seqs, W]
  std::vector<uint32_t> mark;       // duplicate detection within a step
  uint32_t epoch = 0;
};

namespace {

int64_t round256(int64_t x) { return (x + 255) / 256 * 256; }

int64_t blocks_for(int64_t len, int32_t bs) { return (len + bs - 1) / bs; }

pa_bm_layout make_layout(int32_t max_step_seqs, int64_t max_step_tokens, int32_t W) {
  pa_bm_layout l;
  l.context_lens = 0;
  l.cu_seqlens_q = round256(l.context_lens + 4 * (int64_t)max_step_seqs);
  l.slot_mapping = round256(l.cu_seqlens_q + 4 * ((int64_t)max_step_seqs + 1));
  l.block_tables = round256(l.slot_mapping + 8 * max_step_tokens);
  l.bytes = round256(l.block_tables + 4 * (int64_t)max_step_seqs * W);
  return l;
}

}  // namespace

extern "C" pa_status pa_bm_create(int64_t num_blocks, int32_t block_size, int32_t max_seqs,
                                  int32_t max_blocks_per_seq, int32_t max_step_seqs, int64_t max_step_tokens,
                                  pa_block_manager** out) {
  using namespace pa;
  clear_error();
  const char* fn = "pa_bm_create";
  if (!out) return fail(PA_EINVAL, "%s: out is NULL", fn);
  *out = nullptr;
  if (num_blocks <= 0 || num_blocks > INT32_MAX) return fail(PA_EINVAL, "%s: num_blocks must be in [1, 2^31)", fn);
  if (block_size <= 0 || max_seqs <= 0 || max_blocks_per_seq <= 0 || max_step_seqs <= 0 || max_step_tokens <= 0)
    return fail(PA_EINVAL, "%s: sizes must be positive", fn);
  if ((int64_t)max_blocks_per_seq * block_size > INT32_MAX)
    return fail(PA_EINVAL, "%s: max_blocks_per_seq * block_size must fit int32 (context_lens are int32)", fn);
  const pa_bm_layout l = make_layout(max_step_seqs, max_step_tokens, max_blocks_per_seq);
  pa_block_manager* bm = new (std::nothrow) pa_block_manager;
  if (!bm) return fail(PA_EINVAL, "%s: out of host memory", fn);
  try {
    bm->free_stack.resize((size_t)num_blocks);
    for (int64_t i = 0; i < num_blocks; ++i) bm->free_stack[(size_t)i] = (int32_t)(num_blocks - 1 - i);
    bm->len.assign((size_t)max_seqs, 0);
    bm->nblk.assign((size_t)max_seqs, 0);
    bm->table.assign((size_t)max_seqs * max_blocks_per_seq, -1);
    bm->mark.assign((size_t)max_seqs, 0);
  } catch (const std::bad_alloc&) {
    delete bm;
    return fail(PA_EINVAL, "%s: out of host memory for %d sequences x %d blocks", fn, max_seqs, max_blocks_per_seq);
  }
  bm->num_blocks = num_blocks;
  bm->block_size = block_size;
  bm->max_seqs = max_seqs;
  bm->W = max_blocks_per_seq;
  bm->max_step_seqs = max_step_seqs;
  bm->max_step_tokens = max_step_tokens;
  bm->layout = l;
  *out = bm;
  return PA_OK;
}

extern "C" void pa_bm_destroy(pa_block_manager* bm) { delete bm; }

extern "C" pa_status pa_bm_layout_of(const pa_block_manager* bm, pa_bm_layout* out) {
  pa::clear_error();
  if (!bm || !out) return pa::fail(PA_EINVAL, "pa_bm_layout_of: NULL argument");
  *out = bm->layout;
  return PA_OK;
}

extern "C" int64_t pa_bm_free_blocks(const pa_block_manager* bm) {
  return bm ? (int64_t)bm->free_stack.size() : -1;
}

extern "C" int64_t pa_bm_seq_len(const pa_block_manager* bm, int32_t seq) {
  if (!bm || seq < 0 || seq >= bm->max_seqs) return -1;
  return bm->len[(size_t)seq];
}

extern "C" int32_t pa_bm_seq_table(const pa_block_manager* bm, int32_t seq, int32_t* blocks, int32_t capacity) {
  if (!bm || seq < 0 || seq >= bm->max_seqs) return -1;
  const int32_t n = bm->nblk[(size_t)seq];
  if (n > 0 && (!blocks || capacity < n)) return -1;
  if (n > 0) std::memcpy(blocks, &bm->table[(size_t)seq * bm->W], sizeof(int32_t) * (size_t)n);
  return n;
}

extern "C" pa_status pa_bm_release(pa_block_manager* bm, int32_t seq) {
  using namespace pa;
  clear_error();
  if (!bm) return fail(PA_EINVAL, "pa_bm_release: NULL manager");
  if (seq < 0 || seq >= bm->max_seqs) return fail(PA_EINVAL, "pa_bm_release: sequence id %d outside [0, %d)", seq, bm->max_seqs);
  int32_t* row = &bm->table[(size_t)seq * bm->W];
  const int32_t n = bm->nblk[(size_t)seq];
  for (int32_t k = n - 1; k >= 0; --k) {  // the first block ends on top
    bm->free_stack.push_back(row[k]);
    row[k] = -1;
  }
  bm->nblk[(size_t)seq] = 0;
  bm->len[(size_t)seq] = 0;
  return PA_OK;
}

extern "C" pa_status pa_bm_plan_step(pa_block_manager* bm, const int32_t* seqs, const int32_t* num_new,
                                     int32_t num_seqs, int32_t pad_seqs, int64_t pad_tokens, void* host_meta,
                                     int64_t host_meta_bytes, int64_t* num_tokens) {
  using namespace pa;
  clear_error();
  const char* fn = "pa_bm_plan_step";
  if (!bm) return fail(PA_EINVAL, "%s: NULL manager", fn);
  if (num_seqs < 0 || pad_seqs < num_seqs || pad_seqs > bm->max_step_seqs)
    return fail(PA_EINVAL, "%s: need 0 <= num_seqs (%d) <= pad_seqs (%d) <= max_step_seqs (%d)", fn, num_seqs,
                pad_seqs, bm->max_step_seqs);
  if (num_seqs > 0 && (!seqs || !num_new)) return fail(PA_EINVAL, "%s: NULL seqs / num_new", fn);
  if (!host_meta || !aligned(host_meta, 8)) return fail(PA_EINVAL, "%s: host_meta NULL or not 8-byte aligned", fn);
  if (host_meta_bytes < bm->layout.bytes)
    return fail(PA_EINVAL, "%s: host_meta holds %lld bytes, the layout needs %lld", fn, (long long)host_meta_bytes,
                (long long)bm->layout.bytes);

  // Check the whole step before changing anything.
  const int32_t bs = bm->block_size;
  if (++bm->epoch == 0) {  // wrapped: clear the marks once
    std::fill(bm->mark.begin(), bm->mark.end(), 0u);
    bm->epoch = 1;
  }
  int64_t total = 0, need = 0;
  for (int32_t i = 0; i < num_seqs; ++i) {
    const int32_t s = seqs[i];
    if (s < 0 || s >= bm->max_seqs) return fail(PA_EINVAL, "%s: seqs[%d] = %d outside [0, %d)", fn, i, s, bm->max_seqs);
    if (bm->mark[(size_t)s] == bm->epoch) return fail(PA_EINVAL, "%s: sequence %d listed twice", fn, s);
    bm->mark[(size_t)s] = bm->epoch;
    if (num_new[i] < 0) return fail(PA_EINVAL, "%s: num_new[%d] = %d is negative", fn, i, num_new[i]);
    const int64_t nl = bm->len[(size_t)s] + num_new[i];
    const int64_t nb = blocks_for(nl, bs);
    if (nb > bm->W)
      return fail(PA_EINVAL, "%s: sequence %d would need %lld blocks, more than max_blocks_per_seq %d", fn, s,
                  (long long)nb, bm->W);
    need += nb - bm->nblk[(size_t)s];
    total += num_new[i];
  }
  if (total > pad_tokens || pad_tokens > bm->max_step_tokens)
    return fail(PA_EINVAL, "%s: need tokens (%lld) <= pad_tokens (%lld) <= max_step_tokens (%lld)", fn,
                (long long)total, (long long)pad_tokens, (long long)bm->max_step_tokens);
  if (need > (int64_t)bm->free_stack.size())
    return fail(PA_ENOSPACE, "%s: the step needs %lld new blocks, %lld are free", fn, (long long)need,
                (long long)bm->free_stack.size());

  // Apply: allocate, then write the blob.
  char* base = static_cast<char*>(host_meta);
  int32_t* ctx = reinterpret_cast<int32_t*>(base + bm->layout.context_lens);
  int32_t* cu = reinterpret_cast<int32_t*>(base + bm->layout.cu_seqlens_q);
  int64_t* slots = reinterpret_cast<int64_t*>(base + bm->layout.slot_mapping);
  int32_t* tables = reinterpret_cast<int32_t*>(base + bm->layout.block_tables);
  const size_t W = (size_t)bm->W;
  int64_t t = 0;
  for (int32_t i = 0; i < num_seqs; ++i) {
    const size_t s = (size_t)seqs[i];
    int32_t* row = &bm->table[s * W];
    const int64_t old_len = bm->len[s], new_len = old_len + num_new[i];
    const int32_t nb = (int32_t)blocks_for(new_len, bs);
    for (int32_t k = bm->nblk[s]; k < nb; ++k) {
      row[k] = bm->free_stack.back();
      bm->free_stack.pop_back();
    }
    bm->nblk[s] = nb;
    bm->len[s] = new_len;
    ctx[i] = (int32_t)new_len;
    cu[i] = (int32_t)t;
    for (int64_t p = old_len; p < new_len; ++p) slots[t++] = (int64_t)row[p / bs] * bs + p % bs;
    std::memcpy(tables + (size_t)i * W, row, sizeof(int32_t) * (size_t)nb);
    std::fill(tables + (size_t)i * W + nb, tables + (size_t)(i + 1) * W, -1);
  }
  for (int32_t i = num_seqs; i < pad_seqs; ++i) {
    ctx[i] = 0;
    cu[i] = (int32_t)total;
  }
  cu[pad_seqs] = (int32_t)total;
  std::fill(slots + total, slots + pad_tokens, (int64_t)-1);
  std::fill(tables + (size_t)num_seqs * W, tables + (size_t)pad_seqs * W, -1);
  if (num_tokens) *num_tokens = total;
  return PA_OK;
}

extern "C" pa_status pa_bm_upload(const pa_block_manager* bm, const void* host_meta, void* device_meta,
                                  int32_t pad_seqs, void* stream) {
  using namespace pa;
  clear_error();
  const char* fn = "pa_bm_upload";
  if (!bm || !host_meta || !device_meta) return fail(PA_EINVAL, "%s: NULL argument", fn);
  if (pad_seqs < 0 || pad_seqs > bm->max_step_seqs)
    return fail(PA_EINVAL, "%s: pad_seqs %d outside [0, %d]", fn, pad_seqs, bm->max_step_seqs);
  if (!aligned(device_meta, 256)) return fail(PA_EINVAL, "%s: device_meta must be 256-byte aligned", fn);
  const size_t bytes = (size_t)(bm->layout.block_tables + 4 * (int64_t)pad_seqs * bm->W);
  const hipError_t e =
      hipMemcpyAsync(device_meta, host_meta, bytes, hipMemcpyHostToDevice, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(PA_EHIP, "%s: hipMemcpyAsync: %s", fn, hipGetErrorString(e));
  return PA_OK;
}
