// pa_reshape_and_cache: token-major K/V -> paged cache through a slot mapping.
//
// Operation (store_kvcache in section 2.6 "Attention" of the Qwen3-0.6B engine
// walkthrough page; reshape_and_cache_flash in SGLang's cache_ops.py): token t
// resolves a slot (optional second-stage SWA table, negative = skip), the slot
// splits into (block, offset), and the token's [H, D] row is encoded (bit copy,
// or fp32 division by the scale then round-to-nearest-even) into
// cache[block, offset, :, :].
//
// gfx950 design: one wavefront per token (four per 256-thread workgroup). The
// slot chain is read with scalar loads, so the skip test is wave-uniform and
// costs no vector work. A token's [H*D] row is contiguous in both the source
// and the cache, so each lane moves 8-element vectors (16-byte loads of bf16,
// 8- or 16-byte stores) and a wave stores whole contiguous rows. Rows longer
// than 64 lanes x kU vectors are split over gridDim.y. Loads and stores are
// non-temporal: the data is streamed exactly once. The division by a scale is
// a multiply by the fp64 reciprocal (exact for normal quotients, see
// div_by_scale) and the encodes are the hardware packed converts, which keeps
// the vector ALU work per element small enough for the copy to stay HBM-bound.
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

// 8-element vectors per lane per tensor: a wave moves 512 elements of a row and
// longer rows take more workgroup rows (gridDim.y). Half-row waves (1) measured
// 37.2 us against 38.2 us for whole-row waves (2) on the 32,768-token bf16 -> fp8
// write with a cold Infinity Cache; two or four tokens per wave were slower still.
constexpr int kU = 1;

struct RacArgs {
  const void* key;
  const void* value;
  void* key_cache;
  void* value_cache;
  const int64_t* slot_mapping;
  const int64_t* swa;
  const float* k_scale;
  const float* v_scale;
  int64_t swa_len;
  int64_t num_tokens;
  int64_t pool_slots;
  int64_t key_stride;    // elements
  int64_t value_stride;  // elements
  int64_t block_stride;  // elements
  int32_t block_size;
  int32_t bs_shift;      // log2(block_size), or -1 when not a power of two
  int32_t row_elems;     // num_heads * head_size
};

// Final slot of token t, or -1 when the token is skipped (t is wave-uniform).
template <bool kSwa>
__device__ __forceinline__ int64_t resolve_slot(const RacArgs& a, int64_t t) {
  return resolve_token_slot<kSwa>(a.slot_mapping, a.swa, a.swa_len, a.pool_slots, t);
}

__device__ __forceinline__ int64_t row_offset(const RacArgs& a, int64_t s) {
  int64_t blk, off;
  if (a.bs_shift >= 0) {
    blk = s >> a.bs_shift;
    off = s & (int64_t)(a.block_size - 1);
  } else {
    blk = s / a.block_size;
    off = s - blk * a.block_size;
  }
  return blk * a.block_stride + off * (int64_t)a.row_elems;
}

template <Ty S>
__device__ __forceinline__ void store_raw(void* p, const typename Load8<S>::Raw& r);
template <>
__device__ __forceinline__ void store_raw<Ty::BF16>(void* p, const u32x4& r) {
  __builtin_nontemporal_store(r, reinterpret_cast<u32x4*>(p));
}
template <>
__device__ __forceinline__ void store_raw<Ty::F32>(void* p, const F32x8& r) {
  u32x4* q = reinterpret_cast<u32x4*>(p);
  __builtin_nontemporal_store(r.a, q);
  __builtin_nontemporal_store(r.b, q + 1);
}

template <Ty S, Ty C, bool kScale>
__device__ __forceinline__ void encode_store(void* dst, const typename Load8<S>::Raw& r, float scale, double rcp) {
  if constexpr (S == C && !kScale) {
    store_raw<S>(dst, r);  // bit copy keeps -0 and NaN payloads
  } else {
    float f[8];
    Load8<S>::widen(r, f);
    if constexpr (kScale) div_by_scale<8>(f, scale, rcp);  // = IEEE fp32 f / scale, element-wise
    Store8<C>::store(dst, f);
  }
}

template <Ty S, Ty C, bool kScale, bool kSwa>
__global__ __launch_bounds__(256) void rac_vec_kernel(RacArgs a) {
  const int wave = uniform(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + wave;
  if (t >= a.num_tokens) return;
  const int64_t s = resolve_slot<kSwa>(a, t);
  if (s < 0) return;
  constexpr int SB = TyInfo<S>::kBytes, CB = TyInfo<C>::kBytes;
  const int64_t dst_row = row_offset(a, s);
  const int nvec = a.row_elems >> 3;
  const int v0 = (int)blockIdx.y * (64 * kU) + lane;
  const bool has_v = a.value != nullptr;
  float ks = 1.0f, vs = 1.0f;
  double rk = 1.0, rv = 1.0;
  if constexpr (kScale) {
    ks = *a.k_scale;
    rk = 1.0 / (double)ks;
    if (has_v) {
      vs = *a.v_scale;
      rv = 1.0 / (double)vs;
    }
  }
  using L = Load8<S>;
  const char* kp = static_cast<const char*>(a.key) + t * a.key_stride * SB;
  char* kc = static_cast<char*>(a.key_cache) + dst_row * CB;
  typename L::Raw kr[kU], vr[kU];
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    const int v = v0 + u * 64;
    if (v < nvec) kr[u] = L::load(kp + (int64_t)v * 8 * SB);
  }
  if (has_v) {
    const char* vp = static_cast<const char*>(a.value) + t * a.value_stride * SB;
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int v = v0 + u * 64;
      if (v < nvec) vr[u] = L::load(vp + (int64_t)v * 8 * SB);
    }
  }
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    const int v = v0 + u * 64;
    if (v < nvec) encode_store<S, C, kScale>(kc + (int64_t)v * 8 * CB, kr[u], ks, rk);
  }
  if (has_v) {
    char* vc = static_cast<char*>(a.value_cache) + dst_row * CB;
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int v = v0 + u * 64;
      if (v < nvec) encode_store<S, C, kScale>(vc + (int64_t)v * 8 * CB, vr[u], vs, rv);
    }
  }
}

// Element-at-a-time path for rows or pointers that do not allow 8-element
// vectors. Same mapping: one wave per token, lanes stride the row.
template <Ty S, Ty C, bool kScale, bool kSwa>
__global__ __launch_bounds__(256) void rac_scalar_kernel(RacArgs a) {
  const int wave = uniform(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + wave;
  if (t >= a.num_tokens) return;
  const int64_t s = resolve_slot<kSwa>(a, t);
  if (s < 0) return;
  const int64_t dst_row = row_offset(a, s);
  constexpr int SB = TyInfo<S>::kBytes;
  const bool has_v = a.value != nullptr;
  float ks = 1.0f, vs = 1.0f;
  if constexpr (kScale) {
    ks = *a.k_scale;
    if (has_v) vs = *a.v_scale;
  }
  for (int e = lane; e < a.row_elems; e += 64) {
    for (int which = 0; which < (has_v ? 2 : 1); ++which) {
      const void* src = which ? a.value : a.key;
      void* dst = which ? a.value_cache : a.key_cache;
      const int64_t si = t * (which ? a.value_stride : a.key_stride) + e;
      const int64_t di = dst_row + e;
      if constexpr (S == C && !kScale) {
        if constexpr (SB == 2)
          reinterpret_cast<uint16_t*>(dst)[di] = reinterpret_cast<const uint16_t*>(src)[si];
        else
          reinterpret_cast<uint32_t*>(dst)[di] = reinterpret_cast<const uint32_t*>(src)[si];
      } else {
        float f = load1<S>(src, si);
        if constexpr (kScale) f = f / (which ? vs : ks);
        store1<C>(dst, di, f);
      }
    }
  }
}

template <Ty S, Ty C, bool kScale, bool kSwa>
void launch(const RacArgs& a, bool vec, hipStream_t st) {
  const unsigned gx = (unsigned)((a.num_tokens + 3) / 4);
  if (vec) {
    const int nvec = a.row_elems / 8;
    const unsigned gy = (unsigned)((nvec + 64 * kU - 1) / (64 * kU));
    rac_vec_kernel<S, C, kScale, kSwa><<<dim3(gx, gy), 256, 0, st>>>(a);
  } else {
    rac_scalar_kernel<S, C, kScale, kSwa><<<dim3(gx, 1), 256, 0, st>>>(a);
  }
}

template <Ty S, Ty C>
void launch_flags(const RacArgs& a, bool vec, bool scale, bool swa, hipStream_t st) {
  if (scale) {
    if (swa) launch<S, C, true, true>(a, vec, st);
    else launch<S, C, true, false>(a, vec, st);
  } else {
    if (swa) launch<S, C, false, true>(a, vec, st);
    else launch<S, C, false, false>(a, vec, st);
  }
}

template <Ty S>
void launch_cache(pa_dtype cache, const RacArgs& a, bool vec, bool scale, bool swa, hipStream_t st) {
  switch (cache) {
    case PA_BF16: launch_flags<S, Ty::BF16>(a, vec, scale, swa, st); break;
    case PA_F32: launch_flags<S, Ty::F32>(a, vec, scale, swa, st); break;
    default: launch_flags<S, Ty::FP8>(a, vec, scale, swa, st); break;
  }
}

}  // namespace
}  // namespace pa

extern "C" pa_status pa_reshape_and_cache(const void* key, const void* value, pa_dtype src_dtype,
                                          int64_t num_tokens, int32_t num_heads, int32_t head_size,
                                          int64_t key_token_stride, int64_t value_token_stride,
                                          void* key_cache, void* value_cache, pa_dtype cache_dtype,
                                          int64_t num_blocks, int32_t block_size, int64_t block_stride,
                                          const int64_t* slot_mapping, const int64_t* swa_slot_mapping,
                                          int64_t swa_len, const float* k_scale, const float* v_scale,
                                          void* stream) {
  using namespace pa;
  clear_error();
  const char* fn = "pa_reshape_and_cache";
  if (num_tokens < 0) return fail(PA_EINVAL, "%s: num_tokens < 0", fn);
  if (src_dtype != PA_BF16 && src_dtype != PA_F32)
    return fail(PA_EDTYPE, "%s: source dtype %s not supported (bf16, f32)", fn, dtype_name(src_dtype));
  if (cache_dtype != PA_BF16 && cache_dtype != PA_F32 && cache_dtype != PA_FP8_E4M3FN)
    return fail(PA_EDTYPE, "%s: cache dtype %d not supported", fn, (int)cache_dtype);
  if (num_heads <= 0 || head_size <= 0) return fail(PA_EINVAL, "%s: num_heads and head_size must be > 0", fn);
  const int64_t row = (int64_t)num_heads * head_size;
  if (row > (1LL << 30)) return fail(PA_EINVAL, "%s: num_heads*head_size too large", fn);
  if (block_size <= 0) return fail(PA_EINVAL, "%s: block_size must be > 0", fn);
  if (num_blocks < 0) return fail(PA_EINVAL, "%s: num_blocks < 0", fn);
  if (block_stride < (int64_t)block_size * row) return fail(PA_EINVAL, "%s: block_stride < block_size*num_heads*head_size", fn);
  if (num_blocks > 0 && num_blocks > INT64_MAX / block_stride) return fail(PA_EINVAL, "%s: cache too large", fn);
  if ((value == nullptr) != (value_cache == nullptr)) return fail(PA_EINVAL, "%s: value and value_cache must both be given or both be NULL", fn);
  if (k_scale == nullptr && v_scale != nullptr) return fail(PA_EINVAL, "%s: v_scale given without k_scale", fn);
  if (k_scale != nullptr && value != nullptr && v_scale == nullptr) return fail(PA_EINVAL, "%s: k_scale given without v_scale", fn);
  if (swa_slot_mapping != nullptr && swa_len < 0) return fail(PA_EINVAL, "%s: swa_len < 0", fn);
  if (num_tokens == 0) return PA_OK;
  if (!key || !key_cache || !slot_mapping) return fail(PA_EINVAL, "%s: null key, key_cache or slot_mapping", fn);
  if (key_token_stride < row || (value && value_token_stride < row))
    return fail(PA_EINVAL, "%s: token stride smaller than num_heads*head_size", fn);
  if (num_tokens > (int64_t)INT32_MAX * 4) return fail(PA_EINVAL, "%s: num_tokens too large", fn);
  if (checks_on()) {
    const pa_status c = check_slots(fn, reinterpret_cast<hipStream_t>(stream), slot_mapping, num_tokens,
                                    swa_slot_mapping, swa_len, num_blocks, block_size);
    if (c != PA_OK) return c;
  }
  if (num_blocks == 0) return PA_OK;  // every slot lies outside an empty pool

  RacArgs a;
  a.key = key;
  a.value = value;
  a.key_cache = key_cache;
  a.value_cache = value_cache;
  a.slot_mapping = slot_mapping;
  a.swa = swa_slot_mapping;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.swa_len = swa_len;
  a.num_tokens = num_tokens;
  a.pool_slots = num_blocks * (int64_t)block_size;
  a.key_stride = key_token_stride;
  a.value_stride = value ? value_token_stride : 0;
  a.block_stride = block_stride;
  a.block_size = block_size;
  a.bs_shift = (block_size & (block_size - 1)) == 0 ? __builtin_ctz((unsigned)block_size) : -1;
  a.row_elems = (int32_t)row;

  const int sb = dtype_bytes(src_dtype), cb = dtype_bytes(cache_dtype);
  const int dst_align = cache_dtype == PA_FP8_E4M3FN ? 8 : 16;
  bool vec = (row % 8 == 0) && aligned(key, 16) && (key_token_stride * sb) % 16 == 0 &&
             aligned(key_cache, dst_align) && (block_stride * cb) % dst_align == 0;
  if (value) vec = vec && aligned(value, 16) && (value_token_stride * sb) % 16 == 0 && aligned(value_cache, dst_align);
  if (vec && (row / 8 + 64 * kU - 1) / (64 * kU) > 65535) vec = false;

  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const bool scale = k_scale != nullptr, swa = swa_slot_mapping != nullptr;
  if (src_dtype == PA_BF16) launch_cache<Ty::BF16>(cache_dtype, a, vec, scale, swa, st);
  else launch_cache<Ty::F32>(cache_dtype, a, vec, scale, swa, st);
  return after_launch(fn);
}
