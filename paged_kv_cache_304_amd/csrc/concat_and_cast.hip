// pa_concat_and_cast_mla_k: k[t, h, :] = cast(k_nope[t, h, :] ++ k_rope[t, 0, :]).
//
// Operation (concat_and_cast_mha_k in SGLang's cache_ops.py): for every token,
// each head's K row is its own no-RoPE part followed by the RoPE part that all
// heads of the token share; the value is converted to k's dtype at the store.
//
// gfx950 design: one 256-thread workgroup per token. Thread i owns the
// 8-element column vector j = i % V8 of the output row (V8 = (nope+rope)/8) and
// walks the heads h = i / V8, i / V8 + HP, ... (HP = 256 / V8 heads per pass).
// A thread whose column lies in the RoPE part loads its 8 RoPE elements once
// and stores them for every head it visits; a thread in the no-RoPE part
// streams 16 bytes of k_nope per head. Loads and stores are non-temporal.
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

struct CatArgs {
  void* k;
  const void* k_nope;
  const void* k_rope;
  int64_t k_s0, k_s1;        // elements
  int64_t n_s0, n_s1;        // elements
  int64_t r_s0;              // elements
  int64_t num_tokens;
  int32_t num_heads;
  int32_t nope_dim;
  int32_t rope_dim;
};

template <Ty S, Ty K>
__global__ __launch_bounds__(256) void concat_vec_kernel(CatArgs a) {
  const int64_t t = blockIdx.x;
  const int v8 = (a.nope_dim + a.rope_dim) >> 3;
  const int nope8 = a.nope_dim >> 3;
  const int hp = 256 / v8;  // heads per pass (host guarantees v8 <= 256)
  const int i = threadIdx.x;
  const int h0 = i / v8;
  if (h0 >= hp) return;  // the last 256 % v8 threads have no column
  const int j = i - h0 * v8;
  constexpr int SB = TyInfo<S>::kBytes, KB = TyInfo<K>::kBytes;
  using L = Load8<S>;
  char* kt = static_cast<char*>(a.k) + t * a.k_s0 * KB + (int64_t)j * 8 * KB;
  if (j >= nope8) {
    const char* rp = static_cast<const char*>(a.k_rope) + (t * a.r_s0 + (int64_t)(j - nope8) * 8) * SB;
    const typename L::Raw r = L::load(rp);
    float f[8];
    L::widen(r, f);
    for (int h = h0; h < a.num_heads; h += hp) {
      char* dst = kt + (int64_t)h * a.k_s1 * KB;
      if constexpr (S == K) {
        if constexpr (SB == 2) __builtin_nontemporal_store(r, reinterpret_cast<u32x4*>(dst));
        else Store8<K>::store(dst, f);
      } else {
        Store8<K>::store(dst, f);
      }
    }
  } else {
    const char* np = static_cast<const char*>(a.k_nope) + (t * a.n_s0 + (int64_t)j * 8) * SB;
#pragma unroll 4
    for (int h = h0; h < a.num_heads; h += hp) {
      const typename L::Raw r = L::load(np + (int64_t)h * a.n_s1 * SB);
      char* dst = kt + (int64_t)h * a.k_s1 * KB;
      if constexpr (S == K && SB == 2) {
        __builtin_nontemporal_store(r, reinterpret_cast<u32x4*>(dst));
      } else {
        float f[8];
        L::widen(r, f);
        Store8<K>::store(dst, f);
      }
    }
  }
}

// One element per thread-iteration; used when rows or pointers do not allow
// 8-element vectors.
template <Ty S, Ty K>
__global__ __launch_bounds__(256) void concat_scalar_kernel(CatArgs a) {
  const int64_t t = blockIdx.x;
  const int kd = a.nope_dim + a.rope_dim;
  const int total = a.num_heads * kd;
  for (int e = threadIdx.x; e < total; e += 256) {
    const int h = e / kd, d = e - h * kd;
    float f;
    int64_t si;
    const void* src;
    if (d < a.nope_dim) {
      src = a.k_nope;
      si = t * a.n_s0 + (int64_t)h * a.n_s1 + d;
    } else {
      src = a.k_rope;
      si = t * a.r_s0 + (d - a.nope_dim);
    }
    const int64_t di = t * a.k_s0 + (int64_t)h * a.k_s1 + d;
    if constexpr (S == K) {
      if constexpr (TyInfo<S>::kBytes == 2)
        reinterpret_cast<uint16_t*>(a.k)[di] = reinterpret_cast<const uint16_t*>(src)[si];
      else
        reinterpret_cast<uint32_t*>(a.k)[di] = reinterpret_cast<const uint32_t*>(src)[si];
    } else {
      f = load1<S>(src, si);
      store1<K>(a.k, di, f);
    }
  }
}

// ---------------------------------------------------------------------------
// Fused concat -> cast -> paged write of K (pa_concat_and_cache_mla_k): the
// token's [H, nope + rope] row is assembled and encoded straight into its
// cache slot, with no K intermediate in memory. It equals concat_and_cast
// into an fp32 K followed by the K-only cache write, because the widening to
// fp32 is exact: each element is widened, divided by the scale when one is
// given, and rounded once to the cache type.
// ---------------------------------------------------------------------------
struct CacheCatArgs {
  const void* k_nope;
  const void* k_rope;
  void* cache;
  const int64_t* slots;
  const int64_t* swa;
  const float* k_scale;
  int64_t n_s0, n_s1;        // elements
  int64_t r_s0;              // elements
  int64_t swa_len;
  int64_t pool_slots;
  int64_t block_stride;      // elements
  int32_t block_size;
  int32_t num_heads;
  int32_t nope_dim;
  int32_t rope_dim;
};

// 8 fp32 values encoded to the cache type, kept packed so that the RoPE part
// (shared by every head) is encoded once and stored many times.
template <Ty C> struct Pack8;
template <> struct Pack8<Ty::BF16> {
  using V = u32x4;
  __device__ static V pack(const float (&f)[8]) {
    V v;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = f32x2_to_bf16x2(f[2 * i], f[2 * i + 1]);
    return v;
  }
  __device__ static void store(void* p, const V& v) { __builtin_nontemporal_store(v, reinterpret_cast<V*>(p)); }
};
template <> struct Pack8<Ty::FP8> {
  using V = u32x2;
  __device__ static V pack(const float (&f)[8]) {
    return V{f32x4_to_fp8x4(f[0], f[1], f[2], f[3]), f32x4_to_fp8x4(f[4], f[5], f[6], f[7])};
  }
  __device__ static void store(void* p, const V& v) { __builtin_nontemporal_store(v, reinterpret_cast<V*>(p)); }
};
template <> struct Pack8<Ty::F32> {
  using V = F32x8;
  __device__ static V pack(const float (&f)[8]) {
    V v;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v.a[i] = __float_as_uint(f[i]);
      v.b[i] = __float_as_uint(f[4 + i]);
    }
    return v;
  }
  __device__ static void store(void* p, const V& v) {
    u32x4* q = reinterpret_cast<u32x4*>(p);
    __builtin_nontemporal_store(v.a, q);
    __builtin_nontemporal_store(v.b, q + 1);
  }
};

template <Ty S, Ty C, bool kScale>
__device__ __forceinline__ typename Pack8<C>::V encode8(const typename Load8<S>::Raw& r, float scale, double rcp) {
  float f[8];
  Load8<S>::widen(r, f);
  if constexpr (kScale) div_by_scale<8>(f, scale, rcp);  // = IEEE fp32 f / scale
  return Pack8<C>::pack(f);
}

// One 256-thread workgroup per token, the same column walk as concat_vec_kernel.
template <Ty S, Ty C, bool kScale, bool kSwa>
__global__ __launch_bounds__(256) void concat_cache_vec_kernel(CacheCatArgs a) {
  const int64_t t = blockIdx.x;
  const int64_t s = resolve_token_slot<kSwa>(a.slots, a.swa, a.swa_len, a.pool_slots, t);
  if (s < 0) return;  // uniform: the token is skipped
  const int kd = a.nope_dim + a.rope_dim;
  const int v8 = kd >> 3;
  const int nope8 = a.nope_dim >> 3;
  const int hp = 256 / v8;  // host guarantees v8 <= 256
  const int i = threadIdx.x;
  const int h0 = i / v8;
  if (h0 >= hp) return;
  const int j = i - h0 * v8;
  constexpr int SB = TyInfo<S>::kBytes, CBy = TyInfo<C>::kBytes;
  using L = Load8<S>;
  const int64_t blk = s / a.block_size, off = s - blk * a.block_size;
  char* row = static_cast<char*>(a.cache) + (blk * a.block_stride + off * (int64_t)a.num_heads * kd + (int64_t)j * 8) * CBy;
  float scale = 1.0f;
  double rcp = 1.0;
  if constexpr (kScale) {
    scale = *a.k_scale;
    rcp = 1.0 / (double)scale;
  }
  if (j >= nope8) {
    const char* rp = static_cast<const char*>(a.k_rope) + (t * a.r_s0 + (int64_t)(j - nope8) * 8) * SB;
    const typename Pack8<C>::V v = encode8<S, C, kScale>(L::load(rp), scale, rcp);
    for (int h = h0; h < a.num_heads; h += hp) Pack8<C>::store(row + (int64_t)h * kd * CBy, v);
  } else {
    const char* np = static_cast<const char*>(a.k_nope) + (t * a.n_s0 + (int64_t)j * 8) * SB;
#pragma unroll 4
    for (int h = h0; h < a.num_heads; h += hp) {
      const typename L::Raw r = L::load(np + (int64_t)h * a.n_s1 * SB);
      Pack8<C>::store(row + (int64_t)h * kd * CBy, encode8<S, C, kScale>(r, scale, rcp));
    }
  }
}

template <Ty S, Ty C>
void launch_cache_cat(const CacheCatArgs& a, unsigned tokens, bool scale, bool swa, hipStream_t st) {
  if (scale) {
    if (swa) concat_cache_vec_kernel<S, C, true, true><<<tokens, 256, 0, st>>>(a);
    else concat_cache_vec_kernel<S, C, true, false><<<tokens, 256, 0, st>>>(a);
  } else {
    if (swa) concat_cache_vec_kernel<S, C, false, true><<<tokens, 256, 0, st>>>(a);
    else concat_cache_vec_kernel<S, C, false, false><<<tokens, 256, 0, st>>>(a);
  }
}

template <Ty S>
void launch_cache_cat_c(pa_dtype c, const CacheCatArgs& a, unsigned tokens, bool scale, bool swa, hipStream_t st) {
  switch (c) {
    case PA_BF16: launch_cache_cat<S, Ty::BF16>(a, tokens, scale, swa, st); break;
    case PA_F32: launch_cache_cat<S, Ty::F32>(a, tokens, scale, swa, st); break;
    default: launch_cache_cat<S, Ty::FP8>(a, tokens, scale, swa, st); break;
  }
}

template <Ty S, Ty K>
void launch(const CatArgs& a, bool vec, hipStream_t st) {
  const unsigned grid = (unsigned)a.num_tokens;
  if (vec) concat_vec_kernel<S, K><<<grid, 256, 0, st>>>(a);
  else concat_scalar_kernel<S, K><<<grid, 256, 0, st>>>(a);
}

template <Ty S>
void launch_k(pa_dtype kd, const CatArgs& a, bool vec, hipStream_t st) {
  switch (kd) {
    case PA_BF16: launch<S, Ty::BF16>(a, vec, st); break;
    case PA_F32: launch<S, Ty::F32>(a, vec, st); break;
    default: launch<S, Ty::FP8>(a, vec, st); break;
  }
}

}  // namespace
}  // namespace pa

extern "C" pa_status pa_concat_and_cast_mla_k(void* k, pa_dtype k_dtype, int64_t k_stride0, int64_t k_stride1,
                                              const void* k_nope, pa_dtype nope_dtype, int64_t nope_stride0,
                                              int64_t nope_stride1, const void* k_rope, pa_dtype rope_dtype,
                                              int64_t rope_stride0, int64_t num_tokens, int32_t num_heads,
                                              int32_t nope_dim, int32_t rope_dim, void* stream) {
  using namespace pa;
  clear_error();
  const char* fn = "pa_concat_and_cast_mla_k";
  if (num_tokens < 0 || num_heads <= 0 || nope_dim < 0 || rope_dim < 0 || nope_dim + rope_dim <= 0)
    return fail(PA_EINVAL, "%s: invalid sizes (num_tokens=%lld num_heads=%d nope=%d rope=%d)", fn,
                (long long)num_tokens, num_heads, nope_dim, rope_dim);
  if (nope_dtype != PA_BF16 && nope_dtype != PA_F32)
    return fail(PA_EDTYPE, "%s: k_nope dtype %s not supported (bf16, f32)", fn, dtype_name(nope_dtype));
  if (rope_dtype != nope_dtype) return fail(PA_EDTYPE, "%s: k_rope dtype must equal k_nope dtype", fn);
  if (k_dtype != PA_BF16 && k_dtype != PA_F32 && k_dtype != PA_FP8_E4M3FN)
    return fail(PA_EDTYPE, "%s: k dtype %d not supported", fn, (int)k_dtype);
  const int64_t kd = (int64_t)nope_dim + rope_dim;
  if (k_stride1 < kd || k_stride0 < (int64_t)num_heads * k_stride1)
    return fail(PA_EINVAL, "%s: k strides (%lld, %lld) overlap rows of %lld elements", fn,
                (long long)k_stride0, (long long)k_stride1, (long long)kd);
  if (nope_stride1 < nope_dim || nope_stride0 < 0 || rope_stride0 < 0)
    return fail(PA_EINVAL, "%s: invalid source strides", fn);
  if (num_tokens == 0) return PA_OK;
  if (!k || !k_nope || (rope_dim > 0 && !k_rope)) return fail(PA_EINVAL, "%s: null pointer", fn);
  if (num_tokens > INT32_MAX) return fail(PA_EINVAL, "%s: num_tokens too large", fn);

  CatArgs a;
  a.k = k;
  a.k_nope = k_nope;
  a.k_rope = k_rope;
  a.k_s0 = k_stride0;
  a.k_s1 = k_stride1;
  a.n_s0 = nope_stride0;
  a.n_s1 = nope_stride1;
  a.r_s0 = rope_stride0;
  a.num_tokens = num_tokens;
  a.num_heads = num_heads;
  a.nope_dim = nope_dim;
  a.rope_dim = rope_dim;

  const int sb = dtype_bytes(nope_dtype), kb = dtype_bytes(k_dtype);
  const int k_align = k_dtype == PA_FP8_E4M3FN ? 8 : 16;
  const bool vec = nope_dim % 8 == 0 && rope_dim % 8 == 0 && kd / 8 <= 256 && aligned(k, k_align) &&
                   (k_stride0 * kb) % k_align == 0 && (k_stride1 * kb) % k_align == 0 && aligned(k_nope, 16) &&
                   (nope_stride0 * sb) % 16 == 0 && (nope_stride1 * sb) % 16 == 0 &&
                   (rope_dim == 0 || (aligned(k_rope, 16) && (rope_stride0 * sb) % 16 == 0));
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (nope_dtype == PA_BF16) launch_k<Ty::BF16>(k_dtype, a, vec, st);
  else launch_k<Ty::F32>(k_dtype, a, vec, st);
  return after_launch(fn);
}

extern "C" pa_status pa_concat_and_cache_mla_k(const void* k_nope, pa_dtype src_dtype, int64_t nope_stride0,
                                               int64_t nope_stride1, const void* k_rope, int64_t rope_stride0,
                                               int64_t num_tokens, int32_t num_heads, int32_t nope_dim,
                                               int32_t rope_dim, void* key_cache, pa_dtype cache_dtype,
                                               int64_t num_blocks, int32_t block_size, int64_t block_stride,
                                               const int64_t* slot_mapping, const int64_t* swa_slot_mapping,
                                               int64_t swa_len, const float* k_scale, void* stream) {
  using namespace pa;
  clear_error();
  const char* fn = "pa_concat_and_cache_mla_k";
  if (num_tokens < 0 || num_heads <= 0 || nope_dim < 0 || rope_dim < 0 || nope_dim + rope_dim <= 0)
    return fail(PA_EINVAL, "%s: invalid sizes (num_tokens=%lld num_heads=%d nope=%d rope=%d)", fn,
                (long long)num_tokens, num_heads, nope_dim, rope_dim);
  if (src_dtype != PA_BF16 && src_dtype != PA_F32)
    return fail(PA_EDTYPE, "%s: source dtype %s not supported (bf16, f32)", fn, dtype_name(src_dtype));
  if (cache_dtype != PA_BF16 && cache_dtype != PA_F32 && cache_dtype != PA_FP8_E4M3FN)
    return fail(PA_EDTYPE, "%s: cache dtype %d not supported", fn, (int)cache_dtype);
  const int64_t kd = (int64_t)nope_dim + rope_dim;
  const int64_t row = kd * num_heads;
  if (nope_dim % 8 != 0 || rope_dim % 8 != 0 || kd / 8 > 256)
    return fail(PA_EUNSUPPORTED, "%s: nope_dim and rope_dim must be multiples of 8 with (nope+rope)/8 <= 256", fn);
  if (block_size <= 0 || num_blocks < 0) return fail(PA_EINVAL, "%s: invalid pool sizes", fn);
  if (block_stride < (int64_t)block_size * row) return fail(PA_EINVAL, "%s: block_stride < block_size*num_heads*(nope+rope)", fn);
  if (num_blocks > 0 && num_blocks > INT64_MAX / block_stride) return fail(PA_EINVAL, "%s: cache too large", fn);
  if (nope_stride1 < nope_dim || nope_stride0 < 0 || rope_stride0 < 0) return fail(PA_EINVAL, "%s: invalid source strides", fn);
  if (swa_slot_mapping != nullptr && swa_len < 0) return fail(PA_EINVAL, "%s: swa_len < 0", fn);
  if (num_tokens == 0 || num_blocks == 0) return PA_OK;
  if (!k_nope || (rope_dim > 0 && !k_rope) || !key_cache || !slot_mapping) return fail(PA_EINVAL, "%s: null pointer", fn);
  if (num_tokens > INT32_MAX) return fail(PA_EINVAL, "%s: num_tokens too large", fn);
  const int sb = dtype_bytes(src_dtype), cbytes = dtype_bytes(cache_dtype);
  const int c_align = cache_dtype == PA_FP8_E4M3FN ? 8 : 16;
  if (!aligned(key_cache, c_align) || (block_stride * cbytes) % c_align != 0 || !aligned(k_nope, 16) ||
      (nope_stride0 * sb) % 16 != 0 || (nope_stride1 * sb) % 16 != 0 ||
      (rope_dim > 0 && (!aligned(k_rope, 16) || (rope_stride0 * sb) % 16 != 0)))
    return fail(PA_EINVAL, "%s: sources must be 16-byte aligned per row, the cache %d-byte aligned per block", fn, c_align);
  if (checks_on()) {
    const pa_status c = check_slots(fn, reinterpret_cast<hipStream_t>(stream), slot_mapping, num_tokens,
                                    swa_slot_mapping, swa_len, num_blocks, block_size);
    if (c != PA_OK) return c;
  }

  CacheCatArgs a;
  a.k_nope = k_nope;
  a.k_rope = k_rope;
  a.cache = key_cache;
  a.slots = slot_mapping;
  a.swa = swa_slot_mapping;
  a.k_scale = k_scale;
  a.n_s0 = nope_stride0;
  a.n_s1 = nope_stride1;
  a.r_s0 = rope_stride0;
  a.swa_len = swa_len;
  a.pool_slots = num_blocks * (int64_t)block_size;
  a.block_stride = block_stride;
  a.block_size = block_size;
  a.num_heads = num_heads;
  a.nope_dim = nope_dim;
  a.rope_dim = rope_dim;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const bool scale = k_scale != nullptr, swa = swa_slot_mapping != nullptr;
  if (src_dtype == PA_BF16) launch_cache_cat_c<Ty::BF16>(cache_dtype, a, (unsigned)num_tokens, scale, swa, st);
  else launch_cache_cat_c<Ty::F32>(cache_dtype, a, (unsigned)num_tokens, scale, swa, st);
  return after_launch(fn);
}
