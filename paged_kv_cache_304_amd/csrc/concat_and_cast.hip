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
