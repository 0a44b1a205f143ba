// Device-side helpers shared by the gfx950 kernels of the paged KV cache
// library: element conversions, 8-element vector loads/stores and wave-level
// reductions. Everything here is CDNA4-specific (wave64, DPP row operations).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

enum class Ty : int { BF16 = 0, F32 = 2, FP8 = 3 };

template <Ty T> struct TyInfo;
template <> struct TyInfo<Ty::BF16> { using Storage = uint16_t; static constexpr int kBytes = 2; };
template <> struct TyInfo<Ty::F32> { using Storage = float; static constexpr int kBytes = 4; };
template <> struct TyInfo<Ty::FP8> { using Storage = uint8_t; static constexpr int kBytes = 1; };

// ------------------------------------------------------------------ decoding

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Two OCP e4m3fn codes (bytes 0,1 or 2,3 of w) -> two fp32 values. gfx950's
// conversion instruction decodes the OCP format exactly (every code is a
// float32 value).
__device__ __forceinline__ f32x2 fp8x2_lo(uint32_t w) { return __builtin_amdgcn_cvt_pk_f32_fp8(w, false); }
__device__ __forceinline__ f32x2 fp8x2_hi(uint32_t w) { return __builtin_amdgcn_cvt_pk_f32_fp8(w, true); }

// ------------------------------------------------------------------ encoding

// fp32 -> bf16, round to nearest even; overflow gives inf; a NaN keeps its
// sign and top payload bits and gets the quiet bit. gfx950's v_cvt_pk_bf16_f32
// does exactly this (checked against the integer definition on all 2^32 inputs).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}
__device__ __forceinline__ uint32_t f32_to_bf16(float f) { return f32x2_to_bf16x2(f, 0.0f) & 0xFFFFu; }

// fp32 -> OCP e4m3fn, round to nearest even; |y| > 464 (past the midpoint
// above 448) and infinities give 0x7F with the sign of y -- gfx950's
// v_cvt_pk_fp8_f32 does both; it encodes every NaN as 0xFF, so a NaN is first
// replaced by 480 with the NaN's sign (checked on all 2^32 inputs).
__device__ __forceinline__ float fp8_nan_fix(float y) {
  return (y != y) ? __uint_as_float((__float_as_uint(y) & 0x80000000u) | 0x43F00000u) : y;
}
// four values -> four e4m3fn codes, value i in byte i
__device__ __forceinline__ uint32_t f32x4_to_fp8x4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(fp8_nan_fix(a), fp8_nan_fix(b), 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(fp8_nan_fix(c), fp8_nan_fix(d), w, true);
  return (uint32_t)w;
}
__device__ __forceinline__ uint32_t f32_to_fp8(float y) { return f32x4_to_fp8x4(y, 0.0f, 0.0f, 0.0f) & 0xFFu; }

// x / s for a per-tensor scale, as an IEEE fp32 division: x * RN64(1/s) in
// fp64 rounded once to fp32 equals the correctly rounded quotient whenever that
// quotient is a normal number (a bf16 or fp32 x over an fp32 s is never an fp32
// rounding midpoint and lies at least ~2^-49 (relative) away from one, while the
// fp64 product is within 2^-52); subnormal quotients take the real division.
__device__ __forceinline__ bool needs_exact_division(float q) {
  const float aq = fabsf(q);
  return aq != 0.0f && aq <= 1.17549435e-38f;
}
template <int N>
__device__ __forceinline__ void div_by_scale(float (&f)[N], float s, double rcp) {
  float q[N];
  bool any = false;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    q[i] = (float)((double)f[i] * rcp);
    any |= needs_exact_division(q[i]);
  }
  if (__builtin_expect(any, 0)) {
#pragma unroll
    for (int i = 0; i < N; ++i)
      if (needs_exact_division(q[i])) q[i] = f[i] / s;
  }
#pragma unroll
  for (int i = 0; i < N; ++i) f[i] = q[i];
}

// 8 source elements widened to fp32.
template <Ty S> struct Load8;
template <> struct Load8<Ty::BF16> {
  using Raw = u32x4;
  __device__ __forceinline__ static Raw load(const void* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  }
  __device__ __forceinline__ static void widen(const Raw& r, float (&f)[8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = bf16_lo(r[i]);
      f[2 * i + 1] = bf16_hi(r[i]);
    }
  }
};
struct F32x8 { u32x4 a, b; };
template <> struct Load8<Ty::F32> {
  using Raw = F32x8;
  __device__ __forceinline__ static Raw load(const void* p) {
    const u32x4* q = reinterpret_cast<const u32x4*>(p);
    return Raw{__builtin_nontemporal_load(q), __builtin_nontemporal_load(q + 1)};
  }
  __device__ __forceinline__ static void widen(const Raw& r, float (&f)[8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[i] = __uint_as_float(r.a[i]);
      f[4 + i] = __uint_as_float(r.b[i]);
    }
  }
};

// 8 fp32 values rounded to the destination type and stored.
template <Ty D> struct Store8;
template <> struct Store8<Ty::BF16> {
  __device__ __forceinline__ static void store(void* p, const float (&f)[8]) {
    u32x4 v;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = f32x2_to_bf16x2(f[2 * i], f[2 * i + 1]);
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
  }
};
template <> struct Store8<Ty::F32> {
  __device__ __forceinline__ static void store(void* p, const float (&f)[8]) {
    u32x4 a, b;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      a[i] = __float_as_uint(f[i]);
      b[i] = __float_as_uint(f[4 + i]);
    }
    u32x4* q = reinterpret_cast<u32x4*>(p);
    __builtin_nontemporal_store(a, q);
    __builtin_nontemporal_store(b, q + 1);
  }
};
template <> struct Store8<Ty::FP8> {
  __device__ __forceinline__ static void store(void* p, const float (&f)[8]) {
    u32x2 v;
#pragma unroll
    for (int i = 0; i < 2; ++i) v[i] = f32x4_to_fp8x4(f[4 * i], f[4 * i + 1], f[4 * i + 2], f[4 * i + 3]);
    __builtin_nontemporal_store(v, reinterpret_cast<u32x2*>(p));
  }
};

// Single elements (unaligned fallback paths).
template <Ty S> __device__ __forceinline__ float load1(const void* p, int64_t i);
template <> __device__ __forceinline__ float load1<Ty::BF16>(const void* p, int64_t i) {
  return __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(p)[i] << 16);
}
template <> __device__ __forceinline__ float load1<Ty::F32>(const void* p, int64_t i) {
  return reinterpret_cast<const float*>(p)[i];
}
template <Ty D> __device__ __forceinline__ void store1(void* p, int64_t i, float f);
template <> __device__ __forceinline__ void store1<Ty::BF16>(void* p, int64_t i, float f) {
  reinterpret_cast<uint16_t*>(p)[i] = (uint16_t)f32_to_bf16(f);
}
template <> __device__ __forceinline__ void store1<Ty::F32>(void* p, int64_t i, float f) {
  reinterpret_cast<float*>(p)[i] = f;
}
template <> __device__ __forceinline__ void store1<Ty::FP8>(void* p, int64_t i, float f) {
  reinterpret_cast<uint8_t*>(p)[i] = (uint8_t)f32_to_fp8(f);
}

// ------------------------------------------------------- wave-level shuffles

// DPP row operations act inside rows of 16 lanes.
enum : int {
  kDppQuadXor1 = 0xB1,       // quad_perm [1,0,3,2]
  kDppQuadXor2 = 0x4E,       // quad_perm [2,3,0,1]
  kDppRowHalfMirror = 0x141, // lane i <-> 7-i within each half row
  kDppRowMirror = 0x140,     // lane i <-> 15-i within each row
};

template <int Ctrl>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), Ctrl, 0xF, 0xF, false));
}

// Sum over aligned groups of N lanes (N = 2, 4, 8, 16, 32 or 64); every lane of
// a group receives the group's sum.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(N == 1 || N == 2 || N == 4 || N == 8 || N == 16 || N == 32 || N == 64, "group");
  if constexpr (N >= 2) x += dpp<kDppQuadXor1>(x);
  if constexpr (N >= 4) x += dpp<kDppQuadXor2>(x);
  if constexpr (N >= 8) x += dpp<kDppRowHalfMirror>(x);
  if constexpr (N >= 16) x += dpp<kDppRowMirror>(x);
  if constexpr (N >= 32) x += __shfl_xor(x, 16, 64);
  if constexpr (N >= 64) x += __shfl_xor(x, 32, 64);
  return x;
}

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// ------------------------------------------------------- slot resolution

// Final cache slot of token t, or -1 when the token is skipped: a negative
// first-stage slot (tested before the optional second-stage table is read), a
// first-stage slot past that table, a negative second-stage slot, or a slot
// outside the pool's num_blocks * block_size slots. With a wave-uniform t every
// load is a scalar load.
template <bool kSwa>
__device__ __forceinline__ int64_t resolve_token_slot(const int64_t* slot_mapping, const int64_t* swa,
                                                      int64_t swa_len, int64_t pool_slots, int64_t t) {
  int64_t s = slot_mapping[t];
  if (s < 0) return -1;
  if constexpr (kSwa) {
    if (s >= swa_len) return -1;
    s = swa[s];
    if (s < 0) return -1;
  }
  return s < pool_slots ? s : -1;
}

// ------------------------------------------------------- LDS-DMA

// One wave-wide LDS-DMA load: 16 bytes per lane from global memory into LDS at
// lds_base + 16 * lane (global_load_lds_dwordx4, M0 = LDS base, saved and
// restored around it). Written as inline asm so that the compiler does not
// track these LDS writes: it would otherwise put a full vector-memory wait
// (every load in flight) before LDS reads it cannot prove disjoint from them.
// A kernel using it orders every load with its own vmcnt waits and barriers.
// The instruction has no register result; its address registers are read at
// issue.
__device__ __forceinline__ void dma_16B(const void* gptr, uint32_t lds_base) {
  uint32_t saved;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off\n\ts_mov_b32 m0, %0"
               : "=&s"(saved)
               : "v"(gptr), "s"(lds_base)
               : "memory");
}
// The same with 4 bytes per lane (global_load_lds_dword): LDS lds_base + 4 * lane.
__device__ __forceinline__ void dma_4B(const void* gptr, uint32_t lds_base) {
  uint32_t saved;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %1, off\n\ts_mov_b32 m0, %0"
               : "=&s"(saved)
               : "v"(gptr), "s"(lds_base)
               : "memory");
}
// Wait until at most N of this wave's vector-memory operations are in flight
// (they complete in issue order).
template <int N>
__device__ __forceinline__ void wait_vmem() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

}  // namespace pa
