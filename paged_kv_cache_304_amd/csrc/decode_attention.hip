// pa_decode_attention: one query token per sequence against its paged K/V.
//
// Operation (section 2.6 "Attention" of the Qwen3-0.6B engine walkthrough page:
// decode attention reads K/V back along physical blocks through block_tables;
// the PagedAttention principle page: GQA with H_Q an integer multiple of H_KV,
// blocks of [block_size, H_KV, d_h] ordered only by a table): for sequence b
// and q head h, softmax over the first ctx_b cached positions of
// scale * q . K^ (K^ = K * k_scale), weights applied to V^ = V * v_scale.
//
// gfx950 design: split-K over logical positions, then a merge launch.
//  * A workgroup serves one group of KV heads with one wavefront per head, so
//    its waves read every head of the same physical blocks together.
//  * Matrix-core path (block_size a multiple of 16, D <= 128): a persistent
//    kernel. Exactly as many workgroups as the chip holds at once are
//    launched (the hardware hands workgroups to the XCDs round-robin and
//    stalls every XCD when the next one's XCD is full, so a grid of uneven
//    split workgroups leaves compute units idle); each scans the context
//    lengths and takes equal ranges of the flattened (sequence, 16-position
//    tile) list. A tile is 16 positions of one head: QK^T is one
//    v_mfma_f32_16x16x32_bf16 per 32 head dims with the K tile as A (row =
//    position) and the G query heads of the group as B columns, so lane l
//    receives the scores of positions 4*(l/16)+r (r<4) for head l%16. Softmax
//    runs there; P.V runs on the vector ALUs with V in a row layout (16 lanes
//    per cache row, 4 rows per load) in which lane l needs exactly the
//    probabilities of row group l/16, handed over by DPP row_newbcast. K tiles
//    and q rows are fetched straight into LDS (K in whole-row 1 KB wave loads,
//    re-laid out by an XOR swizzle for the MFMA operand reads); fp8 K is
//    widened to bf16 exactly for the MFMA.
//  * Vector path (other block sizes, D = 256): one workgroup per (head group,
//    split, sequence); 8 elements per lane, a cache row spread over D/8
//    lanes, QK dots reduced with DPP row operations, one online-softmax state
//    per row of lanes, merged with lane shuffles at the end.
//  * A sequence that needs one split (chunk) writes its output directly.
//    Otherwise each piece stores (max, sum, normalised output) per q head in
//    the workspace and a second, small launch merges them (lanes over pieces
//    for the weights, lanes over dims for the outputs).
//  * Piece boundaries depend only on the context lengths, so the result is
//    bit-identical under any relabelling of physical blocks.
// Scores are kept in the log2 domain (scale * log2(e) folded in) so that each
// exponential is one v_exp_f32.
#include <math.h>

#include <atomic>
#include <mutex>
#include <type_traits>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

#ifndef PA_DECODE_TARGET_WGS
#define PA_DECODE_TARGET_WGS 8192
#endif
#ifndef PA_DECODE_MIN_SPLIT
#define PA_DECODE_MIN_SPLIT 64
#endif
#ifndef PA_DECODE_MAX_SPLIT
#define PA_DECODE_MAX_SPLIT 128
#endif
#ifndef PA_DECODE_K_DMA
#define PA_DECODE_K_DMA 1
#endif
#ifndef PA_DECODE_NT_V
#define PA_DECODE_NT_V 1
#endif
#ifndef PA_DECODE_MAX_WAVES
#define PA_DECODE_MAX_WAVES 2
#endif
#ifndef PA_DECODE_PRIO
#define PA_DECODE_PRIO 1
#endif
#ifndef PA_DECODE_FP8_WAVES
#define PA_DECODE_FP8_WAVES 4
#endif
constexpr int kMaxWaves = PA_DECODE_MAX_WAVES;        // KV heads (waves) per workgroup
constexpr int kTargetWgs = PA_DECODE_TARGET_WGS;      // split workgroups aimed for if every sequence used all W blocks
constexpr int kMinSplitTokens = PA_DECODE_MIN_SPLIT;  // positions per split, lower bound
constexpr int kMaxSplitTokens = PA_DECODE_MAX_SPLIT;  // positions per split, upper bound

struct DecArgs {
  void* out;
  const void* q;
  const void* kc;
  const void* vc;
  const int32_t* bt;
  const int32_t* ctx_lens;
  const float* k_scale;
  const float* v_scale;
  float* ws_m;
  float* ws_l;
  float* ws_o;
  int32_t* ws_n;           // persistent kernel: chunks per sequence (null for the grid kernel)
  int64_t out_seq_stride;  // elements
  int64_t q_seq_stride;    // elements
  int64_t block_stride;    // elements
  int64_t num_blocks;
  int32_t block_size;
  int32_t W;               // max_blocks_per_seq
  int32_t num_seqs;
  int32_t HQ;
  int32_t HKV;
  int32_t split_blocks;
  int32_t max_splits;
  int32_t waves_per_wg;
  int32_t kv_groups;
  int32_t slots;           // persistent kernel: workgroups per KV-head group
  int32_t out_f32;
  float scale_log2;        // softmax_scale * log2(e)
  // decode step (persistent kernel): the new tokens, bf16 [B, H_KV, D] rows,
  // folded into the attention instead of being read back from the cache
  const uint16_t* new_k;   // null: plain attention
  const uint16_t* new_v;
  const int64_t* new_slots;
  int64_t new_k_stride, new_v_stride;
};

// Persistent kernel: flag in a sequence's chunk count (workspace) that the
// decode step's new token is its last position and is left to the merge pass.
constexpr int kFoldBit = 1 << 30;

__device__ __forceinline__ int clamp_ctx(const DecArgs& a, int b) {
  int ctx = a.ctx_lens[b];
  const int cap = a.W * a.block_size;
  return ctx < 0 ? 0 : (ctx > cap ? cap : ctx);
}

// Decode step: position ctx-1 of sequence b is the new token when the token's
// slot is that position's slot (the normal case). The attention then covers
// positions 0 .. ctx-2 from the cache and takes the last one from the new row
// as the cache write encodes it; otherwise every position comes from the cache.
__device__ __forceinline__ bool new_token_is_last(const DecArgs& a, int b, int ctx) {
  if (ctx < 1) return false;
  const int64_t pool = a.num_blocks * (int64_t)a.block_size;
  const int64_t s = resolve_token_slot<false>(a.new_slots, nullptr, 0, pool, b);
  if (s < 0) return false;
  const int p = ctx - 1;
  const int e = a.bt[(int64_t)b * a.W + p / a.block_size];
  return e >= 0 && (int64_t)e < a.num_blocks && s == (int64_t)e * a.block_size + p % a.block_size;
}

// ------------------------------------------------------------ small helpers

template <int NW> struct Dw { uint32_t w[NW]; };

// Eight elements of a new token's row as the cache write stores them (a bit
// copy for a bf16 cache without scales, else fp32 / scale rounded once to the
// cache type) and as the attention reads them back: the code and the raw
// decoded values (scales are applied by the attention, as for cached rows).
template <Ty C> struct NewCode;
template <> struct NewCode<Ty::BF16> { using T = u32x4; };
template <> struct NewCode<Ty::FP8> { using T = u32x2; };

template <Ty C>
__device__ __forceinline__ void new_token_chunk(const u32x4& raw, bool scaled, float s, double rcp,
                                                typename NewCode<C>::T& code, float (&val)[8]) {
  float f[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = bf16_lo(raw[i]);
    f[2 * i + 1] = bf16_hi(raw[i]);
  }
  if constexpr (C == Ty::BF16) {
    if (!scaled) {
      code = raw;
#pragma unroll
      for (int i = 0; i < 8; ++i) val[i] = f[i];
      return;
    }
    div_by_scale<8>(f, s, rcp);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      code[i] = f32x2_to_bf16x2(f[2 * i], f[2 * i + 1]);
      val[2 * i] = bf16_lo(code[i]);
      val[2 * i + 1] = bf16_hi(code[i]);
    }
  } else {
    if (scaled) div_by_scale<8>(f, s, rcp);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      code[i] = f32x4_to_fp8x4(f[4 * i], f[4 * i + 1], f[4 * i + 2], f[4 * i + 3]);
      const f32x2 lo = fp8x2_lo(code[i]), hi = fp8x2_hi(code[i]);
      val[4 * i] = lo[0];
      val[4 * i + 1] = lo[1];
      val[4 * i + 2] = hi[0];
      val[4 * i + 3] = hi[1];
    }
  }
}

// One element of a new token's row as the attention reads it back from the
// cache (the raw decoded value; see new_token_chunk).
template <Ty C>
__device__ __forceinline__ float new_token_value(float x, bool scaled, float s, double rcp) {
  if (C == Ty::BF16 && !scaled) return x;
  float f[1] = {x};
  if (scaled) div_by_scale<1>(f, s, rcp);
  if constexpr (C == Ty::BF16)
    return bf16_lo(f32_to_bf16(f[0]));
  else
    return fp8x2_lo(f32_to_fp8(f[0]))[0];
}

// Writes chunk `e0 .. e0+7` of head g of the new token of sequence b into its
// cache slot s (K and V).
template <Ty C>
__device__ __forceinline__ void write_new_chunk(const DecArgs& a, int b, int g, int D, int e0, int64_t s,
                                                const u32x4& kraw, const u32x4& vraw, bool scaled, float ks,
                                                double rk, float vs, double rv) {
  (void)b;
  constexpr int CB = TyInfo<C>::kBytes;
  const int64_t blk = s / a.block_size, off = s - blk * a.block_size;
  const int64_t at = (blk * a.block_stride + off * (int64_t)a.HKV * D + (int64_t)g * D + e0) * CB;
  typename NewCode<C>::T code;
  float val[8];
  new_token_chunk<C>(kraw, scaled, ks, rk, code, val);
  *reinterpret_cast<typename NewCode<C>::T*>(static_cast<char*>(const_cast<void*>(a.kc)) + at) = code;
  new_token_chunk<C>(vraw, scaled, vs, rv, code, val);
  *reinterpret_cast<typename NewCode<C>::T*>(static_cast<char*>(const_cast<void*>(a.vc)) + at) = code;
}

// NW dwords; non-temporal when NT (data read once per call, full lines per
// instruction), cached otherwise (a line read in parts by successive loads).
template <int NW, bool NT>
__device__ __forceinline__ Dw<NW> load_dw(const char* p) {
  Dw<NW> r;
  if constexpr (NW == 1) {
    const uint32_t* q = reinterpret_cast<const uint32_t*>(p);
    r.w[0] = NT ? __builtin_nontemporal_load(q) : *q;
  } else if constexpr (NW == 2) {
    const u32x2* q = reinterpret_cast<const u32x2*>(p);
    const u32x2 v = NT ? __builtin_nontemporal_load(q) : *q;
    r.w[0] = v[0];
    r.w[1] = v[1];
  } else {
#pragma unroll
    for (int i = 0; i < NW / 4; ++i) {
      const u32x4* q = reinterpret_cast<const u32x4*>(p) + i;
      const u32x4 v = NT ? __builtin_nontemporal_load(q) : *q;
#pragma unroll
      for (int k = 0; k < 4; ++k) r.w[4 * i + k] = v[k];
    }
  }
  return r;
}

template <int NW>
__device__ __forceinline__ void store_dw(void* p, const uint32_t (&w)[NW]) {
  if constexpr (NW == 1) {
    *reinterpret_cast<uint32_t*>(p) = w[0];
  } else if constexpr (NW == 2) {
    *reinterpret_cast<u32x2*>(p) = u32x2{w[0], w[1]};
  } else {
#pragma unroll
    for (int i = 0; i < NW / 4; ++i)
      reinterpret_cast<u32x4*>(p)[i] = u32x4{w[4 * i], w[4 * i + 1], w[4 * i + 2], w[4 * i + 3]};
  }
}

// N cache elements (packed in dwords) -> fp32.
template <Ty C, int NW, int N>
__device__ __forceinline__ void widen_dw(const Dw<NW>& d, float (&f)[N]) {
  if constexpr (C == Ty::BF16) {
    static_assert(N == 2 * NW, "bf16 count");
#pragma unroll
    for (int i = 0; i < NW; ++i) {
      f[2 * i] = bf16_lo(d.w[i]);
      f[2 * i + 1] = bf16_hi(d.w[i]);
    }
  } else {
    static_assert(N == 4 * NW, "fp8 count");
#pragma unroll
    for (int i = 0; i < NW; ++i) {
      const f32x2 lo = fp8x2_lo(d.w[i]), hi = fp8x2_hi(d.w[i]);
      f[4 * i] = lo[0];
      f[4 * i + 1] = lo[1];
      f[4 * i + 2] = hi[0];
      f[4 * i + 3] = hi[1];
    }
  }
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) x = fmaxf(x, __shfl_xor(x, m, 64));
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) x += __shfl_xor(x, m, 64);
  return x;
}

// N output values of head h at dims d0.. : out (bf16 or fp32).
template <int D, int N>
__device__ __forceinline__ void store_out(const DecArgs& a, int b, int h, int d0, const float (&o)[N]) {
  if (a.out_f32) {
    uint32_t w[N];
#pragma unroll
    for (int k = 0; k < N; ++k) w[k] = __float_as_uint(o[k]);
    store_dw<N>(static_cast<float*>(a.out) + (int64_t)b * a.out_seq_stride + (int64_t)h * D + d0, w);
  } else {
    uint32_t w[N / 2];
#pragma unroll
    for (int k = 0; k < N / 2; ++k) w[k] = f32_to_bf16(o[2 * k]) | (f32_to_bf16(o[2 * k + 1]) << 16);
    store_dw<N / 2>(static_cast<uint16_t*>(a.out) + (int64_t)b * a.out_seq_stride + (int64_t)h * D + d0, w);
  }
}

// Normalised result of one split for head h, dims d0..d0+N: straight to the
// output when the sequence has one split, otherwise to the workspace.
template <int D, int N>
__device__ __forceinline__ void store_split(const DecArgs& a, int b, int h, int split, int nsplit, int d0,
                                            const float (&o)[N], bool write_ml, float m, float l) {
  if (nsplit == 1) {
    store_out<D, N>(a, b, h, d0, o);
    return;
  }
  const int64_t slot = ((int64_t)b * a.HQ + h) * a.max_splits + split;
  if (write_ml) {
    a.ws_m[slot] = m;
    a.ws_l[slot] = l;
  }
  uint32_t w[N];
#pragma unroll
  for (int k = 0; k < N; ++k) w[k] = __float_as_uint(o[k]);
  store_dw<N>(a.ws_o + slot * D + d0, w);
}

// Merge pass: one wave per (sequence, q head), four waves per workgroup. Lane
// s holds piece s's (max, sum); the wave reduces the global max and the
// weights, then sums the pieces' outputs (lane i holds dims i + 64k) with the
// weights broadcast by readlane. The context length, the piece count, the
// first 64 (max, sum) pairs and the first kFirst outputs are all loaded
// together before the count is known (entries past the count are never used),
// so the common case costs one memory round trip. Sequences that fit one
// piece were written by the split pass; after the persistent kernel this pass
// also writes the zeros of empty sequences. (A merge inside the split kernel
// would need an agent-scope release/acquire per workgroup, i.e. an L2
// write-back on its XCD for every piece; the kernel boundary gives that
// ordering for free.)
template <Ty C, int D>
__global__ __launch_bounds__(256) void decode_merge_kernel(DecArgs a) {
  constexpr int PER = D / 64;
  constexpr int kFirst = 4;   // outputs loaded before the piece count is known
  constexpr int kBatch = 16;  // outputs per later round of loads
  const int wid = (int)blockIdx.x * 4 + uniform(threadIdx.x >> 6);
  if (wid >= a.num_seqs * a.HQ) return;
  const int b = wid / a.HQ, h = wid - b * a.HQ;
  const int lane = threadIdx.x & 63;
  const int64_t base = ((int64_t)b * a.HQ + h) * a.max_splits;

  const int ctx_raw = a.ctx_lens[b];
  const int n_raw = a.ws_n ? a.ws_n[b] : 0;
  // Decode step: the new token's elements of this head (q, k, v) and, for the
  // row write, this lane's 8-element chunk are loaded up front, alongside the
  // chunks, whether or not they are needed.
  const bool step = a.new_k != nullptr;
  const int G = a.HQ / a.HKV, g = h / G;
  float q_t[PER], k_t[PER], v_t[PER];
  u32x4 kw8 = {0u, 0u, 0u, 0u}, vw8 = {0u, 0u, 0u, 0u};
  int64_t slot_raw = -1;
  if (step) {
    const uint16_t* nk = a.new_k + (int64_t)b * a.new_k_stride + (int64_t)g * D;
    const uint16_t* nv = a.new_v + (int64_t)b * a.new_v_stride + (int64_t)g * D;
    const uint16_t* qh = static_cast<const uint16_t*>(a.q) + (int64_t)b * a.q_seq_stride + (int64_t)h * D;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      q_t[i] = load1<Ty::BF16>(qh, lane + 64 * i);
      k_t[i] = load1<Ty::BF16>(nk, lane + 64 * i);
      v_t[i] = load1<Ty::BF16>(nv, lane + 64 * i);
    }
    if (lane < D / 8) {
      kw8 = *reinterpret_cast<const u32x4*>(nk + 8 * lane);
      vw8 = *reinterpret_cast<const u32x4*>(nv + 8 * lane);
    }
    slot_raw = a.new_slots[b];
  }
  const int cap0 = min(64, a.max_splits);
  const float m0 = lane < cap0 ? a.ws_m[base + lane] : -INFINITY;
  const float l0 = lane < cap0 ? a.ws_l[base + lane] : 0.0f;
  const int nb0 = min(kFirst, a.max_splits);
  float v0[kFirst][PER];
#pragma unroll
  for (int u = 0; u < kFirst; ++u) {
    const float* wo = a.ws_o + (base + min(u, nb0 - 1)) * D;
#pragma unroll
    for (int i = 0; i < PER; ++i) v0[u][i] = wo[lane + 64 * i];
  }

  const int cap = a.W * a.block_size;
  const int ctx = ctx_raw < 0 ? 0 : (ctx_raw > cap ? cap : ctx_raw);
  // Decode step: the persistent kernel left every chunk here, without the
  // new token when it is the last position; it joins the softmax below as
  // one more position, its row as the cache write encodes it.
  const int64_t pool = a.num_blocks * (int64_t)a.block_size;
  const int64_t slot_new = slot_raw >= 0 && slot_raw < pool ? slot_raw : -1;
  const bool fold = step && ctx >= 1 && (n_raw & kFoldBit) != 0;  // decided by the persistent kernel
  int n;
  if (a.ws_n) {
    n = ctx == 0 ? 0 : (n_raw & (kFoldBit - 1));  // written by the persistent kernel (not for empty sequences)
  } else {
    const int nblk = (ctx + a.block_size - 1) / a.block_size;
    n = (nblk + a.split_blocks - 1) / a.split_blocks;
    if (n <= 1) return;  // written by the split pass (zeros included)
  }
  if (n == 1 && !step) return;

  const bool scaled = a.k_scale != nullptr;
  const float ks = scaled ? *a.k_scale : 1.0f, vs = scaled ? *a.v_scale : 1.0f;
  const double rk = scaled ? 1.0 / (double)ks : 1.0, rv = scaled ? 1.0 / (double)vs : 1.0;
  float s_new = -INFINITY;  // the new token's score (log2 domain) and value
  float v_new[PER];
  if (fold) {
    float dot = 0.0f;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      dot = fmaf(q_t[i], new_token_value<C>(k_t[i], scaled, ks, rk), dot);
      v_new[i] = new_token_value<C>(v_t[i], scaled, vs, rv) * vs;
    }
    s_new = wave_sum(dot) * (a.scale_log2 * ks);
  }

  float o[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) o[i] = 0.0f;
  float M = lane < n ? m0 : -INFINITY;
  for (int s = 64 + lane; s < n; s += 64) M = fmaxf(M, a.ws_m[base + s]);
  M = fmaxf(wave_max(M), s_new);
  if (M != -INFINITY) {
    float den = 0.0f;
    for (int c = 0; c < n; c += 64) {
      const int sl = c + lane;
      float w = 0.0f;
      if (sl < n) w = __builtin_amdgcn_exp2f((c == 0 ? m0 : a.ws_m[base + sl]) - M) * (c == 0 ? l0 : a.ws_l[base + sl]);
      den += w;
      const int cnt = min(64, n - c);
      int s_begin = 0;
      if (c == 0) {
#pragma unroll
        for (int u = 0; u < kFirst; ++u) {
          if (u < cnt) {
            const float ws = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), u));
#pragma unroll
            for (int i = 0; i < PER; ++i) o[i] = fmaf(ws, v0[u][i], o[i]);
          }
        }
        s_begin = kFirst;
      }
      for (int s0 = s_begin; s0 < cnt; s0 += kBatch) {
        float v[kBatch][PER];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          const float* wo = a.ws_o + (base + c + min(s0 + u, cnt - 1)) * D;
#pragma unroll
          for (int i = 0; i < PER; ++i) v[u][i] = wo[lane + 64 * i];
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          if (s0 + u < cnt) {
            const float ws = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), s0 + u));
#pragma unroll
            for (int i = 0; i < PER; ++i) o[i] = fmaf(ws, v[u][i], o[i]);
          }
        }
      }
    }
    float dsum = wave_sum(den);
    if (fold) {
      const float wt = __builtin_amdgcn_exp2f(s_new - M);
      dsum += wt;
#pragma unroll
      for (int i = 0; i < PER; ++i) o[i] = fmaf(wt, v_new[i], o[i]);
    }
    const float inv = 1.0f / dsum;
#pragma unroll
    for (int i = 0; i < PER; ++i) o[i] *= inv;
  }
  // n == 0 (empty sequence) or no attended position: zeros. A decode step
  // writes the new token's row into its slot here, one wave per KV head,
  // after every read of this launch's attention.
  if (step && h % G == 0 && slot_new >= 0 && lane < D / 8)
    write_new_chunk<C>(a, b, g, D, 8 * lane, slot_new, kw8, vw8, scaled, ks, rk, vs, rv);
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int64_t at = (int64_t)b * a.out_seq_stride + (int64_t)h * D + lane + 64 * i;
    if (a.out_f32)
      static_cast<float*>(a.out)[at] = o[i];
    else
      static_cast<uint16_t*>(a.out)[at] = (uint16_t)f32_to_bf16(o[i]);
  }
}

// ---------------------------------------------------------------------------
// Vector-ALU split kernel (any block size that is a multiple of 64 / (D/8)).
// ---------------------------------------------------------------------------
template <Ty C> struct KvRow;
template <> struct KvRow<Ty::BF16> { static constexpr int kW = 4; };
template <> struct KvRow<Ty::FP8> { static constexpr int kW = 2; };

template <Ty C, int D, int G>
__global__ __launch_bounds__(512) void decode_split_valu_kernel(DecArgs a) {
  constexpr int LPR = D / 8;     // lanes per cache row
  constexpr int RPL = 64 / LPR;  // cache rows per wave-load
  constexpr int CB = TyInfo<C>::kBytes;
  constexpr int KW = KvRow<C>::kW;
  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  const int g = (int)blockIdx.x * a.waves_per_wg + wave;
  const bool active = g < a.HKV;
  const int split = blockIdx.y;
  const int b = blockIdx.z;
  const int ctx = clamp_ctx(a, b);
  const int nblk = (ctx + a.block_size - 1) / a.block_size;
  // an empty sequence still gets one (empty) split, which writes zeros
  const int nsplit = max(1, (nblk + a.split_blocks - 1) / a.split_blocks);
  if (split >= nsplit) return;  // uniform over the workgroup
  const int j0 = split * a.split_blocks;
  const int j1 = min(nblk, j0 + a.split_blocks);
  const int r = lane / LPR, c = lane % LPR;

  if (active) {
    float q[G][8];
    {
      const uint16_t* qp = static_cast<const uint16_t*>(a.q) + (int64_t)b * a.q_seq_stride + (int64_t)g * G * D + 8 * c;
#pragma unroll
      for (int gi = 0; gi < G; ++gi) {
        const u32x4 w = *reinterpret_cast<const u32x4*>(qp + gi * D);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          q[gi][2 * i] = bf16_lo(w[i]);
          q[gi][2 * i + 1] = bf16_hi(w[i]);
        }
      }
    }
    const float ks = a.k_scale ? *a.k_scale : 1.0f;
    const float vs = a.v_scale ? *a.v_scale : 1.0f;
    const float sl2 = a.scale_log2 * ks;

    float m[G], l[G], acc[G][8];
#pragma unroll
    for (int gi = 0; gi < G; ++gi) {
      m[gi] = -INFINITY;
      l[gi] = 0.0f;
#pragma unroll
      for (int k = 0; k < 8; ++k) acc[gi][k] = 0.0f;
    }

    const int64_t row_bytes = (int64_t)a.HKV * D * CB;  // between consecutive offsets of a block
    const int steps = a.block_size / RPL;
    const int32_t* bt = a.bt + (int64_t)b * a.W;
    for (int j = j0; j < j1; ++j) {
      const int phys = bt[j];
      if (phys < 0 || (int64_t)phys >= a.num_blocks) continue;  // outside the pool: not attended
      const int valid = min(a.block_size, ctx - j * a.block_size);
      const int64_t base = ((int64_t)phys * a.block_stride + (int64_t)g * D + 8 * c) * CB;
      const char* kb = static_cast<const char*>(a.kc) + base;
      const char* vb = static_cast<const char*>(a.vc) + base;
      for (int st0 = 0; st0 < steps; st0 += 4) {
        Dw<KW> kr[4], vr[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          if (st0 + u < steps) {
            const int64_t off = (int64_t)((st0 + u) * RPL + r) * row_bytes;
            kr[u] = load_dw<KW, true>(kb + off);
            vr[u] = load_dw<KW, true>(vb + off);
          }
        }
        float s[G][4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const bool live = (st0 + u < steps) && ((st0 + u) * RPL + r < valid);
          if (st0 + u < steps) {
            float kf[8];
            widen_dw<C>(kr[u], kf);
#pragma unroll
            for (int gi = 0; gi < G; ++gi) {
              float part = 0.0f;
#pragma unroll
              for (int k = 0; k < 8; ++k) part = fmaf(q[gi][k], kf[k], part);
              const float dot = group_sum<LPR>(part);
              s[gi][u] = live ? dot * sl2 : -INFINITY;
            }
          } else {
#pragma unroll
            for (int gi = 0; gi < G; ++gi) s[gi][u] = -INFINITY;
          }
        }
        float p[G][4];
#pragma unroll
        for (int gi = 0; gi < G; ++gi) {
          const float mx = fmaxf(fmaxf(s[gi][0], s[gi][1]), fmaxf(s[gi][2], s[gi][3]));
          const float mn = fmaxf(m[gi], mx);
          const float mu = (mn == -INFINITY) ? 0.0f : mn;
          const float alpha = __builtin_amdgcn_exp2f(m[gi] - mu);
          float ps = 0.0f;
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            p[gi][u] = __builtin_amdgcn_exp2f(s[gi][u] - mu);
            ps += p[gi][u];
          }
          l[gi] = l[gi] * alpha + ps;
          m[gi] = mn;
#pragma unroll
          for (int k = 0; k < 8; ++k) acc[gi][k] *= alpha;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          if (st0 + u < steps) {
            float vf[8];
            widen_dw<C>(vr[u], vf);
            if ((st0 + u) * RPL + r >= valid) {
#pragma unroll
              for (int k = 0; k < 8; ++k) vf[k] = 0.0f;  // unwritten slots may hold NaN
            }
#pragma unroll
            for (int gi = 0; gi < G; ++gi)
#pragma unroll
              for (int k = 0; k < 8; ++k) acc[gi][k] = fmaf(p[gi][u], vf[k], acc[gi][k]);
          }
        }
      }
    }

    // Merge the RPL row states (rows are LPR lanes apart).
#pragma unroll
    for (int msk = LPR; msk < 64; msk <<= 1) {
#pragma unroll
      for (int gi = 0; gi < G; ++gi) {
        const float mo = __shfl_xor(m[gi], msk, 64);
        const float lo = __shfl_xor(l[gi], msk, 64);
        const float mn = fmaxf(m[gi], mo);
        const float mu = (mn == -INFINITY) ? 0.0f : mn;
        const float a1 = __builtin_amdgcn_exp2f(m[gi] - mu), a2 = __builtin_amdgcn_exp2f(mo - mu);
        l[gi] = l[gi] * a1 + lo * a2;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const float ao = __shfl_xor(acc[gi][k], msk, 64);
          acc[gi][k] = acc[gi][k] * a1 + ao * a2;
        }
        m[gi] = mn;
      }
    }
    if (r == 0) {
#pragma unroll
      for (int gi = 0; gi < G; ++gi) {
        const float inv = l[gi] > 0.0f ? vs / l[gi] : 0.0f;
        float o[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) o[k] = acc[gi][k] * inv;
        store_split<D, 8>(a, b, g * G + gi, split, nsplit, 8 * c, o, c == 0, m[gi], l[gi]);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Matrix-core split kernel (block_size a multiple of 16).
// ---------------------------------------------------------------------------
typedef __bf16 bf16x8 __attribute__((__vector_size__(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// 8 cache elements -> MFMA bf16 operand (fp8 values are exact in bf16).
template <Ty C> __device__ __forceinline__ bf16x8 as_bf16x8(const Dw<8 * TyInfo<C>::kBytes / 4>& d);
template <> __device__ __forceinline__ bf16x8 as_bf16x8<Ty::BF16>(const Dw<4>& d) {
  const u32x4 v = {d.w[0], d.w[1], d.w[2], d.w[3]};
  return __builtin_bit_cast(bf16x8, v);
}
template <> __device__ __forceinline__ bf16x8 as_bf16x8<Ty::FP8>(const Dw<2>& d) {
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const f32x2 lo = fp8x2_lo(d.w[i]), hi = fp8x2_hi(d.w[i]);
    r[4 * i] = (__bf16)lo[0];
    r[4 * i + 1] = (__bf16)lo[1];
    r[4 * i + 2] = (__bf16)hi[0];
    r[4 * i + 3] = (__bf16)hi[1];
  }
  return r;
}

// Value of lane J of this lane's 16-lane row (DPP row_newbcast).
template <int J>
__device__ __forceinline__ float row_bcast(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x150 + J, 0xF, 0xF, false));
}

template <int J, int G, int EPL>
__device__ __forceinline__ void rescale_heads(float (&acc)[G][EPL], float alpha) {
  const float aj = row_bcast<J>(alpha);
#pragma unroll
  for (int k = 0; k < EPL; ++k) acc[J][k] *= aj;
  if constexpr (J + 1 < G) rescale_heads<J + 1, G, EPL>(acc, alpha);
}

template <int J, int G, int EPL>
__device__ __forceinline__ void accumulate_row(float (&acc)[G][EPL], float p, const float (&v)[EPL]) {
  const float pj = row_bcast<J>(p);
#pragma unroll
  for (int k = 0; k < EPL; ++k) acc[J][k] = fmaf(pj, v[k], acc[J][k]);
  if constexpr (J + 1 < G) accumulate_row<J + 1, G, EPL>(acc, p, v);
}

template <int J, int G>
__device__ __forceinline__ void bcast_heads(float x, float (&out)[G]) {
  out[J] = row_bcast<J>(x);
  if constexpr (J + 1 < G) bcast_heads<J + 1, G>(x, out);
}

// One tile = 16 cache positions of one KV head. K is read in row layout (each
// 1 KB wave load covers whole rows, the access pattern that streams at full
// HBM rate) and re-laid out through a per-wave LDS tile into the MFMA operand
// layout; V stays in registers in the row layout the P.V step uses.
template <Ty C, int D>
struct Tile {
  static constexpr int CB = TyInfo<C>::kBytes;
  static constexpr int RB = D * CB;        // bytes of one head's cache row
  static constexpr int KB = 16 * RB;       // bytes of a K tile
  static constexpr int NI = KB / 1024;     // 1 KB wave loads per K tile
  static constexpr int NC = RB / 16;       // 16-byte chunks per row (LDS swizzle period)
  static constexpr int KS = D / 32;        // MFMA steps over the head dim
  static constexpr int EPL = D / 16;       // V dims per lane
  static constexpr int VW = EPL * CB / 4;  // dwords per V chunk
  static_assert(KB % 1024 == 0, "K tile must be whole 1 KB wave loads");
#if !PA_DECODE_K_DMA
  u32x4 k[NI];   // load i, lane l: tile bytes [1024 i + 16 l, +16)
#endif
  Dw<VW> v[4];   // row 4 (l/16) + i of the tile, dims EPL*(l%16) ..
};

template <Ty C, int D>
__device__ __forceinline__ void load_tile(Tile<C, D>& t, const char* kc, const char* vc, int64_t blk_el,
                                          int off, int64_t row_el, int lane, char* lds) {
  using T = Tile<C, D>;
  constexpr int CB = T::CB;
  const char* kb = kc + (blk_el + (int64_t)off * row_el) * CB;
#pragma unroll
  for (int i = 0; i < T::NI; ++i) {
    const int byte = 1024 * i + 16 * lane;
    const int row = byte / T::RB;
#if PA_DECODE_K_DMA
    // straight into this wave's LDS tile: lane l fills LDS slot 1024 i + 16 l,
    // so it fetches the chunk that the swizzle places there
    const int pos = (byte % T::RB) / 16;
    const int col = (pos ^ (row & (T::NC - 1))) * 16;
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(kb + (int64_t)row * row_el * CB + col),
                                     (__attribute__((address_space(3))) void*)(lds + 1024 * i), 16, 0, 0);
#else
    const int col = byte % T::RB;
    t.k[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kb + (int64_t)row * row_el * CB + col));
#endif
  }
  const int li = lane & 15, lg = lane >> 4;
  const char* vp = vc + (blk_el + (int64_t)(off + 4 * lg) * row_el + T::EPL * li) * CB;
#pragma unroll
  for (int i = 0; i < 4; ++i) t.v[i] = load_dw<T::VW, PA_DECODE_NT_V>(vp + (int64_t)i * row_el * CB);
}

// K tile -> this wave's LDS tile, row-major with the 16-byte chunks of row r
// XOR-swizzled by r, so that the 16 rows read at one column land in distinct banks.
template <Ty C, int D>
__device__ __forceinline__ void stage_k(const Tile<C, D>& t, char* lds, int lane) {
#if PA_DECODE_K_DMA
  // the loads wrote LDS directly; the compiler does not track that, so wait
  // for every outstanding vector memory operation before the tile is read
  (void)t;
  (void)lane;
  (void)lds;
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#else
  using T = Tile<C, D>;
#pragma unroll
  for (int i = 0; i < T::NI; ++i) {
    const int byte = 1024 * i + 16 * lane;
    const int row = byte / T::RB, c16 = (byte % T::RB) / 16;
    *reinterpret_cast<u32x4*>(lds + row * T::RB + ((c16 ^ (row & (T::NC - 1))) * 16)) = t.k[i];
  }
#endif
}

// MFMA A operand of step s: dims [32 s + 8 lg, +8) of tile row li.
template <Ty C, int D>
__device__ __forceinline__ bf16x8 k_operand(const char* lds, int s, int li, int lg) {
  using T = Tile<C, D>;
  const int byte = (32 * s + 8 * lg) * T::CB;
  const char* p = lds + li * T::RB + (((byte / 16) ^ (li & (T::NC - 1))) * 16) + (byte % 16);
  if constexpr (C == Ty::BF16) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
  } else {
    const u32x2 w = *reinterpret_cast<const u32x2*>(p);
    Dw<2> d;
    d.w[0] = w[0];
    d.w[1] = w[1];
    return as_bf16x8<C>(d);
  }
}

// Persistent matrix-core kernel. The work of one KV-head group is the list of
// (sequence, 16-position tile) pairs in sequence order, T tiles in all. Each of
// the `slots` workgroups of a group takes ranges of RT consecutive tiles (RT <= 64,
// ranges r = slot, slot + slots, ...), so every workgroup streams the same
// number of tiles and no workgroup is launched without work. A range cuts the
// sequences it touches into segments; the c-th range touching a sequence
// yields its chunk c, stored in the workspace for the merge pass, or written
// straight to the output when the sequence has a single chunk. Chunk
// boundaries depend only on the context lengths (never on physical block ids
// or on the processing order), so results are reproducible.
constexpr int kRangeMaxTiles = 64;  // a segment's blocks then fit one 64-lane table window
constexpr int kRangeMinTiles = 8;   // bounds the chunks per sequence (workspace size)
constexpr int kSegMax = kRangeMaxTiles;  // each segment holds >= 1 tile of the range

__device__ __forceinline__ int tiles_of(int ctx) { return (ctx + 15) >> 4; }

// KV heads (waves) per workgroup of the persistent kernel. An fp8 wave reads
// 128-byte pieces of each 1 KB cache row (eight heads of 128 dims); with four
// heads per workgroup a workgroup reads half of every row, which the memory
// system serves faster than four workgroups each reading a quarter
// (153.6 vs 161.2 us on the batch-256 fp8 workload), while bf16 rows are
// fastest in two-wave workgroups (96.4 vs 98.2 us at batch 64).
template <Ty C> constexpr int persistent_max_waves() { return C == Ty::FP8 ? PA_DECODE_FP8_WAVES : PA_DECODE_MAX_WAVES; }
constexpr int kWavesCap = 8;
static_assert(PA_DECODE_FP8_WAVES >= 1 && PA_DECODE_FP8_WAVES <= kWavesCap && PA_DECODE_MAX_WAVES <= kWavesCap,
              "waves per workgroup");

// Waves per SIMD the persistent kernel is compiled for (its register budget):
// the natural allocation of each shape, except that MFMA accumulator registers
// must not push the D = 128, G <= 2 shapes past 128 registers.
constexpr int persistent_waves_per_eu(int D, int G) {
  return D == 64 ? (G <= 2 ? 5 : (G == 4 ? 4 : 3)) : (G <= 2 ? 4 : (G == 4 ? 3 : 2));
}

template <Ty C, int D, int G, bool kFused>
__global__ __launch_bounds__(64 * persistent_max_waves<C>())
__attribute__((amdgpu_waves_per_eu(persistent_waves_per_eu(D, G), 8)))
void decode_persistent_kernel(DecArgs a) {
  using T = Tile<C, D>;
  constexpr int KS = T::KS;
  constexpr int EPL = T::EPL;
  constexpr int QB = G * D * 2;           // bytes of the group's q rows
  constexpr int QI = (QB + 1023) / 1024;  // 1 KB wave loads per q buffer
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int li = lane & 15, lg = lane >> 4;
  const int wave = uniform(tid >> 6);
  const int nthr = 64 * a.waves_per_wg;
  const int gr = (int)blockIdx.x % a.kv_groups;
  const int slot = (int)blockIdx.x / a.kv_groups;
  const int g = gr * a.waves_per_wg + wave;
  const bool active = g < a.HKV;

  constexpr int kW = persistent_max_waves<C>();
  __shared__ __attribute__((aligned(16))) char k_lds[kW * T::KB];
  __shared__ __attribute__((aligned(16))) char q_lds[kW * 2 * QB];
  __shared__ int seg_b[kSegMax], seg_t0[kSegMax], seg_t1[kSegMax], seg_ctx[kSegMax], seg_k[kSegMax], seg_n[kSegMax];
  __shared__ int seg_x[kSegMax];  // decode step: the new token is this sequence's last position
  __shared__ int64_t wave_tiles[kW];
  __shared__ int seg_count;

  // Tile counts of all sequences and their prefix sums: thread i owns a
  // contiguous run of sequences; a wave scan plus the per-wave totals give the
  // first tile index of each run.
  const int per = (a.num_seqs + nthr - 1) / nthr;
  const int b_lo = min(a.num_seqs, tid * per), b_hi = min(a.num_seqs, b_lo + per);
  int64_t mine = 0;
  for (int b = b_lo; b < b_hi; ++b) mine += tiles_of(clamp_ctx(a, b));
  int64_t incl = mine;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int64_t y = __shfl_up(incl, (unsigned)o, 64);
    if (lane >= o) incl += y;
  }
  if (lane == 63) wave_tiles[wave] = incl;
  __syncthreads();
  int64_t total = 0, before = 0;
  for (int w = 0; w < a.waves_per_wg; ++w) {
    const int64_t v = wave_tiles[w];
    total += v;
    if (w < wave) before += v;
  }
  const int64_t run_first = before + incl - mine;
  if (total == 0) return;  // uniform: every sequence is empty (the merge pass writes zeros)
  const int64_t per_round = (int64_t)kRangeMaxTiles * a.slots;
  const int64_t rounds = (total + per_round - 1) / per_round;
  int64_t RT = (total + rounds * a.slots - 1) / (rounds * a.slots);  // tiles per range
  if (RT < kRangeMinTiles) RT = kRangeMinTiles;
  const int64_t R = (total + RT - 1) / RT;

  const float ks = a.k_scale ? *a.k_scale : 1.0f;
  const float vs = a.v_scale ? *a.v_scale : 1.0f;
  const float sl2 = a.scale_log2 * ks;
  const int64_t row_el = (int64_t)a.HKV * D;  // elements between consecutive slots of a block
  const char* kc = static_cast<const char*>(a.kc);
  const char* vc = static_cast<const char*>(a.vc);
  char* my_lds = k_lds + wave * T::KB;

#if PA_DECODE_PRIO
  // Issue priority from the share of this workgroup's tiles still to do. The
  // sequencer favours older waves, so without this the workgroups placed last
  // on a compute unit fall behind and finish alone, with too few loads in
  // flight to keep HBM busy; a wave that is behind now wins the arbitration.
  int64_t my_tiles = 0;
  for (int64_t r = slot; r < R; r += a.slots) my_tiles += min(total, (r + 1) * RT) - r * RT;
  int64_t tiles_left = my_tiles;
  auto set_priority = [&]() {
    const int p = (int)((4 * tiles_left) / (my_tiles + 1));
    switch (p) {
      case 0: __builtin_amdgcn_s_setprio(0); break;
      case 1: __builtin_amdgcn_s_setprio(1); break;
      case 2: __builtin_amdgcn_s_setprio(2); break;
      default: __builtin_amdgcn_s_setprio(3); break;
    }
  };
#endif

  for (int64_t r = slot; r < R; r += a.slots) {
    // Segment list of range r: [U0, U1) intersected with each sequence.
    const int64_t U0 = r * RT, U1 = min(total, U0 + RT);
    if (tid == 0) seg_count = 0;
    __syncthreads();
    if (run_first < U1 && run_first + mine > U0) {
      int64_t S = run_first;
      for (int b = b_lo; b < b_hi && S < U1; ++b) {
        const int ctx = clamp_ctx(a, b);
        const int nt = tiles_of(ctx);
        if (nt > 0 && S + nt > U0) {
          const int i = atomicAdd(&seg_count, 1);
          const int64_t lo = max(U0, S), hi = min(U1, S + nt);
          seg_b[i] = b;
          seg_t0[i] = (int)(lo - S);
          seg_t1[i] = (int)(hi - S);
          // the positions this segment attends end at ctx -- or at ctx - 1 in
          // a decode step whose new token is the last position: the merge
          // pass takes that one in from the new row (its cache slot is written
          // after this launch)
          int sc = ctx;
          if constexpr (kFused) {
            if (hi == S + nt && new_token_is_last(a, b, ctx)) sc = ctx - 1;
          }
          seg_ctx[i] = sc;
          seg_x[i] = sc < ctx ? 1 : 0;
          seg_k[i] = (int)(lo / RT - S / RT);
          seg_n[i] = (int)((S + nt - 1) / RT - S / RT + 1);
        }
        S += nt;
      }
    }
    __syncthreads();
    const int nseg = seg_count;

    if (active) {
      // q rows of segment i into q buffer `buf` (straight to LDS), and this
      // lane's block-table entry of the segment's 64-block window.
      auto issue = [&](int i, int buf) -> int {
        const int b = seg_b[i];
        const int wb0 = (16 * seg_t0[i]) / a.block_size;
        const char* qs = static_cast<const char*>(a.q) + ((int64_t)b * a.q_seq_stride + (int64_t)g * G * D) * 2;
        char* qd = q_lds + (wave * 2 + buf) * QB;
#pragma unroll
        for (int j = 0; j < QI; ++j) {
          const int byte = 1024 * j + 16 * lane;
          if (byte < QB)
            __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(qs + byte),
                                             (__attribute__((address_space(3))) void*)(qd + 1024 * j), 16, 0, 0);
        }
        return (wb0 + lane < a.W) ? a.bt[(int64_t)b * a.W + wb0 + lane] : -1;
      };

      int bt_cur = nseg > 0 ? issue(0, 0) : -1;
      for (int i = 0; i < nseg; ++i) {
        const int bt_nxt = (i + 1 < nseg) ? issue(i + 1, (i + 1) & 1) : -1;
        const int b = seg_b[i], t0 = seg_t0[i], t1 = seg_t1[i];
        const int chunk = seg_k[i], nch = seg_n[i];
        const int p_end = min(seg_ctx[i], 16 * t1);
        const int wb0 = (16 * t0) / a.block_size;
        // B operand rows: lane column li holds head li of the group (lanes
        // past G repeat a head; their columns are never read).
        const char* qrow = q_lds + (wave * 2 + (i & 1)) * QB + ((li & (G - 1)) * D + 8 * lg) * 2;

        float m_run = -INFINITY, l_run = 0.0f;
        float acc[G][EPL];
#pragma unroll
        for (int j = 0; j < G; ++j)
#pragma unroll
          for (int k = 0; k < EPL; ++k) acc[j][k] = 0.0f;

        auto fetch = [&](T& tile, int t) -> bool {
          const int phys = __builtin_amdgcn_readlane(bt_cur, (16 * t) / a.block_size - wb0);
          const bool ok = phys >= 0 && (int64_t)phys < a.num_blocks;
          load_tile<C, D>(tile, kc, vc, (int64_t)(ok ? phys : 0) * a.block_stride + (int64_t)g * D,
                          (16 * t) % a.block_size, row_el, lane, my_lds);
          return ok;
        };
        // kMask: the tile reaches past the context end (only a sequence's last one can).
        auto compute = [&](const T& tile, int t, auto mask_tag) {
          constexpr bool kMask = decltype(mask_tag)::value;
          stage_k<C, D>(tile, my_lds, lane);
          f32x4 sc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
          for (int s = 0; s < KS; ++s) {
            const bf16x8 qb = *reinterpret_cast<const bf16x8*>(qrow + 64 * s);
            sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k_operand<C, D>(my_lds, s, li, lg), qb, sc, 0, 0, 0);
          }
          const int prow = 16 * t + 4 * lg;  // position of this lane's first score / V row
          float sr[4];
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            sr[r4] = sc[r4] * sl2;
            if constexpr (kMask) sr[r4] = (prow + r4 < p_end) ? sr[r4] : -INFINITY;
          }
          float mx = fmaxf(fmaxf(sr[0], sr[1]), fmaxf(sr[2], sr[3]));
          mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
          mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
          const float mn = fmaxf(m_run, mx);
          const float mu = (mn == -INFINITY) ? 0.0f : mn;
          const float alpha = __builtin_amdgcn_exp2f(m_run - mu);
          float pr[4];
          float ps = 0.0f;
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            pr[r4] = __builtin_amdgcn_exp2f(sr[r4] - mu);
            ps += pr[r4];
          }
          l_run = l_run * alpha + ps;
          m_run = mn;
          rescale_heads<0, G, EPL>(acc, alpha);
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            float vf[EPL];
            widen_dw<C>(tile.v[v], vf);
            if constexpr (kMask) {
              if (prow + v >= p_end) {
#pragma unroll
                for (int k = 0; k < EPL; ++k) vf[k] = 0.0f;  // unwritten slots may hold NaN
              }
            }
            accumulate_row<0, G, EPL>(acc, pr[v], vf);
          }
        };

        for (int t = t0; t < t1; ++t) {
#if PA_DECODE_PRIO
          set_priority();
          --tiles_left;
#endif
          T tile;
          const bool ok = fetch(tile, t);
          if (ok) {
            if (16 * t + 16 <= p_end)
              compute(tile, t, std::false_type{});
            else
              compute(tile, t, std::true_type{});
          }
        }

        // Sum the four row groups (same running max everywhere: no rescaling).
#pragma unroll
        for (int msk = 16; msk < 64; msk <<= 1) {
          l_run += __shfl_xor(l_run, msk, 64);
#pragma unroll
          for (int j = 0; j < G; ++j)
#pragma unroll
            for (int k = 0; k < EPL; ++k) acc[j][k] += __shfl_xor(acc[j][k], msk, 64);
        }
        float lj[G];
        bcast_heads<0, G>(l_run, lj);
        if (lg == 0) {
#pragma unroll
          for (int j = 0; j < G; ++j) {
            const float inv = lj[j] > 0.0f ? vs / lj[j] : 0.0f;
            float o[EPL];
#pragma unroll
            for (int k = 0; k < EPL; ++k) o[k] = acc[j][k] * inv;
            // a decode step always leaves its chunks to the merge pass (it adds the new token)
            store_split<D, EPL>(a, b, g * G + j, chunk, kFused && nch == 1 ? 2 : nch, EPL * li, o, li == j, m_run,
                                lj[j]);
          }
        }
        // the chunk count, and (decode step) whether the merge pass takes in
        // the new token, written once per sequence by its last chunk's group 0
        if (chunk == nch - 1 && g == 0 && lane == 0) a.ws_n[b] = nch | (kFused && seg_x[i] ? kFoldBit : 0);
        bt_cur = bt_nxt;
      }
    }
    __syncthreads();  // the segment list is rebuilt for the next range
  }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
struct Plan {
  bool persistent;  // matrix-core persistent kernel (block_size % 16 == 0, D <= 128)
  int waves_per_wg, kv_groups, split_blocks, max_splits;
  size_t off_n, off_m, off_l, off_o, bytes;
};

inline size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

Plan make_plan(int num_seqs, int HQ, int HKV, int D, int W, int bs) {
  Plan p;
  p.persistent = bs % 16 == 0 && D <= 128;
  p.waves_per_wg = HKV < kMaxWaves ? HKV : kMaxWaves;
  p.kv_groups = (HKV + p.waves_per_wg - 1) / p.waves_per_wg;
  if (p.persistent) {
    // a sequence of n tiles meets at most ceil(n / kRangeMinTiles) + 1 ranges
    const int64_t nt_max = ((int64_t)W * bs + 15) / 16;
    p.split_blocks = 0;
    p.max_splits = (int)((nt_max + kRangeMinTiles - 1) / kRangeMinTiles + 1);
  } else {
    // Aim for kTargetWgs workgroups if every sequence used all W blocks, with
    // splits of kMinSplitTokens..kMaxSplitTokens positions.
    const int64_t per_seq = ((int64_t)kTargetWgs + (int64_t)num_seqs * p.kv_groups - 1) / ((int64_t)num_seqs * p.kv_groups);
    int sb = (int)((W + per_seq - 1) / per_seq);
    const int lo = (kMinSplitTokens + bs - 1) / bs;
    int hi = kMaxSplitTokens / bs > lo ? kMaxSplitTokens / bs : lo;
    sb = sb < lo ? lo : (sb > hi ? hi : sb);
    if (sb > W) sb = W;
    if (sb < 1) sb = 1;
    p.split_blocks = sb;
    p.max_splits = (W + sb - 1) / sb;
  }
  const size_t n = (size_t)num_seqs * HQ * p.max_splits;
  p.off_n = 0;
  p.off_m = p.persistent ? round256((size_t)num_seqs * sizeof(int32_t)) : 0;
  p.off_l = p.off_m + round256(n * sizeof(float));
  p.off_o = p.off_l + round256(n * sizeof(float));
  p.bytes = p.off_o + round256(n * (size_t)D * sizeof(float));
  return p;
}

// Compute units of the current device (cached per device).
int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (dev >= 0 && dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (dev >= 0 && dev < 64) cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

// Resident workgroups per compute unit of the persistent kernel at this
// workgroup size (a property of the kernel binary, cached).
template <Ty C, int D, int G, bool kFused>
int persistent_occupancy(int waves_per_wg) {
  static std::atomic<int> cache[kWavesCap + 1];
  const int c = cache[waves_per_wg].load(std::memory_order_relaxed);
  if (c > 0) return c;
  int nb = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, decode_persistent_kernel<C, D, G, kFused>, 64 * waves_per_wg, 0) !=
      hipSuccess)
    return 0;
  cache[waves_per_wg].store(nb, std::memory_order_relaxed);
  return nb;
}

template <Ty C, int D, int G>
bool launch_split(DecArgs& a, const Plan& p, hipStream_t st) {
  if (p.persistent) {
    if constexpr (D <= 128) {
      const bool fused = a.new_k != nullptr;
      // this kernel's own workgroup width (the plan's is the vector path's)
      constexpr int wmax = persistent_max_waves<C>();
      a.waves_per_wg = a.HKV < wmax ? a.HKV : wmax;
      a.kv_groups = (a.HKV + a.waves_per_wg - 1) / a.waves_per_wg;
      const int cus = device_cus();
      const int occ = fused ? persistent_occupancy<C, D, G, true>(a.waves_per_wg)
                            : persistent_occupancy<C, D, G, false>(a.waves_per_wg);
      if (cus <= 0 || occ <= 0) return false;
      const int64_t resident = (int64_t)cus * occ;
      a.slots = (int)(resident / a.kv_groups > 1 ? resident / a.kv_groups : 1);
      const unsigned grid = (unsigned)(a.slots * a.kv_groups);
      if (fused)
        decode_persistent_kernel<C, D, G, true><<<grid, 64 * a.waves_per_wg, 0, st>>>(a);
      else
        decode_persistent_kernel<C, D, G, false><<<grid, 64 * a.waves_per_wg, 0, st>>>(a);
      decode_merge_kernel<C, D><<<(unsigned)(((int64_t)a.num_seqs * a.HQ + 3) / 4), 256, 0, st>>>(a);
      return true;
    }
    return false;
  }
  // Vector path: one workgroup per (KV-head group, split, sequence), kv-head
  // groups fastest so that sibling workgroups read the same pages together.
  dim3 grid(p.kv_groups, p.max_splits, a.num_seqs);
  decode_split_valu_kernel<C, D, G><<<grid, 64 * p.waves_per_wg, 0, st>>>(a);
  if (p.max_splits > 1)
    decode_merge_kernel<C, D><<<(unsigned)(((int64_t)a.num_seqs * a.HQ + 3) / 4), 256, 0, st>>>(a);
  return true;
}

template <Ty C, int D>
bool launch_g(int G, DecArgs& a, const Plan& p, hipStream_t st) {
  switch (G) {
    case 1: return launch_split<C, D, 1>(a, p, st);
    case 2: return launch_split<C, D, 2>(a, p, st);
    case 4: return launch_split<C, D, 4>(a, p, st);
    case 8: return launch_split<C, D, 8>(a, p, st);
    default: return false;
  }
}

template <Ty C>
bool launch_d(int D, int G, DecArgs& a, const Plan& p, hipStream_t st) {
  switch (D) {
    case 64: return launch_g<C, 64>(G, a, p, st);
    case 128: return launch_g<C, 128>(G, a, p, st);
    case 256: return launch_g<C, 256>(G, a, p, st);
    default: return false;
  }
}

pa_status check_sizes(const char* fn, int32_t num_seqs, int32_t HQ, int32_t HKV, int32_t D, int32_t W, int32_t bs) {
  if (num_seqs < 0 || HQ <= 0 || HKV <= 0 || W <= 0 || bs <= 0)
    return fail(PA_EINVAL, "%s: invalid sizes (num_seqs=%d H_Q=%d H_KV=%d W=%d block_size=%d)", fn, num_seqs, HQ, HKV, W, bs);
  if (HQ % HKV != 0) return fail(PA_EINVAL, "%s: num_q_heads %% num_kv_heads != 0", fn);
  const int G = HQ / HKV;
  if (G != 1 && G != 2 && G != 4 && G != 8)
    return fail(PA_EUNSUPPORTED, "%s: group size H_Q/H_KV = %d not supported (1, 2, 4, 8)", fn, G);
  if (D != 64 && D != 128 && D != 256) return fail(PA_EUNSUPPORTED, "%s: head_size %d not supported (64, 128, 256)", fn, D);
  const int rpl = 64 / (D / 8);
  if (bs % rpl != 0) return fail(PA_EUNSUPPORTED, "%s: block_size %d must be a multiple of %d at head_size %d", fn, bs, rpl, D);
  if ((int64_t)W * bs > INT32_MAX) return fail(PA_EINVAL, "%s: max_blocks_per_seq*block_size too large", fn);
  if (num_seqs > 65535) return fail(PA_EINVAL, "%s: num_seqs > 65535", fn);
  return PA_OK;
}

}  // namespace
}  // namespace pa

extern "C" size_t pa_decode_attention_workspace_size(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                                     int32_t head_size, int32_t max_blocks_per_seq,
                                                     int32_t block_size) {
  using namespace pa;
  clear_error();
  if (check_sizes("pa_decode_attention_workspace_size", num_seqs, num_q_heads, num_kv_heads, head_size,
                  max_blocks_per_seq, block_size) != PA_OK)
    return 0;
  const Plan p = make_plan(num_seqs > 0 ? num_seqs : 1, num_q_heads, num_kv_heads, head_size, max_blocks_per_seq, block_size);
  return p.bytes;
}

namespace pa {
namespace {

// The new tokens of a decode step (one per sequence, bf16 rows of H_KV*head_size).
struct NewTokens {
  const void* k;
  const void* v;
  const int64_t* slots;
  int64_t k_stride, v_stride;
};

pa_status decode_common(const char* fn, void* out, pa_dtype out_dtype, int64_t out_seq_stride, const void* q,
                        pa_dtype q_dtype, int64_t q_seq_stride, const void* key_cache, const void* value_cache,
                        pa_dtype cache_dtype, int64_t num_blocks, int32_t block_size, int64_t block_stride,
                        const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
                        int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_size,
                        float softmax_scale, const float* k_scale, const float* v_scale, void* workspace,
                        size_t workspace_bytes, const NewTokens* nt, void* stream) {
  pa_status s = check_sizes(fn, num_seqs, num_q_heads, num_kv_heads, head_size, max_blocks_per_seq, block_size);
  if (s != PA_OK) return s;
  if (out_dtype != PA_BF16 && out_dtype != PA_F32) return fail(PA_EDTYPE, "%s: out dtype %s not supported", fn, dtype_name(out_dtype));
  if (q_dtype != PA_BF16) return fail(PA_EDTYPE, "%s: q dtype %s not supported (bf16)", fn, dtype_name(q_dtype));
  if (cache_dtype != PA_BF16 && cache_dtype != PA_FP8_E4M3FN)
    return fail(PA_EDTYPE, "%s: cache dtype %s not supported (bf16, fp8_e4m3fn)", fn, dtype_name(cache_dtype));
  if (!(softmax_scale == softmax_scale) || isinf(softmax_scale)) return fail(PA_EINVAL, "%s: softmax_scale is not finite", fn);
  const int64_t row = (int64_t)num_q_heads * head_size;
  if (out_seq_stride < row || q_seq_stride < row) return fail(PA_EINVAL, "%s: sequence strides smaller than H_Q*head_size", fn);
  if (num_blocks < 0) return fail(PA_EINVAL, "%s: num_blocks < 0", fn);
  if (block_stride < (int64_t)block_size * num_kv_heads * head_size) return fail(PA_EINVAL, "%s: block_stride too small", fn);
  if (nt) {
    if ((k_scale == nullptr) != (v_scale == nullptr)) return fail(PA_EINVAL, "%s: give both scales or neither", fn);
    const int64_t kv_row = (int64_t)num_kv_heads * head_size;
    if (nt->k_stride < kv_row || nt->v_stride < kv_row)
      return fail(PA_EINVAL, "%s: new-token strides smaller than H_KV*head_size", fn);
  }
  if (num_seqs == 0) return PA_OK;
  if (!out || !q || !key_cache || !value_cache || !block_tables || !context_lens)
    return fail(PA_EINVAL, "%s: null pointer argument", fn);
  if (nt && (!nt->k || !nt->v || !nt->slots)) return fail(PA_EINVAL, "%s: null new-token pointer", fn);
  if (nt && (!aligned(nt->k, 16) || !aligned(nt->v, 16) || (nt->k_stride * 2) % 16 != 0 || (nt->v_stride * 2) % 16 != 0))
    return fail(PA_EINVAL, "%s: new-token rows must be 16-byte aligned", fn);
  const int cb = dtype_bytes(cache_dtype), ob = dtype_bytes(out_dtype);
  if (!aligned(q, 16) || (q_seq_stride * 2) % 16 != 0) return fail(PA_EINVAL, "%s: q must be 16-byte aligned per sequence", fn);
  if (!aligned(out, 16) || (out_seq_stride * ob) % 16 != 0) return fail(PA_EINVAL, "%s: out must be 16-byte aligned per sequence", fn);
  if (!aligned(key_cache, 16) || !aligned(value_cache, 16) || (block_stride * cb) % 16 != 0)
    return fail(PA_EINVAL, "%s: caches must be 16-byte aligned per block", fn);
  const Plan p = make_plan(num_seqs, num_q_heads, num_kv_heads, head_size, max_blocks_per_seq, block_size);
  if (!workspace || workspace_bytes < p.bytes || !aligned(workspace, 256))
    return fail(PA_EWORKSPACE, "%s: workspace needs %zu bytes, 256-byte aligned (got %zu)", fn, p.bytes, workspace_bytes);
  if (checks_on()) {
    const hipStream_t cs = reinterpret_cast<hipStream_t>(stream);
    s = check_tables(fn, cs, block_tables, num_seqs, max_blocks_per_seq, context_lens, num_blocks, block_size);
    if (s == PA_OK && nt) s = check_slots(fn, cs, nt->slots, num_seqs, nullptr, 0, num_blocks, block_size);
    if (s != PA_OK) return s;
  }

  DecArgs a;
  a.out = out;
  a.q = q;
  a.kc = key_cache;
  a.vc = value_cache;
  a.bt = block_tables;
  a.ctx_lens = context_lens;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.ws_m = reinterpret_cast<float*>(static_cast<char*>(workspace) + p.off_m);
  a.ws_l = reinterpret_cast<float*>(static_cast<char*>(workspace) + p.off_l);
  a.ws_o = reinterpret_cast<float*>(static_cast<char*>(workspace) + p.off_o);
  a.ws_n = p.persistent ? reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + p.off_n) : nullptr;
  a.out_seq_stride = out_seq_stride;
  a.q_seq_stride = q_seq_stride;
  a.block_stride = block_stride;
  a.num_blocks = num_blocks;
  a.block_size = block_size;
  a.W = max_blocks_per_seq;
  a.num_seqs = num_seqs;
  a.HQ = num_q_heads;
  a.HKV = num_kv_heads;
  a.split_blocks = p.split_blocks;
  a.max_splits = p.max_splits;
  a.waves_per_wg = p.waves_per_wg;
  a.kv_groups = p.kv_groups;
  a.slots = 0;
  a.out_f32 = out_dtype == PA_F32;
  a.scale_log2 = softmax_scale * 1.4426950408889634f;

  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  a.new_k = nullptr;
  a.new_v = nullptr;
  a.new_slots = nullptr;
  a.new_k_stride = a.new_v_stride = 0;
  if (nt && p.persistent) {
    // the persistent kernel takes the new tokens in itself and writes them
    a.new_k = static_cast<const uint16_t*>(nt->k);
    a.new_v = static_cast<const uint16_t*>(nt->v);
    a.new_slots = nt->slots;
    a.new_k_stride = nt->k_stride;
    a.new_v_stride = nt->v_stride;
  } else if (nt) {
    // other shapes: the cache write first, on the same stream; it checks its
    // own arguments before it launches anything, so a refusal queues nothing
    s = pa_reshape_and_cache(nt->k, nt->v, PA_BF16, num_seqs, num_kv_heads, head_size, nt->k_stride, nt->v_stride,
                             const_cast<void*>(key_cache), const_cast<void*>(value_cache), cache_dtype, num_blocks,
                             block_size, block_stride, nt->slots, nullptr, 0, k_scale, v_scale, stream);
    if (s != PA_OK) return s;
  }
  const int G = num_q_heads / num_kv_heads;
  const bool ok = cache_dtype == PA_BF16 ? launch_d<Ty::BF16>(head_size, G, a, p, st)
                                         : launch_d<Ty::FP8>(head_size, G, a, p, st);
  if (!ok) return fail(PA_EUNSUPPORTED, "%s: no kernel for this shape", fn);
  return after_launch(fn);
}

}  // namespace
}  // namespace pa

extern "C" pa_status pa_decode_attention(void* out, pa_dtype out_dtype, int64_t out_seq_stride, const void* q,
                                         pa_dtype q_dtype, int64_t q_seq_stride, const void* key_cache,
                                         const void* value_cache, pa_dtype cache_dtype, int64_t num_blocks,
                                         int32_t block_size, int64_t block_stride, const int32_t* block_tables,
                                         int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t num_seqs,
                                         int32_t num_q_heads, int32_t num_kv_heads, int32_t head_size,
                                         float softmax_scale, const float* k_scale, const float* v_scale,
                                         void* workspace, size_t workspace_bytes, void* stream) {
  pa::clear_error();
  return pa::decode_common("pa_decode_attention", out, out_dtype, out_seq_stride, q, q_dtype, q_seq_stride, key_cache,
                           value_cache, cache_dtype, num_blocks, block_size, block_stride, block_tables,
                           max_blocks_per_seq, context_lens, num_seqs, num_q_heads, num_kv_heads, head_size,
                           softmax_scale, k_scale, v_scale, workspace, workspace_bytes, nullptr, stream);
}

// Write then attend, as the engine's decode step orders them: the new token
// enters the cache first, so the attention over context_lens (which count it)
// reads it back from its slot.
extern "C" pa_status pa_decode_step(const void* new_k, const void* new_v, pa_dtype new_dtype, int64_t new_k_stride,
                                    int64_t new_v_stride, const int64_t* new_slots, void* out, pa_dtype out_dtype,
                                    int64_t out_seq_stride, const void* q, pa_dtype q_dtype, int64_t q_seq_stride,
                                    void* key_cache, void* value_cache, pa_dtype cache_dtype, int64_t num_blocks,
                                    int32_t block_size, int64_t block_stride, const int32_t* block_tables,
                                    int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t num_seqs,
                                    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_size, float softmax_scale,
                                    const float* k_scale, const float* v_scale, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  pa::clear_error();
  const char* fn = "pa_decode_step";
  if (new_dtype != PA_BF16)
    return pa::fail(PA_EDTYPE, "%s: new-token dtype %s not supported (bf16)", fn, pa::dtype_name(new_dtype));
  const pa::NewTokens nt{new_k, new_v, new_slots, new_k_stride, new_v_stride};
  return pa::decode_common(fn, out, out_dtype, out_seq_stride, q, q_dtype, q_seq_stride, key_cache, value_cache,
                           cache_dtype, num_blocks, block_size, block_stride, block_tables, max_blocks_per_seq,
                           context_lens, num_seqs, num_q_heads, num_kv_heads, head_size, softmax_scale, k_scale,
                           v_scale, workspace, workspace_bytes, &nt, stream);
}

// ---------------------------------------------------------------------------
// pa_decode_attention_noalloc: pa_decode_attention with its workspace in a
// fixed device array instead of a caller buffer, for callers that cannot
// allocate. The array is a file-scope __device__ object: every GPU the library
// runs on holds its own copy for the life of the process. Host code never uses
// the array's name as a device address (on the host that name is only a
// stand-in): the address is looked up once per device with
// hipGetSymbolAddress and kept in g_scratch_ptr.
namespace pa {
namespace {

constexpr size_t kScratchBytes = (size_t)64 << 20;  // 64 MiB
static __device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's copy of `scratch` (looked up on first use per device).
pa_status scratch_on_current_device(const char* fn, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(PA_EHIP, "%s: hipGetDevice failed: %s", fn, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(PA_EUNSUPPORTED, "%s: device index %d >= %d", fn, dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(PA_EHIP, "%s: hipGetSymbolAddress of the fixed workspace failed: %s", fn, hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return PA_OK;
}

}  // namespace
}  // namespace pa

extern "C" size_t pa_decode_attention_noalloc_max_workspace(void) { return pa::kScratchBytes; }

extern "C" pa_status pa_decode_attention_noalloc(void* out, pa_dtype out_dtype, int64_t out_seq_stride, const void* q,
                                                 pa_dtype q_dtype, int64_t q_seq_stride, const void* key_cache,
                                                 const void* value_cache, pa_dtype cache_dtype, int64_t num_blocks,
                                                 int32_t block_size, int64_t block_stride,
                                                 const int32_t* block_tables, int32_t max_blocks_per_seq,
                                                 const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                                                 int32_t num_kv_heads, int32_t head_size, float softmax_scale,
                                                 const float* k_scale, const float* v_scale, void* stream) {
  using namespace pa;
  clear_error();
  const char* fn = "pa_decode_attention_noalloc";
  pa_status s = check_sizes(fn, num_seqs, num_q_heads, num_kv_heads, head_size, max_blocks_per_seq, block_size);
  if (s != PA_OK) return s;
  if (num_seqs == 0) return PA_OK;
  const Plan p = make_plan(num_seqs, num_q_heads, num_kv_heads, head_size, max_blocks_per_seq, block_size);
  if (p.bytes > kScratchBytes)
    return fail(PA_EWORKSPACE, "%s: these sizes need %zu bytes of workspace; the fixed workspace holds %zu",
                fn, p.bytes, kScratchBytes);
  void* ws = nullptr;
  s = scratch_on_current_device(fn, &ws);
  if (s != PA_OK) return s;
  return decode_common(fn, out, out_dtype, out_seq_stride, q, q_dtype, q_seq_stride, key_cache, value_cache,
                       cache_dtype, num_blocks, block_size, block_stride, block_tables, max_blocks_per_seq,
                       context_lens, num_seqs, num_q_heads, num_kv_heads, head_size, softmax_scale, k_scale,
                       v_scale, ws, kScratchBytes, nullptr, stream);
}
