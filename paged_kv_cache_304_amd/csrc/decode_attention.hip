// pa_decode_attention: one query token per sequence against its paged K/V.
//
// Operation (section 2.6 "Attention" of the Qwen3-0.6B engine walkthrough page:
// decode attention reads K/V back along physical blocks through block_tables;
// the PagedAttention principle page: GQA with H_Q an integer multiple of H_KV,
// blocks of [block_size, H_KV, d_h] ordered only by a table): for sequence b
// and q head h, softmax over the first ctx_b cached positions of
// scale * q . K^ (K^ = K * k_scale), weights applied to V^ = V * v_scale.
//
// gfx950 design (split-K, two launches):
//  * Pass 1: workgroup = (KV split, sequence, KV-head group); one wavefront per
//    KV head, so the waves of a workgroup together read every head of the same
//    physical blocks, i.e. whole contiguous [block_size, H_KV, D] pages. A
//    wave's 64 lanes cover RPL = 64 / (D/8) cache rows of one head per load
//    (8 elements = 16 bytes of bf16 or 8 bytes of fp8 per lane); the QK dot of
//    a row is reduced over its D/8 lanes with DPP row operations. Each row of
//    lanes keeps its own online-softmax state (max, sum, accumulators for the
//    G query heads that share the KV head), updated once per 4 loads; the RPL
//    row states are merged with lane shuffles at the end of the split.
//    Split boundaries depend only on logical block indices, so the result is
//    bit-identical under any relabelling of physical blocks.
//  * Pass 2: one wavefront per (sequence, q head) merges the splits' (max,
//    sum, normalised output) triples; sequences that fit one split were already
//    written by pass 1.
// Scores are kept in the log2 domain (scale * log2(e) folded in) so that the
// exponentials are single v_exp_f32 instructions.
#include <math.h>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kMaxWaves = 8;       // KV heads (waves) per workgroup
constexpr int kTargetWgs = 2048;   // pass-1 workgroups aimed for at full length

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
  int32_t out_f32;
  float scale_log2;        // softmax_scale * log2(e)
};

__device__ __forceinline__ int clamp_ctx(const DecArgs& a, int b) {
  int ctx = a.ctx_lens[b];
  const int cap = a.W * a.block_size;
  return ctx < 0 ? 0 : (ctx > cap ? cap : ctx);
}

template <Ty C> struct KvRow;
template <> struct KvRow<Ty::BF16> {
  using Raw = u32x4;
  __device__ __forceinline__ static Raw load(const char* p) { return *reinterpret_cast<const u32x4*>(p); }
  __device__ __forceinline__ static void widen(const Raw& r, float (&f)[8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = bf16_lo(r[i]);
      f[2 * i + 1] = bf16_hi(r[i]);
    }
  }
};
template <> struct KvRow<Ty::FP8> {
  using Raw = u32x2;
  __device__ __forceinline__ static Raw load(const char* p) { return *reinterpret_cast<const u32x2*>(p); }
  __device__ __forceinline__ static void widen(const Raw& r, float (&f)[8]) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const f32x2 lo = fp8x2_lo(r[i]), hi = fp8x2_hi(r[i]);
      f[4 * i] = lo[0];
      f[4 * i + 1] = lo[1];
      f[4 * i + 2] = hi[0];
      f[4 * i + 3] = hi[1];
    }
  }
};

template <Ty C, int D, int G>
__global__ __launch_bounds__(512) void decode_split_kernel(DecArgs a) {
  constexpr int LPR = D / 8;     // lanes per cache row
  constexpr int RPL = 64 / LPR;  // cache rows per wave-load
  constexpr int CB = TyInfo<C>::kBytes;
  using R = KvRow<C>;
  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  const int g = (int)blockIdx.z * a.waves_per_wg + wave;
  if (g >= a.HKV) return;
  const int b = blockIdx.y;
  const int split = blockIdx.x;
  const int ctx = clamp_ctx(a, b);
  const int nblk = (ctx + a.block_size - 1) / a.block_size;
  // an empty sequence still gets one (empty) split, which writes zeros
  const int nsplit = max(1, (nblk + a.split_blocks - 1) / a.split_blocks);
  if (split >= nsplit) return;
  const int j0 = split * a.split_blocks;
  const int j1 = min(nblk, j0 + a.split_blocks);
  const int r = lane / LPR, c = lane % LPR;

  // q of the G heads of this group: 8 dims per lane, widened to fp32.
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
      typename R::Raw kr[4], vr[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (st0 + u < steps) {
          const int64_t off = (int64_t)((st0 + u) * RPL + r) * row_bytes;
          kr[u] = R::load(kb + off);
          vr[u] = R::load(vb + off);
        }
      }
      float s[G][4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const bool live = (st0 + u < steps) && ((st0 + u) * RPL + r < valid);
        if (st0 + u < steps) {
          float kf[8];
          R::widen(kr[u], kf);
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
          R::widen(vr[u], vf);
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
  if (r != 0) return;

#pragma unroll
  for (int gi = 0; gi < G; ++gi) {
    const int h = g * G + gi;
    const float inv = l[gi] > 0.0f ? vs / l[gi] : 0.0f;
    float o[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) o[k] = acc[gi][k] * inv;
    if (nsplit == 1) {
      if (a.out_f32) {
        float* op = static_cast<float*>(a.out) + (int64_t)b * a.out_seq_stride + (int64_t)h * D + 8 * c;
        u32x4 x, y;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          x[k] = __float_as_uint(o[k]);
          y[k] = __float_as_uint(o[4 + k]);
        }
        reinterpret_cast<u32x4*>(op)[0] = x;
        reinterpret_cast<u32x4*>(op)[1] = y;
      } else {
        uint16_t* op = static_cast<uint16_t*>(a.out) + (int64_t)b * a.out_seq_stride + (int64_t)h * D + 8 * c;
        u32x4 x;
#pragma unroll
        for (int k = 0; k < 4; ++k) x[k] = f32_to_bf16(o[2 * k]) | (f32_to_bf16(o[2 * k + 1]) << 16);
        *reinterpret_cast<u32x4*>(op) = x;
      }
    } else {
      const int64_t slot = ((int64_t)b * a.HQ + h) * a.max_splits + split;
      if (c == 0) {
        a.ws_m[slot] = m[gi];
        a.ws_l[slot] = l[gi];
      }
      float* wo = a.ws_o + slot * D + 8 * c;
      u32x4 x, y;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        x[k] = __float_as_uint(o[k]);
        y[k] = __float_as_uint(o[4 + k]);
      }
      reinterpret_cast<u32x4*>(wo)[0] = x;
      reinterpret_cast<u32x4*>(wo)[1] = y;
    }
  }
}

// ---------------------------------------------------------------------------
// Split pass, matrix-core variant (block_size a multiple of 16).
//
// A tile is 16 consecutive cache positions of one KV head. QK^T of a tile is
// one v_mfma_f32_16x16x32_bf16 per 32 head dims: A = the K tile (row = token,
// lane l holds token l%16, dims 8*(l/16)..+8 of the step), B = the group's q
// heads as columns (columns >= G are zero), so lane l receives the scores of
// tokens 4*(l/16)+r, r = 0..3, for head l%16. The softmax runs on those lanes;
// P.V runs on the vector ALUs with V in a row layout (16 lanes per cache row,
// D/16 dims per lane, 4 rows per load) in which lane l needs exactly the
// probabilities of row-group l/16 -- DPP row_newbcast hands them over. fp8 K
// is widened to bf16 exactly before the MFMA.
// ---------------------------------------------------------------------------
typedef __bf16 bf16x8 __attribute__((__vector_size__(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int NW> struct Dw { uint32_t w[NW]; };

template <int NW>
__device__ __forceinline__ Dw<NW> load_dw(const char* p) {
  Dw<NW> r;
  if constexpr (NW == 1) {
    r.w[0] = *reinterpret_cast<const uint32_t*>(p);
  } else if constexpr (NW == 2) {
    const u32x2 v = *reinterpret_cast<const u32x2*>(p);
    r.w[0] = v[0];
    r.w[1] = v[1];
  } else {
#pragma unroll
    for (int i = 0; i < NW / 4; ++i) {
      const u32x4 v = reinterpret_cast<const u32x4*>(p)[i];
#pragma unroll
      for (int k = 0; k < 4; ++k) r.w[4 * i + k] = v[k];
    }
  }
  return r;
}

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

// NW dwords of cache elements -> fp32.
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

// Value of lane j of this lane's 16-lane row (DPP row_newbcast).
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

template <Ty C, int D, int G, int TPI>
__global__ __launch_bounds__(512) void decode_split_mfma_kernel(DecArgs a) {
  constexpr int KS = D / 32;               // MFMA steps over the head dim
  constexpr int EPL = D / 16;              // V dims per lane
  constexpr int CB = TyInfo<C>::kBytes;
  constexpr int KW = 8 * CB / 4;           // dwords per K operand chunk
  constexpr int VW = EPL * CB / 4;         // dwords per V chunk
  static_assert(VW >= 1, "V chunk");
  const int lane = threadIdx.x & 63;
  const int li = lane & 15, lg = lane >> 4;
  const int wave = uniform(threadIdx.x >> 6);
  const int g = (int)blockIdx.z * a.waves_per_wg + wave;
  if (g >= a.HKV) return;
  const int b = blockIdx.y;
  const int split = blockIdx.x;
  const int ctx = clamp_ctx(a, b);
  const int nblk = (ctx + a.block_size - 1) / a.block_size;
  const int nsplit = max(1, (nblk + a.split_blocks - 1) / a.split_blocks);
  if (split >= nsplit) return;
  const int j0 = split * a.split_blocks;
  const int j1 = min(nblk, j0 + a.split_blocks);
  const int p_begin = j0 * a.block_size;
  const int p_end = min(ctx, j1 * a.block_size);
  const int n_tiles = p_end > p_begin ? (p_end - p_begin + 15) >> 4 : 0;

  bf16x8 qb[KS];
  {
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) + (int64_t)b * a.q_seq_stride +
                         (int64_t)(g * G + (li < G ? li : 0)) * D + 8 * lg;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      u32x4 w = *reinterpret_cast<const u32x4*>(qp + 32 * s);
      if (li >= G) w = u32x4{0, 0, 0, 0};
      qb[s] = __builtin_bit_cast(bf16x8, w);
    }
  }
  const float ks = a.k_scale ? *a.k_scale : 1.0f;
  const float vs = a.v_scale ? *a.v_scale : 1.0f;
  const float sl2 = a.scale_log2 * ks;

  float m_run = -INFINITY, l_run = 0.0f;
  float acc[G][EPL];
#pragma unroll
  for (int j = 0; j < G; ++j)
#pragma unroll
    for (int k = 0; k < EPL; ++k) acc[j][k] = 0.0f;

  const int64_t row_el = (int64_t)a.HKV * D;  // elements between consecutive slots of a block
  const int32_t* bt = a.bt + (int64_t)b * a.W;
  const char* kc = static_cast<const char*>(a.kc);
  const char* vc = static_cast<const char*>(a.vc);

  for (int t0 = 0; t0 < n_tiles; t0 += TPI) {
    Dw<KW> kr[TPI][KS];
    Dw<VW> vr[TPI][4];
    bool tv[TPI];
    int tp0[TPI];
#pragma unroll
    for (int tt = 0; tt < TPI; ++tt) {
      const int p0 = p_begin + (t0 + tt) * 16;
      tp0[tt] = p0;
      bool valid = (t0 + tt) < n_tiles;
      int phys = 0;
      if (valid) {
        phys = bt[p0 / a.block_size];
        valid = phys >= 0 && (int64_t)phys < a.num_blocks;  // outside the pool: not attended
      }
      tv[tt] = valid;
      if (valid) {
        const int off = p0 % a.block_size;
        const int64_t blk = (int64_t)phys * a.block_stride + (int64_t)g * D;
        const char* kp = kc + (blk + (int64_t)(off + li) * row_el + 8 * lg) * CB;
#pragma unroll
        for (int s = 0; s < KS; ++s) kr[tt][s] = load_dw<KW>(kp + 32 * s * CB);
        const char* vp = vc + (blk + (int64_t)(off + 4 * lg) * row_el + EPL * li) * CB;
#pragma unroll
        for (int i = 0; i < 4; ++i) vr[tt][i] = load_dw<VW>(vp + i * row_el * CB);
      }
    }
#pragma unroll
    for (int tt = 0; tt < TPI; ++tt) {
      if (!tv[tt]) continue;
      f32x4 sc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int s = 0; s < KS; ++s)
        sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8<C>(kr[tt][s]), qb[s], sc, 0, 0, 0);
      const int prow = tp0[tt] + 4 * lg;  // position of this lane's first score / V row
      float sr[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) sr[r] = (prow + r < p_end) ? sc[r] * sl2 : -INFINITY;
      float mx = fmaxf(fmaxf(sr[0], sr[1]), fmaxf(sr[2], sr[3]));
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float mn = fmaxf(m_run, mx);
      const float mu = (mn == -INFINITY) ? 0.0f : mn;
      const float alpha = __builtin_amdgcn_exp2f(m_run - mu);
      float pr[4];
      float ps = 0.0f;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        pr[r] = __builtin_amdgcn_exp2f(sr[r] - mu);
        ps += pr[r];
      }
      l_run = l_run * alpha + ps;
      m_run = mn;
      rescale_heads<0, G, EPL>(acc, alpha);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float vf[EPL];
        widen_dw<C>(vr[tt][i], vf);
        if (prow + i >= p_end) {
#pragma unroll
          for (int k = 0; k < EPL; ++k) vf[k] = 0.0f;  // unwritten slots may hold NaN
        }
        accumulate_row<0, G, EPL>(acc, pr[i], vf);
      }
    }
  }

  // Sum the four row groups (same running max everywhere, so no rescaling).
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
  if (lg != 0) return;

#pragma unroll
  for (int j = 0; j < G; ++j) {
    const int h = g * G + j;
    const float inv = lj[j] > 0.0f ? vs / lj[j] : 0.0f;
    float o[EPL];
#pragma unroll
    for (int k = 0; k < EPL; ++k) o[k] = acc[j][k] * inv;
    if (nsplit == 1) {
      if (a.out_f32) {
        float* op = static_cast<float*>(a.out) + (int64_t)b * a.out_seq_stride + (int64_t)h * D + EPL * li;
#pragma unroll
        for (int k = 0; k < EPL; ++k) op[k] = o[k];
      } else {
        uint16_t* op = static_cast<uint16_t*>(a.out) + (int64_t)b * a.out_seq_stride + (int64_t)h * D + EPL * li;
        uint32_t w[EPL / 2];
#pragma unroll
        for (int k = 0; k < EPL / 2; ++k) w[k] = f32_to_bf16(o[2 * k]) | (f32_to_bf16(o[2 * k + 1]) << 16);
#pragma unroll
        for (int k = 0; k < EPL / 2; ++k) reinterpret_cast<uint32_t*>(op)[k] = w[k];
      }
    } else {
      const int64_t slot = ((int64_t)b * a.HQ + h) * a.max_splits + split;
      if (li == j) {
        a.ws_m[slot] = m_run;
        a.ws_l[slot] = lj[j];
      }
      float* wo = a.ws_o + slot * D + EPL * li;
#pragma unroll
      for (int k = 0; k < EPL; ++k) wo[k] = o[k];
    }
  }
}

// Pass 2: one wavefront per (sequence, q head); lane i holds dims i, i+64, ...
template <int D>
__global__ __launch_bounds__(256) void decode_merge_kernel(DecArgs a) {
  constexpr int PER = D / 64;
  const int lane = threadIdx.x & 63;
  const int wid = (int)blockIdx.x * 4 + uniform(threadIdx.x >> 6);
  if (wid >= a.num_seqs * a.HQ) return;
  const int b = wid / a.HQ, h = wid - b * a.HQ;
  const int ctx = clamp_ctx(a, b);
  const int nblk = (ctx + a.block_size - 1) / a.block_size;
  const int nsplit = (nblk + a.split_blocks - 1) / a.split_blocks;
  if (nsplit <= 1) return;  // written by pass 1
  float o[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) o[i] = 0.0f;
  {
    const int64_t base = ((int64_t)b * a.HQ + h) * a.max_splits;
    float M = -INFINITY;
    for (int s = 0; s < nsplit; ++s) M = fmaxf(M, a.ws_m[base + s]);
    if (M != -INFINITY) {
      float den = 0.0f;
      for (int s = 0; s < nsplit; ++s) {
        const float w = __builtin_amdgcn_exp2f(a.ws_m[base + s] - M) * a.ws_l[base + s];
        den += w;
        const float* wo = a.ws_o + (base + s) * D;
#pragma unroll
        for (int i = 0; i < PER; ++i) o[i] = fmaf(w, wo[lane + 64 * i], o[i]);
      }
      const float inv = 1.0f / den;
#pragma unroll
      for (int i = 0; i < PER; ++i) o[i] *= inv;
    }
  }
  if (a.out_f32) {
    float* op = static_cast<float*>(a.out) + (int64_t)b * a.out_seq_stride + (int64_t)h * D;
#pragma unroll
    for (int i = 0; i < PER; ++i) op[lane + 64 * i] = o[i];
  } else {
    uint16_t* op = static_cast<uint16_t*>(a.out) + (int64_t)b * a.out_seq_stride + (int64_t)h * D;
#pragma unroll
    for (int i = 0; i < PER; ++i) op[lane + 64 * i] = (uint16_t)f32_to_bf16(o[i]);
  }
}

struct Plan {
  int waves_per_wg, kv_groups, split_blocks, max_splits;
  size_t off_l, off_o, bytes;
};

inline size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

Plan make_plan(int num_seqs, int HQ, int HKV, int D, int W, int bs) {
  Plan p;
  p.waves_per_wg = HKV < kMaxWaves ? HKV : kMaxWaves;
  p.kv_groups = (HKV + p.waves_per_wg - 1) / p.waves_per_wg;
  // Aim for kTargetWgs workgroups if every sequence used all W blocks, but
  // never split finer than 4 blocks (per-split merge traffic).
  const int64_t per_seq = ((int64_t)kTargetWgs + (int64_t)num_seqs * p.kv_groups - 1) / ((int64_t)num_seqs * p.kv_groups);
  int sb = (int)((W + per_seq - 1) / per_seq);
  const int min_sb = (64 + bs - 1) / bs;  // at least 64 tokens per split
  if (sb < min_sb) sb = min_sb;
  if (sb > W) sb = W;
  if (sb < 1) sb = 1;
  p.split_blocks = sb;
  p.max_splits = (W + sb - 1) / sb;
  const size_t n = (size_t)num_seqs * HQ * p.max_splits;
  p.off_l = round256(n * sizeof(float));
  p.off_o = p.off_l + round256(n * sizeof(float));
  p.bytes = p.off_o + round256(n * (size_t)D * sizeof(float));
  return p;
}

template <Ty C, int D, int G>
void launch_split(const DecArgs& a, const Plan& p, hipStream_t st) {
  dim3 grid(p.max_splits, a.num_seqs, p.kv_groups);
  if (a.block_size % 16 == 0)
    decode_split_mfma_kernel<C, D, G, (D >= 256 ? 1 : 2)><<<grid, 64 * p.waves_per_wg, 0, st>>>(a);
  else
    decode_split_kernel<C, D, G><<<grid, 64 * p.waves_per_wg, 0, st>>>(a);
}

template <Ty C, int D>
bool launch_g(int G, const DecArgs& a, const Plan& p, hipStream_t st) {
  switch (G) {
    case 1: launch_split<C, D, 1>(a, p, st); return true;
    case 2: launch_split<C, D, 2>(a, p, st); return true;
    case 4: launch_split<C, D, 4>(a, p, st); return true;
    case 8: launch_split<C, D, 8>(a, p, st); return true;
    default: return false;
  }
}

template <Ty C>
bool launch_d(int D, int G, const DecArgs& a, const Plan& p, hipStream_t st) {
  switch (D) {
    case 64: return launch_g<C, 64>(G, a, p, st);
    case 128: return launch_g<C, 128>(G, a, p, st);
    case 256: return launch_g<C, 256>(G, a, p, st);
    default: return false;
  }
}

bool launch_merge(int D, const DecArgs& a, hipStream_t st) {
  const unsigned grid = (unsigned)(((int64_t)a.num_seqs * a.HQ + 3) / 4);
  switch (D) {
    case 64: decode_merge_kernel<64><<<grid, 256, 0, st>>>(a); return true;
    case 128: decode_merge_kernel<128><<<grid, 256, 0, st>>>(a); return true;
    case 256: decode_merge_kernel<256><<<grid, 256, 0, st>>>(a); return true;
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

extern "C" pa_status pa_decode_attention(void* out, pa_dtype out_dtype, int64_t out_seq_stride, const void* q,
                                         pa_dtype q_dtype, int64_t q_seq_stride, const void* key_cache,
                                         const void* value_cache, pa_dtype cache_dtype, int64_t num_blocks,
                                         int32_t block_size, int64_t block_stride, const int32_t* block_tables,
                                         int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t num_seqs,
                                         int32_t num_q_heads, int32_t num_kv_heads, int32_t head_size,
                                         float softmax_scale, const float* k_scale, const float* v_scale,
                                         void* workspace, size_t workspace_bytes, void* stream) {
  using namespace pa;
  clear_error();
  const char* fn = "pa_decode_attention";
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
  if (num_seqs == 0) return PA_OK;
  if (!out || !q || !key_cache || !value_cache || !block_tables || !context_lens)
    return fail(PA_EINVAL, "%s: null pointer argument", fn);
  const int cb = dtype_bytes(cache_dtype), ob = dtype_bytes(out_dtype);
  if (!aligned(q, 16) || (q_seq_stride * 2) % 16 != 0) return fail(PA_EINVAL, "%s: q must be 16-byte aligned per sequence", fn);
  if (!aligned(out, 16) || (out_seq_stride * ob) % 16 != 0) return fail(PA_EINVAL, "%s: out must be 16-byte aligned per sequence", fn);
  if (!aligned(key_cache, 16) || !aligned(value_cache, 16) || (block_stride * cb) % 16 != 0)
    return fail(PA_EINVAL, "%s: caches must be 16-byte aligned per block", fn);
  const Plan p = make_plan(num_seqs, num_q_heads, num_kv_heads, head_size, max_blocks_per_seq, block_size);
  if (!workspace || workspace_bytes < p.bytes || !aligned(workspace, 256))
    return fail(PA_EWORKSPACE, "%s: workspace needs %zu bytes, 256-byte aligned (got %zu)", fn, p.bytes, workspace_bytes);

  DecArgs a;
  a.out = out;
  a.q = q;
  a.kc = key_cache;
  a.vc = value_cache;
  a.bt = block_tables;
  a.ctx_lens = context_lens;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.ws_m = static_cast<float*>(workspace);
  a.ws_l = reinterpret_cast<float*>(static_cast<char*>(workspace) + p.off_l);
  a.ws_o = reinterpret_cast<float*>(static_cast<char*>(workspace) + p.off_o);
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
  a.out_f32 = out_dtype == PA_F32;
  a.scale_log2 = softmax_scale * 1.4426950408889634f;

  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const int G = num_q_heads / num_kv_heads;
  const bool ok = cache_dtype == PA_BF16 ? launch_d<Ty::BF16>(head_size, G, a, p, st)
                                         : launch_d<Ty::FP8>(head_size, G, a, p, st);
  if (!ok) return fail(PA_EUNSUPPORTED, "%s: no kernel for this shape", fn);
  s = after_launch(fn);
  if (s != PA_OK) return s;
  if (p.max_splits > 1) {
    launch_merge(head_size, a, st);
    s = after_launch("pa_decode_attention (merge)");
  }
  return s;
}
