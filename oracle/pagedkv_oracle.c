/*
 * CPU oracle for the paged KV cache hot path.
 *
 * TEST INFRASTRUCTURE ONLY. This file states, as plainly as possible, what the
 * cache write, the MLA-style K concat, single-token paged decode attention,
 * chunked-prefill (variable-length, causal) paged attention and MLA decode over
 * a latent paged cache compute, so that the GPU kernels can be checked against it. Only the test
 * suite, the smoke check and the benchmark's CPU-baseline leg may load it; the
 * product library never links or calls it, and it shares no source, header,
 * table or helper with the HIP path.
 *
 * Sources (the web pages this project follows):
 *  - Qwen3-0.6B engine walkthrough page, section 2.6 "Attention": the Triton
 *    store_kvcache kernel, its cache layout [num_blocks, block_size, H_KV, d_h],
 *    the slot -> (block, offset) split and the skip of slot -1, and the worked
 *    source-offset example (token 5, head 3 -> elements 5504..5631).
 *  - "PagedAttention principle" page, sections on GQA/MLA shapes (H_Q is an
 *    integer multiple of H_KV; per token the cache holds k, v of [H_KV, d_h]),
 *    the decode dataflow (the new token is written before attention) and the
 *    block allocation paragraph (a block is [block_size, H_KV, d_h]; blocks are
 *    physically scattered and found through a table).
 *  - Qwen3-0.6B engine walkthrough page, section 2.4 (the LM head): queries of a
 *    prefill batch are packed token-major and delimited by cu_seqlens_q
 *    (prefix sums of the per-sequence query counts); section 2.6 names the
 *    variable-length flash path of prefill.
 *  - "PagedAttention principle" page, autoregressive dataflow section: prefill
 *    computes causal attention over the prompt while caching its K/V.
 *  - "PagedAttention principle" page, MLA paragraphs of the GQA/MLA shapes
 *    section: MLA caches the latent c_kv = x W_DKV ([d_c] per token) instead of
 *    K and V, which are recovered as c_kv W_UK and c_kv W_UV ([H_Q * d_h],
 *    reshaped per head); the q.k dimension carries a RoPE part that v lacks.
 *  - SGLang cache_ops.py (Triton): concat_and_cast_mha_k (per-head k_nope with
 *    one shared k_rope, cast at the store) and reshape_and_cache_flash (source
 *    token strides, optional second-stage SWA slot remap, optional division by
 *    a per-tensor k/v scale before the store, block stride of the cache).
 *
 * Readings taken where the pages leave a step open:
 *  R1  Any negative slot skips the token; a negative first-stage slot skips it
 *      before the SWA table is consulted (the SGLang kernel would index the
 *      table with -1).
 *  R2  Memory-safety superset: a first-stage slot >= swa_len, or a final slot
 *      >= num_blocks*block_size, also skips the token.
 *  R3  The scale is divided out on write (the SGLang code divides, although its
 *      docstring says "dequantization") as an IEEE fp32 division of the value
 *      widened to fp32 by the fp32 scale; the quotient is then rounded once
 *      more to the cache type.
 *  R4  fp8 is OCP e4m3fn: bias 7, no infinities, max 448, NaN = S.1111.111.
 *      Rounding is to nearest, ties to even; any value whose rounded magnitude
 *      would exceed 448 (|y| > 464), every infinity and every NaN becomes
 *      NaN with the input's sign (0x7F | sign).
 *  R5  fp32 -> bf16 is round to nearest, ties to even (overflow goes to inf);
 *      a NaN keeps its sign and top payload bits and gets the quiet bit.
 *  R6  GQA groups are contiguous: q head h reads kv head h / (H_Q / H_KV).
 *  R7  Decode attention is textbook softmax attention of one query token over
 *      the first context_lens[b] cached positions of sequence b, read through
 *      block_tables[b]; K and V are dequantised by multiplying with k_scale
 *      and v_scale. context_lens is clamped to [0, W*block_size]; ctx == 0
 *      gives an all-zero output; a position whose table entry lies outside
 *      [0, num_blocks) does not take part (memory-safety superset).
 *  R10 Chunked prefill: sequence b contributes n_b = cu_seqlens_q[b+1] -
 *      cu_seqlens_q[b] query tokens, the last n_b positions of its context
 *      (their K/V are already in the cache), so query i sits at position
 *      p = ctx_b - n_b + i and attends causally to cached positions 0..p
 *      through block_tables[b] (the same clamping, dequantisation, GQA mapping
 *      and table-entry rule as R7). A query with p < 0 (n_b > ctx_b) has no
 *      key and gives zeros. n_b = 1 is exactly R7's decode step.
 *  R13 MLA over a latent cache: per token the cache holds one row, the latent
 *      c (latent_dim values) followed by a RoPE key part k_r (rope_dim values,
 *      possibly none) shared by every head. Head h's key and value are the
 *      page's up-projections k_h = (c W_UK)[h*qk_dim ..], v_h = (c W_UV)[h*v_dim
 *      ..] with W_UK [latent_dim, H*qk_dim], W_UV [latent_dim, H*v_dim]; the
 *      query of head h is q_nope[h] (qk_dim) and q_rope[h] (rope_dim), and the
 *      score is scale * (q_nope[h].k_h + q_rope[h].k_r) -- the page says only
 *      that the q.k dimension carries a RoPE part that v lacks; the decoupled,
 *      shared RoPE key is the form the MLA-style concat of a shared k_rope
 *      produces. Context clamping and the table-entry rule are R7's.
 *
 * Build: gcc -O2 -std=c11 -fopenmp -ffp-contract=off -fPIC -shared
 * (no fast-math: IEEE single division and round-to-nearest are required).
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Threads of the OpenMP loops below (for timing the oracle; no effect on results). */
int orc_max_threads(void) { return omp_get_max_threads(); }
void orc_set_num_threads(int n) { omp_set_num_threads(n > 0 ? n : 1); }

/* dtype codes of this file (independent of the product library's) */
enum { ORC_BF16 = 0, ORC_F32 = 2, ORC_FP8_E4M3FN = 3 };

static int orc_elem_size(int dt) {
  switch (dt) {
    case ORC_BF16: return 2;
    case ORC_F32: return 4;
    case ORC_FP8_E4M3FN: return 1;
    default: return 0;
  }
}

/* ---------------------------------------------------------------- decoding */

/* bf16 is the top half of an fp32 bit pattern. */
static float orc_bf16_to_f32(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* OCP e4m3fn: value = (-1)^s * m * 2^-9 for e == 0 (subnormal),
 * (-1)^s * (8 + m) * 2^(e - 10) otherwise; e == 15 && m == 7 is NaN. */
double orc_e4m3fn_to_f64(uint8_t c) {
  int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
  double v;
  if (e == 15 && m == 7) return s ? -NAN : NAN;
  if (e == 0)
    v = ldexp((double)m, -9);
  else
    v = ldexp((double)(8 + m), e - 10);
  return s ? -v : v;
}

/* Value of one stored element, widened exactly to double. */
static double orc_load_f64(const void* base, int64_t idx, int dt) {
  switch (dt) {
    case ORC_BF16: return (double)orc_bf16_to_f32(((const uint16_t*)base)[idx]);
    case ORC_F32: return (double)((const float*)base)[idx];
    case ORC_FP8_E4M3FN: return orc_e4m3fn_to_f64(((const uint8_t*)base)[idx]);
  }
  return NAN;
}

/* The element widened to fp32 (exact for bf16 and fp32 sources). */
static float orc_load_f32(const void* base, int64_t idx, int dt) {
  switch (dt) {
    case ORC_BF16: return orc_bf16_to_f32(((const uint16_t*)base)[idx]);
    case ORC_F32: return ((const float*)base)[idx];
    case ORC_FP8_E4M3FN: return (float)orc_e4m3fn_to_f64(((const uint8_t*)base)[idx]);
  }
  return NAN;
}

/* ---------------------------------------------------------------- encoding */

/* R5: fp32 -> bf16, round to nearest even on the discarded 16 bits.
 * IEEE magnitudes are ordered like their bit patterns, so the two bf16
 * neighbours of x are the truncation and the truncation plus one bf16 ulp. */
uint16_t orc_f32_to_bf16(float x) {
  uint32_t u;
  memcpy(&u, &x, 4);
  if (isnan(x)) return (uint16_t)((u >> 16) | 0x0040u);
  uint32_t down = u & 0xFFFF0000u;
  uint32_t rem = u & 0x0000FFFFu;
  uint32_t up = down + 0x00010000u; /* next magnitude away from zero */
  uint32_t pick;
  if (rem < 0x8000u)
    pick = down;
  else if (rem > 0x8000u)
    pick = up;
  else
    pick = ((down >> 16) & 1u) ? up : down; /* tie: keep the even one */
  return (uint16_t)(pick >> 16);
}

/* R4: fp32 -> e4m3fn. The representable magnitudes are a grid whose step is
 * 2^-9 below 2^-6 and 2^(E-3) in the binade [2^E, 2^(E+1)); round |x| to the
 * nearest grid point with ties to the even multiple (an even multiple is an
 * even code), then encode. Work is in double, where every step is exact. */
uint8_t orc_f32_to_e4m3fn(float xf) {
  double x = (double)xf;
  uint8_t sign = signbit(x) ? 0x80 : 0x00;
  if (isnan(x) || isinf(x)) return sign | 0x7F;
  double a = fabs(x);
  int E;
  double q; /* grid step at a */
  if (a < ldexp(1.0, -6)) {
    q = ldexp(1.0, -9);
  } else {
    (void)frexp(a, &E); /* a = f * 2^E, f in [0.5, 1) -> binade 2^(E-1) */
    q = ldexp(1.0, (E - 1) - 3);
  }
  double r = nearbyint(a / q); /* default rounding mode: ties to even */
  double v = r * q;
  if (v > 448.0) return sign | 0x7F;
  if (v < ldexp(1.0, -6)) return sign | (uint8_t)r; /* subnormal: code = m */
  int k;
  double f = frexp(v, &k);                  /* v = f * 2^k */
  int e = (k - 1) + 7;                      /* biased exponent */
  int m = (int)((2.0 * f - 1.0) * 8.0);     /* 3-bit mantissa, exact */
  return sign | (uint8_t)((e << 3) | m);
}

/* Store fp32 y into element idx of a tensor of type dt (one rounding). */
static void orc_store_from_f32(void* base, int64_t idx, int dt, float y) {
  switch (dt) {
    case ORC_BF16: ((uint16_t*)base)[idx] = orc_f32_to_bf16(y); break;
    case ORC_F32: ((float*)base)[idx] = y; break;
    case ORC_FP8_E4M3FN: ((uint8_t*)base)[idx] = orc_f32_to_e4m3fn(y); break;
  }
}

/* enc(): a bit copy when the types agree and there is no scale (this keeps
 * -0 and NaN payloads); otherwise widen to fp32, divide by the scale if any
 * (R3), and round once to the destination type. */
static void orc_encode(const void* src, int64_t si, int sdt, void* dst, int64_t di, int ddt,
                       const float* scale) {
  if (sdt == ddt && scale == NULL) {
    int es = orc_elem_size(sdt);
    memcpy((char*)dst + di * es, (const char*)src + si * es, (size_t)es);
    return;
  }
  float x = orc_load_f32(src, si, sdt);
  float y = scale ? x / *scale : x;
  orc_store_from_f32(dst, di, ddt, y);
}

/* n fp32 values rounded once to dst_dt (R4, R5), element by element: the
 * scalar encodes above applied to an array (used to check a conversion over
 * every fp32 bit pattern). Returns 0, or -1 for an unsupported type. */
int orc_encode_f32_array(const float* src, int64_t n, void* dst, int dst_dt) {
  if (dst_dt != ORC_BF16 && dst_dt != ORC_FP8_E4M3FN) return -1;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) orc_store_from_f32(dst, i, dst_dt, src[i]);
  return 0;
}

/* Exposed for the pin tests. */
uint8_t orc_encode_bf16_to_fp8_scaled(uint16_t h, float scale) {
  float x = orc_bf16_to_f32(h);
  return orc_f32_to_e4m3fn(x / scale);
}

/* ----------------------------------------------------- slot resolution (a1) */

/* Returns the final slot of token t, or -1 when the token is skipped.
 * Step order (R1, R2): first-stage slot; a negative one skips; with an SWA
 * table, the first-stage slot indexes it and a negative entry skips; a final
 * slot outside the pool skips. */
int64_t orc_resolve_slot(const int64_t* slot_mapping, int64_t t, const int64_t* swa,
                         int64_t swa_len, int64_t pool_slots) {
  int64_t s = slot_mapping[t];
  if (s < 0) return -1;
  if (swa) {
    if (s >= swa_len) return -1;
    s = swa[s];
    if (s < 0) return -1;
  }
  if (s >= pool_slots) return -1;
  return s;
}

/* ------------------------------------------------- reshape_and_cache (a1,a2) */

/* Writes key[t, h, d] (and value[t, h, d] when value != NULL) to
 * cache[block, off, h, d] with block = slot / block_size, off = slot % block_size.
 * Source element (t, h, d) sits at t*token_stride + h*head_size + d; cache
 * element (blk, off, h, d) at blk*block_stride + (off*num_heads + h)*head_size + d.
 * Returns the number of tokens written. */
int64_t orc_reshape_and_cache(const void* key, const void* value, int src_dt, int64_t num_tokens,
                              int num_heads, int head_size, int64_t key_token_stride,
                              int64_t value_token_stride, void* key_cache, void* value_cache,
                              int cache_dt, int64_t num_blocks, int block_size,
                              int64_t block_stride, const int64_t* slot_mapping,
                              const int64_t* swa, int64_t swa_len, const float* k_scale,
                              const float* v_scale) {
  int64_t written = 0;
  int64_t pool_slots = num_blocks * (int64_t)block_size;
#pragma omp parallel for reduction(+ : written) schedule(static)
  for (int64_t t = 0; t < num_tokens; ++t) {
    int64_t s = orc_resolve_slot(slot_mapping, t, swa, swa_len, pool_slots);
    if (s < 0) continue;
    int64_t blk = s / block_size, off = s % block_size;
    for (int h = 0; h < num_heads; ++h) {
      for (int d = 0; d < head_size; ++d) {
        int64_t dst = blk * block_stride + (off * num_heads + h) * (int64_t)head_size + d;
        orc_encode(key, t * key_token_stride + (int64_t)h * head_size + d, src_dt, key_cache, dst,
                   cache_dt, k_scale);
        if (value)
          orc_encode(value, t * value_token_stride + (int64_t)h * head_size + d, src_dt,
                     value_cache, dst, cache_dt, v_scale);
      }
    }
    written += 1;
  }
  return written;
}

/* --------------------------------------------------- concat_and_cast (a3) */

/* k[t, h, d] = cast(k_nope[t, h, d]) for d < nope_dim and
 * k[t, h, d] = cast(k_rope[t, 0, d - nope_dim]) for nope_dim <= d < nope_dim + rope_dim;
 * the rope part is shared by every head. Innermost strides are 1. */
void orc_concat_and_cast(void* k, int k_dt, int64_t k_s0, int64_t k_s1, const void* k_nope,
                         int nope_dt, int64_t n_s0, int64_t n_s1, const void* k_rope, int rope_dt,
                         int64_t r_s0, int64_t num_tokens, int num_heads, int nope_dim,
                         int rope_dim) {
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < num_tokens; ++t)
    for (int h = 0; h < num_heads; ++h) {
      for (int d = 0; d < nope_dim; ++d)
        orc_encode(k_nope, t * n_s0 + h * n_s1 + d, nope_dt, k, t * k_s0 + h * k_s1 + d, k_dt,
                   NULL);
      for (int d = 0; d < rope_dim; ++d)
        orc_encode(k_rope, t * r_s0 + d, rope_dt, k, t * k_s0 + h * k_s1 + nope_dim + d, k_dt,
                   NULL);
    }
}

/* --------------------------------------------- paged decode attention (a4-a7) */

/* Element index of cache position p of sequence b, kv head g, dim 0; -1 when
 * the position's block-table entry is outside the pool (R7). */
static int64_t orc_gather_row(const int32_t* block_tables, int64_t b, int W, int64_t p,
                              int block_size, int64_t block_stride, int num_kv_heads,
                              int head_size, int g, int64_t num_blocks) {
  int32_t phys = block_tables[b * (int64_t)W + p / block_size];
  if (phys < 0 || phys >= num_blocks) return -1;
  int64_t off = p % block_size;
  return (int64_t)phys * block_stride + (off * num_kv_heads + g) * (int64_t)head_size;
}

/* out[b, h, :] (fp64, unrounded) = softmax_p(scale * q[b,h,:].K^[p,g,:]) . V^[p,g,:]
 * over p < ctx_b, g = h / (num_q_heads / num_kv_heads), K^ = K * k_scale,
 * V^ = V * v_scale (a NULL scale means 1). The softmax is computed in two
 * passes: max, then exp(s - max) and its sum. q is [B, H_Q, D] with sequence
 * stride q_seq_stride. */
void orc_decode_attention(double* out, const void* q, int q_dt, int64_t q_seq_stride,
                          const void* key_cache, const void* value_cache, int cache_dt,
                          int64_t num_blocks, int block_size, int64_t block_stride,
                          const int32_t* block_tables, int W, const int32_t* context_lens,
                          int num_seqs, int num_q_heads, int num_kv_heads, int head_size,
                          double softmax_scale, const float* k_scale, const float* v_scale) {
  int group = num_q_heads / num_kv_heads;
  double ks = k_scale ? (double)*k_scale : 1.0;
  double vs = v_scale ? (double)*v_scale : 1.0;
#pragma omp parallel for collapse(2) schedule(dynamic)
  for (int b = 0; b < num_seqs; ++b)
    for (int h = 0; h < num_q_heads; ++h) {
      int g = h / group;
      int64_t ctx = context_lens[b];
      if (ctx < 0) ctx = 0;
      if (ctx > (int64_t)W * block_size) ctx = (int64_t)W * block_size;
      double* o = out + ((int64_t)b * num_q_heads + h) * head_size;
      for (int d = 0; d < head_size; ++d) o[d] = 0.0;
      if (ctx == 0) continue;
      const int64_t qb = (int64_t)b * q_seq_stride + (int64_t)h * head_size;
      /* pass 1: scores and their maximum */
      double m = -INFINITY;
      double* s = (double*)malloc(sizeof(double) * (size_t)ctx);
      for (int64_t p = 0; p < ctx; ++p) {
        int64_t row = orc_gather_row(block_tables, b, W, p, block_size, block_stride,
                                     num_kv_heads, head_size, g, num_blocks);
        if (row < 0) {
          s[p] = -INFINITY;
          continue;
        }
        double dot = 0.0;
        for (int d = 0; d < head_size; ++d)
          dot += orc_load_f64(q, qb + d, q_dt) * (orc_load_f64(key_cache, row + d, cache_dt) * ks);
        s[p] = softmax_scale * dot;
        if (s[p] > m) m = s[p];
      }
      if (m == -INFINITY) { /* no position took part */
        free(s);
        continue;
      }
      /* pass 2: weights, their sum, and the weighted sum of V^ */
      double l = 0.0;
      for (int64_t p = 0; p < ctx; ++p) {
        if (s[p] == -INFINITY) continue;
        double w = exp(s[p] - m);
        l += w;
        int64_t row = orc_gather_row(block_tables, b, W, p, block_size, block_stride,
                                     num_kv_heads, head_size, g, num_blocks);
        for (int d = 0; d < head_size; ++d)
          o[d] += w * (orc_load_f64(value_cache, row + d, cache_dt) * vs);
      }
      for (int d = 0; d < head_size; ++d) o[d] /= l;
      free(s);
    }
}

/* MLA decode attention over a latent paged cache (R13), with K and V written
 * out as the page defines them: for each cached position the latent row c is
 * multiplied by W_UK and W_UV (k_raw = c W_UK, v_raw = c W_UV, then split per
 * head), and each head runs R7's two-pass softmax attention with the RoPE term
 * added to its scores. All inputs are bf16 bit patterns; out is fp64
 * [num_seqs, num_heads, v_dim], unrounded. latent_cache is [num_blocks,
 * block_size, latent_dim + rope_dim] with block stride block_stride. */
void orc_mla_decode(double* out, const uint16_t* q_nope, int64_t q_nope_stride, const uint16_t* q_rope,
                    int64_t q_rope_stride, const uint16_t* w_uk, const uint16_t* w_uv,
                    const uint16_t* latent_cache, int64_t num_blocks, int block_size, int64_t block_stride,
                    const int32_t* block_tables, int W, const int32_t* context_lens, int num_seqs,
                    int num_heads, int qk_dim, int rope_dim, int latent_dim, int v_dim,
                    double softmax_scale) {
  const int row_len = latent_dim + rope_dim;
  const int64_t kw = (int64_t)num_heads * qk_dim, vw = (int64_t)num_heads * v_dim;
  for (int b = 0; b < num_seqs; ++b) {
    int64_t ctx = context_lens[b];
    if (ctx < 0) ctx = 0;
    if (ctx > (int64_t)W * block_size) ctx = (int64_t)W * block_size;
    for (int64_t i = 0; i < vw; ++i) out[(int64_t)b * vw + i] = 0.0;
    if (ctx == 0) continue;
    /* the up-projected keys and values of every position (k_raw, v_raw) */
    double* K = (double*)malloc(sizeof(double) * (size_t)(ctx * kw));
    double* V = (double*)malloc(sizeof(double) * (size_t)(ctx * vw));
    int64_t* row = (int64_t*)malloc(sizeof(int64_t) * (size_t)ctx);
#pragma omp parallel for schedule(dynamic)
    for (int64_t p = 0; p < ctx; ++p) {
      int32_t phys = block_tables[(int64_t)b * W + p / block_size];
      if (phys < 0 || phys >= num_blocks) {
        row[p] = -1;
        continue;
      }
      row[p] = (int64_t)phys * block_stride + (p % block_size) * (int64_t)row_len;
      for (int64_t j = 0; j < kw; ++j) {
        double acc = 0.0;
        for (int c = 0; c < latent_dim; ++c)
          acc += orc_load_f64(latent_cache, row[p] + c, ORC_BF16) * orc_load_f64(w_uk, (int64_t)c * kw + j, ORC_BF16);
        K[p * kw + j] = acc;
      }
      for (int64_t j = 0; j < vw; ++j) {
        double acc = 0.0;
        for (int c = 0; c < latent_dim; ++c)
          acc += orc_load_f64(latent_cache, row[p] + c, ORC_BF16) * orc_load_f64(w_uv, (int64_t)c * vw + j, ORC_BF16);
        V[p * vw + j] = acc;
      }
    }
#pragma omp parallel for schedule(dynamic)
    for (int h = 0; h < num_heads; ++h) {
      double* o = out + (int64_t)b * vw + (int64_t)h * v_dim;
      const int64_t qn = (int64_t)b * q_nope_stride + (int64_t)h * qk_dim;
      const int64_t qr = (int64_t)b * q_rope_stride + (int64_t)h * rope_dim;
      double* s = (double*)malloc(sizeof(double) * (size_t)ctx);
      double m = -INFINITY;
      for (int64_t p = 0; p < ctx; ++p) {
        if (row[p] < 0) {
          s[p] = -INFINITY;
          continue;
        }
        double dot = 0.0;
        for (int j = 0; j < qk_dim; ++j) dot += orc_load_f64(q_nope, qn + j, ORC_BF16) * K[p * kw + (int64_t)h * qk_dim + j];
        for (int r = 0; r < rope_dim; ++r)
          dot += orc_load_f64(q_rope, qr + r, ORC_BF16) * orc_load_f64(latent_cache, row[p] + latent_dim + r, ORC_BF16);
        s[p] = softmax_scale * dot;
        if (s[p] > m) m = s[p];
      }
      if (m != -INFINITY) {
        double l = 0.0;
        for (int64_t p = 0; p < ctx; ++p) {
          if (s[p] == -INFINITY) continue;
          double w = exp(s[p] - m);
          l += w;
          for (int j = 0; j < v_dim; ++j) o[j] += w * V[p * vw + (int64_t)h * v_dim + j];
        }
        for (int j = 0; j < v_dim; ++j) o[j] /= l;
      }
      free(s);
    }
    free(K);
    free(V);
    free(row);
  }
}

/* Chunked-prefill paged attention (R10): for sequence b with n_b queries and
 * clamped context length L, query i (packed row t = cu_seqlens_q[b] + i) sits
 * at position p = L - n_b + i and
 *   out[t, h, :] = softmax_{j <= p}(scale * q[t,h,:].K^[j,g,:]) . V^[j,g,:]
 * with g = h / (num_q_heads / num_kv_heads); zeros when p < 0 or when no
 * position takes part. q is [T, H_Q, D] with token stride q_token_stride;
 * out is [T, H_Q, D] fp64. Rows of cu_seqlens_q are non-decreasing. */
void orc_prefill_attention(double* out, const void* q, int q_dt, int64_t q_token_stride,
                           const int32_t* cu_seqlens_q, int num_seqs,
                           const void* key_cache, const void* value_cache, int cache_dt,
                           int64_t num_blocks, int block_size, int64_t block_stride,
                           const int32_t* block_tables, int W, const int32_t* context_lens,
                           int num_q_heads, int num_kv_heads, int head_size,
                           double softmax_scale, const float* k_scale, const float* v_scale) {
  int group = num_q_heads / num_kv_heads;
  double ks = k_scale ? (double)*k_scale : 1.0;
  double vs = v_scale ? (double)*v_scale : 1.0;
  for (int b = 0; b < num_seqs; ++b) {
    int64_t t0 = cu_seqlens_q[b], n = (int64_t)cu_seqlens_q[b + 1] - t0;
    int64_t L = context_lens[b];
    if (L < 0) L = 0;
    if (L > (int64_t)W * block_size) L = (int64_t)W * block_size;
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int64_t i = 0; i < n; ++i)
      for (int h = 0; h < num_q_heads; ++h) {
        int g = h / group;
        int64_t p = L - n + i; /* this query's position */
        double* o = out + ((t0 + i) * num_q_heads + h) * (int64_t)head_size;
        for (int d = 0; d < head_size; ++d) o[d] = 0.0;
        if (p < 0) continue;
        const int64_t qb = (t0 + i) * q_token_stride + (int64_t)h * head_size;
        /* pass 1: scores of positions 0..p and their maximum */
        double m = -INFINITY;
        double* s = (double*)malloc(sizeof(double) * (size_t)(p + 1));
        for (int64_t j = 0; j <= p; ++j) {
          int64_t row = orc_gather_row(block_tables, b, W, j, block_size, block_stride,
                                       num_kv_heads, head_size, g, num_blocks);
          if (row < 0) {
            s[j] = -INFINITY;
            continue;
          }
          double dot = 0.0;
          for (int d = 0; d < head_size; ++d)
            dot += orc_load_f64(q, qb + d, q_dt) * (orc_load_f64(key_cache, row + d, cache_dt) * ks);
          s[j] = softmax_scale * dot;
          if (s[j] > m) m = s[j];
        }
        if (m == -INFINITY) {
          free(s);
          continue;
        }
        /* pass 2: weights, their sum, and the weighted sum of V^ */
        double l = 0.0;
        for (int64_t j = 0; j <= p; ++j) {
          if (s[j] == -INFINITY) continue;
          double w = exp(s[j] - m);
          l += w;
          int64_t row = orc_gather_row(block_tables, b, W, j, block_size, block_stride,
                                       num_kv_heads, head_size, g, num_blocks);
          for (int d = 0; d < head_size; ++d)
            o[d] += w * (orc_load_f64(value_cache, row + d, cache_dt) * vs);
        }
        for (int d = 0; d < head_size; ++d) o[d] /= l;
        free(s);
      }
  }
}
