// MLA decode attention over a latent paged cache, with absorbed weights.
//
// The "PagedAttention principle" page (MLA paragraphs of the GQA/MLA shapes
// section) has MLA cache one latent row per token, c = x W_DKV, and recover
// head h's key and value as (c W_UK) and (c W_UV) split per head; the q.k
// dimension also carries a RoPE part that v lacks. Here each cached row is c
// (512 values) followed by a RoPE key part k_r (64 values or none) shared by
// all heads, the form the MLA-style concat of a shared k_rope writes.
//
// Writing K and V out per position would cost latent_dim * H * (qk + v) MACs
// per cached token. Instead the products are re-associated (the same sums):
//   q.k_h = (W_UK,h q_h) . c          -- absorb W_UK into the query once
//   o_h   = (sum_p P_p c_p) W_UV,h    -- attend over the latent, then W_UV
// so the hot loop is multi-query attention of all 16 heads over the latent
// rows themselves, and the cache is read once.
//
// Three kernels:
//  * absorb: q~ = scale*log2(e) * [W_UK,h^T q_nope,h ; q_rope,h], a small
//    matrix-core GEMM per head accumulated in fp32, then split into bf16
//    hi + lo (x - hi rounded again), so that the products below keep ~16 more
//    bits than a bf16 q~ would.
//  * split: one workgroup per live (sequence, 256-position piece) -- found by
//    a scan of the sequences' piece counts, so the grid holds no idle runs --,
//    4 waves, tiles of 32 positions staged in LDS (three workgroups per CU).
//    Scores S^T = C q~^T on v_mfma_f32_16x16x32_bf16 (hi and lo; each wave
//    takes a quarter of the 576-dim contraction with its q~ operands held in
//    registers, and the partial sums meet in LDS); online softmax in the log2
//    domain; O += P C with P split into hi + lo as well and C's operand from
//    LDS by transposing reads, each wave owning 128 of the 512 latent dims.
//    Writes the unnormalised O, its running max and sum per head.
//  * merge: combines the pieces of a sequence and applies W_UV per head.
#include <math.h>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

typedef __bf16 bf16x8 __attribute__((__vector_size__(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kDC = 512;        // latent (kv_lora_rank) dims
constexpr int kHeads = 16;      // query heads (the MFMA's 16-wide operand)
constexpr int kTile = 32;       // positions per tile
constexpr int kSplit = 256;     // positions per workgroup piece
constexpr int kWaves = 4;
constexpr int kPad = 16;        // LDS row padding (bytes)

template <int DR>
struct MlaGeo {
  static constexpr int ROW = kDC + DR;           // values per cached row
  static constexpr int RB = ROW * 2;             // bytes per cached row
  static constexpr int RS = RB + kPad;           // LDS row stride
  static constexpr int KSTEPS = ROW / 32;        // MFMA steps over the row
  static constexpr int HALF = KSTEPS / 2;        // steps per wave pair
  static constexpr int LOADS = RB / 128;          // 16-byte loads per thread and tile:
                                                  // 8 threads per row, 32 rows
  static_assert(RB % 128 == 0 && kTile * 8 == 64 * kWaves, "row-per-8-threads tile loads");
};

struct MlaArgs {
  void* out;
  const void* q_nope;
  const void* q_rope;
  const void* w_uk;
  const void* w_uv;
  const void* cache;
  const int32_t* bt;
  const int32_t* ctx_lens;
  uint16_t* q_hi;   // [B, 16, ROW]
  uint16_t* q_lo;
  float* ws_m;      // [B, S, 16]
  float* ws_l;
  float* ws_o;      // [B, S, 16, 512]
  int64_t out_seq_stride, qn_seq_stride, qr_seq_stride;
  int64_t block_stride, num_blocks;
  int32_t block_size, W, num_seqs, qk, dr, dv, splits;
  int32_t out_f32;
  float scale_log2;
};

__device__ __forceinline__ int clamp_ctx(const MlaArgs& a, int b) {
  int c = a.ctx_lens[b];
  const int64_t cap = (int64_t)a.W * a.block_size;
  c = c < 0 ? 0 : c;
  return (int64_t)c > cap ? (int)cap : c;
}

__device__ __forceinline__ void split_hi_lo(float x, uint16_t& hi, uint16_t& lo) {
  hi = (uint16_t)f32_to_bf16(x);
  lo = (uint16_t)f32_to_bf16(x - __uint_as_float((uint32_t)hi << 16));
}

// ---------------------------------------------------------------- absorb
// q~^T [512 c x B] = W_UK,h [512 x qk] q_h^T [qk x B] per head on the matrix
// cores (bf16 x bf16 products are exact in fp32, sums in fp32). grid (16
// heads, 8 blocks of 64 latent dims, ceil(B / 16)); wave w computes latent
// dims 64 cb + 16 w .. +15 for 16 sequences. The A operand is 16 bytes of a
// W_UK row (dims 8 (l/16) .. of row l%16), the B operand 16 bytes of a q row.
__global__ __launch_bounds__(256) void mla_absorb_kernel(MlaArgs a, int row) {
  const int h = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, lg = lane >> 4;
  const int c0 = 64 * blockIdx.y + 16 * wave, b0 = 16 * blockIdx.z;
  const int bq = b0 + li;                         // this lane's sequence in the B operand
  const bool bq_ok = bq < a.num_seqs;
  const uint16_t* wr = static_cast<const uint16_t*>(a.w_uk) + (int64_t)(c0 + li) * kHeads * a.qk + (int64_t)h * a.qk;
  const uint16_t* qr = static_cast<const uint16_t*>(a.q_nope) + (int64_t)(bq_ok ? bq : 0) * a.qn_seq_stride +
                       (int64_t)h * a.qk;
  const u32x4 z = {0u, 0u, 0u, 0u};
  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  constexpr int kMaxSteps = 256 / 32;             // qk <= 256: every load issued before the products
  u32x4 wa[kMaxSteps], qb[kMaxSteps];
#pragma unroll
  for (int s = 0; s < kMaxSteps; ++s) {
    const int j = 32 * s + 8 * lg;
    const int jc = j < a.qk ? j : 0;              // qk is a multiple of 8, not always of 32
    wa[s] = *reinterpret_cast<const u32x4*>(wr + jc);
    qb[s] = *reinterpret_cast<const u32x4*>(qr + jc);
  }
#pragma unroll
  for (int s = 0; s < kMaxSteps; ++s) {
    const bool in = 32 * s + 8 * lg < a.qk;
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, in ? wa[s] : z),
                                                  __builtin_bit_cast(bf16x8, (in && bq_ok) ? qb[s] : z), acc, 0,
                                                  0, 0);
  }
  // lane l holds latent dims c0 + 4 (l/16) + r of sequence b0 + l%16
  if (bq_ok) {  // four consecutive dims: one 8-byte store each for hi and lo
    const int64_t base = ((int64_t)bq * kHeads + h) * row + c0 + 4 * lg;
    uint16_t hi[4], lo[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) split_hi_lo(acc[r] * a.scale_log2, hi[r], lo[r]);
    *reinterpret_cast<u32x2*>(a.q_hi + base) = u32x2{hi[0] | ((uint32_t)hi[1] << 16), hi[2] | ((uint32_t)hi[3] << 16)};
    *reinterpret_cast<u32x2*>(a.q_lo + base) = u32x2{lo[0] | ((uint32_t)lo[1] << 16), lo[2] | ((uint32_t)lo[3] << 16)};
  }
  if (blockIdx.y == 0) {  // the RoPE part: scaled and split as it is (16 * dr <= 1024 values)
    float x[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = tid + 256 * u;
      const int bb = b0 + i / (a.dr > 0 ? a.dr : 1), r = i % (a.dr > 0 ? a.dr : 1);
      const bool ok = i < 16 * a.dr && bb < a.num_seqs;
      x[u] = ok ? load1<Ty::BF16>(a.q_rope, (int64_t)bb * a.qr_seq_stride + (int64_t)h * a.dr + r) : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = tid + 256 * u;
      const int bb = b0 + i / (a.dr > 0 ? a.dr : 1), r = i % (a.dr > 0 ? a.dr : 1);
      if (!(i < 16 * a.dr && bb < a.num_seqs)) continue;
      uint16_t hi, lo;
      split_hi_lo(x[u] * a.scale_log2, hi, lo);
      const int64_t base = ((int64_t)bb * kHeads + h) * row + kDC;
      a.q_hi[base + r] = hi;
      a.q_lo[base + r] = lo;
    }
  }
}

// ---------------------------------------------------------------- split
// A workgroup barrier for LDS traffic only: the next tile's global loads stay
// in flight across it (a full __syncthreads would wait for them too).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

__device__ __forceinline__ float bcast_lane(float x, int src) {
  return __int_as_float(__builtin_amdgcn_ds_bpermute(src << 2, __float_as_int(x)));
}

__device__ __forceinline__ int pieces_of(const MlaArgs& a, int b) { return (clamp_ctx(a, b) + kSplit - 1) / kSplit; }

// Workgroup L serves the L-th live piece in (sequence, piece) order: wave 0
// scans the sequences' piece counts (each lane a run of sequences) and finds
// it. Returns false when L is past the last piece.
__device__ bool find_piece(const MlaArgs& a, int L, int lane, int& b_out, int& s_out) {
  const int per = (a.num_seqs + 63) / 64;
  const int lo = min(a.num_seqs, lane * per), hi = min(a.num_seqs, lo + per);
  int mine = 0;
  for (int b = lo; b < hi; ++b) mine += pieces_of(a, b);
  int incl = mine;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, (unsigned)o, 64);
    if (lane >= o) incl += y;
  }
  const uint64_t past = __builtin_amdgcn_ballot_w64(incl <= L);  // lanes wholly before L
  const int owner = __builtin_popcountll(past);
  if (owner >= 64) return false;
  int found_b = -1, found_s = 0;
  if (lane == owner) {
    int run = incl - mine;
    for (int b = lo; b < hi; ++b) {
      const int n = pieces_of(a, b);
      if (L < run + n) {
        found_b = b;
        found_s = L - run;
        break;
      }
      run += n;
    }
  }
  b_out = __shfl(found_b, owner, 64);
  s_out = __shfl(found_s, owner, 64);
  return b_out >= 0;
}

template <int DR>
__global__ __launch_bounds__(64 * kWaves) __attribute__((amdgpu_waves_per_eu(3, 3))) void mla_split_kernel(MlaArgs a) {
  using Gm = MlaGeo<DR>;
  constexpr int ROW = Gm::ROW, RS = Gm::RS, LOADS = Gm::LOADS;
  constexpr int KSTEPS = ROW / 32, QMAX = (KSTEPS + kWaves - 1) / kWaves;
  const int tid = threadIdx.x, lane = tid & 63, li = lane & 15, lg = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  __shared__ __attribute__((aligned(16))) char tile_lds[kTile * RS];
  __shared__ f32x4 sx[kWaves][2][64];
  __shared__ int64_t rowoff[kSplit];  // byte offset of each position's row; -1: none
  __shared__ int which[2];

  if (wave == 0) {
    int b, s;
    const bool ok = find_piece(a, (int)blockIdx.x, lane, b, s);
    if (lane == 0) {
      which[0] = ok ? b : -1;
      which[1] = s;
    }
  }
  __syncthreads();
  const int b = which[0], sp = which[1];
  if (b < 0) return;  // uniform: past the last live piece
  const int ctx = clamp_ctx(a, b);
  const int p0 = sp * kSplit;
  const int p1 = min(ctx, p0 + kSplit);
  const int ntiles = (p1 - p0 + kTile - 1) / kTile;
  const int64_t piece = (int64_t)b * a.splits + sp;
  if (a.num_blocks == 0) {  // uniform: an empty pool -- no position takes part
    if (tid < kHeads) {
      a.ws_m[piece * kHeads + tid] = -INFINITY;
      a.ws_l[piece * kHeads + tid] = 0.0f;
    }
    return;
  }

  // where each position's row lives (the only division by block_size)
  const int bs = a.block_size;
  for (int i = tid; i < kSplit; i += 64 * kWaves) {
    const int pos = p0 + i;
    int64_t off = -1;
    if (pos < p1) {
      const int e = a.bt[(int64_t)b * a.W + pos / bs];
      if (e >= 0 && (int64_t)e < a.num_blocks) off = ((int64_t)e * a.block_stride + (int64_t)(pos % bs) * ROW) * 2;
    }
    rowoff[i] = off;
  }

  // This wave's share of the score contraction: steps s0 .. s0 + nst - 1 of
  // KSTEPS (32 dims each); its q~ operands (head li, dims 32 s + 8 lg ..) stay
  // in registers for the whole piece.
  const int base_n = KSTEPS / kWaves, rem = KSTEPS % kWaves;
  const int nst = base_n + (wave < rem ? 1 : 0);
  const int s0 = wave * base_n + min(wave, rem);
  bf16x8 qh[QMAX], ql[QMAX];
  {
    const uint16_t* qhb = a.q_hi + ((int64_t)b * kHeads + li) * ROW;
    const uint16_t* qlb = a.q_lo + ((int64_t)b * kHeads + li) * ROW;
#pragma unroll
    for (int i = 0; i < QMAX; ++i) {
      const int k0 = 32 * (s0 + (i < nst ? i : 0)) + 8 * lg;
      qh[i] = *reinterpret_cast<const bf16x8*>(qhb + k0);
      ql[i] = *reinterpret_cast<const bf16x8*>(qlb + k0);
    }
  }
  __syncthreads();

  // Tile loads: thread t loads row t / 8 of the tile, 16 bytes at columns
  // 16 (t % 8) + 128 i -- one row offset per thread and tile, immediate
  // offsets after it. Every thread loads (a row past the piece or with a bad
  // table entry reads the pool's first row instead) and such rows are zeroed
  // when stored to LDS: a load under a divergent branch would make the
  // compiler wait for it before the other branch writes the register. Their
  // scores are -inf, and 0 * 0 keeps P V finite.
  const char* cache = static_cast<const char*>(a.cache) + 16 * (tid & 7);
  const int lrow = tid >> 3;
  char* const lds_dst = tile_lds + lrow * RS + 16 * (tid & 7);
  u32x4 pre[LOADS];
  bool row_ok = false;
  auto load_tile = [&](int t) {
    const int64_t ro = rowoff[kTile * t + lrow];
    row_ok = ro >= 0;
    const char* src = cache + (row_ok ? ro : 0);
#pragma unroll
    for (int i = 0; i < LOADS; ++i) pre[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + 128 * i));
  };
  auto store_tile = [&]() {
    const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < LOADS; ++i) *reinterpret_cast<u32x4*>(lds_dst + 128 * i) = row_ok ? pre[i] : z;
  };

  const int dim0 = 128 * wave;  // this wave's 128 latent dims of O
  float m_run = -INFINITY, l_run = 0.0f;
  f32x4 acc[8];
#pragma unroll
  for (int cb = 0; cb < 8; ++cb) acc[cb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  load_tile(0);
  for (int t = 0; t < ntiles; ++t) {
    lds_barrier();  // every wave is done reading the previous tile
    store_tile();
    lds_barrier();
    if (t + 1 < ntiles) load_tile(t + 1);

    // partial S^T of both 16-position blocks over this wave's contraction
    // steps: rows = positions 16 pb + 4 lg + r, column = head li
    f32x4 spb[2] = {{0.0f, 0.0f, 0.0f, 0.0f}, {0.0f, 0.0f, 0.0f, 0.0f}};
#pragma unroll
    for (int i = 0; i < QMAX; ++i) {
      if (i < nst) {
        const int k0 = 32 * (s0 + i) + 8 * lg;
#pragma unroll
        for (int pb = 0; pb < 2; ++pb) {
          const bf16x8 cop = *reinterpret_cast<const bf16x8*>(tile_lds + (16 * pb + li) * RS + 2 * k0);
          spb[pb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cop, qh[i], spb[pb], 0, 0, 0);
          spb[pb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cop, ql[i], spb[pb], 0, 0, 0);
        }
      }
    }
    sx[wave][0][lane] = spb[0];
    sx[wave][1][lane] = spb[1];
    lds_barrier();
    // full scores of head li at positions 4 lg + r (block 0) and 16 + 4 lg + r
    // (block 1), summed over the waves in one fixed order
    float sc[8];
#pragma unroll
    for (int pb = 0; pb < 2; ++pb) {
      f32x4 s4 = sx[0][pb][lane];
#pragma unroll
      for (int w = 1; w < kWaves; ++w) s4 += sx[w][pb][lane];
#pragma unroll
      for (int r = 0; r < 4; ++r) sc[4 * pb + r] = s4[r];
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const bool ok = rowoff[kTile * t + 16 * (k >> 2) + 4 * lg + (k & 3)] >= 0;  // -1 past p1 too
      sc[k] = ok ? sc[k] : -INFINITY;
    }
    float mx = sc[0];
#pragma unroll
    for (int k = 1; k < 8; ++k) mx = fmaxf(mx, sc[k]);
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float mn = fmaxf(m_run, mx);
    const float mu = (mn == -INFINITY) ? 0.0f : mn;
    const float alpha = __builtin_amdgcn_exp2f(m_run - mu);
    float pr[8];
    float ps = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      pr[k] = __builtin_amdgcn_exp2f(sc[k] - mu);
      ps += pr[k];
    }
    l_run = l_run * alpha + ps;
    m_run = mn;
    // rescale O rows (heads 4 lg + r) by their heads' alpha
    if (__builtin_amdgcn_ballot_w64(alpha != 1.0f) != 0) {
      float al[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) al[r] = bcast_lane(alpha, 4 * lg + r);
#pragma unroll
      for (int cb = 0; cb < 8; ++cb)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[cb][r] *= al[r];
    }
    // P as the A operand (row = head li, contraction = this lane's 8 positions)
    // in hi + lo halves
    uint32_t phw[4], plw[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      phw[e] = f32x2_to_bf16x2(pr[2 * e], pr[2 * e + 1]);
      plw[e] = f32x2_to_bf16x2(pr[2 * e] - bf16_lo(phw[e]), pr[2 * e + 1] - bf16_hi(phw[e]));
    }
    const bf16x8 ph = __builtin_bit_cast(bf16x8, u32x4{phw[0], phw[1], phw[2], phw[3]});
    const bf16x8 pl = __builtin_bit_cast(bf16x8, u32x4{plw[0], plw[1], plw[2], plw[3]});
    // O += P C over this wave's dims: transposing reads give lane (m, g)
    // C[4g + j][d0 + m] (low half) and C[16 + 4g + j][d0 + m] (high half)
    const int trow = 4 * lg + (li >> 2);
#pragma unroll
    for (int cb = 0; cb < 8; ++cb) {
      const int col = 2 * (dim0 + 16 * cb + 4 * (li & 3));
      const i16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4*)(tile_lds + trow * RS + col));
      const i16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4*)(tile_lds + (trow + 16) * RS + col));
      const bf16x8 vop = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
      acc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ph, vop, acc[cb], 0, 0, 0);
      acc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pl, vop, acc[cb], 0, 0, 0);
    }
  }

  // the four lane groups saw different positions under one running max
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);
  if (wave == 0 && lane < kHeads) {
    a.ws_m[piece * kHeads + lane] = m_run;
    a.ws_l[piece * kHeads + lane] = l_run;
  }
  float* o = a.ws_o + piece * kHeads * kDC;
#pragma unroll
  for (int cb = 0; cb < 8; ++cb)
#pragma unroll
    for (int r = 0; r < 4; ++r) o[(4 * lg + r) * kDC + dim0 + 16 * cb + li] = acc[cb][r];
}

// ---------------------------------------------------------------- merge
// grid (16 heads, ceil(B / 4)): the pieces of each of 4 sequences combined
// into o~ [512] (normalised), then o = o~ W_UV,h.
__global__ __launch_bounds__(256) void mla_merge_kernel(MlaArgs a) {
  const int h = blockIdx.x, b0 = 4 * blockIdx.y, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  __shared__ float ot[4][kDC];
  __shared__ float mM[4], mInv[4];
  __shared__ int nps[4];
  __shared__ float red[256 * 32];
  const int nb = min(4, a.num_seqs - b0);
  {  // wave bb: pieces, global max and 1 / sum of sequence b0 + bb
    const int bb = wave;
    int n = 0;
    float M = -INFINITY;
    if (bb < nb) {
      n = pieces_of(a, b0 + bb);
      for (int s = lane; s < n; s += 64) M = fmaxf(M, a.ws_m[((int64_t)(b0 + bb) * a.splits + s) * kHeads + h]);
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o, 64));
    }
    float L = 0.0f;
    if (M != -INFINITY) {
      for (int s = lane; s < n; s += 64) {
        const int64_t i = ((int64_t)(b0 + bb) * a.splits + s) * kHeads + h;
        L += __builtin_amdgcn_exp2f(a.ws_m[i] - M) * a.ws_l[i];
      }
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) L += __shfl_xor(L, o, 64);
    }
    if (lane == 0) {
      nps[bb] = (M == -INFINITY || !(L > 0.0f)) ? 0 : n;
      mM[bb] = M;
      mInv[bb] = L > 0.0f ? 1.0f / L : 0.0f;
    }
  }
  __syncthreads();
  {  // thread (bb, c8): o~[bb][8 c8 .. +8] as a weighted sum over the pieces
    const int bb = wave, c = 8 * lane;
    const int n = nps[bb];
    const float M = mM[bb];
    float v[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
    const int64_t p0 = (int64_t)(b0 + bb) * a.splits;
    constexpr int kBatch = 4;  // pieces whose loads are in flight together
    for (int s0 = 0; s0 < n; s0 += kBatch) {
      f32x4 x[kBatch][2];
      float w[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int s = s0 + u < n ? s0 + u : s0;
        const float* src = a.ws_o + ((p0 + s) * kHeads + h) * kDC + c;
        x[u][0] = *reinterpret_cast<const f32x4*>(src);
        x[u][1] = *reinterpret_cast<const f32x4*>(src + 4);
        w[u] = s0 + u < n ? __builtin_amdgcn_exp2f(a.ws_m[(p0 + s) * kHeads + h] - M) : 0.0f;
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[e] = fmaf(w[u], x[u][0][e], v[e]);
          v[4 + e] = fmaf(w[u], x[u][1][e], v[4 + e]);
        }
    }
    const float inv = mInv[bb];
#pragma unroll
    for (int e = 0; e < 8; ++e) ot[bb][c + e] = v[e] * inv;
  }
  __syncthreads();
  // o = o~ W_UV,h: thread (jg, cg) takes 8 output dims 8 jg.. and a slice of
  // the 512 latent dims; the slices meet in LDS.
  const int jgs = a.dv / 8, cgs = 256 / jgs;
  const int jg = tid % jgs, cg = tid / jgs;
  const int per = kDC / cgs;
  float acc[4][8];
#pragma unroll
  for (int bb = 0; bb < 4; ++bb)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[bb][e] = 0.0f;
  const int64_t wrow = (int64_t)kHeads * a.dv;
  const uint16_t* wbase = static_cast<const uint16_t*>(a.w_uv) + (int64_t)h * a.dv + 8 * jg;
#pragma unroll 8
  for (int c = cg * per; c < (cg + 1) * per; ++c) {
    const u32x4 w = *reinterpret_cast<const u32x4*>(wbase + c * wrow);
    float wf[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      wf[2 * e] = bf16_lo(w[e]);
      wf[2 * e + 1] = bf16_hi(w[e]);
    }
#pragma unroll
    for (int bb = 0; bb < 4; ++bb) {
      const float x = ot[bb][c];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[bb][e] = fmaf(x, wf[e], acc[bb][e]);
    }
  }
#pragma unroll
  for (int bb = 0; bb < 4; ++bb)
#pragma unroll
    for (int e = 0; e < 8; ++e) red[(cg * 4 + bb) * a.dv + 8 * jg + e] = acc[bb][e];
  __syncthreads();
  for (int i = tid; i < 4 * a.dv; i += 256) {
    const int bb = i / a.dv, j = i % a.dv;
    if (bb >= nb) continue;
    float v = 0.0f;
    for (int g = 0; g < cgs; ++g) v += red[(g * 4 + bb) * a.dv + j];
    const int64_t oi = (int64_t)(b0 + bb) * a.out_seq_stride + (int64_t)h * a.dv + j;
    if (a.out_f32)
      static_cast<float*>(a.out)[oi] = v;
    else
      static_cast<uint16_t*>(a.out)[oi] = (uint16_t)f32_to_bf16(v);
  }
}

struct MlaPlan {
  int row, splits;
  size_t off_qhi, off_qlo, off_m, off_l, off_o, bytes;
};

size_t round256(size_t x) { return (x + 255) / 256 * 256; }

MlaPlan mla_plan(int32_t num_seqs, int32_t rope_dim, int32_t max_blocks_per_seq, int32_t block_size) {
  MlaPlan p;
  p.row = kDC + rope_dim;
  p.splits = (int)(((int64_t)max_blocks_per_seq * block_size + kSplit - 1) / kSplit);
  const size_t B = (size_t)(num_seqs > 0 ? num_seqs : 1);
  size_t off = 0;
  p.off_qhi = off;
  off = round256(off + B * kHeads * p.row * 2);
  p.off_qlo = off;
  off = round256(off + B * kHeads * p.row * 2);
  p.off_m = off;
  off = round256(off + B * p.splits * kHeads * 4);
  p.off_l = off;
  off = round256(off + B * p.splits * kHeads * 4);
  p.off_o = off;
  off = round256(off + B * p.splits * kHeads * (size_t)kDC * 4);
  p.bytes = off;
  return p;
}

pa_status check_mla_shape(const char* fn, int32_t num_seqs, int32_t num_heads, int32_t qk_dim, int32_t rope_dim,
                          int32_t kv_lora_rank, int32_t v_dim, int32_t max_blocks_per_seq, int32_t block_size) {
  if (num_seqs < 0 || max_blocks_per_seq <= 0 || block_size <= 0) return fail(PA_EINVAL, "%s: bad sizes", fn);
  if ((int64_t)max_blocks_per_seq * block_size > INT32_MAX) return fail(PA_EINVAL, "%s: W * block_size overflows", fn);
  if (num_heads != kHeads) return fail(PA_EUNSUPPORTED, "%s: num_heads %d (supported: 16 per call)", fn, num_heads);
  if (kv_lora_rank != kDC) return fail(PA_EUNSUPPORTED, "%s: kv_lora_rank %d (supported: 512)", fn, kv_lora_rank);
  if (rope_dim != 0 && rope_dim != 64) return fail(PA_EUNSUPPORTED, "%s: rope_dim %d (supported: 0, 64)", fn, rope_dim);
  if (qk_dim <= 0 || qk_dim > 256 || qk_dim % 8 != 0)
    return fail(PA_EUNSUPPORTED, "%s: qk_nope_dim %d (supported: multiples of 8 up to 256)", fn, qk_dim);
  if (v_dim <= 0 || v_dim > 256 || v_dim % 8 != 0 || 256 % (v_dim / 8) != 0)
    return fail(PA_EUNSUPPORTED, "%s: v_dim %d (supported: 8 * a divisor of 256, up to 256)", fn, v_dim);
  return PA_OK;
}

}  // namespace
}  // namespace pa

extern "C" size_t pa_mla_decode_workspace_size(int32_t num_seqs, int32_t num_heads, int32_t qk_nope_dim,
                                               int32_t rope_dim, int32_t kv_lora_rank, int32_t v_dim,
                                               int32_t max_blocks_per_seq, int32_t block_size) {
  using namespace pa;
  clear_error();
  if (check_mla_shape("pa_mla_decode_workspace_size", num_seqs, num_heads, qk_nope_dim, rope_dim, kv_lora_rank, v_dim,
                      max_blocks_per_seq, block_size) != PA_OK)
    return 0;
  return mla_plan(num_seqs, rope_dim, max_blocks_per_seq, block_size).bytes;
}

extern "C" pa_status pa_mla_decode_attention(void* out, pa_dtype out_dtype, int64_t out_seq_stride, const void* q_nope,
                                             int64_t q_nope_seq_stride, const void* q_rope, int64_t q_rope_seq_stride,
                                             pa_dtype q_dtype, const void* w_uk, const void* w_uv, pa_dtype w_dtype,
                                             const void* latent_cache, pa_dtype cache_dtype, int64_t num_blocks,
                                             int32_t block_size, int64_t block_stride, const int32_t* block_tables,
                                             int32_t max_blocks_per_seq, const int32_t* context_lens,
                                             int32_t num_seqs, int32_t num_heads, int32_t qk_nope_dim,
                                             int32_t rope_dim, int32_t kv_lora_rank, int32_t v_dim,
                                             float softmax_scale, void* workspace, size_t workspace_bytes,
                                             void* stream) {
  using namespace pa;
  clear_error();
  const char* fn = "pa_mla_decode_attention";
  pa_status s = check_mla_shape(fn, num_seqs, num_heads, qk_nope_dim, rope_dim, kv_lora_rank, v_dim,
                                max_blocks_per_seq, block_size);
  if (s != PA_OK) return s;
  if (out_dtype != PA_BF16 && out_dtype != PA_F32) return fail(PA_EDTYPE, "%s: out dtype %s not supported", fn, dtype_name(out_dtype));
  if (q_dtype != PA_BF16 || w_dtype != PA_BF16 || cache_dtype != PA_BF16)
    return fail(PA_EDTYPE, "%s: q, weights and latent cache must be bf16", fn);
  if (!(softmax_scale == softmax_scale) || isinf(softmax_scale)) return fail(PA_EINVAL, "%s: softmax_scale is not finite", fn);
  const int row = kDC + rope_dim;
  if (num_blocks < 0) return fail(PA_EINVAL, "%s: num_blocks < 0", fn);
  if (block_stride < (int64_t)block_size * row) return fail(PA_EINVAL, "%s: block_stride below block_size * (512 + rope_dim)", fn);
  if (out_seq_stride < (int64_t)num_heads * v_dim) return fail(PA_EINVAL, "%s: out_seq_stride below H * v_dim", fn);
  if (q_nope_seq_stride < (int64_t)num_heads * qk_nope_dim) return fail(PA_EINVAL, "%s: q_nope_seq_stride below H * qk_nope_dim", fn);
  if (rope_dim > 0 && q_rope_seq_stride < (int64_t)num_heads * rope_dim)
    return fail(PA_EINVAL, "%s: q_rope_seq_stride below H * rope_dim", fn);
  if (num_seqs == 0) return PA_OK;
  if (!out || !q_nope || (rope_dim > 0 && !q_rope) || !w_uk || !w_uv || !latent_cache || !block_tables || !context_lens)
    return fail(PA_EINVAL, "%s: null pointer argument", fn);
  if (!aligned(latent_cache, 16) || (block_stride * 2) % 16 != 0)
    return fail(PA_EINVAL, "%s: latent cache must be 16-byte aligned per block", fn);
  if (!aligned(w_uk, 16) || !aligned(w_uv, 16)) return fail(PA_EINVAL, "%s: weights must be 16-byte aligned", fn);
  if (!aligned(q_nope, 16) || (q_nope_seq_stride * 2) % 16 != 0)
    return fail(PA_EINVAL, "%s: q_nope must be 16-byte aligned per sequence", fn);
  const MlaPlan p = mla_plan(num_seqs, rope_dim, max_blocks_per_seq, block_size);
  if (!workspace || workspace_bytes < p.bytes || !aligned(workspace, 256))
    return fail(PA_EWORKSPACE, "%s: workspace needs %zu bytes, 256-byte aligned (got %zu)", fn, p.bytes, workspace_bytes);

  MlaArgs a;
  a.out = out;
  a.q_nope = q_nope;
  a.q_rope = q_rope;
  a.w_uk = w_uk;
  a.w_uv = w_uv;
  a.cache = latent_cache;
  a.bt = block_tables;
  a.ctx_lens = context_lens;
  char* ws = static_cast<char*>(workspace);
  a.q_hi = reinterpret_cast<uint16_t*>(ws + p.off_qhi);
  a.q_lo = reinterpret_cast<uint16_t*>(ws + p.off_qlo);
  a.ws_m = reinterpret_cast<float*>(ws + p.off_m);
  a.ws_l = reinterpret_cast<float*>(ws + p.off_l);
  a.ws_o = reinterpret_cast<float*>(ws + p.off_o);
  a.out_seq_stride = out_seq_stride;
  a.qn_seq_stride = q_nope_seq_stride;
  a.qr_seq_stride = q_rope_seq_stride;
  a.block_stride = block_stride;
  a.num_blocks = num_blocks;
  a.block_size = block_size;
  a.W = max_blocks_per_seq;
  a.num_seqs = num_seqs;
  a.qk = qk_nope_dim;
  a.dr = rope_dim;
  a.dv = v_dim;
  a.splits = p.splits;
  a.out_f32 = out_dtype == PA_F32;
  a.scale_log2 = softmax_scale * 1.4426950408889634f;

  // one workgroup per live piece at most: sum over sequences of ceil(ctx / 256)
  // <= num_seqs * splits; workgroups past the last live piece exit at once.
  // Checked before the first launch, so a refusal leaves nothing enqueued.
  const int64_t items = (int64_t)num_seqs * p.splits;
  if (items > INT32_MAX / 2) return fail(PA_EINVAL, "%s: too many (sequence, piece) items", fn);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  mla_absorb_kernel<<<dim3(kHeads, kDC / 64, (unsigned)((num_seqs + 15) / 16)), 256, 0, st>>>(a, row);
  if (rope_dim == 64)
    mla_split_kernel<64><<<(unsigned)items, 64 * kWaves, 0, st>>>(a);
  else
    mla_split_kernel<0><<<(unsigned)items, 64 * kWaves, 0, st>>>(a);
  mla_merge_kernel<<<dim3(kHeads, (unsigned)((num_seqs + 3) / 4)), 256, 0, st>>>(a);
  return after_launch(fn);
}
