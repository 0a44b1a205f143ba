// pa_prefill_attention: chunked-prefill (variable-length, causal) attention of
// packed query tokens against their sequences' paged K/V.
//
// Operation (Qwen3-0.6B engine walkthrough page, section 2.4: prefill queries are
// packed token-major and delimited by cu_seqlens_q; section 2.6: the
// variable-length flash path of prefill; "PagedAttention principle" page,
// autoregressive dataflow: prefill attends causally over the prompt while its
// K/V are cached): sequence b owns query rows cu[b] .. cu[b+1]-1, the last
// n_b = cu[b+1]-cu[b] positions of its context of ctx_b positions; query i sits
// at position p = ctx_b - n_b + i and attends to cached positions 0..p through
// block_tables[b], K^ = K * k_scale, V^ = V * v_scale, q head h reading KV
// head h / G. A query with p < 0 gives zeros.
//
// gfx950 design (matrix cores for both products):
//  * Workgroup = 128 (token, head) rows of one KV head: 128/G consecutive
//    query tokens of one sequence times the G query heads of the group (row R
//    -> token R / G, head R % G), two waves per SIMD (256 registers per lane
//    each). For D = 64 and 128, 4 waves own 32 rows each as two 16-row MFMA
//    blocks that share every K/V operand read (two workgroups per compute
//    unit); for D = 256, 8 waves own one 16-row block each (one workgroup per
//    compute unit). Workgroups are ordered so that each XCD runs the query
//    tiles of the same (KV head, sequence) together and its L2 serves their K/V.
//  * Key tiles of 32 positions: the tile's K and V arrive as 1 KB
//    global_load_lds_dwordx4 wave loads dealt over the waves, straight into an
//    LDS ring in the order the operand reads consume them (every read is one
//    contiguous, conflict-free block), tiles ahead of the compute. The ring
//    comes first in LDS (64 KB for D = 128, 128 KB for D = 256).
//  * S^T = K Q^T on v_mfma_f32_16x16x32_bf16 (K rows from LDS as A, the
//    wave's q rows from registers as B): lane l gets the scores of keys
//    16*kb + 4*(l/16) + r for query row l%16, so each lane keeps one row's
//    online-softmax state and the row max needs two cross-row lane swaps.
//    The running max is raised lazily (only when a tile passes it by more
//    than 2^8 in probability), so the accumulator is rarely rescaled.
//  * O = P V: the lane's own probabilities of keys {4g..4g+3} and
//    {16+4g..16+4g+3} (g = l/16) are its A operand (a permutation of the
//    contraction index, applied to both operands), split into bf16 hi + lo
//    (two products) so that P enters at fp32 accuracy, and V's B operand comes
//    from LDS with ds_read_b64_tr_b16 (transposing reads: lane i of a 16-lane
//    group receives element (i mod 4) of the 8-byte chunk addressed by lane
//    4j + i/4, j = 0..3), which returns V[key][d] for four consecutive keys
//    of column d from the row-major tile.
//  * Only tiles that reach the diagonal, the context end or an invalid table
//    entry take the masking path (causal / out-of-range scores -> -inf and
//    the matching V operand elements -> 0, as unwritten slots may hold NaN).
// Scores are kept in the log2 domain (scale * log2(e) folded in).
#include <math.h>

#include <type_traits>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

typedef __bf16 bf16x8 __attribute__((__vector_size__(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// two waves per SIMD (256 registers each)
#define PA_PREFILL_OCCUPANCY __attribute__((amdgpu_waves_per_eu(2, 2)))

#ifndef PA_PREFILL_KEYS
#define PA_PREFILL_KEYS 32
#endif
#ifndef PA_PREFILL_PRIO_SM
#define PA_PREFILL_PRIO_SM 1
#endif
#ifndef PA_PREFILL_SCHED
#define PA_PREFILL_SCHED 0   // vector instructions scheduled after each score MFMA (0: no hint)
#endif
// Issue priority of a wave during a tile's softmax (0 for the products).
constexpr int kPrioSM = PA_PREFILL_PRIO_SM;
template <int P> __device__ __forceinline__ void set_prio() {
  static_assert(P >= 0 && P <= 3, "priority 0..3");
  __builtin_amdgcn_s_setprio(P);
}
// A workgroup holds kRows (token, head) rows: four waves of two 16-row MFMA
// blocks for D = 64 and 128; for D = 256, whose accumulators and q operands are
// twice as wide, eight waves of one block (one workgroup per compute unit: its
// K/V ring is 128 KB).
constexpr int kRows = 128;
template <int D>
struct Shape {
  static constexpr int RB = D == 256 ? 1 : 2;       // 16-row MFMA blocks per wave
  static constexpr int WAVES = kRows / (16 * RB);   // waves per workgroup
};
constexpr int kKeys = PA_PREFILL_KEYS;        // positions per key tile
constexpr int kKB = kKeys / 16;               // 16-key blocks per tile
constexpr int kBufs = 4;                      // LDS ring: tiles in P.V, in S, and two in flight
constexpr float kLazyMax = 8.0f;              // log2 headroom of the running max
static_assert(kKeys == 32 || kKeys == 64, "key tile");

// Workgroup barrier without a memory fence. __syncthreads() would also wait
// for every outstanding vector-memory operation, i.e. drain the K/V tiles in
// flight; LDS-DMA landing is waited for explicitly with wait_vmem, and every
// LDS read a wave issued has been consumed (by an MFMA) before it gets here.
__device__ __forceinline__ void barrier_no_vmem_wait() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

constexpr int kTab = 2048;  // block-table entries staged in LDS at a time
constexpr int kBins = 64;   // length classes of the dispatch order

struct PfArgs {
  void* out;
  const void* q;
  const void* kc;
  const void* vc;
  const int32_t* bt;
  const int32_t* ctx_lens;
  const int32_t* cu;
  const float* k_scale;
  const float* v_scale;
  int64_t out_tok_stride;  // elements
  int64_t q_tok_stride;    // elements
  int64_t block_stride;    // elements
  int64_t num_blocks;
  int64_t num_tokens;
  int32_t block_size;
  int32_t W;
  int32_t num_seqs;
  int32_t HQ;
  int32_t HKV;
  int32_t out_f32;
  int64_t tiles_ub;        // query tiles per KV head, upper bound (grid = HKV * tiles_ub, rounded up to 8)
  int32_t bin_w;           // key tiles per length class of the dispatch order
  float scale_log2;
};

// LDS tile geometry for head size D. Both tiles are stored in the order their
// readers consume them (the DMA lets every lane choose the 16-byte chunk it
// fetches), so each operand read is one contiguous, conflict-free block at
// base + lane * (bytes per lane) and needs no per-read address arithmetic:
//  * K: read (kb, s) -- rows 16kb + l%16, dims 32s + 8(l/16) .. +7 -- is the
//    1 KB at ((kb * KS + s) * 64 + l) * 16.
//  * V: transposing read (st, cb, half) -- lane (m, g) = (l%16, l/16) needs
//    row 32st + 16half + 4g + m/4, dims 16cb + 4(m%4) .. +3 -- is the 512 B at
//    ((st * CB + cb) * 2 + half) * 512 + 8 l; its 16-byte chunk q holds row
//    32st + 16half + 4(q/8) + (q%8)/2, dims 8(2cb + q%2) .. +7.
template <int D>
struct Geo {
  static constexpr int RB = D * 2;                 // bytes per cache row of one head
  static constexpr int TB = kKeys * RB;            // bytes per K (or V) tile
  static constexpr int KS = D / 32;                // MFMA steps over the head dim
  static constexpr int CB = D / 16;                // 16-column output blocks
  static constexpr int TI = TB / 1024;             // 1 KB wave loads per K (or V) tile
  static constexpr int IPW = 2 * TI / Shape<D>::WAVES;  // ... per wave and tile, K and V together
  static_assert(TB % 1024 == 0 && (2 * TI) % Shape<D>::WAVES == 0, "tile / wave split");
  static_assert(TI == (kKeys / 16) * KS && TI == (kKeys / 32) * CB, "reader-ordered layout");
  __device__ static int k_off(int kb, int s, int lane) { return ((kb * KS + s) * 64 + lane) * 16; }
  __device__ static int v_off(int st, int cb, int half, int lane) { return ((st * CB + cb) * 2 + half) * 512 + 8 * lane; }
};

// Max over the lanes l, l^16, l^32 and l^48 (the four lanes that hold one
// query row's scores): gfx950's cross-row lane swaps, no LDS round trip. Each
// swap exchanges one half of a copy of x with the other half of a second copy,
// so the two results hold, lane by lane, x at l and at its partner lane.
__device__ __forceinline__ float row_max4(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto a = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  const float m = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const uint32_t w = __float_as_uint(m);
  const auto b = __builtin_amdgcn_permlane16_swap(w, w, false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float bcast_lane(float x, int src) {
  return __int_as_float(__builtin_amdgcn_ds_bpermute(src << 2, __float_as_int(x)));
}

// fp8 caches: the tile's K and V arrive as e4m3fn into a staging ring in row
// order (row r of the tile at r * D bytes), and each lane converts the 16-byte
// chunks it fetched into the bf16 reader-ordered tiles (fp8 values are exact
// in bf16) before the tile's products read them.
template <int D>
struct Geo8 {
  static constexpr int TB = kKeys * D;         // bytes per fp8 K (or V) tile
  static constexpr int TI = TB / 1024;         // 1 KB wave loads per K (or V) tile
  static constexpr int IPW = 2 * TI / Shape<D>::WAVES;  // ... per wave and tile, K and V together
  static_assert(TB % 1024 == 0 && (2 * TI) % Shape<D>::WAVES == 0 && IPW >= 1, "fp8 tile / wave split");
};

template <int D, int G, bool kFp8>
__global__ __launch_bounds__(64 * Shape<D>::WAVES) PA_PREFILL_OCCUPANCY void prefill_mfma_kernel(PfArgs a) {
  using Gm = Geo<D>;
  using G8 = Geo8<D>;
  constexpr int kRB = Shape<D>::RB, kWaves = Shape<D>::WAVES, kRowsPerWave = 16 * kRB;
  constexpr int KS = Gm::KS, CB = Gm::CB;
  constexpr int QT = kRows / G;  // query tokens per workgroup
  const int tid = threadIdx.x, lane = tid & 63, li = lane & 15, lg = lane >> 4;
  const int wave = uniform(tid >> 6);
  // XCD-aware work order: the hardware deals workgroups to the 8 XCDs
  // round-robin (linear id mod 8), so workgroup L takes work item
  // (L mod 8) * per_xcd + L / 8. The workgroups one XCD runs at a time then hold
  // consecutive items -- the query tiles of the same (KV head, sequence) --
  // and that XCD's L2 serves their shared K/V tiles once.
  const int64_t per_xcd = ((int64_t)gridDim.x + 7) / 8;
  const int64_t item = (int64_t)(blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  const int g = (int)(item / a.tiles_ub);  // KV head
  const int64_t t = item % a.tiles_ub;     // query tile among this head's
  if (g >= a.HKV) return;  // uniform

  // One shared object with the K/V ring first (the LDS-DMA destinations).
  // bf16 caches: a kBufs-slot ring of bf16 tiles filled by the DMA. fp8
  // caches: a kBufs-slot ring of fp8 tiles filled by the DMA (first) and two bf16 tiles (the tile in P.V and the tile in S).
  constexpr int kDmaBufs = kBufs, kBfBufs = kFp8 ? 2 : kBufs;
  constexpr int kDmaTile = kFp8 ? G8::TB : Gm::TB;
  struct Smem {
    char dma[kDmaBufs][2][kDmaTile];  // [slot][K, V]: the DMA ring (bf16: the operand tiles)
    char bf[kFp8 ? kBfBufs : 1][2][kFp8 ? Gm::TB : 16];  // fp8: converted operand tiles
    int tab[kTab];              // validated table entries of blocks tab_base ..
    int64_t wave_tiles[kWaves];
    int found[2];               // sequence, tile index within it
    int bins[kBins];            // query tiles per length class
    int64_t pick[2];            // the class holding this workgroup's tile, its rank inside
  };
  static_assert(sizeof(Smem) <= 160 * 1024, "one compute unit's LDS");
  __shared__ __attribute__((aligned(16))) Smem sm;
  // operand tiles (bf16, reader-ordered) of key tile t
  auto ktile = [&](int t) -> const char* { return kFp8 ? sm.bf[t % kBfBufs][0] : sm.dma[t % kBufs][0]; };
  auto vtile = [&](int t) -> const char* { return kFp8 ? sm.bf[t % kBfBufs][1] : sm.dma[t % kBufs][1]; };
  auto& wave_tiles = sm.wave_tiles;
  auto& found = sm.found;
  auto& tab = sm.tab;

  // ---- which (sequence, query tile) this workgroup serves. Dispatch order:
  // sequences in descending length classes (class = key tiles of the
  // sequence's longest query tile / bin_w), by index within a class; each
  // sequence's query tiles together and last-first. The workgroups dispatched
  // first -- those resident from the start -- take the longest work, and the
  // tiles of one (KV head, sequence) stay consecutive, which keeps them on
  // one XCD. Tiles are found by thread-run scans over cu_seqlens.
  const int nthr = 64 * kWaves;
  const int per = (a.num_seqs + nthr - 1) / nthr;
  const int b_lo = min(a.num_seqs, tid * per), b_hi = min(a.num_seqs, b_lo + per);
  auto seq_rows = [&](int b) -> int {
    int lo = a.cu[b], hi = a.cu[b + 1];
    lo = lo < 0 ? 0 : (lo > a.num_tokens ? (int)a.num_tokens : lo);
    hi = hi < lo ? lo : (hi > a.num_tokens ? (int)a.num_tokens : hi);
    return hi - lo;
  };
  const int cap_all = a.W * a.block_size;
  auto seq_class = [&](int b) -> int {
    int L = a.ctx_lens[b];
    L = L < 0 ? 0 : (L > cap_all ? cap_all : L);
    return min(kBins - 1, ((L + kKeys - 1) / kKeys) / a.bin_w);
  };
  if (tid < kBins) sm.bins[tid] = 0;
  __syncthreads();
  for (int b = b_lo; b < b_hi; ++b) {
    const int nt = (seq_rows(b) + QT - 1) / QT;
    if (nt > 0) atomicAdd(&sm.bins[seq_class(b)], nt);
  }
  __syncthreads();
  if (wave == 0) {  // classes in descending order: lane c holds class kBins-1-c
    const int64_t cnt = sm.bins[kBins - 1 - lane];
    int64_t inc = cnt;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int64_t y = __shfl_up(inc, (unsigned)o, 64);
      if (lane >= o) inc += y;
    }
    const uint64_t below = __builtin_amdgcn_ballot_w64(inc <= t);  // classes wholly before t
    const int sel = __builtin_popcountll(below);
    if (lane == (sel < 64 ? sel : 0)) {
      sm.pick[0] = sel < 64 ? kBins - 1 - sel : -1;
      sm.pick[1] = t - (inc - cnt);
    }
  }
  __syncthreads();
  const int cls = (int)sm.pick[0];
  const int64_t t_in = sm.pick[1];  // rank of this workgroup's tile inside class cls
  int64_t mine = 0;
  if (cls >= 0)
    for (int b = b_lo; b < b_hi; ++b)
      if (seq_class(b) == cls) mine += (seq_rows(b) + QT - 1) / QT;
  int64_t incl = mine;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int64_t y = __shfl_up(incl, (unsigned)o, 64);
    if (lane >= o) incl += y;
  }
  if (lane == 63) wave_tiles[wave] = incl;
  if (tid == 0) found[0] = -1;
  __syncthreads();
  int64_t before = 0;
  for (int w = 0; w < wave; ++w) before += wave_tiles[w];
  if (cls >= 0) {
    int64_t S = before + incl - mine;
    if (t_in >= S && t_in < S + mine) {
      for (int b = b_lo; b < b_hi; ++b) {
        if (seq_class(b) != cls) continue;
        const int nt = (seq_rows(b) + QT - 1) / QT;
        if (t_in < S + nt) {
          found[0] = b;
          found[1] = nt - 1 - (int)(t_in - S);
          break;
        }
        S += nt;
      }
    }
  }
  __syncthreads();
  const int b = found[0];
  if (b < 0) return;  // uniform: more workgroups than query tiles
  const int qtile = found[1];

  int row0 = a.cu[b];
  row0 = row0 < 0 ? 0 : (row0 > a.num_tokens ? (int)a.num_tokens : row0);
  const int n = seq_rows(b);
  const int cap = a.W * a.block_size;
  int L = a.ctx_lens[b];
  L = L < 0 ? 0 : (L > cap ? cap : L);
  const int tq0 = qtile * QT;                    // first query token of the tile
  const int tq_end = min(n, tq0 + QT);
  const int p_first = L - n + tq0;               // position of the tile's first query
  const int p_last = L - n + tq_end - 1;         // ... and of its last
  const int n_kt = p_last >= 0 ? (p_last + kKeys) / kKeys : 0;

  const float ks = a.k_scale ? *a.k_scale : 1.0f;
  const float vs = a.v_scale ? *a.v_scale : 1.0f;
  // Scores enter as raw q.K dot products; exp2 takes fma(s, sl2, -max). A
  // negative scale is folded into q by flipping its sign bits (exact), so
  // sl2 >= 0 and the row max of raw scores scales to the max of scaled ones.
  const float sl2_signed = a.scale_log2 * ks;
  const bool flip_q = sl2_signed < 0.0f;
  const float sl2 = flip_q ? -sl2_signed : sl2_signed;

  // ---- this wave's rows: block rb, lane row li -> token / head
  int pos_row[kRB];  // query position of the lane's row in each block (-1: no key / no query)
  bf16x8 qop[kRB][KS];
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) {
    const int R = wave * kRowsPerWave + 16 * rb + li;
    const int tq = tq0 + R / G, hh = g * G + R % G;
    const bool live = tq < tq_end;
    pos_row[rb] = live ? L - n + tq : -1;
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) + (int64_t)(row0 + (live ? tq : 0)) * a.q_tok_stride +
                         (int64_t)hh * D + 8 * lg;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      u32x4 w = *reinterpret_cast<const u32x4*>(qp + 32 * s);
      if (flip_q) w ^= u32x4{0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
      qop[rb][s] = __builtin_bit_cast(bf16x8, w);
    }
  }

  // ---- block-table entries, staged in LDS (so that the key loop never waits
  // on a vector load of its own: vector-memory counters drain in order and
  // would also wait for the K/V tiles in flight). An entry outside the table or
  // the pool is stored as -1.
  const int32_t* btrow = a.bt + (int64_t)b * a.W;
  const int64_t row_el = (int64_t)a.HKV * D;  // elements between consecutive slots of a block
  const int nthreads = 64 * kWaves;
  int tab_base = 0;
  auto stage_table = [&](int base) {
    for (int i = tid; i < kTab; i += nthreads) {
      const int j = base + i;
      int ph = -1;
      if (j < a.W) {
        ph = btrow[j];
        if (ph < 0 || (int64_t)ph >= a.num_blocks) ph = -1;
      }
      tab[i] = ph;
    }
    tab_base = base;
  };
  stage_table(0);
  __syncthreads();
  // Key tiles are visited strictly in order: a uniform cursor holds the block
  // and offset of the next tile's first key and advances by kKeys (no integer
  // division in the loop). For each 16-key block of the tile, base[kb] is the
  // element offset of its first row in the pool (block 0 when the block lies
  // outside the table or the pool, which okbits records).
  struct TileAddr {
    int64_t base[kKB];
    int okbits;
  };
  int cur_jb = 0, cur_ob = 0;  // block index / offset of the next tile's first key
  auto next_tile_addr = [&](int t, TileAddr& ta) {
    int ok = 0;
#pragma unroll
    for (int kb = 0; kb < kKB; ++kb) {
      int o = cur_ob + 16 * kb, j = cur_jb;
      while (o >= a.block_size) {
        o -= a.block_size;
        ++j;
      }
      const int ph = (t < n_kt && j < a.W) ? tab[j - tab_base] : -1;
      ok |= (ph >= 0 ? 1 : 0) << kb;
      ta.base[kb] = (int64_t)(ph >= 0 ? ph : 0) * a.block_stride + (int64_t)o * row_el;
    }
    ta.okbits = ok;
    cur_ob += kKeys;
    while (cur_ob >= a.block_size) {
      cur_ob -= a.block_size;
      ++cur_jb;
    }
  };
  auto cursor_last_block = [&]() {  // block of the last key of the cursor's tile
    int o = cur_ob + kKeys - 1, j = cur_jb;
    while (o >= a.block_size) {
      o -= a.block_size;
      ++j;
    }
    return j;
  };

  // fetch of key tile kt into ring buffer buf (a block outside the pool is read
  // as block 0 and masked later)
  const char* kc = static_cast<const char*>(a.kc);
  const char* vc = static_cast<const char*>(a.vc);
  // This wave's IPW of the tile's 2*TI 1 KB loads (K loads first, then V):
  // lane l of a load fills LDS slot l of that kilobyte. bf16: it fetches the
  // chunk the reader-ordered layout puts there. fp8: the tile is staged in row
  // order, slot l of load ii holding row (1024 ii + 16 l) / D, 16 dims from
  // 16 * (((1024 ii + 16 l) % D) / 16). The lane's element offset inside its
  // 16-key block is fixed; only the blocks' bases change per tile.
  constexpr int kIPW = kFp8 ? G8::IPW : Gm::IPW;
  constexpr int kTI = kFp8 ? G8::TI : Gm::TI;
  constexpr int kEB = kFp8 ? 1 : 2;  // bytes per cache element
  int64_t lane_el[kIPW];
  int lane_kb[kIPW];
  int lane_row[kIPW], lane_chunk[kIPW];  // fp8: tile row and 16-dim chunk of the staged slot
#pragma unroll
  for (int i = 0; i < kIPW; ++i) {
    const int ii = wave * kIPW + i;
    int row, el;
    if constexpr (kFp8) {
      const int byte = 1024 * (ii % kTI) + 16 * lane;
      row = byte / D;
      lane_row[i] = row;
      lane_chunk[i] = (byte % D) / 16;
      el = 16 * lane_chunk[i];
    } else if (ii < Gm::TI) {  // K read (kb, s) = (ii / KS, ii % KS)
      row = 16 * (ii / Gm::KS) + (lane & 15);
      el = 8 * (4 * (ii % Gm::KS) + (lane >> 4));
    } else {            // V regions 2(ii - TI) and 2(ii - TI) + 1
      const int region = 2 * (ii - Gm::TI) + (lane >> 5);
      const int q = lane & 31;
      const int st = region / (2 * Gm::CB), cb = (region >> 1) % Gm::CB, half = region & 1;
      row = 32 * st + 16 * half + 4 * (q >> 3) + ((q & 7) >> 1);
      el = 8 * (2 * cb + (q & 1));
    }
    lane_kb[i] = row >> 4;
    lane_el[i] = (int64_t)(row & 15) * row_el + (int64_t)g * D + el;
  }
  auto fetch = [&](int buf, const TileAddr& ta) {
#pragma unroll
    for (int i = 0; i < kIPW; ++i) {
      const int ii = wave * kIPW + i;
      int64_t base = ta.base[0];
#pragma unroll
      for (int kb = 1; kb < kKB; ++kb) base = lane_kb[i] == kb ? ta.base[kb] : base;
      const char* src0 = ii < kTI ? kc : vc;
      char* dst = sm.dma[buf][ii < kTI ? 0 : 1] + (ii % kTI) * 1024;
      dma_16B(src0 + (base + lane_el[i]) * kEB, lds_addr(dst));
    }
  };
  // fp8: this lane's staged chunks of tile t (landed) -> the bf16 operand tiles.
  // K chunk (row r, dims 16c..+15) -> reads (kb, s) = (r/16, c/2), lanes
  // 16 (2(c%2)) + r%16 and 16 (2(c%2) + 1) + r%16; V chunk -> 16-byte slots q0,
  // q0 + 1 of block (cb, half) = (c, r/16), q0 = 8 ((r%16)/4) + 2 (r%4).
  auto convert = [&](int t) {
    if constexpr (kFp8) {
#pragma unroll
      for (int i = 0; i < kIPW; ++i) {
        const int ii = wave * kIPW + i;
        const bool is_k = ii < kTI;
        const u32x4 w = *reinterpret_cast<const u32x4*>(sm.dma[t % kBufs][is_k ? 0 : 1] + (ii % kTI) * 1024 +
                                                         16 * lane);
        u32x4 lo8, hi8;  // dims +0..7 and +8..15 as bf16
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const f32x2 a0 = fp8x2_lo(w[e]), a1 = fp8x2_hi(w[e]);
          lo8[2 * e] = f32x2_to_bf16x2(a0[0], a0[1]);
          lo8[2 * e + 1] = f32x2_to_bf16x2(a1[0], a1[1]);
          const f32x2 b0 = fp8x2_lo(w[2 + e]), b1 = fp8x2_hi(w[2 + e]);
          hi8[2 * e] = f32x2_to_bf16x2(b0[0], b0[1]);
          hi8[2 * e + 1] = f32x2_to_bf16x2(b1[0], b1[1]);
        }
        const int r = lane_row[i], c = lane_chunk[i];
        char* bt = sm.bf[t % kBfBufs][is_k ? 0 : 1];
        if (is_k) {
          const int kb = r >> 4, s = c >> 1, l0 = 16 * (2 * (c & 1)) + (r & 15);
          *reinterpret_cast<u32x4*>(bt + Gm::k_off(kb, s, l0)) = lo8;
          *reinterpret_cast<u32x4*>(bt + Gm::k_off(kb, s, l0 + 16)) = hi8;
        } else {
          const int q0 = 8 * ((r & 15) >> 2) + 2 * (r & 3);
          char* blk = bt + ((0 * CB + c) * 2 + (r >> 4)) * 512 + 16 * q0;
          *reinterpret_cast<u32x4*>(blk) = lo8;
          *reinterpret_cast<u32x4*>(blk + 16) = hi8;
        }
      }
    }
  };

  float m_run[kRB], l_run[kRB];
  f32x4 acc[kRB][CB];
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) {
    m_run[rb] = -INFINITY;
    l_run[rb] = 0.0f;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) acc[rb][cb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  }

  // The tile step in three parts. qk: S^T of a tile (sc[rb][kb] holds keys
  // 16kb + 4lg + r of row (rb, li)). softmax: the online-softmax update of
  // the running max and sum and the tile's probabilities as bf16 hi + lo P.V
  // operands; it returns, per 16-row block, whether some row's max moved
  // (alpha then holds the rescale factor of the lane's row). pv: O += P V.
  // kMask: some score of the tile is causal-masked, past the context end, or
  // in a block outside the pool.
  constexpr int kSt = kKeys / 32;  // 32-key steps of P.V
  auto qk = [&](int t, f32x4 (&sc)[kRB][kKB]) {
    const char* kl = ktile(t);
#pragma unroll
    for (int kb = 0; kb < kKB; ++kb) {
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb) sc[rb][kb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const bf16x8 kop = *reinterpret_cast<const bf16x8*>(kl + Gm::k_off(kb, s, lane));
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb)
          sc[rb][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, qop[rb][s], sc[rb][kb], 0, 0, 0);
      }
    }
  };
  auto softmax = [&](int kt, int okbits, const f32x4 (&sc)[kRB][kKB], bf16x8 (&pop)[kRB][kSt],
                     bf16x8 (&plo)[kRB][kSt], float (&alpha)[kRB], bool (&moved)[kRB], auto mask_tag) {
    constexpr bool kMask = decltype(mask_tag)::value;
    const int key0 = kt * kKeys;
    bool kb_ok[kKB];
#pragma unroll
    for (int kb = 0; kb < kKB; ++kb) kb_ok[kb] = kMask ? ((okbits >> kb) & 1) != 0 : true;
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) {
      bool ok[kKB][4];
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          ok[kb][r] = true;
          if constexpr (kMask) {
            const int key = key0 + 16 * kb + 4 * lg + r;
            ok[kb][r] = kb_ok[kb] && key <= pos_row[rb];
          }
          mx = fmaxf(mx, ok[kb][r] ? sc[rb][kb][r] : -INFINITY);
        }
      mx = row_max4(mx);
      const float mxs = mx == -INFINITY ? -INFINITY : mx * sl2;  // max of the scaled scores
      // The running max m is raised only when the tile's max passes it by more
      // than kLazyMax (first tile: any finite max): probabilities 2^(s - m) then
      // stay below 2^kLazyMax, and the accumulator rescale is rare.
      const bool raise = mxs > m_run[rb] + kLazyMax;
      const float mn = raise ? mxs : m_run[rb];
      const float mu = (mn == -INFINITY) ? 0.0f : mn;
      alpha[rb] = raise ? __builtin_amdgcn_exp2f(m_run[rb] - mu) : 1.0f;
      float ps = 0.0f;
      float pr[kKB][4];
#pragma unroll
      for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float e2 = __builtin_amdgcn_exp2f(fmaf(sc[rb][kb][r], sl2, -mu));
          pr[kb][r] = kMask ? (ok[kb][r] ? e2 : 0.0f) : e2;
          ps += pr[kb][r];
        }
      l_run[rb] = l_run[rb] * alpha[rb] + ps;
      moved[rb] = raise;
      m_run[rb] = mn;
      // p = hi + lo with hi = bf16(p) and lo = bf16(p - hi), both rounded to
      // nearest even: hi + lo is within 2^-17 (relative) of the fp32 p, so P.V
      // on the bf16 matrix core stays fp32-accurate (l above sums the same p)
#pragma unroll
      for (int st = 0; st < kSt; ++st) {
        uint32_t wh[4], wl[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float x0 = pr[2 * st + (e >> 1)][2 * (e & 1)], x1 = pr[2 * st + (e >> 1)][2 * (e & 1) + 1];
          wh[e] = f32x2_to_bf16x2(x0, x1);
          wl[e] = f32x2_to_bf16x2(x0 - bf16_lo(wh[e]), x1 - bf16_hi(wh[e]));
        }
        pop[rb][st] = __builtin_bit_cast(bf16x8, u32x4{wh[0], wh[1], wh[2], wh[3]});
        plo[rb][st] = __builtin_bit_cast(bf16x8, u32x4{wl[0], wl[1], wl[2], wl[3]});
      }
    }
  };
  // Rescale the accumulator rows 4lg + r of block rb by their rows' alpha --
  // only when some row's max was raised (otherwise every alpha is exactly 1).
  // Issue order of the block holding tile kt+1's score product and tile kt's
  // softmax: the K operand reads first, then the products one by one with a
  // few vector instructions between them.
  auto interleave_hint = [&]() {
#if PA_PREFILL_SCHED
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * KS, 0);  // DS reads: K operands
#pragma unroll
    for (int i = 0; i < kRB * kKB * KS; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, PA_PREFILL_SCHED, 0);  // vector ALU
    }
#endif
  };
  auto rescale = [&](const float (&alpha)[kRB], const bool (&moved)[kRB]) {
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) {
      if (__builtin_amdgcn_ballot_w64(moved[rb]) != 0) {
        float al[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) al[r] = bcast_lane(alpha[rb], (lane & 48) + 4 * lg + r);
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[rb][cb][r] *= al[r];
      }
    }
  };
  // O += P V, V's operand by transposing reads (lane m of a 16-lane group
  // reads row kbase + m/4, columns 16cb + 4(m%4) .. +3, kbase = 32st + 4g,
  // then + 16); the two reads are the operand's low and high halves.
  auto pv = [&](int kt, int okbits, const bf16x8 (&pop)[kRB][kSt], const bf16x8 (&plo)[kRB][kSt],
                auto mask_tag) {
    constexpr bool kMask = decltype(mask_tag)::value;
    const char* vl = vtile(kt);
    const int key0 = kt * kKeys;
#pragma unroll
    for (int st = 0; st < kSt; ++st) {
      u32x4 vmask = {~0u, ~0u, ~0u, ~0u};  // V elements of masked-out keys -> 0
      if constexpr (kMask) {
        uint32_t m16[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int kb = 2 * st + (j >> 2);
          const int key = key0 + 16 * kb + 4 * lg + (j & 3);
          m16[j] = (((okbits >> kb) & 1) && key < L) ? 0xFFFFu : 0u;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) vmask[i] = m16[2 * i] | (m16[2 * i + 1] << 16);
      }
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4*)(vl + Gm::v_off(st, cb, 0, lane)));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4*)(vl + Gm::v_off(st, cb, 1, lane)));
        u32x4 w = __builtin_bit_cast(u32x4, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        if constexpr (kMask) w &= vmask;
        const bf16x8 vop = __builtin_bit_cast(bf16x8, w);
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb)
          acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pop[rb][st], vop, acc[rb][cb], 0, 0, 0);
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb)
          acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(plo[rb][st], vop, acc[rb][cb], 0, 0, 0);
      }
    }
  };

  // ---- key loop (fp8 caches: after a tile's barrier each lane converts its
  // staged chunks into the tile's bf16 slot, then a second barrier; the bf16
  // slot of tile t is free once tile t - 2's P.V is done). Ring of kBufs = 4 tiles: tile kt (P.V), kt + 1 (its
  // scores, computed while tile kt's softmax runs) and two tiles in flight.
  // Iteration kt: wait for this wave's share of tile kt + 1, one barrier
  // (every wave's share has landed, and every wave is done with tile kt - 1,
  // whose buffer the fetch of tile kt + 3 then refills), S of tile kt + 1,
  // then the softmax and P.V of tile kt. Table entries of a tile are read one
  // tile before its fetch; the validity of the 16-key blocks of the tiles in
  // the ring is kept as 4 bits per slot. Every wave issues the same number of
  // loads per tile, so a wait leaves exactly the later tile's loads
  // outstanding.
  static_assert(kBufs == 4, "ring: tile in P.V, tile in S, two in flight");
  constexpr int kLoadsPerTile = kIPW;
  static_assert(2 * kLoadsPerTile <= 63, "vmcnt range");
  constexpr int kAll = (1 << kKB) - 1;
  int okring = 0;  // bits 4 * (t % kBufs) ..: 16-key blocks of tile t inside the pool
  auto start_tile = [&](int t, const TileAddr& ta) {
    fetch(t % kBufs, ta);
    okring = (okring & ~(15 << (4 * (t % kBufs)))) | (ta.okbits << (4 * (t % kBufs)));
  };
  TileAddr ta_next;
  for (int t = 0; t < 3; ++t) {
    next_tile_addr(t, ta_next);
    if (t < n_kt) start_tile(t, ta_next);
  }
  next_tile_addr(3, ta_next);
  // (t >= 1) Wait until this wave's share of tile t has landed (tile t + 1's
  // loads stay in flight), then a barrier; then fetch tile t + 2 into the
  // buffer of tile t - 2, which every wave is done with.
  auto bring_in = [&](int t) {
    if (t + 1 < n_kt)
      wait_vmem<kLoadsPerTile>();
    else
      wait_vmem<0>();
    barrier_no_vmem_wait();
    const int tn = t + 2;
    if (tn < n_kt) start_tile(tn, ta_next);
    // next tile's addresses; restage the table window when the tile runs past
    // it (uniform; once per kTab blocks)
    if (tn + 1 < n_kt && cursor_last_block() >= tab_base + kTab) {
      barrier_no_vmem_wait();
      stage_table(cur_jb);
      __syncthreads();
    }
    next_tile_addr(tn + 1, ta_next);
    if constexpr (kFp8) {  // tile t into its bf16 slot (freed by tile t - 2's P.V), then visible
      convert(t);
      barrier_no_vmem_wait();
    }
  };
  f32x4 sc_cur[kRB][kKB], sc_nxt[kRB][kKB];
  bf16x8 pop[kRB][kSt], plo[kRB][kSt];
  float alpha[kRB];
  bool moved[kRB];
  if (n_kt > 0) {  // tile 0 in, with tiles 1 and 2 (if any) still in flight
    if (n_kt > 2)
      wait_vmem<2 * kLoadsPerTile>();
    else if (n_kt > 1)
      wait_vmem<kLoadsPerTile>();
    else
      wait_vmem<0>();
    barrier_no_vmem_wait();
    if constexpr (kFp8) {  // tile 0 into bf16, visible to every wave
      convert(0);
      barrier_no_vmem_wait();
    }
    qk(0, sc_cur);
  }
  // Two loops, each with one variant of the softmax and P.V (both variants in
  // one loop need more registers than a lane has and spill inside the loop,
  // and a scratch reload waits on the vector-memory counter the tile pipeline
  // runs on): tiles are clean (no causal, context-end or table mask) up to the
  // first one that is not; from there on every tile takes the masked variant.
  int kt = 0;
  for (; kt < n_kt; ++kt) {
    const int okb = (okring >> (4 * (kt % kBufs))) & 15;
    if (!(kt * kKeys + kKeys - 1 <= p_first && okb == kAll)) break;
    if (kt + 1 < n_kt) bring_in(kt + 1);
    // tile kt+1's scores (after the last tile: a stale buffer, never used) in
    // the same block as tile kt's softmax, so their issue interleaves
    if (kPrioSM) set_prio<kPrioSM>();
    qk(kt + 1, sc_nxt);
    softmax(kt, okb, sc_cur, pop, plo, alpha, moved, std::false_type{});
    interleave_hint();
    rescale(alpha, moved);
    if (kPrioSM) set_prio<0>();
    pv(kt, okb, pop, plo, std::false_type{});
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb)
#pragma unroll
      for (int kb = 0; kb < kKB; ++kb) sc_cur[rb][kb] = sc_nxt[rb][kb];
  }
  for (; kt < n_kt; ++kt) {
    const int okb = (okring >> (4 * (kt % kBufs))) & 15;
    if (kt + 1 < n_kt) bring_in(kt + 1);
    // tile kt+1's scores (after the last tile: a stale buffer, never used) in
    // the same block as tile kt's softmax, so their issue interleaves
    if (kPrioSM) set_prio<kPrioSM>();
    qk(kt + 1, sc_nxt);
    softmax(kt, okb, sc_cur, pop, plo, alpha, moved, std::true_type{});
    interleave_hint();
    rescale(alpha, moved);
    if (kPrioSM) set_prio<0>();
    pv(kt, okb, pop, plo, std::true_type{});
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb)
#pragma unroll
      for (int kb = 0; kb < kKB; ++kb) sc_cur[rb][kb] = sc_nxt[rb][kb];
  }

  // ---- finish: sum the row sums over the four lane groups, normalise, store
  // (the grid is launched with 64 * kWaves threads per workgroup)
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) {
    float l = l_run[rb];
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    float inv[4];
    int tok[4], head[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float lr = bcast_lane(l, (lane & 48) + 4 * lg + r);
      inv[r] = lr > 0.0f ? vs / lr : 0.0f;
      const int R = wave * kRowsPerWave + 16 * rb + 4 * lg + r;
      tok[r] = tq0 + R / G;
      head[r] = g * G + R % G;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if (tok[r] >= tq_end) continue;
      const int64_t base = (int64_t)(row0 + tok[r]) * a.out_tok_stride + (int64_t)head[r] * D + li;
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const float o = acc[rb][cb][r] * inv[r];
        if (a.out_f32)
          static_cast<float*>(a.out)[base + 16 * cb] = o;
        else
          static_cast<uint16_t*>(a.out)[base + 16 * cb] = (uint16_t)f32_to_bf16(o);
      }
    }
  }
}

template <int D, bool kFp8>
bool launch_g(int G, const PfArgs& a, hipStream_t st) {
  const unsigned grid = (unsigned)((a.tiles_ub * a.HKV + 7) / 8 * 8);
  switch (G) {
    case 1: prefill_mfma_kernel<D, 1, kFp8><<<grid, 64 * Shape<D>::WAVES, 0, st>>>(a); return true;
    case 2: prefill_mfma_kernel<D, 2, kFp8><<<grid, 64 * Shape<D>::WAVES, 0, st>>>(a); return true;
    case 4: prefill_mfma_kernel<D, 4, kFp8><<<grid, 64 * Shape<D>::WAVES, 0, st>>>(a); return true;
    case 8: prefill_mfma_kernel<D, 8, kFp8><<<grid, 64 * Shape<D>::WAVES, 0, st>>>(a); return true;
    default: return false;
  }
}

}  // namespace
}  // namespace pa

extern "C" pa_status pa_prefill_attention(void* out, pa_dtype out_dtype, int64_t out_token_stride,
                                          const void* q, pa_dtype q_dtype, int64_t q_token_stride,
                                          int64_t num_tokens, const int32_t* cu_seqlens_q,
                                          const void* key_cache, const void* value_cache,
                                          pa_dtype cache_dtype, int64_t num_blocks, int32_t block_size,
                                          int64_t block_stride, const int32_t* block_tables,
                                          int32_t max_blocks_per_seq, const int32_t* context_lens,
                                          int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                          int32_t head_size, float softmax_scale, const float* k_scale,
                                          const float* v_scale, void* stream) {
  using namespace pa;
  clear_error();
  const char* fn = "pa_prefill_attention";
  if (num_seqs < 0 || num_tokens < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || max_blocks_per_seq <= 0 ||
      block_size <= 0)
    return fail(PA_EINVAL, "%s: invalid sizes", fn);
  if (num_tokens > INT32_MAX) return fail(PA_EINVAL, "%s: num_tokens must fit in int32", fn);
  if (num_seqs > 65535) return fail(PA_EINVAL, "%s: num_seqs > 65535", fn);
  if (num_q_heads % num_kv_heads != 0) return fail(PA_EINVAL, "%s: num_q_heads %% num_kv_heads != 0", fn);
  const int G = num_q_heads / num_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8)
    return fail(PA_EUNSUPPORTED, "%s: group size H_Q/H_KV = %d not supported (1, 2, 4, 8)", fn, G);
  if (head_size != 64 && head_size != 128 && head_size != 256)
    return fail(PA_EUNSUPPORTED, "%s: head_size %d not supported (64, 128, 256)", fn, head_size);
  if (block_size % 16 != 0) return fail(PA_EUNSUPPORTED, "%s: block_size %d must be a multiple of 16", fn, block_size);
  if ((int64_t)max_blocks_per_seq * block_size > INT32_MAX) return fail(PA_EINVAL, "%s: max_blocks_per_seq*block_size too large", fn);
  if (out_dtype != PA_BF16 && out_dtype != PA_F32) return fail(PA_EDTYPE, "%s: out dtype %s not supported", fn, dtype_name(out_dtype));
  if (q_dtype != PA_BF16) return fail(PA_EDTYPE, "%s: q dtype %s not supported (bf16)", fn, dtype_name(q_dtype));
  if (cache_dtype != PA_BF16 && cache_dtype != PA_FP8_E4M3FN)
    return fail(PA_EDTYPE, "%s: cache dtype %s not supported (bf16, fp8_e4m3fn)", fn, dtype_name(cache_dtype));
  if (!(softmax_scale == softmax_scale) || isinf(softmax_scale)) return fail(PA_EINVAL, "%s: softmax_scale is not finite", fn);
  const int64_t row = (int64_t)num_q_heads * head_size;
  if (out_token_stride < row || q_token_stride < row) return fail(PA_EINVAL, "%s: token strides smaller than H_Q*head_size", fn);
  if (num_blocks < 0) return fail(PA_EINVAL, "%s: num_blocks < 0", fn);
  if (block_stride < (int64_t)block_size * num_kv_heads * head_size) return fail(PA_EINVAL, "%s: block_stride too small", fn);
  if (num_seqs == 0 || num_tokens == 0) return PA_OK;
  if (!out || !q || !key_cache || !value_cache || !block_tables || !context_lens || !cu_seqlens_q)
    return fail(PA_EINVAL, "%s: null pointer argument", fn);
  const int ob = dtype_bytes(out_dtype);
  if (!aligned(q, 16) || (q_token_stride * 2) % 16 != 0) return fail(PA_EINVAL, "%s: q must be 16-byte aligned per token", fn);
  if (!aligned(out, 16) || (out_token_stride * ob) % 16 != 0) return fail(PA_EINVAL, "%s: out must be 16-byte aligned per token", fn);
  const int cbytes = dtype_bytes(cache_dtype);
  if (!aligned(key_cache, 16) || !aligned(value_cache, 16) || (block_stride * cbytes) % 16 != 0)
    return fail(PA_EINVAL, "%s: caches must be 16-byte aligned per block", fn);
  if (((int64_t)num_kv_heads * head_size * cbytes) % 16 != 0)
    return fail(PA_EINVAL, "%s: cache rows must be a multiple of 16 bytes", fn);
  if (checks_on()) {
    const hipStream_t cs = reinterpret_cast<hipStream_t>(stream);
    pa_status c = check_tables(fn, cs, block_tables, num_seqs, max_blocks_per_seq, context_lens, num_blocks, block_size);
    if (c == PA_OK) c = check_chunks(fn, cs, cu_seqlens_q, num_seqs, num_tokens, context_lens);
    if (c != PA_OK) return c;
  }

  PfArgs a;
  a.out = out;
  a.q = q;
  a.kc = key_cache;
  a.vc = value_cache;
  a.bt = block_tables;
  a.ctx_lens = context_lens;
  a.cu = cu_seqlens_q;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.out_tok_stride = out_token_stride;
  a.q_tok_stride = q_token_stride;
  a.block_stride = block_stride;
  a.num_blocks = num_blocks;
  a.num_tokens = num_tokens;
  a.block_size = block_size;
  a.W = max_blocks_per_seq;
  a.num_seqs = num_seqs;
  a.HQ = num_q_heads;
  a.HKV = num_kv_heads;
  a.out_f32 = out_dtype == PA_F32;
  a.scale_log2 = softmax_scale * 1.4426950408889634f;
  // query tiles: at most ceil(T / QT) + num_seqs (one partial tile per sequence)
  const int64_t qt = kRows / G;
  a.tiles_ub = (num_tokens + qt - 1) / qt + num_seqs;
  {  // length classes: the key tiles of the longest possible query tile over kBins classes
    const int64_t kt_max = ((int64_t)max_blocks_per_seq * block_size + kKeys - 1) / kKeys;
    a.bin_w = (int)((kt_max + kBins - 1) / kBins);
    if (a.bin_w < 1) a.bin_w = 1;
  }
  if (a.tiles_ub * num_kv_heads + 7 > 0x7FFFFFFF) return fail(PA_EINVAL, "%s: too many query tiles", fn);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const bool fp8 = cache_dtype == PA_FP8_E4M3FN;
  const bool ok = head_size == 64    ? (fp8 ? launch_g<64, true>(G, a, st) : launch_g<64, false>(G, a, st))
                  : head_size == 128 ? (fp8 ? launch_g<128, true>(G, a, st) : launch_g<128, false>(G, a, st))
                                     : (fp8 ? launch_g<256, true>(G, a, st) : launch_g<256, false>(G, a, st));
  if (!ok) return fail(PA_EUNSUPPORTED, "%s: no kernel for this shape", fn);
  return after_launch(fn);
}
