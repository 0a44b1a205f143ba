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
//  * split: persistent, one workgroup per compute unit over an even share of
//    the items of all sequences (each sequence's q~, then its 32-position
//    tiles); 2 fetching waves move each item by LDS-DMA into a 4-deep LDS
//    ring, and the computing waves meet them and each other through LDS
//    counters (no workgroup barrier per tile). Two score waves (8 heads each)
//    form S^T = C [q~hi | q~lo] on v_mfma_f32_16x16x32_bf16 with q~ held in
//    registers, add the hi and lo columns, run the online softmax in the log2
//    domain and hand P over as bf16 hi + lo rows; four P.V waves (128 latent
//    dims each) form O += P C on v_mfma_f32_32x32x16_bf16 with C's operand
//    from LDS by transposing reads. Writes the unnormalised O, its running
//    max and sum per head for each (workgroup, sequence) segment.
//  * merge: combines the pieces of a sequence and applies W_UV per head.
#include <math.h>

#include <type_traits>

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
constexpr int kScore = 2;       // score waves of a split workgroup (8 heads each)
constexpr int kPV = 4;          // P.V waves (128 latent dims each)
constexpr int kWaves = kScore + kPV;  // computing waves: each takes part in every item
constexpr int kProducers = 2;   // ... and its fetching waves (16 rows of an item each)
constexpr int kRing = 4;        // LDS item buffers: one being computed, three in flight
constexpr int kTabSlots = 8;    // LDS slots of fetched block-table entries
constexpr int kAhead = 3;       // items a fetching wave keeps in flight
constexpr uint32_t kSpinLimit = 1u << 20;  // polls before a wait gives up (never, when the counts are right)

template <int DR>
struct MlaGeo {
  static constexpr int ROW = kDC + DR;           // values per cached row
  static constexpr int RB = ROW * 2;             // bytes per cached row
  static constexpr int CH = RB / 16;             // 16-byte chunks per row (64 or 72)
  static constexpr int TILE = kTile * RB;        // bytes per LDS tile (rows back to back)
  static constexpr int LOADS = TILE / 1024;      // 1 KB LDS-DMA wave loads per tile
  static constexpr int LPP = LOADS / kProducers; // ... per fetching wave: 16 rows
  static constexpr int KS = ROW / 32;            // 16x16x32 MFMA steps over the row
  static_assert(CH % 8 == 0 && TILE % 1024 == 0 && LPP * 1024 == 16 * RB, "tile geometry");
  // Chunk swizzle: physical chunk of logical chunk lc in row r is lc ^ sw(r),
  // so that 16 consecutive rows read at one logical chunk hit 16 different
  // 16-byte bank groups (a row start advances 8 groups when CH % 16 == 8).
  __device__ static int sw(int r) { return CH % 16 == 0 ? (r & 15) : ((r >> 1) & 7); }
  __device__ static int phys(int r, int lc) { return lc ^ sw(r); }
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
  int32_t* ts;      // [B + 1] first work unit of each sequence; ts[B] = all units (q~ items and tiles)
  int32_t* flag;    // set when a wait of the split ran past its bound (the outputs are then NaN)
  float* ws_m;      // [G + B, 16] per (workgroup, sequence) partial
  float* ws_l;
  float* ws_o;      // [G + B, 16, 512]
  int64_t out_seq_stride, qn_seq_stride, qr_seq_stride;
  int64_t block_stride, num_blocks;
  int32_t block_size, W, num_seqs, qk, dr, dv, grid;
  int32_t bs_log2;  // log2(block_size) when a power of two, else -1
  int32_t out_f32;
  float scale_log2;
  // decode step only (new_slots null otherwise): the batch's new latent rows,
  // written by the absorb launch before the split reads the cache
  uint16_t* wcache;            // the latent cache, writable
  const uint16_t* new_c;       // [B, 512], row stride new_c_stride
  const uint16_t* new_r;       // [B, rope_dim], row stride new_r_stride
  const int64_t* new_slots;    // [B]; negative or outside the pool: no write
  int64_t new_c_stride, new_r_stride;
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

// The work of all sequences in sequence order forms one list of T units: a
// sequence with tiles contributes one unit for its q~ item followed by one per
// tile (an empty sequence none), so that the q~ items a workgroup fetches are
// part of its even share. Workgroup w of G serves units range_start(w) ..
// range_start(w + 1) - 1; unit u belongs to workgroup tile_owner(u). A
// workgroup whose share holds some of a sequence's tiles fetches that
// sequence's q~ item even when the q~ unit itself lies in the previous share.
__device__ __forceinline__ int range_start(int w, int T, int G) {
  const int q = T / G, r = T % G;
  return w * q + min(w, r);
}
__device__ __forceinline__ int tile_owner(int t, int T, int G) {
  const int q = T / G, r = T % G, big = r * (q + 1);
  return t < big ? t / (q + 1) : r + (t - big) / q;
}
__device__ __forceinline__ int tiles_of(const MlaArgs& a, int b) { return (clamp_ctx(a, b) + kTile - 1) / kTile; }
__device__ __forceinline__ int units_of(const MlaArgs& a, int b) {
  const int t = tiles_of(a, b);
  return t > 0 ? t + 1 : 0;
}

// ts[b] = units of sequences 0 .. b - 1 (ts[B] = T), by one workgroup of 256:
// each thread sums a run of sequences, a lane scan per wave and the four wave
// totals give each run's first tile (one workgroup barrier).
__device__ void plan_tiles(const MlaArgs& a) {
  __shared__ int wsum[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, B = a.num_seqs;
  const int per = (B + 255) / 256;
  const int lo = min(B, tid * per), hi = min(B, lo + per);
  int mine = 0;
  for (int b = lo; b < hi; ++b) mine += units_of(a, b);
  int incl = mine;  // inclusive prefix over this wave's lanes
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_up(incl, (unsigned)o, 64);
    if (lane >= o) incl += v;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  int run = incl - mine;
  for (int w = 0; w < wave; ++w) run += wsum[w];
  if (per == 1) {  // (B <= 256: the run is one sequence, its count already summed)
    if (lo < hi) a.ts[lo] = run;
    run += mine;
  } else {
    for (int b = lo; b < hi; ++b) {
      a.ts[b] = run;
      run += units_of(a, b);
    }
  }
  if (tid == 255) {  // the last run ends at T
    a.ts[B] = run;
    *a.flag = 0;
  }
}

// Decode step: sequence r's new latent row (c ++ RoPE key) into cache slot
// new_slots[r], one wave a row (a lane moves 16 bytes of c, lanes < dr / 8 16
// bytes of the RoPE key); workgroup wg of nwg takes rows 4 wg + wave, + 4 nwg, ...
__device__ void write_new_rows(const MlaArgs& a, int row, int wg, int nwg) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t pool = a.num_blocks * (int64_t)a.block_size;
  for (int r = 4 * wg + wave; r < a.num_seqs; r += 4 * nwg) {
    const int64_t slot = a.new_slots[r];
    if (slot < 0 || slot >= pool) continue;  // (uniform across the wave)
    const int64_t blk = slot / a.block_size, off = slot - blk * a.block_size;
    uint16_t* dst = a.wcache + blk * a.block_stride + off * row;
    *reinterpret_cast<u32x4*>(dst + 8 * lane) = *reinterpret_cast<const u32x4*>(a.new_c + (int64_t)r * a.new_c_stride + 8 * lane);
    if (lane < a.dr / 8)
      *reinterpret_cast<u32x4*>(dst + kDC + 8 * lane) =
          *reinterpret_cast<const u32x4*>(a.new_r + (int64_t)r * a.new_r_stride + 8 * lane);
  }
}

// ---------------------------------------------------------------- absorb
// q~^T [512 c x B] = W_UK,h [512 x qk] q_h^T [qk x B] per head on the matrix
// cores (bf16 x bf16 products are exact in fp32, sums in fp32). grid (16
// heads, 8 blocks of 64 latent dims, ceil(B / 16) + 1: the last layer writes the
// tile plan of the split and, in a decode step, the new latent rows); wave w computes latent
// dims 64 cb + 16 w .. +15 for 16 sequences. The A operand is 16 bytes of a
// W_UK row (dims 8 (l/16) .. of row l%16), the B operand 16 bytes of a q row.
__global__ __launch_bounds__(256) void mla_absorb_kernel(MlaArgs a, int row) {
  if (blockIdx.z == gridDim.z - 1) {  // the extra layer: its first workgroup writes the tile plan,
    // and in a decode step the others write the new latent rows
    const int lid = (int)(blockIdx.y * gridDim.x + blockIdx.x);
    if (lid == 0)
      plan_tiles(a);
    else if (a.new_slots)
      write_new_rows(a, row, lid - 1, (int)(gridDim.x * gridDim.y) - 1);
    return;
  }
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
  // the RoPE part (latent block 0 only; 16 * dr <= 1024 values), loaded in the
  // same round as the operands above, before any store
  float xr[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  const int drr = a.dr > 0 ? a.dr : 1;
  if (blockIdx.y == 0) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = tid + 256 * u;
      const int bb = b0 + i / drr, r = i % drr;
      if (i < 16 * a.dr && bb < a.num_seqs)
        xr[u] = load1<Ty::BF16>(a.q_rope, (int64_t)bb * a.qr_seq_stride + (int64_t)h * a.dr + r);
    }
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
  if (blockIdx.y == 0) {  // the RoPE part: scaled and split as it is
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = tid + 256 * u;
      const int bb = b0 + i / drr, r = i % drr;
      if (!(i < 16 * a.dr && bb < a.num_seqs)) continue;
      uint16_t hi, lo;
      split_hi_lo(xr[u] * a.scale_log2, hi, lo);
      const int64_t base = ((int64_t)bb * kHeads + h) * row + kDC;
      a.q_hi[base + r] = hi;
      a.q_lo[base + r] = lo;
    }
  }
}

// ---------------------------------------------------------------- split
// A workgroup barrier for LDS traffic only: loads in flight stay in flight
// across it (a full __syncthreads would wait for them too).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

__device__ __forceinline__ float bcast_lane(float x, int src) {
  return __int_as_float(__builtin_amdgcn_ds_bpermute(src << 2, __float_as_int(x)));
}

// max over the four lanes l % 16 + 16 j: each permlane swap exchanges one half
// of a copy of x with the other half of a second copy, so the two results hold,
// lane by lane, x at l and at its partner lane (l ^ 32, then l ^ 16).
__device__ __forceinline__ float max_over_groups(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto a = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  const float m = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const uint32_t v = __float_as_uint(m);
  const auto b = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// sum over the four lanes l % 16 + 16 j (every lane gets the same sum)
__device__ __forceinline__ float sum_over_groups(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto a = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  const float m = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const uint32_t v = __float_as_uint(m);
  const auto b = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// block and offset of a position (a shift when the block size is a power of two)
__device__ __forceinline__ void block_of(const MlaArgs& a, int pos, int& blk, int& off) {
  if (a.bs_log2 >= 0) {
    blk = pos >> a.bs_log2;
    off = pos & (a.block_size - 1);
  } else {
    blk = pos / a.block_size;
    off = pos - blk * a.block_size;
  }
}

constexpr float kLazyMax = 8.0f;  // log2 headroom of a segment's running max

// Persistent: one workgroup per compute unit, each over an even share of the
// T units of all sequences (sequence order). Its share falls into segments,
// one per sequence it touches; a segment is processed as an item stream --
// the sequence's q~ (hi and lo, 32 rows of the row length: exactly one tile's
// bytes), then its tiles -- and ends with a partial (running max, sum and
// unnormalised O of the 16 heads) at slot w + b of the workspace (w + b is
// unique: a later workgroup never serves an earlier sequence).
//
// Roles: waves 0 and 1 score (8 heads each), waves 2..5 multiply P by the
// latent rows (128 latent dims of O each), waves 6 and 7 fetch. Every item
// goes global -> LDS by LDS-DMA into a ring of kRing buffers; fetching wave p
// moves rows 16 p .. 16 p + 15 of each item and, kAhead + 1 items ahead, the
// block-table entries of those rows (4 bytes a lane), so that no load the
// compiler sees sits in its loop (vector-memory counters complete in order;
// waiting for such a load would wait for the items in flight too). Every
// computing wave reads what it needs of an item into registers and gives the
// buffer back at once; the roles meet through LDS counters instead of
// workgroup barriers, so that a fetching wave whose DMA issue stalls on a full
// memory pipeline never holds a computing wave, nor the other way round:
//  * ready[p]: items whose share from fetching wave p has landed (raised
//    after its own vmcnt wait); a computing wave starts item i when both are
//    past i;
//  * consumed[r]: +1 per computing wave once it has read the item in buffer
//    r; a fetching wave puts item j there only when it reaches
//    kWaves (j / kRing), every earlier item of that buffer read by every
//    computing wave (one count per buffer, not one for the ring: waves of
//    different roles drift apart, and a sum over the ring would let a fast
//    wave's reads stand in for a slow wave's);
//  * p_ready[pb] / p_done[pb]: the score waves' P of the k-th tile (bf16 hi
//    and lo) goes into LDS buffer pb = k % 2; +1 per score wave once written,
//    +1 per P.V wave once read, counted per buffer for the same reason.
// Every wait polls with a bound: counts that never arrive end the kernel
// instead of hanging the device, and set a flag in the workspace that makes
// the merge write NaN outputs.
__device__ __forceinline__ uint32_t lds_load_u32(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void lds_add_u32(uint32_t* p, uint32_t v) {
  __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void lds_store_u32(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }
// Polls until *p >= target (uniform); false after kSpinLimit polls.
__device__ __forceinline__ bool wait_at_least(const uint32_t* p, uint32_t target) {
  for (uint32_t n = 0; n < kSpinLimit; ++n) {
    if (__builtin_amdgcn_readfirstlane(lds_load_u32(p)) >= target) {
      compiler_fence();
      return true;
    }
    __builtin_amdgcn_s_sleep(1);
  }
  return false;
}

// A wait ran past its bound: the call's outputs become NaN (the merge reads the flag).
__device__ __forceinline__ void timed_out(const MlaArgs& a) {
  if ((threadIdx.x & 63) == 0) *a.flag = 1;
}

template <int DR>
__global__ __launch_bounds__(64 * (kWaves + kProducers)) void mla_split_kernel(MlaArgs a) {
  using Gm = MlaGeo<DR>;
  constexpr int ROW = Gm::ROW, RB = Gm::RB, LPP = Gm::LPP;
  constexpr int KS = Gm::KS;
  const int tid = threadIdx.x, lane = tid & 63, li = lane & 15, lg = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = (int)gridDim.x, w = (int)blockIdx.x, B = a.num_seqs;

  __shared__ __attribute__((aligned(16))) char ring[kRing][Gm::TILE];
  constexpr int kPRow = 64;  // bytes per P row (32 positions)
  __shared__ __attribute__((aligned(16))) char pbuf[2][32 * kPRow];  // P of tiles k, k + 1 (hi rows, then lo)
  __shared__ float palpha[2][kHeads];                                // their rescale factors of O
  __shared__ int praise[2][kScore];                                  // some head's max was raised
  __shared__ __attribute__((aligned(16))) int32_t tab[kProducers][kTabSlots][64];
  __shared__ int desc[kRing][4];  // item: local tile (-1 q~, -2 none), sequence, last tile of its segment
  __shared__ uint32_t rowmask[kRing][kProducers];
  __shared__ uint32_t ready[kProducers], consumed[kRing], p_ready[2], p_done[2];
  if (tid == 0) {
    for (int p2 = 0; p2 < kProducers; ++p2) ready[p2] = 0u;
    for (int r = 0; r < kRing; ++r) consumed[r] = 0u;
    p_ready[0] = p_ready[1] = p_done[0] = p_done[1] = 0u;
  }
  __syncthreads();  // the counters start at zero (before any load is in flight)

  const int T = uniform(a.ts[B]);
  const int t0 = range_start(w, T, G), t1 = range_start(w + 1, T, G);
  if (t0 >= t1) return;  // uniform: no tiles for this workgroup

  if (wave >= kWaves) {
    // ================================================================ fetch
    const int pw = wave - kWaves;
    // ---- segments: lane j of sg_* holds the j-th segment of the current list
    // (up to 64 sequences at a time): sequence, first local tile, tiles, length.
    int b_first;
    {  // the last sequence whose first tile is <= t0 (it holds tile t0)
      int lo = 0, hi = B;
      while (hi - lo > 1) {
        const int step = (hi - lo + 63) / 64;
        const int idx = lo + lane * step;
        const int v = idx < hi ? a.ts[idx] : INT32_MAX;
        const uint64_t le = __builtin_amdgcn_ballot_w64(v <= t0);  // a prefix of the lanes, lane 0 included
        const int j = 63 - __builtin_clzll(le);
        lo = lo + j * step;
        hi = min(hi, lo + step);
      }
      b_first = uniform(lo);
    }
    int sg_b = 0, sg_lt0 = 0, sg_nt = 0, sg_ctx = 0, nseg = 0, b_next = b_first;
    bool more = true;
    auto fill = [&]() {  // the next 64 sequences from b_next, compacted to the live ones
      const int b = b_next + lane;
      bool live = false;
      int lt0 = 0, nt = 0, cx = 0;
      if (b < B) {  // its tiles are units tsb + 1 .. tse - 1
        const int tsb = a.ts[b], tse = a.ts[b + 1];
        const int lo_t = max(t0, tsb + 1), hi_t = min(t1, tse);
        live = hi_t > lo_t;
        lt0 = lo_t - tsb - 1;
        nt = hi_t - lo_t;
        cx = clamp_ctx(a, b);
      }
      const uint64_t m = __builtin_amdgcn_ballot_w64(live);
      const int below = __builtin_popcountll(m & ((1ull << lane) - 1ull));
      const int cnt = __builtin_popcountll(m);
      const int dst = 4 * (live ? below : cnt + (lane - below));  // a permutation: live lanes first
      sg_b = __builtin_amdgcn_ds_permute(dst, b);
      sg_lt0 = __builtin_amdgcn_ds_permute(dst, lt0);
      sg_nt = __builtin_amdgcn_ds_permute(dst, nt);
      sg_ctx = __builtin_amdgcn_ds_permute(dst, cx);
      nseg = cnt;
      const int nb = b_next + 64;
      more = nb < B && uniform(a.ts[nb < B ? nb : B]) + 1 < t1;  // tiles of later sequences remain
      b_next = nb;
    };
    int cur_k = 0, cur_idx = 0;  // item cursor: segment, item within it (0: q~)
    fill();
    // descriptor of the next item: lt (-1: q~, -2: none, else local tile),
    // sequence, length, last tile of its segment
    auto next_item = [&](int& lt, int& bb, int& cx, int& last) {
      while (cur_k >= nseg && more) {  // uniform; a refill waits for every load in flight (rare)
        fill();
        cur_k = 0;
      }
      if (cur_k >= nseg) {
        lt = -2;
        bb = 0;
        cx = 0;
        last = 0;
        return;
      }
      const int sb = __builtin_amdgcn_readlane(sg_b, cur_k), s0 = __builtin_amdgcn_readlane(sg_lt0, cur_k);
      const int sn = __builtin_amdgcn_readlane(sg_nt, cur_k), sc = __builtin_amdgcn_readlane(sg_ctx, cur_k);
      bb = sb;
      cx = sc;
      lt = cur_idx == 0 ? -1 : s0 + cur_idx - 1;
      last = cur_idx == sn ? 1 : 0;
      if (++cur_idx > sn) {
        cur_idx = 0;
        ++cur_k;
      }
    };

    if (a.num_blocks == 0) {  // an empty pool -- every position is masked (the computing waves left)
      if (pw == 0) {
        for (;;) {
          if (lane < nseg) {
#pragma unroll
            for (int h = 0; h < kHeads; ++h) {
              a.ws_m[(int64_t)(w + sg_b) * kHeads + h] = -INFINITY;
              a.ws_l[(int64_t)(w + sg_b) * kHeads + h] = 0.0f;
            }
          }
          if (!more) break;
          fill();
        }
      }
      return;
    }

    const char* cache = static_cast<const char*>(a.cache);
    // entries of rows 16 pw + lane % 16 of a tile item (a fixed valid entry otherwise)
    auto fetch_tab = [&](int slot, int lt, int bb) {
      const int32_t* src = a.bt;
      if (lt >= 0) {
        int blk, o;
        block_of(a, kTile * lt + 16 * pw + (lane & 15), blk, o);
        src = a.bt + (int64_t)bb * a.W + min(blk, a.W - 1);
      }
      dma_4B(src, lds_addr(&tab[pw][slot][0]));
    };
    // This wave's LPP loads of an item fill buffer bytes 1024 (pw LPP + k) ..
    // +1023: exactly rows 16 pw .. 16 pw + 15, a load spanning at most two
    // rows. Lane l's 16 bytes of load k are physical chunk pc of one of them,
    // so it fetches logical chunk phys(row, pc) of that row. Lanes r < 16 find
    // row 16 pw + r's source (an offset from base in 16-byte units; a masked
    // position reads the base's first row instead, its values masked) and the
    // rows that take part (bit r for row 16 pw + r); the sixteen offsets reach
    // every lane through readlane.
    const int64_t qlo_delta16 = ((const char*)a.q_lo - (const char*)a.q_hi) / 16;
    struct RowSrc {
      const char* base;
      uint32_t roff[16];
      uint32_t rows;
    };
    auto find_rows = [&](int tslot, int lt, int bb, int cx, RowSrc& rs) {
      const int r = lane & 15;
      int64_t off16;
      bool ok;
      if (lt == -1) {  // q~: rows 0..15 the hi parts of heads 0..15, rows 16..31 the lo parts
        rs.base = reinterpret_cast<const char*>(a.q_hi);
        off16 = (pw == 0 ? 0 : qlo_delta16) + ((int64_t)bb * kHeads + r) * (RB / 16);
        ok = true;
      } else {
        rs.base = cache;
        const int e = tab[pw][tslot][lane];
        const int pos = kTile * lt + 16 * pw + r;
        int blk, o;
        block_of(a, pos, blk, o);
        (void)blk;
        ok = pos < cx && e >= 0 && (int64_t)e < a.num_blocks;
        off16 = ok ? ((int64_t)e * a.block_stride + (int64_t)o * ROW) / 8 : 0;  // bf16 elements / 8
      }
      rs.rows = (uint32_t)__builtin_amdgcn_ballot_w64(ok) & 0xFFFFu;
#pragma unroll
      for (int j2 = 0; j2 < 16; ++j2) rs.roff[j2] = __builtin_amdgcn_readlane((uint32_t)off16, j2);
    };
    // loads k0 .. k1 - 1 of this wave's share of an item into ring slot rslot
    auto issue = [&](int rslot, const RowSrc& rs, auto k0c, auto k1c) {
      constexpr int k0 = decltype(k0c)::value, k1 = decltype(k1c)::value;
      char* dst = ring[rslot] + 1024 * (pw * LPP);
#pragma unroll
      for (int k = k0; k < k1; ++k) {
        const int ra = (1024 * k) / RB;                     // first of the load's rows (wave-local)
        const int split = (RB * (ra + 1) - 1024 * k) / 16;  // lanes below it are in row ra
        const bool second = lane >= split;
        const int rl = second ? ra + 1 : ra;
        const int pc = (1024 * k + 16 * lane - RB * rl) / 16;
        const int lc = Gm::phys(16 * pw + rl, pc);
        const uint32_t ro = second ? rs.roff[ra + 1 < 16 ? ra + 1 : 15] : rs.roff[ra];
        dma_16B(rs.base + 16 * ((uint64_t)ro + lc), lds_addr(dst + 1024 * k));
      }
    };
    using KZero = std::integral_constant<int, 0>;
    using KAll = std::integral_constant<int, LPP>;
    auto post = [&](int slot, int lt, int bb, int last, uint32_t rows) {  // to the computing waves
      if (lane == 0) {
        rowmask[slot][pw] = rows << (16 * pw);
        if (pw == 0) {
          desc[slot][0] = lt;
          desc[slot][1] = bb;
          desc[slot][2] = last;
        }
      }
    };

    // descriptors of items j .. j + kAhead + 1
    constexpr int ND = kAhead + 2;
    int dl[ND], db[ND], dc[ND], dz[ND];
#pragma unroll
    for (int s2 = 0; s2 < ND; ++s2) next_item(dl[s2], db[s2], dc[s2], dz[s2]);
    // entries of items 0 .. kAhead
#pragma unroll
    for (int s2 = 0; s2 <= kAhead; ++s2) fetch_tab(s2, dl[s2], db[s2]);
    bool ok_run = true;
    for (int j = 0; ok_run; ++j) {
      // Step j: item j - kAhead is published once this wave's share of it has
      // landed -- this wave's later operations, the entries and data of items
      // j - kAhead + 1 .. j - 1 (entries run kAhead + 1 items ahead of data),
      // are then all that may be in flight --, before the wait for a buffer,
      // so that a landed item never waits for one; item j goes into buffer
      // j % kRing once item j - kRing is done with.
      // In flight at the start of step j: the prologue's entries of items
      // min(j, kAhead + 1) .. kAhead, then per earlier step the entries of
      // one item and the data of another (LPP + 1 operations). Item 0 is a
      // segment's q~ (it needs no entries); steps 2 and 3 wait for items 0
      // and 1 themselves, so that the first tile is published a step early.
      static_assert(kAhead == 3, "the waits below count steps of (LPP + 1) operations");
      if (j == 1) wait_vmem<LPP + 3>();  // item 1's entries (the prologue's second)
      if (j == 2 || j == 3) {
        wait_vmem<LPP + 1>();  // items j - 2 and all before them, with the prologue's entries
        compiler_fence();
        if (lane == 0) lds_store_u32(&ready[pw], (uint32_t)(j - 1));
      } else if (j > kAhead) {
        wait_vmem<2 * (LPP + 1)>();
        compiler_fence();
        if (lane == 0) lds_store_u32(&ready[pw], (uint32_t)(j - kAhead + 1));
      }
      if (j >= kRing) ok_run = wait_at_least(&consumed[j % kRing], (uint32_t)(kWaves * (j / kRing)));
      if (!ok_run) {
        timed_out(a);
        break;
      }
      if (dl[0] == -2) {  // item j is past the last one: the end marker in its buffer's slot
        if (pw == 0 && lane == 0) desc[j % kRing][0] = -2;
        break;
      }
      RowSrc rs;
      find_rows(j % kTabSlots, dl[0], db[0], dc[0], rs);  // its entries arrived with item j - kAhead - 1
      fetch_tab((j + kAhead + 1) % kTabSlots, dl[ND - 1], db[ND - 1]);
      issue(j % kRing, rs, KZero{}, KAll{});
      post(j % kRing, dl[0], db[0], dz[0], rs.rows);
#pragma unroll
      for (int s2 = 0; s2 < ND - 1; ++s2) {
        dl[s2] = dl[s2 + 1];
        db[s2] = db[s2 + 1];
        dc[s2] = dc[s2 + 1];
        dz[s2] = dz[s2 + 1];
      }
      next_item(dl[ND - 1], db[ND - 1], dc[ND - 1], dz[ND - 1]);
    }
    // everything issued has landed: publish the rest and the end marker
    wait_vmem<0>();
    compiler_fence();
    if (lane == 0) lds_store_u32(&ready[pw], 0x7FFFFFFFu);
    return;
  }

  // ================================================================ score waves
  if (a.num_blocks == 0) return;  // uniform: the fetching waves write the partials
  typedef float f32x16 __attribute__((ext_vector_type(16)));
  const int r32 = lane & 31, h32 = lane >> 5;
  if (wave < kScore) {
    // Score wave sw takes heads 8 sw .. 8 sw + 7: S^T = C [q~hi | q~lo] on
    // v_mfma_f32_16x16x32_bf16 per 16-position block rb, A = positions
    // 16 rb + li (dims 32 s + 8 lg ..), B = 16 columns: the hi parts of its 8
    // heads, then their lo parts (held in registers for the segment). Lane l
    // gets column li at positions 16 rb + 4 lg + r; columns li and li ^ 8 add
    // up to head 8 sw + li % 8's score.
    const int sw = wave;
    const int qrow = (li < 8 ? 0 : 16) + 8 * sw + (li & 7);  // q~ item row of column li, and P row
    bf16x8 qb[KS];
    float m_run = -INFINITY, l_run = 0.0f;  // of head 8 sw + li % 8 (every lane of that head agrees)
    uint32_t k = 0;                         // tiles scored in this workgroup
    for (int i = 0;; ++i) {
      bool ok = true;
#pragma unroll
      for (int p2 = 0; p2 < kProducers; ++p2) ok = ok && wait_at_least(&ready[p2], (uint32_t)(i + 1));
      if (!ok) {
        timed_out(a);
        break;
      }
      const int slot = i % kRing;
      const int lt = uniform(desc[slot][0]);
      if (lt == -2) break;
      const int bb = uniform(desc[slot][1]);
      const int last = uniform(desc[slot][2]);
      const char* tile = ring[slot];
      if (lt == -1) {  // q~ of a new segment: rows 0..15 its hi parts, 16..31 its lo parts
#pragma unroll
        for (int s = 0; s < KS; ++s)
          qb[s] = *reinterpret_cast<const bf16x8*>(tile + qrow * RB + 16 * Gm::phys(qrow, 4 * s + lg));
        m_run = -INFINITY;
        l_run = 0.0f;
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // its reads are done: the buffer may be refilled
        if (lane == 0) lds_add_u32(&consumed[slot], 1u);
        continue;
      }
      const uint32_t valid = uniform(rowmask[slot][0]) | uniform(rowmask[slot][1]);  // bit r: position r takes part
      f32x4 S[2] = {{0.0f, 0.0f, 0.0f, 0.0f}, {0.0f, 0.0f, 0.0f, 0.0f}};
#pragma unroll
      for (int s = 0; s < KS; ++s)
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          const int r = 16 * rb + li;
          const bf16x8 cop = *reinterpret_cast<const bf16x8*>(tile + r * RB + 16 * Gm::phys(r, 4 * s + lg));
          S[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cop, qb[s], S[rb], 0, 0, 0);
        }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the tile's reads are done
      if (lane == 0) lds_add_u32(&consumed[slot], 1u);
      float sc[8];
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float x = S[rb][r];
          const float y = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xF, 0xF, false));  // lane li ^ 8
          const int p = 16 * rb + 4 * lg + r;
          sc[4 * rb + r] = ((valid >> p) & 1u) ? x + y : -INFINITY;
        }
      float mx = sc[0];
#pragma unroll
      for (int v = 1; v < 8; ++v) mx = fmaxf(mx, sc[v]);
      mx = max_over_groups(mx);
      // lazy running max: raised only when the tile's max passes it by more
      // than kLazyMax (first tile: any finite max), so p = 2^(s - m) <= 2^kLazyMax
      const bool raise = mx > m_run + kLazyMax;
      const float mn = raise ? mx : m_run;
      const float mu = (mn == -INFINITY) ? 0.0f : mn;
      const float alpha = raise ? __builtin_amdgcn_exp2f(m_run - mu) : 1.0f;
      float pr[8], ps = 0.0f;
#pragma unroll
      for (int v = 0; v < 8; ++v) {
        pr[v] = __builtin_amdgcn_exp2f(sc[v] - mu);
        ps += pr[v];
      }
      ps = sum_over_groups(ps);
      l_run = l_run * alpha + ps;
      m_run = mn;
      // P to the P.V waves: P row qrow holds head 8 sw + li % 8's bf16 hi part
      // (li < 8) or its lo part, lo = bf16(p - hi): hi + lo is within 2^-17 of
      // the fp32 p. Lane l writes positions 16 rb + 4 lg .. + 3 (8 bytes each).
      const uint32_t pb = k & 1u;
      if (k >= 2 && !wait_at_least(&p_done[pb], kPV * (k / 2u))) {  // tiles k - 2, k - 4, .. have left this buffer
        timed_out(a);
        break;
      }
      char* prow = pbuf[pb] + qrow * kPRow;
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        uint32_t wd[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const float x0 = pr[4 * rb + 2 * e], x1 = pr[4 * rb + 2 * e + 1];
          const uint32_t hi = f32x2_to_bf16x2(x0, x1);
          wd[e] = li < 8 ? hi : f32x2_to_bf16x2(x0 - bf16_lo(hi), x1 - bf16_hi(hi));
        }
        *reinterpret_cast<u32x2*>(prow + 2 * (16 * rb + 4 * lg)) = u32x2{wd[0], wd[1]};
      }
      if (lane < 8) palpha[pb][8 * sw + lane] = alpha;
      if (lane == 0) praise[pb][sw] = __builtin_amdgcn_ballot_w64(raise) != 0 ? 1 : 0;
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      if (lane == 0) lds_add_u32(&p_ready[pb], 1u);
      ++k;
      if (last && lane < 8) {  // the segment's running max and sum of this wave's heads
        const int64_t pslot = (int64_t)w + bb;
        a.ws_m[pslot * kHeads + 8 * sw + lane] = m_run;
        a.ws_l[pslot * kHeads + 8 * sw + lane] = l_run;
      }
    }
    return;
  }

  // ================================================================ P.V waves
  // O2 [32 x 512] += P2 [32 x 32] C [32 x 512] on v_mfma_f32_32x32x16_bf16:
  // P2's rows are the heads' P hi parts, then their lo parts (so O = rows h
  // + rows 16 + h); wave pv owns latent dims 128 pv .. + 127 as 4 blocks of
  // 32. P2's A operand: lane l row r32, positions 16 ks + 8 h32 .. + 7. C's B
  // operand (lane: dim r32 of a block, the same positions) comes by
  // transposing reads: the read of a 16-lane group with base row R and base
  // column Q gives lane i C[R + j][Q + i], j = 0..3. Lane l gets O2's column
  // r32 at rows 8 (v / 4) + 4 h32 + v % 4.
  const int pv = wave - kScore;
  f32x16 acc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) acc[db] = f32x16{};
  uint32_t k = 0;  // tiles multiplied in this workgroup
  const int g = lane >> 4, li16 = lane & 15;
  for (int i = 0;; ++i) {
    bool ok = true;
#pragma unroll
    for (int p2 = 0; p2 < kProducers; ++p2) ok = ok && wait_at_least(&ready[p2], (uint32_t)(i + 1));
    if (!ok) {
      timed_out(a);
      break;
    }
    const int slot = i % kRing;
    const int lt = uniform(desc[slot][0]);
    if (lt == -2) break;
    const int bb = uniform(desc[slot][1]);
    const int last = uniform(desc[slot][2]);
    if (lt == -1) {  // a new segment
#pragma unroll
      for (int db = 0; db < 4; ++db) acc[db] = f32x16{};
      if (lane == 0) lds_add_u32(&consumed[slot], 1u);
      continue;
    }
    const uint32_t valid = uniform(rowmask[slot][0]) | uniform(rowmask[slot][1]);
    const char* tile = ring[slot];
    u32x4 cv[4][2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const int q0 = 128 * pv + 32 * db + 16 * (g & 1) + 4 * (li16 & 3);  // this lane's column address
        const int lc = (2 * q0) >> 4, within = (2 * q0) & 15;
        const int R0 = 16 * ks + 8 * (g >> 1) + (li16 >> 2), R1 = R0 + 4;
        const i16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4*)(tile + R0 * RB + 16 * Gm::phys(R0, lc) + within));
        const i16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4*)(tile + R1 * RB + 16 * Gm::phys(R1, lc) + within));
        cv[db][ks] = __builtin_bit_cast(u32x4, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the tile's reads are done: its buffer may be refilled
    if (lane == 0) lds_add_u32(&consumed[slot], 1u);
    // C elements of masked positions -> 0 (their slots may hold NaN; their p are 0)
    u32x4 vmask[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int p0 = 16 * ks + 8 * h32 + 2 * q;
        vmask[ks][q] = (((valid >> p0) & 1u) ? 0xFFFFu : 0u) | (((valid >> (p0 + 1)) & 1u) ? 0xFFFF0000u : 0u);
      }
    const uint32_t pb = k & 1u;
    if (!wait_at_least(&p_ready[pb], kScore * (k / 2u + 1u))) {  // both score waves' P of tile k
      timed_out(a);
      break;
    }
    // rescale O's rows by their heads' alpha when a score wave raised the max
    if ((uniform(praise[pb][0]) | uniform(praise[pb][1])) != 0) {
      float al[8];  // heads 8 jj + 4 h32 + r: rows 8 j + 4 h32 + r, j = jj, jj + 2
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
#pragma unroll
        for (int r = 0; r < 4; ++r) al[4 * jj + r] = palpha[pb][8 * jj + 4 * h32 + r];
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[db][v] *= al[4 * ((v >> 2) & 1) + (v & 3)];
    }
    bf16x8 pa[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
      pa[ks] = *reinterpret_cast<const bf16x8*>(pbuf[pb] + r32 * kPRow + 2 * (16 * ks + 8 * h32));
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if (lane == 0) lds_add_u32(&p_done[pb], 1u);
    ++k;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int db = 0; db < 4; ++db)
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa[ks], __builtin_bit_cast(bf16x8, cv[db][ks] & vmask[ks]),
                                                         acc[db], 0, 0, 0);
    if (last) {  // the segment's partial O: rows h and 16 + h summed
      const int64_t pslot = (int64_t)w + bb;
      float* o = a.ws_o + pslot * kHeads * kDC + 128 * pv + r32;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int v = 0; v < 8; ++v) {
          const int h = 8 * (v >> 2) + 4 * h32 + (v & 3);
          o[h * kDC + 32 * db] = acc[db][v] + acc[db][v + 8];
        }
    }
  }
}

// ---------------------------------------------------------------- merge
// grid (16 heads, ceil(B / 4)), 8 waves: the partials of each of 4 sequences
// combined into o~ [512] (normalised), then o = o~ W_UV,h. This thread's first
// kMergeW rows of W_UV,h are loaded first; once the tile plan is read (scalar
// loads), the partials' maxima, sums and first kMergeBatch outputs go out in
// one round. Wave w combines sequence b0 + w % 4 over latent dims
// 256 (w / 4) + 4 lane .. + 3; thread (jg, cg) of the product takes 8 output
// dims 8 jg .. and latent rows cg * rows .., and the row groups meet in LDS.
constexpr int kMergeThreads = 512;
constexpr int kMergeBatch = 12; // partial outputs of a sequence loaded in the first round
constexpr int kMergeW = 16;     // W_UV rows of a thread loaded in the first round

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

__global__ __launch_bounds__(kMergeThreads) void mla_merge_kernel(MlaArgs a) {
  const int h = blockIdx.x, b0 = 4 * blockIdx.y, tid = threadIdx.x;
  const int lane = tid & 63, wave = uniform(tid >> 6);
  __shared__ __attribute__((aligned(16))) float ot[4][kDC];
  __shared__ float red[4 * 8 * kMergeThreads];  // [cg][4][dv]: cgs * dv = 8 * kMergeThreads
  const int jgs = a.dv / 8, cgs = kMergeThreads / jgs, rows = kDC / cgs;
  const int jg = tid % jgs, cg = tid / jgs;
  const int64_t wrow = (int64_t)kHeads * a.dv;
  const uint16_t* wbase = static_cast<const uint16_t*>(a.w_uv) + (int64_t)h * a.dv + 8 * jg + (int64_t)cg * rows * wrow;

  // this thread's first rows of W_UV,h: they need nothing the split wrote, so
  // they go out first (the plan below comes by scalar loads, which do not wait
  // behind them)
  u32x4 wv[kMergeW];
#pragma unroll
  for (int r = 0; r < kMergeW; ++r)
    wv[r] = r < rows ? *reinterpret_cast<const u32x4*>(wbase + (int64_t)r * wrow) : u32x4{0u, 0u, 0u, 0u};

  // ---- sequence b0 + bb's partials sit in slots w + b of the workgroups w that served its tiles
  const int bb = wave & 3, hd = wave >> 2;
  const int b = b0 + bb;
  int n = 0, p0 = 0;
  if (b < a.num_seqs) {
    const int T = a.ts[a.num_seqs], tsb = a.ts[b], tse = a.ts[b + 1];
    if (tse > tsb) {  // its tiles are units tsb + 1 .. tse - 1
      const int wf = tile_owner(tsb + 1, T, a.grid), wl = tile_owner(tse - 1, T, a.grid);
      n = wl - wf + 1;
      p0 = wf + b;
    }
  }
  n = uniform(n);
  p0 = uniform(p0);

  // ---- one round of loads
  const int c4 = 256 * hd + 4 * lane;
  float ms = -INFINITY, ls = 0.0f;  // lane s: piece s's max and sum
  if (lane < n) {
    const int64_t i = ((int64_t)p0 + lane) * kHeads + h;
    ms = a.ws_m[i];
    ls = a.ws_l[i];
  }
  f32x4 x[kMergeBatch];
#pragma unroll
  for (int u = 0; u < kMergeBatch; ++u)  // (n is uniform: no load past the count)
    x[u] = u < n ? *reinterpret_cast<const f32x4*>(a.ws_o + (((int64_t)p0 + u) * kHeads + h) * kDC + c4)
                 : f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  // ---- weights 2^(m_s - M), the sum L of their l_s, and o~ = sum_s w_s o_s / L
  float M = ms;
  for (int s = lane + 64; s < n; s += 64) M = fmaxf(M, a.ws_m[((int64_t)p0 + s) * kHeads + h]);
  M = wave_max(M);
  float v[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  float inv = 0.0f;
  if (n > 0 && M != -INFINITY) {  // uniform
    const float wl = lane < n ? __builtin_amdgcn_exp2f(ms - M) : 0.0f;
    float L = wl * ls;
    for (int s = lane + 64; s < n; s += 64) {
      const int64_t i = ((int64_t)p0 + s) * kHeads + h;
      L += __builtin_amdgcn_exp2f(a.ws_m[i] - M) * a.ws_l[i];
    }
    L = wave_sum(L);
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) {
      const float wu = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), u));  // 0 past the count
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = fmaf(wu, x[u][e], v[e]);
    }
    for (int s = kMergeBatch; s < n; ++s) {  // sequences with more pieces
      const int64_t i = ((int64_t)p0 + s) * kHeads + h;
      const float ws = __builtin_amdgcn_exp2f(a.ws_m[i] - M);
      const f32x4 xs = *reinterpret_cast<const f32x4*>(a.ws_o + i * kDC + c4);
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = fmaf(ws, xs[e], v[e]);
    }
    inv = L > 0.0f ? 1.0f / L : 0.0f;
  }
  *reinterpret_cast<f32x4*>(&ot[bb][c4]) = f32x4{v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv};
  __syncthreads();

  // ---- o = o~ W_UV,h over this thread's rows
  float acc[4][8];
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[q][e] = 0.0f;
  auto row_step = [&](const u32x4& w, int c) {
    float wf[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      wf[2 * e] = bf16_lo(w[e]);
      wf[2 * e + 1] = bf16_hi(w[e]);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float xo = ot[q][c];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[q][e] = fmaf(xo, wf[e], acc[q][e]);
    }
  };
#pragma unroll
  for (int r = 0; r < kMergeW; ++r)
    if (r < rows) row_step(wv[r], cg * rows + r);
  for (int r = kMergeW; r < rows; ++r) row_step(*reinterpret_cast<const u32x4*>(wbase + (int64_t)r * wrow), cg * rows + r);
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int e = 0; e < 8; ++e) red[(cg * 4 + q) * a.dv + 8 * jg + e] = acc[q][e];
  __syncthreads();
  const bool failed = uniform(*a.flag) != 0;
  for (int i = tid; i < 4 * a.dv; i += kMergeThreads) {
    const int q = i / a.dv, j = i % a.dv;
    if (b0 + q >= a.num_seqs) continue;
    float o = 0.0f;
    for (int g = 0; g < cgs; ++g) o += red[(g * 4 + q) * a.dv + j];
    if (failed) o = __builtin_nanf("");
    const int64_t oi = (int64_t)(b0 + q) * a.out_seq_stride + (int64_t)h * a.dv + j;
    if (a.out_f32)
      static_cast<float*>(a.out)[oi] = o;
    else
      static_cast<uint16_t*>(a.out)[oi] = (uint16_t)f32_to_bf16(o);
  }
}

struct MlaPlan {
  int row;
  size_t off_qhi, off_qlo, off_ts, off_flag, off_m, off_l, off_o, bytes;
};

size_t round256(size_t x) { return (x + 255) / 256 * 256; }

// One split workgroup per compute unit of the current device, at most
// kMaxGrid (the workspace holds kMaxGrid + B partial slots).
constexpr int kMaxGrid = 256;
pa_status split_grid(const char* fn, int* grid) {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    return fail(PA_EHIP, "%s: cannot read the device's compute-unit count", fn);
  *grid = cus < kMaxGrid ? cus : kMaxGrid;
  return PA_OK;
}

MlaPlan mla_plan(int32_t num_seqs, int32_t rope_dim) {
  MlaPlan p;
  p.row = kDC + rope_dim;
  const size_t B = (size_t)(num_seqs > 0 ? num_seqs : 1);
  const size_t slots = (size_t)kMaxGrid + B;  // partial slot w + b
  size_t off = 0;
  p.off_qhi = off;
  off = round256(off + B * kHeads * p.row * 2);
  p.off_qlo = off;
  off = round256(off + B * kHeads * p.row * 2);
  p.off_ts = off;
  off = round256(off + (B + 1) * 4);
  p.off_flag = off;
  off = round256(off + 4);
  p.off_m = off;
  off = round256(off + slots * kHeads * 4);
  p.off_l = off;
  off = round256(off + slots * kHeads * 4);
  p.off_o = off;
  off = round256(off + slots * kHeads * (size_t)kDC * 4);
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
  return mla_plan(num_seqs, rope_dim).bytes;
}

namespace pa {
namespace {

// The new latent rows of a decode step (null for plain attention).
struct MlaNewRows {
  const void* c;
  int64_t c_stride;
  const void* r;
  int64_t r_stride;
  pa_dtype dtype;
  const int64_t* slots;
};

pa_status mla_launch(const char* fn, const MlaNewRows* nr, void* out, pa_dtype out_dtype, int64_t out_seq_stride,
                     const void* q_nope, int64_t q_nope_seq_stride, const void* q_rope, int64_t q_rope_seq_stride,
                     pa_dtype q_dtype, const void* w_uk, const void* w_uv, pa_dtype w_dtype, const void* latent_cache,
                     pa_dtype cache_dtype, int64_t num_blocks, int32_t block_size, int64_t block_stride,
                     const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
                     int32_t num_seqs, int32_t num_heads, int32_t qk_nope_dim, int32_t rope_dim, int32_t kv_lora_rank,
                     int32_t v_dim, float softmax_scale, void* workspace, size_t workspace_bytes, void* stream) {
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
  if (num_blocks > 0 && (num_blocks * block_stride * 2) / 16 > (int64_t)UINT32_MAX)
    return fail(PA_EUNSUPPORTED, "%s: latent cache above 64 GiB", fn);
  if (num_seqs > (1 << 20)) return fail(PA_EUNSUPPORTED, "%s: more than 2^20 sequences per call", fn);
  if (!aligned(w_uk, 16) || !aligned(w_uv, 16)) return fail(PA_EINVAL, "%s: weights must be 16-byte aligned", fn);
  if (!aligned(q_nope, 16) || (q_nope_seq_stride * 2) % 16 != 0)
    return fail(PA_EINVAL, "%s: q_nope must be 16-byte aligned per sequence", fn);
  if (nr) {
    if (nr->dtype != PA_BF16) return fail(PA_EDTYPE, "%s: new latent rows must be bf16", fn);
    if (!nr->c || !nr->slots || (rope_dim > 0 && !nr->r)) return fail(PA_EINVAL, "%s: null new-row argument", fn);
    if (nr->c_stride < kDC || (rope_dim > 0 && nr->r_stride < rope_dim))
      return fail(PA_EINVAL, "%s: new-row strides below the row widths", fn);
    if (!aligned(nr->c, 16) || (nr->c_stride * 2) % 16 != 0 ||
        (rope_dim > 0 && (!aligned(nr->r, 16) || (nr->r_stride * 2) % 16 != 0)))
      return fail(PA_EINVAL, "%s: new latent rows must be 16-byte aligned per row", fn);
  }
  // the split's units (tiles of 32 positions over all sequences, plus one
  // query item per sequence: at most 2^20 more) must count in 32 bits
  if ((int64_t)num_seqs * (((int64_t)max_blocks_per_seq * block_size + kTile - 1) / kTile) > INT32_MAX / 2)
    return fail(PA_EINVAL, "%s: too many (sequence, tile) items", fn);
  const MlaPlan p = mla_plan(num_seqs, rope_dim);
  if (!workspace || workspace_bytes < p.bytes || !aligned(workspace, 256))
    return fail(PA_EWORKSPACE, "%s: workspace needs %zu bytes, 256-byte aligned (got %zu)", fn, p.bytes, workspace_bytes);
  if (checks_on()) {
    pa_status c = check_tables(fn, reinterpret_cast<hipStream_t>(stream), block_tables, num_seqs,
                               max_blocks_per_seq, context_lens, num_blocks, block_size);
    if (c == PA_OK && nr)
      c = check_slots(fn, reinterpret_cast<hipStream_t>(stream), nr->slots, num_seqs, nullptr, 0, num_blocks,
                      block_size);
    if (c != PA_OK) return c;
  }

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
  a.ts = reinterpret_cast<int32_t*>(ws + p.off_ts);
  a.flag = reinterpret_cast<int32_t*>(ws + p.off_flag);
  a.ws_m = reinterpret_cast<float*>(ws + p.off_m);
  a.ws_l = reinterpret_cast<float*>(ws + p.off_l);
  a.ws_o = reinterpret_cast<float*>(ws + p.off_o);
  a.out_seq_stride = out_seq_stride;
  a.qn_seq_stride = q_nope_seq_stride;
  a.qr_seq_stride = q_rope_seq_stride;
  a.block_stride = block_stride;
  a.num_blocks = num_blocks;
  a.block_size = block_size;
  a.bs_log2 = (block_size & (block_size - 1)) == 0 ? __builtin_ctz((unsigned)block_size) : -1;
  a.W = max_blocks_per_seq;
  a.num_seqs = num_seqs;
  a.qk = qk_nope_dim;
  a.dr = rope_dim;
  a.dv = v_dim;
  a.out_f32 = out_dtype == PA_F32;
  a.scale_log2 = softmax_scale * 1.4426950408889634f;
  a.wcache = nr ? const_cast<uint16_t*>(static_cast<const uint16_t*>(latent_cache)) : nullptr;
  a.new_c = nr ? static_cast<const uint16_t*>(nr->c) : nullptr;
  a.new_r = nr ? static_cast<const uint16_t*>(nr->r) : nullptr;
  a.new_slots = nr ? nr->slots : nullptr;
  a.new_c_stride = nr ? nr->c_stride : 0;
  a.new_r_stride = nr ? nr->r_stride : 0;

  int grid = 0;
  s = split_grid(fn, &grid);
  if (s != PA_OK) return s;
  a.grid = grid;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  mla_absorb_kernel<<<dim3(kHeads, kDC / 64, (unsigned)((num_seqs + 15) / 16 + 1)), 256, 0, st>>>(a, row);
  if (rope_dim == 64)
    mla_split_kernel<64><<<(unsigned)grid, 64 * (kWaves + kProducers), 0, st>>>(a);
  else
    mla_split_kernel<0><<<(unsigned)grid, 64 * (kWaves + kProducers), 0, st>>>(a);
  mla_merge_kernel<<<dim3(kHeads, (unsigned)((num_seqs + 3) / 4)), kMergeThreads, 0, st>>>(a);
  return after_launch(fn);
}

}  // namespace
}  // namespace pa

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
  pa::clear_error();
  return pa::mla_launch("pa_mla_decode_attention", nullptr, out, out_dtype, out_seq_stride, q_nope, q_nope_seq_stride,
                        q_rope, q_rope_seq_stride, q_dtype, w_uk, w_uv, w_dtype, latent_cache, cache_dtype, num_blocks,
                        block_size, block_stride, block_tables, max_blocks_per_seq, context_lens, num_seqs, num_heads,
                        qk_nope_dim, rope_dim, kv_lora_rank, v_dim, softmax_scale, workspace, workspace_bytes, stream);
}

extern "C" pa_status pa_mla_decode_step(const void* new_c, int64_t new_c_stride, const void* new_rope,
                                        int64_t new_rope_stride, pa_dtype new_dtype, const int64_t* new_slots,
                                        void* out, pa_dtype out_dtype, int64_t out_seq_stride, const void* q_nope,
                                        int64_t q_nope_seq_stride, const void* q_rope, int64_t q_rope_seq_stride,
                                        pa_dtype q_dtype, const void* w_uk, const void* w_uv, pa_dtype w_dtype,
                                        void* latent_cache, pa_dtype cache_dtype, int64_t num_blocks,
                                        int32_t block_size, int64_t block_stride, const int32_t* block_tables,
                                        int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t num_seqs,
                                        int32_t num_heads, int32_t qk_nope_dim, int32_t rope_dim,
                                        int32_t kv_lora_rank, int32_t v_dim, float softmax_scale, void* workspace,
                                        size_t workspace_bytes, void* stream) {
  pa::clear_error();
  const pa::MlaNewRows nr = {new_c, new_c_stride, new_rope, new_rope_stride, new_dtype, new_slots};
  return pa::mla_launch("pa_mla_decode_step", &nr, out, out_dtype, out_seq_stride, q_nope, q_nope_seq_stride, q_rope,
                        q_rope_seq_stride, q_dtype, w_uk, w_uv, w_dtype, latent_cache, cache_dtype, num_blocks,
                        block_size, block_stride, block_tables, max_blocks_per_seq, context_lens, num_seqs, num_heads,
                        qk_nope_dim, rope_dim, kv_lora_rank, v_dim, softmax_scale, workspace, workspace_bytes, stream);
}
