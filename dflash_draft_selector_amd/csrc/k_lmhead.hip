// LM head with the top-16 taken in its epilogue: the draft logits
// l[r, v] = bf16(sum_d h[r, d] W[v, d]) never reach memory, only every row's
// top-16 per 256-column tile does ([FT] "Details", runtime: the target's LM head gives
// 16 candidates per slot; [RFC] "Questions", item 4: the draft shares the target's LM
// head).
//
// Stage 1, k_lmhead_tiles: 512-thread work-groups, one round of them resident, each
// running a sequence of 256-column vocabulary tiles (per group of up to 128 rows).  Each
// wave owns two 16-column tiles for every 16-row tile, on v_mfma_f32_16x16x32_bf16 with
// fp32 accumulators.  W rows go straight from HBM into the MFMA B operand (each lane 16
// contiguous bytes of one W row per step), loaded a stage (eight steps) ahead in a
// register ring that runs on from one tile into the next; the hidden rows (read by every
// work-group, so cache-resident) are staged 256 dims at a time through LDS with an XOR
// swizzle, so the 16 rows a wave reads per instruction sit in distinct banks.  The
// epilogue rounds the accumulators to bf16, sorts each row's 32 columns per wave with
// DPP bitonic networks and merges the eight wave lists of every row through LDS, while
// the next tile's first W loads are in flight.
// Stage 2, k_lmhead_merge: one work-group per row merges the row's sorted tile lists.
//
// Selection order: value descending, token id ascending, NaN below -inf (the order of
// dflash2_topk16).
#include "dflash2_internal.h"
#include "topk_dev.h"

namespace df2 {

constexpr int kLmThreads = 512;                       // 8 waves
constexpr int kLmWaves = kLmThreads / kWave;
constexpr int kLmCols = kLmWaves * 2 * 16;            // 256 vocabulary columns per work-group
constexpr int kLmSteps = 8;                           // 32-wide MFMA steps per LDS stage
constexpr int kLmStageDims = kLmSteps * 32;           // 256 hidden dims per stage
constexpr int kLmSlots = kLmStageDims / 8;            // 16-byte slots per staged row (32)
constexpr int kLmMergeThreads = 1024;
constexpr int kLmMaxParts = 8;                        // hidden-dimension parts of a split tile
constexpr int kLmBurst = 2;                           // W ring refills per burst (steps)
static_assert(kLmSteps % kLmBurst == 0, "bursts must tile a stage");

int lmhead_tiles(int64_t vocab) { return (int)((vocab + kLmCols - 1) / kLmCols); }

size_t lmhead_tail_bytes();

LmheadWs carve_lmhead(Carver& c, int64_t rows, int64_t vocab) {
  LmheadWs w;
  w.partials = c.take<unsigned long long>((size_t)rows * lmhead_tiles(vocab) * kNC);
  w.tail_bytes = lmhead_tail_bytes();
  w.tail = c.take<unsigned char>(w.tail_bytes);
  return w;
}

// Byte offset of 16-byte slot c of staged row r: slot c ^ (r % 16) within each group of
// 16 slots, so rows r..r+15 at one slot land on 16 different bank groups.
__device__ __forceinline__ int lm_lds_off(int r, int c) { return r * (kLmSlots * 16) + ((c ^ (r & 15)) << 4); }

// Signed 32-bit rank of a logit in tile column lc (0..255): order key in the high half
// (offset to signed), 0xffff - lc in the low half.  INT_MIN marks a column past the
// vocabulary (below every logit, NaN included).
__device__ __forceinline__ int lm_rank(float x, int lc, bool valid) {
  const int key = (int)bf16_key(f32_to_bf16_rne(x));
  return valid ? (int)(((unsigned)(key - 0x8000) << 16) | (unsigned)(0xffff - lc)) : (int)0x80000000;
}

// Per-lane bounds of the sorting networks' compare-exchanges.  A lane's new value is
// med3(x, partner, c): the larger of the two where c = INT_MAX, the smaller where
// c = INT_MIN, so a compare-exchange is a DPP move and one v_med3_i32 instead of a
// maximum, a minimum and a select.  The bounds go through an empty asm so that the
// compiler, which knows c is one of the two extremes, does not fold the median back.
struct LmBounds {
  int b[10];       // stages (K, J): (2,1) (4,2) (4,1) (8,4) (8,2) (8,1) (16,8) (16,4) (16,2) (16,1)
};

template <int K, int J>
constexpr int lm_bound_index() {
  return K == 2 ? 0 : K == 4 ? (J == 2 ? 1 : 2) : K == 8 ? (J == 4 ? 3 : J == 2 ? 4 : 5)
                                                : (J == 8 ? 6 : J == 4 ? 7 : J == 2 ? 8 : 9);
}

__device__ __forceinline__ int lm_bound(int i, int K, int J) {
  // the orientation of bitonic_stage_i32: blocks of K lanes largest first where lane bit
  // K is clear (and for K = 16); the lower lane of a pair at distance J keeps the larger
  const bool desc = K >= 16 || (i & K) == 0;
  int c = (((i & J) == 0) == desc) ? 0x7fffffff : (int)0x80000000;
  asm("" : "+v"(c));
  return c;
}

// This lane's index in its wave, computed where it is used: the tile kernel runs its
// epilogue inside the loop over tiles, and a lane-derived value the compiler hoisted out
// of that loop would stay live (and spill) across the main loop.
__device__ __forceinline__ int lm_lane_here() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

__device__ __forceinline__ LmBounds lm_bounds(int lane) {
  const int i = lane & 15;
  return LmBounds{{lm_bound(i, 2, 1), lm_bound(i, 4, 2), lm_bound(i, 4, 1), lm_bound(i, 8, 4), lm_bound(i, 8, 2),
                   lm_bound(i, 8, 1), lm_bound(i, 16, 8), lm_bound(i, 16, 4), lm_bound(i, 16, 2),
                   lm_bound(i, 16, 1)}};
}

template <int K, int J>
__device__ __forceinline__ int lm_stage(int x, const LmBounds& bd) {
  const int p = row_partner_i32<J>(x);
  const int c = bd.b[lm_bound_index<K, J>()];
  return max(min(x, p), min(max(x, p), c));     // med3(x, p, c)
}

// Full descending sort of the 16 values held by each 16-lane row, for N independent
// registers at once (Batcher's bitonic sort: blocks of 2, 4, 8, then the 16-lane
// half-cleaners).  Each stage is applied to all N before the next, so the independent
// DPP moves fill each other's wait states.
template <int N>
__device__ __forceinline__ void row16_full_sort_i32(int (&x)[N], const LmBounds& bd) {
#define DF2_STAGE(K, J)                                              \
  _Pragma("unroll") for (int n = 0; n < N; ++n) x[n] = lm_stage<K, J>(x[n], bd);
  DF2_STAGE(2, 1) DF2_STAGE(4, 2) DF2_STAGE(4, 1) DF2_STAGE(8, 4) DF2_STAGE(8, 2) DF2_STAGE(8, 1)
  DF2_STAGE(16, 8) DF2_STAGE(16, 4) DF2_STAGE(16, 2) DF2_STAGE(16, 1)
#undef DF2_STAGE
}

// The bitonic half-cleaners (distances 8, 4, 2, 1) on N independent registers.
template <int N>
__device__ __forceinline__ void row16_bitonic_sort_i32(int (&x)[N], const LmBounds& bd) {
#pragma unroll
  for (int n = 0; n < N; ++n) x[n] = lm_stage<16, 8>(x[n], bd);
#pragma unroll
  for (int n = 0; n < N; ++n) x[n] = lm_stage<16, 4>(x[n], bd);
#pragma unroll
  for (int n = 0; n < N; ++n) x[n] = lm_stage<16, 2>(x[n], bd);
#pragma unroll
  for (int n = 0; n < N; ++n) x[n] = lm_stage<16, 1>(x[n], bd);
}

// Tile list entry -> row composite of dflash2_topk16 (0 = empty).
__device__ __forceinline__ unsigned long long lm_rank_to_rc(int rank, int col0) {
  if (rank == (int)0x80000000) return 0ull;
  const uint32_t key = (uint32_t)((rank >> 16) + 0x8000);
  const uint32_t id = (uint32_t)(col0 + (0xffff - (rank & 0xffff)));
  uint32_t bits;
  if (key == 0u)
    bits = 0x7fc0u;                                   // NaN
  else if (key >= 0x8000u)
    bits = key - 0x8000u;                             // +0 and positive values
  else
    bits = 0x8000u | (0x8000u - key);                 // negative values
  return make_rc(key, id, bits);
}

// Per-row top-16 of one tile from the accumulators (the whole work-group calls it):
// acc[m][nt][r] is row 16 m + 4 g + r, column 32 wv + 16 nt + i16 of the tile.  Rounds
// to bf16, sorts each row's 32 columns per wave, merges the eight wave lists of every
// row through LDS (`lists`, [MT * 16 rows][8 waves][16], MT * 8 KB, free on entry) and
// writes the tile's lists.  wv: this wave's index in the work-group.
template <int MT>
__device__ __forceinline__ void lm_tile_top16(const f32x4 (&acc)[MT][2], int* lists, int tile, int rows, int row0,
                                              int vocab, int ntiles, int wv,
                                              unsigned long long* __restrict__ partials) {
  const int lane = lm_lane_here();
  const int g = lane >> 4, i16 = lane & 15;
  const int col0 = tile * kLmCols;
  const LmBounds bd = lm_bounds(lane);
  // (m, r) pairs two at a time: sort both halves of each pair's 32 columns, keep the
  // top 16 of the two sorted halves (the maximum against the other half reversed is
  // bitonic) and sort that
  static_assert((MT * 4) % 2 == 0, "pairs are taken two at a time");
  const int lc0 = 32 * wv + i16, lc1 = lc0 + 16;
  const bool v0 = col0 + lc0 < vocab, v1 = col0 + lc1 < vocab;
#pragma unroll
  for (int k = 0; k < MT * 4; k += 2) {
    const int m0 = k >> 2, r0 = k & 3, m1 = (k + 1) >> 2, r1 = (k + 1) & 3;
    int x[4] = {lm_rank(acc[m0][0][r0], lc0, v0), lm_rank(acc[m0][1][r0], lc1, v1),
                lm_rank(acc[m1][0][r1], lc0, v0), lm_rank(acc[m1][1][r1], lc1, v1)};
    row16_full_sort_i32<4>(x, bd);
    int y[2] = {max(x[0], dpp_i32<0x140>(x[1])), max(x[2], dpp_i32<0x140>(x[3]))};   // row_mirror
    row16_bitonic_sort_i32<2>(y, bd);
    lists[((16 * m0 + 4 * g + r0) * kLmWaves + wv) * kNC + i16] = y[0];
    lists[((16 * m1 + 4 * g + r1) * kLmWaves + wv) * kNC + i16] = y[1];
  }
  __syncthreads();
  // every wave merges the eight lists of rows wv, wv + 8, ..., two rows at a time:
  // lane row q takes lists 2q and 2q + 1 (the second reversed), then the rows merge
  // pairwise (the maximum against the mirrored partner row is bitonic)
  static_assert((MT * 16) % (2 * kLmWaves) == 0, "two rows per wave per pass");
  for (int rl = wv; rl < MT * 16; rl += 2 * kLmWaves) {
    const int* L0 = lists + rl * kLmWaves * kNC;
    const int* L1 = lists + (rl + kLmWaves) * kLmWaves * kNC;
    int x[2] = {max(L0[(2 * g) * kNC + i16], L0[(2 * g + 1) * kNC + (kNC - 1 - i16)]),
                max(L1[(2 * g) * kNC + i16], L1[(2 * g + 1) * kNC + (kNC - 1 - i16)])};
    row16_bitonic_sort_i32<2>(x, bd);
#pragma unroll
    for (int msk = 16; msk <= 32; msk *= 2) {
      x[0] = max(x[0], xor_lane_i32(dpp_i32<0x140>(x[0]), msk));
      x[1] = max(x[1], xor_lane_i32(dpp_i32<0x140>(x[1]), msk));
      row16_bitonic_sort_i32<2>(x, bd);
    }
    if (lane < kNC && row0 + rl < rows)
      partials[((size_t)(row0 + rl) * ntiles + tile) * kNC + lane] = lm_rank_to_rc(x[0], col0);
    if (lane < kNC && row0 + rl + kLmWaves < rows)
      partials[((size_t)(row0 + rl + kLmWaves) * ntiles + tile) * kNC + lane] = lm_rank_to_rc(x[1], col0);
  }
}

// The work of one group of rows is a sequence of units: units [0, nfull) are whole tiles
// (tile k over the whole hidden dimension, ending with its top-16); the rest split the
// remaining tiles along the hidden dimension, nparts units per tile (the last round of a
// vocabulary that does not fill the chip in whole rounds would otherwise run few
// work-groups): each sums its share of the stages and stores the fp32 tile
// (tail[(tail tile, part)][wave][m][nt][lane], f32x4), and k_lmhead_combine adds the
// parts in order and takes the top-16 of each 16-row tile.
struct LmUnit {
  int tile, s0, ns;    // the unit's tile and its stages s0 .. s0 + ns - 1
};

__device__ __forceinline__ LmUnit lm_unit(int k, int nfull, int nparts, int nstages) {
  if (k < nfull) return LmUnit{k, 0, nstages};
  const int u = k - nfull, part = u % nparts;
  const int s0 = (int)((long long)nstages * part / nparts);
  return LmUnit{nfull + u / nparts, s0, (int)((long long)nstages * (part + 1) / nparts) - s0};
}

// Each work-group runs units blockIdx.x, blockIdx.x + gridDim.x, ... back to back (the
// grid is one round of resident work-groups), and its W ring runs on across them: the
// last half-stages of a unit refill the ring with the next unit's first ones, and the
// next unit's first hidden stage is loaded with them, so those loads are in flight while
// the unit's epilogue sorts.
// PACKED: W in the packed layout of lm_packed_offset (each load instruction one contiguous 1 KB), else
// row-major [vocab][hidden] (each instruction 64 bytes of 16 rows).
template <int MT, bool PACKED>
__global__ void __launch_bounds__(kLmThreads) k_lmhead_tiles(const uint16_t* __restrict__ h,
                                                              const uint16_t* __restrict__ w, int rows, int hidden,
                                                              int vocab, int row0, int ntiles, int nfull, int nparts,
                                                              unsigned long long* __restrict__ partials,
                                                              f32x4* __restrict__ tail) {
  // the staged hidden rows, and the epilogue's sorted lists (apart, so that the next
  // unit's first stage is staged before the epilogue)
  __shared__ __align__(16) unsigned char lds[MT * 16 * kLmSlots * 16];
  __shared__ int lists[MT * 16 * kLmWaves * kNC];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, i16 = lane & 15;
  const int nstages = hidden / kLmStageDims;
  const int nunits = nfull + (ntiles - nfull) * nparts;
  const int stride = (int)gridDim.x;
  constexpr int kHalf = kLmSteps / 2;
  constexpr int kPk = kLmWaves * 512;                  // elements of one packed (step, column tile) slice

  // W of tile t, half-stage ha of the hidden dimension: a uniform base, plus per lane
  // its 16 bytes of every packed 1 KB slice, or the offset of its row (column of the
  // tile; a column past the vocabulary reads the last row, unused) and dims
  auto wbase = [&](int t, int ha) -> const uint16_t* {
    if constexpr (PACKED)
      return w + (size_t)t * kLmCols * hidden + (size_t)ha * kHalf * 2 * kPk;
    else
      return w + (size_t)t * kLmCols * hidden + (size_t)ha * (kLmStageDims / 2);
  };
  auto wlane = [&](int t, int nt) -> unsigned {
    if constexpr (PACKED) {
      return (unsigned)(nt * kPk + wv * 512 + lane * 8);
    } else {
      const int last = vocab - 1 - t * kLmCols;
      const int lc = 32 * wv + 16 * nt + i16;
      return (unsigned)((lc < last ? lc : last) * hidden + 8 * g);
    }
  };
  // The half-stage at b as a buffer resource; `live` false gives one of no records,
  // whose loads return zero without touching memory (past the last unit: the loads are
  // still issued, so that the compiler's wait counts stay the same on every path).
  auto wres = [&](const uint16_t* b, bool live) -> __amdgpu_buffer_rsrc_t {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(b), (short)0, live ? 0x7fffffff : 0, 0x00020000);
  };
  // W fragment of step s of a half-stage, column tile nt (lane element offset o)
  auto wfrag = [&](__amdgpu_buffer_rsrc_t rs, unsigned o, int s) -> u32x4 {
    return __builtin_amdgcn_raw_buffer_load_b128(rs, 2 * (o + (PACKED ? s * 2 * kPk : 32 * s)), 0, 0);
  };

  // staging of one 256-dim stage of the hidden rows: thread slot e covers row
  // (tid + 512 e) / 32, 16-byte slot (tid + 512 e) % 32; rows past the group are zero,
  // their loads skipped (reading a valid row for them instead, so that every path issues
  // the same loads, measured 2-5% slower: every padding lane of the chip then reads the
  // same few lines)
  auto load_h = [&](int st, u32x4 (&hp)[MT]) {
#pragma unroll
    for (int e = 0; e < MT; ++e) {
      const int idx = tid + kLmThreads * e;
      const int r = idx / kLmSlots, c = idx % kLmSlots;
      const int grow = row0 + r;
      const u32x4 v = *reinterpret_cast<const u32x4*>(h + (size_t)(grow < rows ? grow : rows - 1) * hidden +
                                                      st * kLmStageDims + 8 * c);
      hp[e] = grow < rows ? v : (u32x4){0u, 0u, 0u, 0u};
    }
  };
  auto store_h = [&](const u32x4 (&hp)[MT]) {
    // row tid / 32 + 16 e has the swizzle of row tid / 32: one offset, plus e rows of 16
    const int base = lm_lds_off(tid / kLmSlots, tid % kLmSlots);
#pragma unroll
    for (int e = 0; e < MT; ++e)
      *reinterpret_cast<u32x4*>(lds + base + e * (kLmThreads / kLmSlots) * kLmSlots * 16) = hp[e];
  };

  // this work-group's units k, k + gridDim.x, ...: the current one and the next.
  int k = (int)blockIdx.x;
  if (k >= nunits) return;
  LmUnit cu = lm_unit(k, nfull, nparts, nstages);
  bool more = k + stride < nunits;
  LmUnit nu = more ? lm_unit(k + stride, nfull, nparts, nstages) : cu;

  f32x4 acc[MT][2];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) acc[m][nt] = (f32x4){0.f, 0.f, 0.f, 0.f};

  // W ring: the two half-stages (4 MFMA steps each) of a stage in registers, wr0 and
  // wr1.  Each half refills its slot, kLmBurst steps at a time, with the same half of the
  // unit's next stage or, on the unit's last stage, of the next unit's first one, so
  // that the next unit starts with its first stage loaded; past the last unit it reloads
  // nothing (loads of no records).  Every path issues the same W loads, so that waiting
  // for a hidden slice leaves the ring's loads in flight.
  // The two 64-byte halves of every 128-byte line of a row-major W row are requested back
  // to back.  Plain loads: the line stays in L2 for its second half (non-temporal loads
  // measured 25% slower).
  u32x4 wr0[kHalf][2], wr1[kHalf][2];
  auto fill = [&](u32x4 (&wr)[kHalf][2], int part_h) {
    const __amdgpu_buffer_rsrc_t rs = wres(wbase(cu.tile, 2 * cu.s0 + part_h), true);
    const unsigned o0 = wlane(cu.tile, 0), o1 = wlane(cu.tile, 1);
#pragma unroll
    for (int s = 0; s < kHalf; ++s) {
      wr[s][0] = wfrag(rs, o0, s);
      wr[s][1] = wfrag(rs, o1, s);
    }
  };
  fill(wr0, 0);
  fill(wr1, 1);

  u32x4 hp[MT];
  load_h(cu.s0, hp);
  store_h(hp);
  __syncthreads();

  // Half part_h of a stage, on ring slot part_h.  sn: the stage loaded meanwhile, of
  // tile tn (this unit's next stage or the next unit's first); live false past the last
  // unit (sn is then this stage: its hidden slice is staged again, to no use, and the W
  // refills read nothing).  The W refills stay where they are written
  // (scheduling barriers), a half-stage ahead of their use, and the hidden slice is
  // staged on every path, so that the compiler does not sink its loads next to their use
  // (into the branch that would stage it), which would wait for the whole ring there.
  auto half = [&](u32x4 (&wr)[kHalf][2], const int part_h, const int tn, const int sn, const bool live) {
    if (part_h == 0) load_h(sn, hp);                  // the next staged hidden slice
    const __amdgpu_buffer_rsrc_t rs = wres(wbase(tn, 2 * sn + part_h), live);   // this ring slot's refill
    const unsigned o0 = wlane(tn, 0), o1 = wlane(tn, 1);
#pragma unroll
    for (int s = 0; s < kHalf; ++s) {
      const int step = kHalf * part_h + s;
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(lds + lm_lds_off(16 * m + i16, 4 * step + g));
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
          acc[m][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                               __builtin_bit_cast(bf16x8, wr[s][nt]), acc[m][nt],
                                                               0, 0, 0);
      }
      if ((s + 1) % kLmBurst == 0) {
#pragma unroll
        for (int q = s + 1 - kLmBurst; q <= s; ++q) {
          wr[q][0] = wfrag(rs, o0, q);
          wr[q][1] = wfrag(rs, o1, q);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (part_h == 1) {
      __syncthreads();
      store_h(hp);
      __syncthreads();
    }
  };

  for (;;) {
    for (int st = 0; st < cu.ns; ++st) {
      const bool own = st + 1 < cu.ns;
      const int tn = own || !more ? cu.tile : nu.tile;
      const int sn = own ? cu.s0 + st + 1 : more ? nu.s0 : cu.s0 + st;
      half(wr0, 0, tn, sn, own || more);
      half(wr1, 1, tn, sn, own || more);
    }
    // the unit is done: its top-16, or its part
    if (k < nfull) {
      lm_tile_top16<MT>(acc, lists, cu.tile, rows, row0, vocab, ntiles, wv, partials);
    } else {
      f32x4* dst = tail + ((size_t)(k - nfull) * kLmWaves + wv) * MT * 2 * kWave + lm_lane_here();
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) dst[(m * 2 + nt) * kWave] = acc[m][nt];
    }
    if (!more) break;
    k += stride;
    cu = nu;
    more = k + stride < nunits;
    if (more) nu = lm_unit(k + stride, nfull, nparts, nstages);
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) acc[m][nt] = (f32x4){0.f, 0.f, 0.f, 0.f};
  }
}

// The split tiles: one work-group per (tile, 16-row tile) adds the nparts partial
// accumulators of its rows in part order (two parts' loads in flight at a time), then
// takes their top-16 as the whole-tile work-groups do.  Spreading the combine over
// MT x as many work-groups keeps its sorting off a few compute units.
template <int MT>
__global__ void __launch_bounds__(kLmThreads) k_lmhead_combine(const f32x4* __restrict__ tail, int nparts, int rows,
                                                                int vocab, int row0, int ntiles, int nfull,
                                                                unsigned long long* __restrict__ partials) {
  __shared__ int lists[16 * kLmWaves * kNC];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int tt = (int)blockIdx.x / MT, m = (int)blockIdx.x % MT;
  constexpr size_t kPart = (size_t)kLmWaves * MT * 2 * kWave;
  const f32x4* src = tail + ((size_t)tt * nparts * kLmWaves + wv) * MT * 2 * kWave + m * 2 * kWave + lane;
  f32x4 acc[1][2];
  for (int p0 = 0; p0 < nparts; p0 += 2) {
    const bool two = p0 + 1 < nparts;
    const f32x4* s0 = src + (size_t)p0 * kPart;
    const f32x4* s1 = src + (size_t)(two ? p0 + 1 : p0) * kPart;   // a missing second part is not added
    f32x4 v0[2], v1[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      v0[nt] = s0[nt * kWave];
      v1[nt] = s1[nt * kWave];
    }
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      acc[0][nt] = p0 == 0 ? v0[nt] : acc[0][nt] + v0[nt];
      if (two) acc[0][nt] += v1[nt];
    }
  }
  lm_tile_top16<1>(acc, lists, nfull + tt, rows, row0 + 16 * m, vocab, ntiles, wv, partials);
}

// Top-16 of a row's ntiles sorted tile lists: 64 lane rows each merge every 64th list
// in registers, the waves merge their four rows, and wave 0 the sixteen wave lists.
__global__ void __launch_bounds__(kLmMergeThreads) k_lmhead_merge(const unsigned long long* __restrict__ partials,
                                                                   int ntiles, int32_t* __restrict__ cand_idx,
                                                                   float* __restrict__ cand_val,
                                                                   int32_t* __restrict__ row_status) {
  constexpr int kGroups = kLmMergeThreads / kNC;      // 64 lane rows
  constexpr int kBatch = 16;                          // lists loaded before merging (one pass up to 1024 tiles)
  __shared__ unsigned long long wl[kLmMergeThreads / kWave][kNC];
  const int row = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int grp = tid >> 4, i = tid & 15;
  const unsigned long long* src = partials + (size_t)row * ntiles * kNC;
  unsigned long long x = 0ull;
  for (int base = grp; base < ntiles; base += kGroups * kBatch) {
    unsigned long long y[kBatch];
#pragma unroll
    for (int c = 0; c < kBatch; ++c) {
      const int t = base + kGroups * c;
      y[c] = t < ntiles ? src[(size_t)t * kNC + (kNC - 1 - i)] : 0ull;   // reversed: merge16 takes b reversed
    }
#pragma unroll
    for (int c = 0; c < kBatch; ++c) x = merge16(x, y[c]);
  }
  x = merge16(x, xor_lane_u64(dpp_u64<0x140>(x), 16));
  x = merge16(x, xor_lane_u64(dpp_u64<0x140>(x), 32));
  if (lane < kNC) wl[wv][lane] = x;
  __syncthreads();
  if (wv != 0) return;
  const int q = lane >> 4;
  x = wl[4 * q][i];
#pragma unroll
  for (int c = 1; c < 4; ++c) x = merge16(x, wl[4 * q + c][kNC - 1 - i]);
  x = merge16(x, xor_lane_u64(dpp_u64<0x140>(x), 16));
  x = merge16(x, xor_lane_u64(dpp_u64<0x140>(x), 32));
  const float v = bf16_to_f32(rc_bits(x));
  const bool bad = __ballot(lane < kNC && !__builtin_isfinite(v)) != 0ull;
  if (lane < kNC) {
    cand_idx[(size_t)row * kNC + lane] = x ? rc_id(x) : 0;
    cand_val[(size_t)row * kNC + lane] = v;
  }
  if (row_status && lane == 0) row_status[row] = bad ? 1 : 0;
}

// Work-groups of k_lmhead_tiles<MT, PACKED> resident per compute unit.
template <int MT, bool PACKED>
static int lmhead_per_cu() {
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_lmhead_tiles<MT, PACKED>, kLmThreads, 0) !=
          hipSuccess ||
      per_cu < 1)
    per_cu = 1;
  return per_cu;
}

template <int MT, bool PACKED>
static void lmhead_group(hipStream_t s, const uint16_t* h, const uint16_t* w, int rows, int hidden, int vocab,
                         int row0, int dev_cus, const LmheadWs& ws) {
  const int ntiles = lmhead_tiles(vocab);
  const int nstages = hidden / kLmStageDims;
  const int per_cu = lmhead_per_cu<MT, PACKED>();
  const int round = per_cu * dev_cus;                  // the work-groups of one full round
  const int tail = ntiles % round;
  int nparts = 1;
  // a last round under half full: split its tiles so that it fills the chip
  if (tail > 0 && 2 * tail <= round && ntiles > round) {
    nparts = round / tail;
    if (nparts > nstages) nparts = nstages;
    if (nparts > kLmMaxParts) nparts = kLmMaxParts;
    const size_t need = (size_t)tail * nparts * kLmWaves * MT * 2 * kWave * sizeof(f32x4);
    if (need > ws.tail_bytes) nparts = 1;
  }
  const int nfull = nparts > 1 ? ntiles - tail : ntiles;
  const int nunits = nfull + (nparts > 1 ? tail * nparts : 0);
  // one round of work-groups runs the units in turn (each every grid-th one), so that a
  // tile's epilogue overlaps the next tile's first loads
  const int grid = nunits < round ? nunits : round;
  hipLaunchKernelGGL((k_lmhead_tiles<MT, PACKED>), dim3((unsigned)grid), dim3(kLmThreads), 0, s, h, w, rows, hidden,
                     vocab, row0, ntiles, nfull, nparts, ws.partials, reinterpret_cast<f32x4*>(ws.tail));
  if (nparts > 1)
    hipLaunchKernelGGL((k_lmhead_combine<MT>), dim3((unsigned)(tail * MT)), dim3(kLmThreads), 0, s,
                       reinterpret_cast<const f32x4*>(ws.tail), nparts, rows, vocab, row0, ntiles, nfull,
                       ws.partials);
}

size_t lmhead_tail_bytes() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
    cus = 256;
  // a split round holds at most one round of work-groups, and (work-groups per compute
  // unit) x MT <= 8 for every instance, so one round needs at most cus x 8 x 16 KB
  return (size_t)cus * 8 * 16 * 1024;
}

template <bool PACKED>
static void lmhead_groups(hipStream_t s, const uint16_t* h, const uint16_t* w, int rows, int hidden, int vocab,
                          int cus, const LmheadWs& ws) {
  for (int row0 = 0; row0 < rows; row0 += kLmMaxRows) {
    const int n = rows - row0 < kLmMaxRows ? rows - row0 : kLmMaxRows;
    if (n <= 16)
      lmhead_group<1, PACKED>(s, h, w, rows, hidden, vocab, row0, cus, ws);
    else if (n <= 32)
      lmhead_group<2, PACKED>(s, h, w, rows, hidden, vocab, row0, cus, ws);
    else if (n <= 64)
      lmhead_group<4, PACKED>(s, h, w, rows, hidden, vocab, row0, cus, ws);
    else if (n <= 112)
      lmhead_group<7, PACKED>(s, h, w, rows, hidden, vocab, row0, cus, ws);
    else
      lmhead_group<8, PACKED>(s, h, w, rows, hidden, vocab, row0, cus, ws);
  }
}

hipError_t launch_lmhead_topk16(const uint16_t* h, const uint16_t* w, bool packed, int rows, int hidden, int vocab,
                                int32_t* cand_idx, float* cand_val, int32_t* row_status, LmheadWs ws,
                                hipStream_t s) {
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  if (packed)
    lmhead_groups<true>(s, h, w, rows, hidden, vocab, cus, ws);
  else
    lmhead_groups<false>(s, h, w, rows, hidden, vocab, cus, ws);
  hipLaunchKernelGGL(k_lmhead_merge, dim3((unsigned)rows), dim3(kLmMergeThreads), 0, s, ws.partials,
                     lmhead_tiles(vocab), cand_idx, cand_val, row_status);
  return hipGetLastError();
}

// ---- the packed weight ---------------------------------------------------------------
// Tile T of 256 vocabulary columns, 32-dim step k of the hidden dimension: 16 KB laid out
// [column tile nt (2)][wave (8)][dim group g (4)][column i (16)][8 dims], column
// 256 T + 32 wave + 16 nt + i, dims 32 k + 8 g .. + 7: each 1 KB is one MFMA B-operand
// slice of one wave, lane 16 g + i reading its 16 bytes.  Columns past the vocabulary
// are zero.
size_t lmhead_packed_elems(int64_t vocab, int64_t hidden) { return (size_t)lmhead_tiles(vocab) * kLmCols * hidden; }

// One thread per 16-byte piece of the packed weight.
__global__ void __launch_bounds__(256) k_lmhead_pack(const uint16_t* __restrict__ w, int vocab, int hidden,
                                                      uint16_t* __restrict__ wp, size_t npieces) {
  const size_t p = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (p >= npieces) return;
  const int lane = (int)(p & 63);
  const size_t q = p >> 6;                           // (T * nsteps + k) * 16 + nt * 8 + wave
  const int wave = (int)(q & 7), nt = (int)((q >> 3) & 1);
  const size_t tk = q >> 4;
  const int nsteps = hidden / 32;
  const int k = (int)(tk % nsteps);
  const int T = (int)(tk / nsteps);
  const int col = T * kLmCols + 32 * wave + 16 * nt + (lane & 15);
  const int d0 = 32 * k + 8 * (lane >> 4);
  u32x4 v = (u32x4){0u, 0u, 0u, 0u};
  if (col < vocab) v = *reinterpret_cast<const u32x4*>(w + (size_t)col * hidden + d0);
  *reinterpret_cast<u32x4*>(wp + p * 8) = v;
}

hipError_t launch_lmhead_pack(const uint16_t* w, int vocab, int hidden, uint16_t* wp, hipStream_t s) {
  const size_t npieces = lmhead_packed_elems(vocab, hidden) / 8;
  hipLaunchKernelGGL(k_lmhead_pack, dim3((unsigned)((npieces + 255) / 256)), dim3(256), 0, s, w, vocab, hidden, wp,
                     npieces);
  return hipGetLastError();
}

}  // namespace df2
