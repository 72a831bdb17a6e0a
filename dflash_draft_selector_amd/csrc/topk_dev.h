// Split-vocabulary top-16 over bf16 logits rows.  A work-group streams one chunk of a
// row.  Its waves sort their lanes' maxima, and the 16th largest of the block's 512 lane
// maxima bounds the chunk's 16th best logit from below (16 lanes hold a logit at least
// that large), so only the few logits at or above it are gathered, with exact keys, and
// one wave ranks them into the chunk's sorted top-16.  When too few or too many survive,
// every wave selects its own top-16 exactly and one wave merges the eight lists with a
// bitonic network.  The chunks of a row are merged afterwards with the same network.
// Selection order: value descending, token id ascending, -0 == +0, NaN below -inf
// (pegainfer issue "DFlash 2 proposer", section "What upstream shipped", item 1: keep
// the top-16 candidates per position).
#pragma once

#include "device_common.h"

namespace df2 {

constexpr int kTopkThreads = 512;                            // 8 waves
constexpr int kTopkWaves = kTopkThreads / kWave;
constexpr int kTopkVecPerThread = 19;                        // 19 x 16 B loads in flight per lane
constexpr int kChunkVec = kTopkThreads * kTopkVecPerThread;  // 9728 vectors = 77824 logits
constexpr int kWaveCapVec = 64;                              // candidate vectors kept per wave
constexpr int kBlockCapCand = 128;                           // candidate logits kept per block
constexpr int kMaxChunks = 7;                                // vocab <= 7 * 77824 (2^19 and more)

typedef short s16x2 __attribute__((ext_vector_type(2)));

// Row composite of a logit: (order key << 48) | ((0xfffff - token id) << 28) | bf16 bits.
// Larger = better (higher value, then lower id); unique per token; 0 = empty slot.
__device__ __forceinline__ unsigned long long make_rc(uint32_t key, uint32_t id, uint32_t bits) {
  return ((unsigned long long)key << 48) | ((unsigned long long)(0xfffffu - id) << 28) | (unsigned long long)bits;
}
__device__ __forceinline__ int rc_id(unsigned long long rc) { return (int)(0xfffffu - (uint32_t)((rc >> 28) & 0xfffffu)); }
__device__ __forceinline__ uint32_t rc_bits(unsigned long long rc) { return (uint32_t)(rc & 0xffffu); }

struct ChunkShared {
  u32x4 vec_data[kTopkWaves][kWaveCapVec];                  // each wave's candidate vectors
  unsigned int vec_pos[kTopkWaves][kWaveCapVec];            // and their positions in the chunk
  int lane_top[2][kTopkWaves][kNC];                         // sorted lane maxima (raw, signed order)
  unsigned long long cand[kBlockCapCand + 8];               // the block's candidate logits
  unsigned long long lists[kTopkWaves * kNC];               // exact per-wave top-16s (fallback)
  unsigned int ncand;
  unsigned int overflow;
};

// Signed 16-bit order of a bf16 pattern, two per word: flip the magnitude bits of
// negative values.  Monotone in the value for non-NaN inputs except that -0 sits one
// below +0; +NaN lands above +inf and -NaN below -inf.
__device__ __forceinline__ s16x2 signed_order2(uint32_t w) {
  const s16x2 x = __builtin_bit_cast(s16x2, w);
  const s16x2 sm = x >> (s16x2){15, 15};
  return x ^ (sm & (s16x2){0x7fff, 0x7fff});
}

// The two patterns of a word as signed 16-bit integers.  The word is taken by value:
// clang's __builtin_bit_cast applied directly to an ext_vector component reads the
// vector's first component instead.
__device__ __forceinline__ s16x2 raw_order2(uint32_t w) { return __builtin_bit_cast(s16x2, w); }

__device__ __forceinline__ int max_halves(s16x2 v) { return v.x > v.y ? (int)v.x : (int)v.y; }

// Inverse of the signed order (it is an involution on 16-bit patterns).
__device__ __forceinline__ uint32_t order_to_bits(int s) {
  const uint32_t u = (uint32_t)s & 0xffffu;
  return u ^ ((u & 0x8000u) ? 0x7fffu : 0u);
}

__device__ __forceinline__ uint32_t elem_bits(const u32x4& d, int e) {
  const uint32_t w = d[e >> 1];
  return (e & 1) ? (w >> 16) : (w & 0xffffu);
}

// Orders this wave's LDS writes before its later LDS reads by other lanes.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ---- bitonic merging of sorted top-16 lists ------------------------------------------
// A 16-lane row of a wave holds one list, slot i in lane i (row lane = lane & 15).
// The 64-bit moves use DPP within a row and ds_bpermute across rows.

template <int CTRL>
__device__ __forceinline__ unsigned long long dpp_u64(unsigned long long v) {
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, CTRL, 0xf, 0xf, true);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v >> 32), CTRL, 0xf, 0xf, true);
  return ((unsigned long long)(uint32_t)hi << 32) | (uint32_t)lo;
}

// Value of lane (lane ^ m) of the wave.
__device__ __forceinline__ unsigned long long xor_lane_u64(unsigned long long v, int m) {
  const int addr = ((threadIdx.x & 63) ^ m) << 2;
  const int lo = __builtin_amdgcn_ds_bpermute(addr, (int)(uint32_t)v);
  const int hi = __builtin_amdgcn_ds_bpermute(addr, (int)(uint32_t)(v >> 32));
  return ((unsigned long long)(uint32_t)hi << 32) | (uint32_t)lo;
}

// Compare-exchange with the partner's value: the lane keeps the larger when keep_max.
__device__ __forceinline__ unsigned long long cmpx(unsigned long long x, unsigned long long p, bool keep_max) {
  return ((x > p) == keep_max) ? x : p;
}

// Sorts, largest first, a bitonic sequence held by each 16-lane row: half-cleaners at
// distances 8, 4, 2, 1 (Batcher's bitonic sorter).
__device__ __forceinline__ unsigned long long row16_bitonic_sort(unsigned long long x) {
  const int i = threadIdx.x & 15;
  x = cmpx(x, dpp_u64<0x128>(x), (i & 8) == 0);                       // row_ror:8 = lane ^ 8
  const unsigned long long up = dpp_u64<0x12C>(x);                    // row_ror:12 = lane + 4
  const unsigned long long dn = dpp_u64<0x124>(x);                    // row_ror:4 = lane - 4
  x = cmpx(x, (i & 4) ? dn : up, (i & 4) == 0);
  x = cmpx(x, dpp_u64<0x4e>(x), (i & 2) == 0);                        // quad_perm [2,3,0,1]
  x = cmpx(x, dpp_u64<0xb1>(x), (i & 1) == 0);                        // quad_perm [1,0,3,2]
  return x;
}

// Top-16, sorted, of the union of two disjoint sorted lists a (slot i) and b (slot
// 15 - i in this lane): the elementwise maximum of a list and the other reversed holds
// the 16 largest of both and is bitonic.
__device__ __forceinline__ unsigned long long merge16(unsigned long long a, unsigned long long b_rev) {
  return row16_bitonic_sort(a > b_rev ? a : b_rev);
}

// 32-bit forms for the lanes' own values.
template <int CTRL>
__device__ __forceinline__ int dpp_i32(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xf, 0xf, true);
}
__device__ __forceinline__ int xor_lane_i32(int v, int m) {
  return __builtin_amdgcn_ds_bpermute(((threadIdx.x & 63) ^ m) << 2, v);
}
__device__ __forceinline__ int cmpx_i32(int x, int p, bool keep_max) { return keep_max ? max(x, p) : min(x, p); }

// Partner of a lane at distance j (1, 2, 4 or 8) inside its 16-lane row.
template <int J>
__device__ __forceinline__ int row_partner_i32(int x) {
  if constexpr (J == 8) return dpp_i32<0x128>(x);                    // row_ror:8
  if constexpr (J == 2) return dpp_i32<0x4e>(x);                     // quad_perm [2,3,0,1]
  if constexpr (J == 1) return dpp_i32<0xb1>(x);                     // quad_perm [1,0,3,2]
  const int up = dpp_i32<0x12C>(x), dn = dpp_i32<0x124>(x);          // row_ror:12 / row_ror:4
  return (threadIdx.x & 4) ? dn : up;
}

// One stage of Batcher's bitonic sort on the rows: blocks of K lanes ordered largest
// first where lane bit K is clear (and for K = 16), partners at distance J.
template <int K, int J>
__device__ __forceinline__ int bitonic_stage_i32(int x) {
  const int i = threadIdx.x & 15;
  const bool desc = K >= 16 || (i & K) == 0;
  return cmpx_i32(x, row_partner_i32<J>(x), ((i & J) == 0) == desc);
}

// Maximum of the lanes' values over the whole wave (DPP within each 16-lane row, then
// the four row results through readlane); every lane gets it.
__device__ __forceinline__ int wave_max_i32(int x) {
  x = max(x, dpp_i32<0xb1>(x));                                      // quad_perm [1,0,3,2]
  x = max(x, dpp_i32<0x4e>(x));                                      // quad_perm [2,3,0,1]
  x = max(x, dpp_i32<0x141>(x));                                     // row_half_mirror
  x = max(x, dpp_i32<0x140>(x));                                     // row_mirror
  const int a = max(__builtin_amdgcn_readlane(x, 0), __builtin_amdgcn_readlane(x, 16));
  const int b = max(__builtin_amdgcn_readlane(x, 32), __builtin_amdgcn_readlane(x, 48));
  return max(a, b);
}

// Half-cleaners at distances 8, 4, 2, 1: sorts, largest first, a bitonic sequence held
// by each 16-lane row.
__device__ __forceinline__ int row16_bitonic_sort_i32(int x) {
  x = bitonic_stage_i32<16, 8>(x);
  x = bitonic_stage_i32<16, 4>(x);
  x = bitonic_stage_i32<16, 2>(x);
  return bitonic_stage_i32<16, 1>(x);
}

// Keeps in each row the best 16 of it and its partner row (lane ^ m, m = 16 or 32),
// sorted: the elementwise maximum with the mirrored partner row is bitonic.
__device__ __forceinline__ int row16_merge_rows_i32(int x, int m) {
  return row16_bitonic_sort_i32(max(x, xor_lane_i32(dpp_i32<0x140>(x), m)));   // row_mirror
}

// The 16 largest of the wave's lane values, largest first, in lanes 0..15 (each row
// sorted by a full bitonic sort, then the rows merged pairwise).  All on the vector unit.
__device__ __forceinline__ int wave_top16_i32(int x) {
  x = bitonic_stage_i32<2, 1>(x);
  x = bitonic_stage_i32<4, 2>(x);
  x = bitonic_stage_i32<4, 1>(x);
  x = bitonic_stage_i32<8, 4>(x);
  x = bitonic_stage_i32<8, 2>(x);
  x = bitonic_stage_i32<8, 1>(x);
  x = row16_bitonic_sort_i32(x);
  x = row16_merge_rows_i32(x, 16);
  return row16_merge_rows_i32(x, 32);
}

// 16th largest of the union of kTopkWaves sorted top-16 lists (LDS, 16 each), taken by
// every wave that calls it: lists merge pairwise in the four rows, then the rows.
__device__ __forceinline__ int block_kth16(const int* lists) {
  static_assert(kTopkWaves == 8, "the merge tree assumes eight wave lists");
  const int lane = threadIdx.x & 63;
  const int r = lane >> 4, i = lane & 15;
  int x = row16_bitonic_sort_i32(max(lists[(2 * r) * kNC + i], lists[(2 * r + 1) * kNC + (kNC - 1 - i)]));
  x = row16_merge_rows_i32(x, 16);
  x = row16_merge_rows_i32(x, 32);
  return __builtin_amdgcn_readlane(x, 15);
}

// Top-16, best first, of the block's kTopkWaves sorted wave lists (LDS, 16 each) by one
// whole wave: pairs of lists merge in the four rows, then pairs of rows (through the
// mirrored partner row), twice.  Lane i < 16 returns slot i.
__device__ __forceinline__ unsigned long long wave_merge_block(const unsigned long long* lists) {
  static_assert(kTopkWaves == 8, "the merge tree assumes eight wave lists");
  const int lane = threadIdx.x & 63;
  const int r = lane >> 4, i = lane & 15;
  unsigned long long x = merge16(lists[(2 * r) * kNC + i], lists[(2 * r + 1) * kNC + (kNC - 1 - i)]);
  x = merge16(x, xor_lane_u64(dpp_u64<0x140>(x), 16));                // row_mirror, then the row above/below
  x = merge16(x, xor_lane_u64(dpp_u64<0x140>(x), 32));
  return x;
}

// ---- one chunk of a row -------------------------------------------------------------
// Lane L of wave w loads vectors v0 + 64 w + L + kTopkThreads k of the chunk [v0, v1)
// of `row`, so a block's loads are contiguous; vector v holds logits 8v..8v+7, only
// those < V exist, the rest read as -NaN (below every logit).

__device__ __forceinline__ void load_chunk(const uint16_t* __restrict__ row, int V, int v0, int v1,
                                           u32x4 (&d)[kTopkVecPerThread]) {
  const int nfull = V >> 3;
  const u32x4* __restrict__ rowv = reinterpret_cast<const u32x4*>(row);
  // whole vectors, branch-free: a slot past the chunk or the row reads the chunk's first
  // vector (always whole) and is replaced by -NaN padding
#pragma unroll
  for (int k = 0; k < kTopkVecPerThread; ++k) {
    const int v = v0 + (int)threadIdx.x + k * kTopkThreads;
    const bool whole = v < v1 && v < nfull;
    d[k] = __builtin_nontemporal_load(rowv + (whole ? v : v0));
    if (!whole) d[k] = (u32x4){0xffffffffu, 0xffffffffu, 0xffffffffu, 0xffffffffu};
  }
  // the row's ragged last vector (V % 8 != 0), in the one lane that owns it
  const int vr = nfull - v0;
  if ((V & 7) != 0 && nfull < v1 && vr >= 0 && (int)threadIdx.x == vr % kTopkThreads) {
    uint32_t w4[4] = {0xffffffffu, 0xffffffffu, 0xffffffffu, 0xffffffffu};
#pragma unroll 1
    for (int e = 0; e < (V & 7); ++e) {
      const uint32_t b = row[8 * nfull + e];
      w4[e >> 1] = (e & 1) ? ((w4[e >> 1] & 0xffffu) | (b << 16)) : ((w4[e >> 1] & 0xffff0000u) | b);
    }
    const u32x4 x = (u32x4){w4[0], w4[1], w4[2], w4[3]};
    const int kr = vr / kTopkThreads;
#pragma unroll
    for (int k = 0; k < kTopkVecPerThread; ++k)
      if (k == kr) d[k] = x;
  }
}

// Per-vector maxima and the lane maximum, on the raw patterns read as signed 16-bit
// integers (SIGNED = false) or in the signed order (SIGNED = true).  On non-negative
// values (and +NaN, above +inf) the raw order is the value order and every negative
// value sits below +0, so a threshold above +0 found in it is exact; the signed order
// follows the value order everywhere (-0 one below +0).
template <bool SIGNED>
__device__ __forceinline__ int vector_maxima(const u32x4 (&d)[kTopkVecPerThread], int (&vmax)[kTopkVecPerThread]) {
  int lmax = -32768;
#pragma unroll
  for (int k = 0; k < kTopkVecPerThread; ++k) {
    s16x2 a, b;
    if constexpr (SIGNED) {
      a = __builtin_elementwise_max(signed_order2(d[k].x), signed_order2(d[k].y));
      b = __builtin_elementwise_max(signed_order2(d[k].z), signed_order2(d[k].w));
    } else {
      a = __builtin_elementwise_max(raw_order2(d[k].x), raw_order2(d[k].y));
      b = __builtin_elementwise_max(raw_order2(d[k].z), raw_order2(d[k].w));
    }
    vmax[k] = max_halves(__builtin_elementwise_max(a, b));
    lmax = vmax[k] > lmax ? vmax[k] : lmax;
  }
  return lmax;
}

// Exact top-16 of the logits this wave's lanes load, best first, into list[0..16)
// (written by lane 0), zero-padded when the wave holds fewer than 16: sixteen rounds of
// a wave maximum below the previous one.  Each round re-reads the share (cache-resident
// by now) four vectors per lane at a time, so that the common path keeps its register
// budget.  Only chunks with heavy ties at the bound, NaN lanes or few logits take it.
__device__ __noinline__ void wave_exact_list(const uint16_t* __restrict__ row, int V, int v0, int v1,
                                             unsigned long long* list) {
  constexpr int kBatch = 4;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int nfull = V >> 3;
  const u32x4* __restrict__ rowv = reinterpret_cast<const u32x4*>(row);
  unsigned long long prev = ~0ull;
  for (int r = 0; r < kNC; ++r) {
    unsigned long long best = 0ull;
#pragma unroll 1
    for (int k0 = 0; k0 < kTopkVecPerThread; k0 += kBatch) {
      u32x4 x[kBatch];
#pragma unroll
      for (int i = 0; i < kBatch; ++i) {
        const int v = v0 + tid + (k0 + i) * kTopkThreads;
        x[i] = (u32x4){0u, 0u, 0u, 0u};
        if (k0 + i < kTopkVecPerThread && v < v1) {
          if (v < nfull) {
            x[i] = rowv[v];
          } else {
            uint32_t w4[4] = {0u, 0u, 0u, 0u};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              if (8 * v + e < V) {
                const uint32_t b = row[8 * v + e];
                w4[e >> 1] |= (e & 1) ? (b << 16) : b;
              }
            }
            x[i] = (u32x4){w4[0], w4[1], w4[2], w4[3]};
          }
        }
      }
#pragma unroll
      for (int i = 0; i < kBatch; ++i) {
        const int v = v0 + tid + (k0 + i) * kTopkThreads;
        if (k0 + i < kTopkVecPerThread && v < v1) {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            if (8 * v + e < V) {
              const uint32_t bits = elem_bits(x[i], e);
              const unsigned long long comp = make_rc(bf16_key(bits), (unsigned)(8 * v + e), bits);
              if (comp < prev && comp > best) best = comp;
            }
          }
        }
      }
    }
    best = wave_max_u64(best);
    if (lane == 0) list[r] = best;
    prev = best;
  }
}

// The chunk's top-16 row composites, best first, written to out[0..16) (global memory),
// zero-padded when the chunk holds fewer than 16 logits.  The whole block calls it.
__device__ __forceinline__ void chunk_top16(const uint16_t* __restrict__ row, int V, int v0, int v1, ChunkShared& sm,
                                            unsigned long long* __restrict__ out) {
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid >> 6;
  if (tid == 0) {
    sm.ncand = 0;
    sm.overflow = 0;
  }

  // ---- stream: every lane issues all its 16-byte loads before using any ------------
  u32x4 d[kTopkVecPerThread];
  load_chunk(row, V, v0, v1, d);

  // ---- the block's 16th largest lane maximum, first in the raw order ----------------
  int vmax[kTopkVecPerThread];
  const int lmax_raw = vector_maxima<false>(d, vmax);
  int t = wave_top16_i32(lmax_raw);
  if (lane < kNC) sm.lane_top[0][wave][lane] = t;
  __syncthreads();
  int tau = block_kth16(&sm.lane_top[0][0][0]);
  const bool raw = tau > 0;                      // the same in every wave
  if (!raw) {
    t = wave_top16_i32(vector_maxima<true>(d, vmax));
    if (lane < kNC) sm.lane_top[1][wave][lane] = t;
    __syncthreads();
    tau = block_kth16(&sm.lane_top[1][0][0]);
  }
  if (tau > 0x7f80) tau = 0x7f80;                // never above +inf
  const uint32_t tau_key = bf16_key(raw ? (uint32_t)tau : order_to_bits(tau));
  const int slack = raw ? 0 : 1;                 // signed order: -0 sits one below +0

  // ---- this wave's vectors that may hold a logit >= tau -----------------------------
  // Few qualify, so each slot k costs one ballot and a wave-uniform branch unless some
  // lane's vector k does.
  uint32_t nv = 0;
#pragma unroll
  for (int k = 0; k < kTopkVecPerThread; ++k) {
    const bool f = vmax[k] >= tau - slack;
    const unsigned long long m = __ballot(f);
    if (m != 0ull) {
      const uint32_t slot = nv + __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
      if (f && slot < (uint32_t)kWaveCapVec) {
        sm.vec_data[wave][slot] = d[k];
        sm.vec_pos[wave][slot] = (unsigned)(tid + k * kTopkThreads);
      }
      nv += (uint32_t)__popcll(m);
    }
  }
  wave_lds_sync();

  // ---- their logits >= tau, with exact keys, into the block's candidates -----------
  if (nv > (uint32_t)kWaveCapVec) {
    if (lane == 0) sm.overflow = 1u;
  } else {
    for (uint32_t base = 0; base < nv * 8u; base += kWave) {
      const uint32_t e = base + (uint32_t)lane;
      bool f = false;
      unsigned long long comp = 0ull;
      if (e < nv * 8u) {
        const uint32_t slot = e >> 3;
        const uint32_t pos = sm.vec_pos[wave][slot];
        const uint32_t w = reinterpret_cast<const uint32_t*>(&sm.vec_data[wave][slot])[(e & 7u) >> 1];
        const uint32_t bits = (e & 1u) ? (w >> 16) : (w & 0xffffu);
        const uint32_t key = bf16_key(bits);
        f = key != 0u && key >= tau_key;
        comp = make_rc(key, (uint32_t)v0 * 8u + pos * 8u + (e & 7u), bits);
      }
      const unsigned long long m = __ballot(f);
      if (m != 0ull) {
        uint32_t at = 0;
        if (lane == 0) at = atomicAdd(&sm.ncand, (uint32_t)__popcll(m));
        at = __builtin_amdgcn_readfirstlane(at);
        const uint32_t slot = at + __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
        if (f && slot < (uint32_t)kBlockCapCand) sm.cand[slot] = comp;
      }
    }
  }
  __syncthreads();

  // ---- rank the candidates: every wave takes two at a time, one per half-wave, and --
  // counts the larger ones by ballot, 32 at a time; ranks 0..15 each occur once.
  const uint32_t n = sm.ncand;
  if (sm.overflow == 0u && n >= (uint32_t)kNC && n <= (uint32_t)kBlockCapCand) {
    const int half = lane >> 5, j = lane & 31;
    for (uint32_t c0 = 0; c0 < n; c0 += 2 * kTopkWaves) {
      const uint32_t c = c0 + 2u * (uint32_t)wave + (uint32_t)half;
      const unsigned long long mine = c < n ? sm.cand[c] : 0ull;
      uint32_t rank = 0;
      for (uint32_t j0 = 0; j0 < n; j0 += 32) {
        const uint32_t jj = j0 + (uint32_t)j;
        const bool gt = jj < n && sm.cand[jj] > mine;
        const unsigned long long m = __ballot(gt);
        rank += (uint32_t)__popc((uint32_t)(m >> (32 * half)));
      }
      if (j == 0 && c < n && rank < (uint32_t)kNC) out[rank] = mine;
    }
    return;
  }

  // ---- fallback (NaN-heavy, constant, heavily tied or tiny chunks) -------------------
  wave_exact_list(row, V, v0, v1, sm.lists + wave * kNC);
  __syncthreads();
  if (wave == 0) {
    const unsigned long long top = wave_merge_block(sm.lists);
    if (lane < kNC) out[lane] = top;
  }
}

// Top-16, best first, of L <= kMaxChunks sorted lists of 16 (global memory) by one whole
// wave: 16-lane row g merges lists g, g + 4, g + 8, ... one after another (all of them
// loaded first), then the rows merge pairwise.  Lane i of every row returns slot i.
__device__ __forceinline__ unsigned long long wave_merge_lists(const unsigned long long* __restrict__ src, int L) {
  constexpr int kPerRow = (kMaxChunks + 3) / 4;
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4, i = lane & 15;
  unsigned long long y[kPerRow];
#pragma unroll
  for (int k = 0; k < kPerRow; ++k) {
    const int l = g + 4 * k;
    y[k] = l < L ? src[(size_t)l * kNC + (k == 0 ? i : kNC - 1 - i)] : 0ull;
  }
  unsigned long long x = y[0];
#pragma unroll
  for (int k = 1; k < kPerRow; ++k)
    if (4 * k < L) x = merge16(x, y[k]);                            // wave-uniform: every row merges
  x = merge16(x, xor_lane_u64(dpp_u64<0x140>(x), 16));
  return merge16(x, xor_lane_u64(dpp_u64<0x140>(x), 32));
}

// Placement of a stream over the rows of several requests: the rows_per * nchunks
// chunk work-groups of request b take the work-group ids 8 * slot + b % 8, which the
// dispatcher deals to one XCD (work-group id mod 8 picks the XCD), so that the kernel
// after the stream, which reads request b's chunk results from work-group b (also on
// XCD b % 8), finds them in the L2 they were written to.  Returns the chunk block
// (row * nchunks + chunk, rows counted over all requests) of work-group id, or -1 for the
// padding ids of the last lanes; the grid has 8 * ceil(batch / 8) * rows_per * nchunks ids.
__device__ __forceinline__ int xcd_chunk_block(int id, int batch, int rows_per, int nchunks) {
  const int per = rows_per * nchunks;
  const int x = id & 7, slot = id >> 3;
  const int b = x + 8 * (slot / per);
  return b < batch ? b * per + (slot - (slot / per) * per) : -1;
}
__host__ __device__ __forceinline__ long long xcd_chunk_grid(long long batch, long long rows_per, long long nchunks) {
  return 8 * ((batch + 7) / 8) * rows_per * nchunks;
}

// Chunking of a row: n chunks of near-equal vector counts, each <= kChunkVec.
__host__ __device__ __forceinline__ int topk_num_chunks(long long vocab) {
  const long long nvec = (vocab + 7) / 8;
  return (int)((nvec + kChunkVec - 1) / kChunkVec);
}
__host__ __device__ __forceinline__ int chunk_begin(long long vocab, int nchunks, int c) {
  const long long nvec = (vocab + 7) / 8;
  return (int)(nvec * c / nchunks);
}

}  // namespace df2
