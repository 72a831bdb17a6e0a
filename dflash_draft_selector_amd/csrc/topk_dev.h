// Split-vocabulary top-16 over bf16 logits rows.  Every wave of the streaming pass
// reduces the logits its lanes load to a short candidate list that contains the wave's
// best 16; the lists of a row are then merged into the row's top-16.
// Selection order: value descending, token id ascending, -0 == +0, NaN below -inf
// (pegainfer issue "DFlash 2 proposer", section "What upstream shipped", item 1: keep
// the top-16 candidates per position).
#pragma once

#include "device_common.h"

namespace df2 {

constexpr int kTopkThreads = 256;                            // 4 waves
constexpr int kTopkWaves = kTopkThreads / kWave;
constexpr int kTopkVecPerThread = 16;                        // 16 x 16 B loads in flight per lane
constexpr int kChunkVec = kTopkThreads * kTopkVecPerThread;  // 4096 vectors = 32768 logits
constexpr int kWaveCapVec = 64;                              // candidate vectors kept per wave
constexpr int kWaveCapCand = 128;                            // candidate logits kept per wave
constexpr int kListLen = 32;                                 // entries of a wave's candidate list
constexpr int kMaxChunks = 16;                               // vocab <= 16 * 32768 = 2^19
constexpr int kMaxLists = kMaxChunks * kTopkWaves;           // candidate lists per row (64)
constexpr int kMaxListEntries = kMaxLists * kListLen;        // 2048
constexpr int kMergeCandCap = 2 * kWave;                     // merge survivors ranked in LDS

typedef short s16x2 __attribute__((ext_vector_type(2)));
typedef unsigned long long u64x2 __attribute__((ext_vector_type(2)));

// Row composite of a logit: (order key << 48) | ((0xfffff - token id) << 28) | bf16 bits.
// Larger = better (higher value, then lower id); unique per token; 0 = empty slot.
__device__ __forceinline__ unsigned long long make_rc(uint32_t key, uint32_t id, uint32_t bits) {
  return ((unsigned long long)key << 48) | ((unsigned long long)(0xfffffu - id) << 28) | (unsigned long long)bits;
}
__device__ __forceinline__ int rc_id(unsigned long long rc) { return (int)(0xfffffu - (uint32_t)((rc >> 28) & 0xfffffu)); }
__device__ __forceinline__ uint32_t rc_bits(unsigned long long rc) { return (uint32_t)(rc & 0xffffu); }

// Per-wave scratch of the chunk selection (each wave uses only its own slot, so the
// waves of a block never wait for one another).
struct WaveSelShared {
  u32x4 vec_data[kWaveCapVec];
  unsigned int vec_pos[kWaveCapVec];
  unsigned long long cand[kWaveCapCand + 8];
  unsigned long long top[kNC];
};

struct ChunkShared {
  WaveSelShared w[kTopkWaves];
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

__device__ __forceinline__ unsigned long long lanemask_lt() {
  const int lane = threadIdx.x & 63;
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

// Orders this wave's LDS writes before its later LDS reads by other lanes.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// rank[i] = number of entries of list[0..n) larger than mine_i, for the (up to) two
// keys a lane owns.  `list` is in LDS and zero-padded to a multiple of 8 (a zero is
// never larger); all lanes read the same address in each step (a broadcast), and eight
// independent reads are in flight per step.
__device__ __forceinline__ void rank2(const unsigned long long* list, unsigned int n, unsigned long long mine0,
                                      unsigned long long mine1, unsigned int& r0, unsigned int& r1) {
  r0 = 0;
  r1 = 0;
  for (unsigned int j = 0; j < n; j += 8) {
    unsigned long long x[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) x[u] = list[j + u];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      r0 += x[u] > mine0 ? 1u : 0u;
      r1 += x[u] > mine1 ? 1u : 0u;
    }
  }
}

// 16th largest of the lanes' values v (signed 16-bit range): a radix select on ballots.
__device__ __forceinline__ int lane_threshold(int v) {
  const uint32_t u = (uint32_t)(v + 32768);
  uint32_t T = 0;
#pragma unroll
  for (int bit = 15; bit >= 0; --bit) {
    const uint32_t c = T | (1u << bit);
    if (__popcll(__ballot(u >= c)) >= kNC) T = c;
  }
  return (int)T - 32768;
}

// Candidate list of the logits this wave's lanes load from the chunk of vectors
// [v0, v1) of `row` (lane L of wave w loads vectors v0 + 64 w + L + 256 k, so a
// block's loads are contiguous); vector v holds logits 8v..8v+7, only those < V
// exist.  Writes kListLen row composites to list[] (lanes < kListLen): a set that
// contains the wave's best 16, in no particular order, zero-padded.  Called by every
// wave of the block; no wave waits for another.
//
// The wave finds the 16th largest of its lanes' maxima (a radix select on ballots):
// at least 16 of its logits reach it, so only logits at or above it can be among the
// wave's best 16.  Those few are gathered with exact keys (ballot compaction); when
// they fit the list they are the list, otherwise they are ranked and the best 16 kept.
// If fewer than 16 or too many survive (NaN-heavy, constant or heavily tied data), an
// exact 16-round selection over the wave's logits decides instead.
__device__ __forceinline__ void wave_list(const uint16_t* __restrict__ row, int V, int v0, int v1, WaveSelShared& sm,
                                          unsigned long long* __restrict__ list) {
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int nfull = V >> 3;
  const u32x4* __restrict__ rowv = reinterpret_cast<const u32x4*>(row);

  // ---- stream: every lane issues all its 16-byte loads before using any ----------
  u32x4 d[kTopkVecPerThread];
#pragma unroll
  for (int k = 0; k < kTopkVecPerThread; ++k) {
    const int v = v0 + tid + k * kTopkThreads;
    if (v < v1 && v < nfull) {
      d[k] = __builtin_nontemporal_load(rowv + v);
    } else {
      uint32_t w4[4] = {0xffffffffu, 0xffffffffu, 0xffffffffu, 0xffffffffu};   // -NaN padding
      if (v < v1) {                                                            // ragged last vector
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          if (8 * v + e < V) {
            const uint32_t b = row[8 * v + e];
            w4[e >> 1] = (e & 1) ? ((w4[e >> 1] & 0xffffu) | (b << 16)) : ((w4[e >> 1] & 0xffff0000u) | b);
          }
        }
      }
      d[k] = (u32x4){w4[0], w4[1], w4[2], w4[3]};
    }
  }

  // ---- pass 1: per-vector and per-lane maxima --------------------------------------
  // First on the raw patterns read as signed 16-bit integers: on non-negative values
  // (and +NaN, above +inf) that is the value order, and every negative value sits
  // below +0, so a threshold above +0 found in it is exact.  Otherwise the pass is
  // redone in the signed order, which follows the value order everywhere.
  int vmax[kTopkVecPerThread];
  int lmax = -32768;
#pragma unroll
  for (int k = 0; k < kTopkVecPerThread; ++k) {
    const s16x2 a = __builtin_elementwise_max(raw_order2(d[k].x), raw_order2(d[k].y));
    const s16x2 b = __builtin_elementwise_max(raw_order2(d[k].z), raw_order2(d[k].w));
    vmax[k] = max_halves(__builtin_elementwise_max(a, b));
    lmax = vmax[k] > lmax ? vmax[k] : lmax;
  }
  int tau = lane_threshold(lmax);
  const bool raw = tau > 0;
  if (!raw) {
    lmax = -32768;
#pragma unroll
    for (int k = 0; k < kTopkVecPerThread; ++k) {
      const s16x2 a = __builtin_elementwise_max(signed_order2(d[k].x), signed_order2(d[k].y));
      const s16x2 b = __builtin_elementwise_max(signed_order2(d[k].z), signed_order2(d[k].w));
      vmax[k] = max_halves(__builtin_elementwise_max(a, b));
      lmax = vmax[k] > lmax ? vmax[k] : lmax;
    }
    tau = lane_threshold(lmax);
  }
  if (tau > 0x7f80) tau = 0x7f80;                // never above +inf
  const uint32_t tau_key = bf16_key(raw ? (uint32_t)tau : order_to_bits(tau));
  const int slack = raw ? 0 : 1;                 // signed order: -0 sits one below +0

  // ---- vectors that may hold a logit >= tau (ballot compaction) -------------------
  unsigned int nv = 0;
#pragma unroll
  for (int k = 0; k < kTopkVecPerThread; ++k) {
    const bool f = vmax[k] >= tau - slack;
    const unsigned long long m = __ballot(f);
    if (f) {
      const unsigned int slot = nv + (unsigned)__popcll(m & lanemask_lt());
      if (slot < (unsigned)kWaveCapVec) {
        sm.vec_data[slot] = d[k];
        sm.vec_pos[slot] = (unsigned)(tid + k * kTopkThreads);
      }
    }
    nv += (unsigned)__popcll(m);
  }
  wave_lds_sync();

  // ---- their logits >= tau, with exact keys ---------------------------------------
  unsigned int nc = 0;
  bool exact = nv > (unsigned)kWaveCapVec;
  if (!exact) {
    for (unsigned int base = 0; base < nv * 8u; base += kWave) {
      const unsigned int e = base + (unsigned)lane;
      bool f = false;
      unsigned long long comp = 0ull;
      if (e < nv * 8u) {
        const unsigned int slot = e >> 3;
        const uint32_t w = reinterpret_cast<const uint32_t*>(&sm.vec_data[slot])[(e & 7u) >> 1];
        const uint32_t bits = (e & 1u) ? (w >> 16) : (w & 0xffffu);
        const uint32_t key = bf16_key(bits);
        f = key != 0u && key >= tau_key;
        comp = make_rc(key, (unsigned)v0 * 8u + sm.vec_pos[slot] * 8u + (e & 7u), bits);
      }
      const unsigned long long m = __ballot(f);
      if (f) {
        const unsigned int slot = nc + (unsigned)__popcll(m & lanemask_lt());
        if (slot < (unsigned)kWaveCapCand) sm.cand[slot] = comp;
      }
      nc += (unsigned)__popcll(m);
    }
    exact = nc < (unsigned)kNC || nc > (unsigned)kWaveCapCand;
  }
  if (!exact && nc <= (unsigned)kListLen) {
    // ---- the survivors are the list ----------------------------------------------------
    if (lane < kListLen) list[lane] = (unsigned)lane < nc ? sm.cand[lane] : 0ull;
    return;
  }
  if (!exact) {
    // ---- rank the survivors (at most two per lane) ---------------------------------
    const unsigned int npad = (nc + 7u) & ~7u;
    for (unsigned int c = nc + (unsigned)lane; c < npad; c += kWave) sm.cand[c] = 0ull;
    wave_lds_sync();
    const unsigned long long m0 = (unsigned)lane < nc ? sm.cand[lane] : 0ull;
    const unsigned long long m1 = (unsigned)lane + kWave < nc ? sm.cand[lane + kWave] : 0ull;
    unsigned int r0, r1;
    rank2(sm.cand, npad, m0, m1, r0, r1);
    if (m0 && r0 < (unsigned)kNC) sm.top[r0] = m0;
    if (m1 && r1 < (unsigned)kNC) sm.top[r1] = m1;
  } else {
    // ---- exact 16-round selection over the wave's logits -----------------------------
    // It re-reads them from memory (cache-resident by now) so that the common path
    // keeps its register budget.
    unsigned long long prev = ~0ull;
    for (int r = 0; r < kNC; ++r) {
      unsigned long long best = 0ull;
#pragma unroll 1
      for (int k = 0; k < kTopkVecPerThread; ++k) {
        const int v = v0 + tid + k * kTopkThreads;
        if (v >= v1) break;
        u32x4 x;
        if (v < nfull) {
          x = rowv[v];
        } else {
          uint32_t w4[4] = {0u, 0u, 0u, 0u};
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            if (8 * v + e < V) {
              const uint32_t b = row[8 * v + e];
              w4[e >> 1] |= (e & 1) ? (b << 16) : b;
            }
          }
          x = (u32x4){w4[0], w4[1], w4[2], w4[3]};
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          if (8 * v + e < V) {
            const uint32_t bits = elem_bits(x, e);
            const unsigned long long comp = make_rc(bf16_key(bits), (unsigned)(8 * v + e), bits);
            if (comp < prev && comp > best) best = comp;
          }
        }
      }
      best = wave_max_u64(best);
      if (lane == 0) sm.top[r] = best;
      prev = best;
    }
  }
  wave_lds_sync();
  if (lane < kListLen) list[lane] = lane < kNC ? sm.top[lane] : 0ull;
}

// Copy a row's candidate lists (n composites, n a multiple of 128, at most
// kMaxListEntries) from global memory to dst (LDS).  One whole wave; every load is
// issued before the first store.
__device__ __forceinline__ void wave_stage_lists(const unsigned long long* __restrict__ src, int n,
                                                 unsigned long long* dst) {
  constexpr int kPer = kMaxListEntries / 2 / kWave;
  const int lane = threadIdx.x & 63;
  const int nvec = n / 2;                               // a multiple of 64
  const u64x2* __restrict__ s2 = reinterpret_cast<const u64x2*>(src);
  u64x2* d2 = reinterpret_cast<u64x2*>(dst);
  u64x2 x[kPer];
#pragma unroll
  for (int k = 0; k < kPer; ++k)
    if (k * kWave < nvec) x[k] = s2[lane + k * kWave];
#pragma unroll
  for (int k = 0; k < kPer; ++k)
    if (k * kWave < nvec) d2[lane + k * kWave] = x[k];
  wave_lds_sync();
}

// Top-16 of a row, best first, from its n candidate-list entries ent[] (LDS; row
// composites in no order, zero-padded) into out16[] (LDS).  One whole wave; lane l
// looks at entries l + 64 j.  The 16th largest lane-maximum order key T bounds the
// row's 16th best from below (16 lanes hold an entry at least that large), so only
// entries with key >= T are compacted into cbuf (LDS, kMergeCandCap + 8) and ranked
// among themselves.  Rows where fewer than 16 lanes see a key above the NaN key, or
// with too many survivors, take an exact 16-round selection over all entries.
__device__ __forceinline__ void wave_merge_lists(const unsigned long long* ent, int n, unsigned long long* cbuf,
                                                 unsigned long long* out16) {
  const int lane = threadIdx.x & 63;
  const int m = n / kWave;
  uint32_t lmax = 0;
#pragma unroll 4
  for (int j = 0; j < m; ++j) {
    const uint32_t k = (uint32_t)(ent[lane + kWave * j] >> 48);
    lmax = k > lmax ? k : lmax;
  }
  uint32_t T = 0;
#pragma unroll
  for (int bit = 15; bit >= 0; --bit) {
    const uint32_t c = T | (1u << bit);
    if (__popcll(__ballot(lmax >= c)) >= kNC) T = c;
  }
  unsigned int nc = 0;
  if (T != 0u) {
#pragma unroll 4
    for (int j = 0; j < m; ++j) {
      const unsigned long long x = ent[lane + kWave * j];
      const bool f = (uint32_t)(x >> 48) >= T;
      const unsigned long long mk = __ballot(f);
      if (f) {
        const unsigned int slot = nc + (unsigned)__popcll(mk & lanemask_lt());
        if (slot < (unsigned)kMergeCandCap) cbuf[slot] = x;
      }
      nc += (unsigned)__popcll(mk);
    }
  }
  if (T != 0u && nc <= (unsigned)kMergeCandCap) {
    const unsigned int npad = (nc + 7u) & ~7u;
    for (unsigned int c = nc + (unsigned)lane; c < npad; c += kWave) cbuf[c] = 0ull;
    wave_lds_sync();
    const unsigned long long m0 = (unsigned)lane < nc ? cbuf[lane] : 0ull;
    const unsigned long long m1 = (unsigned)lane + kWave < nc ? cbuf[lane + kWave] : 0ull;
    unsigned int r0, r1;
    rank2(cbuf, npad, m0, m1, r0, r1);
    if (m0 && r0 < (unsigned)kNC) out16[r0] = m0;
    if (m1 && r1 < (unsigned)kNC) out16[r1] = m1;
  } else {
    unsigned long long prev = ~0ull;
    for (int r = 0; r < kNC; ++r) {
      unsigned long long best = 0ull;
      for (int j = 0; j < m; ++j) {
        const unsigned long long x = ent[lane + kWave * j];
        if (x < prev && x > best) best = x;
      }
      best = wave_max_u64(best);
      if (lane == 0) out16[r] = best;
      prev = best;
    }
  }
  wave_lds_sync();
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
