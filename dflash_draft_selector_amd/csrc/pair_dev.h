// Pair scores S_t(a, b) = U_t(b) + <A(a) (.) H(h_t), B(b)> for the 16 x 16 adjacent
// candidate pairs of one draft position, and the per-row decisions of the walk over
// them (pegainfer issue "DFlash 2 proposer", section "What upstream shipped", item 1,
// and section "Proposal", phase 1: block_size x 16 predecessors x 16 candidates x 256
// dims, then a <= block_size-step argmax walk).
#pragma once

#include "device_common.h"

namespace df2 {

__device__ __forceinline__ int clamp_id(int id, int V, int* bad) {
  if (id < 0 || id >= V) {
    *bad = 1;
    return id < 0 ? 0 : V - 1;
  }
  return id;
}

__device__ __forceinline__ uint32_t bf16_bits(__bf16 x) { return (uint32_t)__builtin_bit_cast(uint16_t, x); }

constexpr int kTileThreads = 256;     // the block of one draft position: 4 waves

// Waves that share a tile: each covers DIM / NW of the selector dims, at least one MFMA
// step (32 dims with bf16 tables, 16 with fp32 ones).
template <int DIM, bool BF16>
constexpr int tile_waves() {
  constexpr int steps = DIM / (BF16 ? 32 : 16);
  return steps >= 4 ? 4 : (steps >= 1 ? steps : 1);
}

struct TileShared {
  float red[4][kNC][kNC];             // each wave's partial tile
  int any[4];                         // per-wave flags of block_any
};

// Whether any thread of the kTileThreads-thread block passes f (a barrier).
__device__ __forceinline__ bool block_any(bool f, TileShared& sm) {
  const unsigned long long m = __ballot(f);
  if ((threadIdx.x & 63) == 0) sm.any[threadIdx.x >> 6] = m != 0ull;
  __syncthreads();
  return (sm.any[0] | sm.any[1] | sm.any[2] | sm.any[3]) != 0;
}

// Partial tile of wave w over the selector dims [w, w + 1) * DIM / NW.  Lane l
// (g = l / 16, r = l % 16) passes the (clamped) id of predecessor row r as `prev` and of
// candidate column r as `cur`; it gets back, in register i, the part of
// sum_d A[prev of row 4 g + i][d] H[d] B[cur of column r][d] over the wave's dims.
//
// bf16 tables, on v_mfma_f32_16x16x32_bf16: x = A(prev)[d] H[d] is split into
// hi = bf16(fp32(x)) (nearest even) and lo = bf16(fma(A, H, -hi)), the remainder of the
// exact product rounded once to fp32 and then to bf16; hi and lo each go through the
// MFMA against the bf16 row of B, whose products are exact, so a term departs from
// x B by at most about 2^-18 |x B| and the sums accumulate in fp32.  The remainder is an
// explicit fused multiply-add so that no kernel's contraction choice changes a bit.
// In MFMA step s, lane l feeds row / column r with the dims base + 32 s + 8 g + [0, 8)
// (with 16 dims the two upper groups feed zeros).
// fp32 tables, on v_mfma_f32_16x16x4_f32: lane l loads the dims base + 16 m + 4 g +
// [0, 4) and feeds A[prev][d] H[d] and B[cur][d] of dim base + 16 m + 4 g + c to step
// (m, c).
// Either way the four lanes of a row read 64 contiguous bytes of it per load, so each
// load instruction touches 16 cache lines of the tables, and the contraction over d is
// a permutation of the plain sum.
template <int DIM, bool BF16>
__device__ __forceinline__ f32x4 wave_pair_part(const void* __restrict__ emb_a, const void* __restrict__ emb_b,
                                                int prev, int cur, const float* __restrict__ Hrow, int w) {
  static_assert(DIM >= 16 && DIM <= 1024 && (DIM & (DIM - 1)) == 0, "selector dims: a power of two in [16, 1024]");
  constexpr int SUB = DIM / tile_waves<DIM, BF16>();           // dims per wave
  const int g = (threadIdx.x & 63) >> 4;
  const int base = w * SUB;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  if constexpr (BF16) {
    constexpr int NS = SUB >= 32 ? SUB / 32 : 1;               // MFMA steps
    constexpr int NB = NS < 16 ? NS : 16;                      // steps whose rows are loaded at once
    const bool live = 8 * g < SUB;
    const int off = base + (live ? 8 * g : 0);
    const uint16_t* ap = static_cast<const uint16_t*>(emb_a) + (size_t)prev * DIM + off;
    const uint16_t* bp = static_cast<const uint16_t*>(emb_b) + (size_t)cur * DIM + off;
    const float* hp = Hrow + off;
#pragma unroll
    for (int s0 = 0; s0 < NS; s0 += NB) {
      u32x4 av[NB], bv[NB];
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        av[i] = *reinterpret_cast<const u32x4*>(ap + 32 * (s0 + i));
        bv[i] = *reinterpret_cast<const u32x4*>(bp + 32 * (s0 + i));
      }
      __builtin_amdgcn_sched_barrier(0);                       // every gather of the batch in flight first
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        const f32x4 h0 = *reinterpret_cast<const f32x4*>(hp + 32 * (s0 + i));
        const f32x4 h1 = *reinterpret_cast<const f32x4*>(hp + 32 * (s0 + i) + 4);
        const f32x2 h2[4] = {{h0.x, h0.y}, {h0.z, h0.w}, {h1.x, h1.y}, {h1.z, h1.w}};
        u32x4 hi, lo;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const f32x2 a2 = {bf16_lo(av[i][p]), bf16_hi(av[i][p])};
          const f32x2 x = a2 * h2[p];
          const uint32_t hb = __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2));
          const f32x2 r = __builtin_elementwise_fma(a2, h2[p], -(f32x2){bf16_lo(hb), bf16_hi(hb)});
          hi[p] = hb;
          lo[p] = __builtin_bit_cast(uint32_t, __builtin_convertvector(r, bf16x2));
        }
        if (!live) hi = lo = (u32x4){0u, 0u, 0u, 0u};
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, hi), __builtin_bit_cast(bf16x8, bv[i]),
                                                      acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, lo), __builtin_bit_cast(bf16x8, bv[i]),
                                                      acc, 0, 0, 0);
      }
    }
  } else {
    constexpr int NV = SUB / 16;                               // 16-byte loads per lane and row
    constexpr int NB = NV < 16 ? NV : 16;
    const float* ap = static_cast<const float*>(emb_a) + (size_t)prev * DIM + base + 4 * g;
    const float* bp = static_cast<const float*>(emb_b) + (size_t)cur * DIM + base + 4 * g;
    const float* hp = Hrow + base + 4 * g;
#pragma unroll
    for (int v0 = 0; v0 < NV; v0 += NB) {
      f32x4 av[NB], bv[NB];
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        av[i] = *reinterpret_cast<const f32x4*>(ap + 16 * (v0 + i));
        bv[i] = *reinterpret_cast<const f32x4*>(bp + 16 * (v0 + i));
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        const f32x4 h = *reinterpret_cast<const f32x4*>(hp + 16 * (v0 + i));
#pragma unroll
        for (int c = 0; c < 4; ++c) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[i][c] * h[c], bv[i][c], acc, 0, 0, 0);
      }
    }
  }
  return acc;
}

// One position's 16 x 16 tile by the whole block (kTileThreads threads, every one calls
// it): waves w < NW compute their partial tiles (every lane passes its prev / cur ids as
// in wave_pair_part) and the partials are added in wave order after a barrier.  Thread
// 16 i + j gets S[i][j] = U_j + (partial sums), with u_col = U of its column j.
template <int DIM, bool BF16>
__device__ __forceinline__ float block_pair_tile(const void* __restrict__ emb_a, const void* __restrict__ emb_b,
                                                 int prev, int cur, const float* __restrict__ Hrow, float u_col,
                                                 TileShared& sm) {
  constexpr int NW = tile_waves<DIM, BF16>();
  const int tid = threadIdx.x, w = tid >> 6;
  if (w < NW) {
    const f32x4 acc = wave_pair_part<DIM, BF16>(emb_a, emb_b, prev, cur, Hrow, w);
    const int lane = tid & 63, g = lane >> 4, r = lane & 15;
    // D layout: lane l, register i -> row 4 (l / 16) + i, column l % 16
#pragma unroll
    for (int i = 0; i < 4; ++i) sm.red[w][4 * g + i][r] = acc[i];
  }
  __syncthreads();
  const int i = tid >> 4, j = tid & 15;
  float sum = sm.red[0][i][j];
#pragma unroll
  for (int v = 1; v < NW; ++v) sum += sm.red[v][i][j];
  return u_col + sum;
}

}  // namespace df2
