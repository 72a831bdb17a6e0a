// Context gate tiles H = act(W_H h + b) (pegainfer issue "DFlash 2 proposer", section
// "What upstream shipped", item 1: 256-dim token embeddings + context gate).
//
// h comes as fp32 or as bf16 (HB).  bf16 weight: fp32 h is rounded to bf16 (nearest
// even) as it is loaded, bf16 h goes in as it is, and the product runs on
// v_mfma_f32_16x16x32_bf16 with fp32 accumulation.  A work-group owns a 16-row
// x (16 NB)-column output tile over one slice of the hidden dimension; its NW waves take
// interleaved 32-wide steps of the slice and their partial tiles are summed in LDS in
// wave order.  With several slices the tile is stored as a partial sum and the slices
// are added later in slice order, then the bias and the activation, so results never
// depend on scheduling.
#pragma once

#include "device_common.h"

namespace df2 {

__device__ __forceinline__ float gate_act(float x, int act) { return act == 0 ? 1.f / (1.f + expf(-x)) : x; }

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_rne(lo) | (f32_to_bf16_rne(hi) << 16);
}

// The 32-wide steps [s0, s1) of slice `split` of nsplit over ceil(hidden / 32) steps.
__host__ __device__ __forceinline__ void gate_slice(int hidden, int split, int nsplit, int& s0, int& s1) {
  const int nsteps = (hidden + 31) / 32;
  s0 = (int)((long long)nsteps * split / nsplit);
  s1 = (int)((long long)nsteps * (split + 1) / nsplit);
}

// Tile (mt, nt) of slice `split`; red = LDS [NW][16][16 NB].  With nsplit == 1 and H
// given it writes H (bias and activation applied), else partial[split][row][col].  The
// first NW * 64 threads of the block call it.
template <int NB, int NW, int ROUND, bool HB>
__device__ __forceinline__ void gate_tile(const void* __restrict__ h, const uint16_t* __restrict__ w,
                                          const float* __restrict__ bias, int rows, int hidden, int dim, int act,
                                          int mt, int nt, int split, int nsplit, float* red, float* __restrict__ H,
                                          float* __restrict__ partial) {
  constexpr int kCols = 16 * NB;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const int g = lane >> 4, r16 = lane & 15;
  int s0, s1;
  gate_slice(hidden, split, nsplit, s0, s1);

  const int arow = mt * 16 + r16;
  const bool arow_ok = arow < rows;
  const size_t hoff = (size_t)(arow_ok ? arow : 0) * hidden;
  const float* hrow = static_cast<const float*>(h) + hoff;
  const uint16_t* hrow16 = static_cast<const uint16_t*>(h) + hoff;
  const uint16_t* wcol[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) wcol[j] = w + (size_t)(nt * kCols + j * 16 + r16) * hidden;

  f32x4 acc[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) acc[j] = (f32x4){0.f, 0.f, 0.f, 0.f};

  for (int base = s0 + wv; base < s1; base += NW * ROUND) {
    f32x4 x0[ROUND], x1[ROUND];
    u32x4 xb[ROUND];
    u32x4 bw[ROUND][NB];
#pragma unroll
    for (int i = 0; i < ROUND; ++i) {
      const int st = base + NW * i;
      const int k = st * 32 + g * 8;
      const bool kok = st < s1 && k < hidden;
      x0[i] = x1[i] = (f32x4){0.f, 0.f, 0.f, 0.f};
      xb[i] = (u32x4){0u, 0u, 0u, 0u};
      if (kok && arow_ok) {
        if constexpr (HB) {
          xb[i] = *reinterpret_cast<const u32x4*>(hrow16 + k);
        } else {
          x0[i] = *reinterpret_cast<const f32x4*>(hrow + k);
          x1[i] = *reinterpret_cast<const f32x4*>(hrow + k + 4);
        }
      }
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        bw[i][j] = (u32x4){0u, 0u, 0u, 0u};
        if (kok) bw[i][j] = *reinterpret_cast<const u32x4*>(wcol[j] + k);
      }
    }
#pragma unroll
    for (int i = 0; i < ROUND; ++i) {
      u32x4 a = xb[i];
      if constexpr (!HB) {
        a.x = pack_bf16x2(x0[i].x, x0[i].y);
        a.y = pack_bf16x2(x0[i].z, x0[i].w);
        a.z = pack_bf16x2(x1[i].x, x1[i].y);
        a.w = pack_bf16x2(x1[i].z, x1[i].w);
      }
#pragma unroll
      for (int j = 0; j < NB; ++j)
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                         __builtin_bit_cast(bf16x8, bw[i][j]), acc[j], 0, 0, 0);
    }
  }

  // D layout: lane l, register r -> row 4 * (l / 16) + r, column l % 16 of each block
#pragma unroll
  for (int j = 0; j < NB; ++j)
#pragma unroll
    for (int r = 0; r < 4; ++r) red[(wv * 16 + 4 * g + r) * kCols + j * 16 + r16] = acc[j][r];
  __syncthreads();
  for (int e = tid; e < 16 * kCols; e += NW * 64) {
    const int rr = e / kCols, c = e - rr * kCols;
    const int row = mt * 16 + rr;
    if (row >= rows) continue;
    const int n = nt * kCols + c;
    float sum = red[rr * kCols + c];
#pragma unroll
    for (int v = 1; v < NW; ++v) sum += red[(v * 16 + rr) * kCols + c];
    if (H != nullptr && nsplit == 1)
      H[(size_t)row * dim + n] = gate_act(sum + (bias ? bias[n] : 0.f), act);
    else
      partial[((size_t)split * rows + row) * dim + n] = sum;
  }
}

// fp32 weight: the same tiling on v_mfma_f32_16x16x4f32 with 16-wide steps of hidden.
// In step st lane l loads h[row][16 st + 4 g .. + 3] and W[col][16 st + 4 g .. + 3]
// (g = l / 16, row / col = l % 16 of the tile) and feeds component j of both to MFMA j,
// so the four MFMAs of a step contract over all 16 of its hidden indices (a permutation
// of the sum, exact up to fp32 rounding order).  bf16 h (HB) is widened to fp32, which
// is exact.
template <int NB, int NW, int ROUND, bool HB>
__device__ __forceinline__ void gate_tile_f32(const void* __restrict__ h, const float* __restrict__ w,
                                              const float* __restrict__ bias, int rows, int hidden, int dim,
                                              int act, int mt, int nt, int split, int nsplit, float* red,
                                              float* __restrict__ H, float* __restrict__ partial) {
  constexpr int kCols = 16 * NB;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const int g = lane >> 4, r16 = lane & 15;
  const int nsteps = (hidden + 15) / 16;
  const int s0 = (int)((long long)nsteps * split / nsplit), s1 = (int)((long long)nsteps * (split + 1) / nsplit);

  const int arow = mt * 16 + r16;
  const bool arow_ok = arow < rows;
  const size_t hoff = (size_t)(arow_ok ? arow : 0) * hidden;
  const float* hrow = static_cast<const float*>(h) + hoff;
  const uint16_t* hrow16 = static_cast<const uint16_t*>(h) + hoff;
  const float* wcol[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) wcol[j] = w + (size_t)(nt * kCols + j * 16 + r16) * hidden;

  f32x4 acc[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) acc[j] = (f32x4){0.f, 0.f, 0.f, 0.f};

  for (int base = s0 + wv; base < s1; base += NW * ROUND) {
    f32x4 x[ROUND];
    f32x4 y[ROUND][NB];
#pragma unroll
    for (int i = 0; i < ROUND; ++i) {
      const int st = base + NW * i;
      const int k = st * 16 + g * 4;
      const bool kok = st < s1 && k < hidden;
      x[i] = (f32x4){0.f, 0.f, 0.f, 0.f};
      if (kok && arow_ok) {
        if constexpr (HB) {
          const u32x2 v = *reinterpret_cast<const u32x2*>(hrow16 + k);
          x[i] = (f32x4){bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y)};
        } else {
          x[i] = *reinterpret_cast<const f32x4*>(hrow + k);
        }
      }
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        y[i][j] = (f32x4){0.f, 0.f, 0.f, 0.f};
        if (kok) y[i][j] = *reinterpret_cast<const f32x4*>(wcol[j] + k);
      }
    }
#pragma unroll
    for (int i = 0; i < ROUND; ++i)
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int j = 0; j < NB; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(x[i][c], y[i][j][c], acc[j], 0, 0, 0);
  }

#pragma unroll
  for (int j = 0; j < NB; ++j)
#pragma unroll
    for (int r = 0; r < 4; ++r) red[(wv * 16 + 4 * g + r) * kCols + j * 16 + r16] = acc[j][r];
  __syncthreads();
  for (int e = tid; e < 16 * kCols; e += NW * 64) {
    const int rr = e / kCols, c = e - rr * kCols;
    const int row = mt * 16 + rr;
    if (row >= rows) continue;
    const int n = nt * kCols + c;
    float sum = red[rr * kCols + c];
#pragma unroll
    for (int v = 1; v < NW; ++v) sum += red[(v * 16 + rr) * kCols + c];
    if (H != nullptr && nsplit == 1)
      H[(size_t)row * dim + n] = gate_act(sum + (bias ? bias[n] : 0.f), act);
    else
      partial[((size_t)split * rows + row) * dim + n] = sum;
  }
}

// Gate value of (row, n) from the nsplit partial sums, added in slice order.  Loads
// go out sixteen at a time, so up to sixteen slices cost one memory round trip.
__device__ __forceinline__ float gate_finish(const float* __restrict__ partial, const float* __restrict__ bias,
                                             int rows, int dim, int nsplit, int act, int row, int n) {
  constexpr int kBatch = 16;
  const size_t stride = (size_t)rows * dim;
  const float* p = partial + (size_t)row * dim + n;
  float sum = 0.f;
  for (int s0 = 0; s0 < nsplit; s0 += kBatch) {
    float v[kBatch];
#pragma unroll
    for (int i = 0; i < kBatch; ++i) v[i] = s0 + i < nsplit ? p[(size_t)(s0 + i) * stride] : 0.f;
#pragma unroll
    for (int i = 0; i < kBatch; ++i)
      if (s0 + i < nsplit) sum += v[i];
  }
  return gate_act(sum + (bias ? bias[n] : 0.f), act);
}

}  // namespace df2
