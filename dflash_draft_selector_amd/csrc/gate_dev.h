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

// ---- wide tiles for many rows (bf16 weight) ---------------------------------------------
// At hundreds of rows the 16 x 64 tiles re-read W once per 16 rows and h once per 64
// columns, about 1 MB per compute unit at 960 rows, and each compute unit's load path
// (not HBM, not the matrix cores) sets the time.  A wide tile is 64 rows x 256 columns
// over a part of the hidden dimension: the 64 hidden rows of each 128-dim stage go
// through LDS (rounded to bf16 as they are staged), double-buffered with one barrier per
// stage, and each wave streams the W rows of its own 32 columns straight into the MFMA B
// operand, two stages ahead in registers.  The parts' sums go to partial[part][row][col]
// and k_gate_finish adds them in part order, so results never depend on scheduling.
constexpr int kWideRows = 64;
constexpr int kWideCols = 256;
constexpr int kWideStage = 128;                        // hidden dims per stage (4 MFMA steps)
constexpr int kWideSlots = kWideStage / 8;             // 16-byte bf16 slots per staged row
constexpr int kWideMinRows = 256;

constexpr int kWideLdsBuf = kWideRows * kWideSlots * 16;   // one staged stage of hidden rows (16 KB)

__device__ __forceinline__ int wide_lds_off(int r, int c) { return r * (kWideSlots * 16) + ((c ^ (r & 15)) << 4); }

// Wide tile (mg, ct) of part `part` of nparts, by a 512-thread work-group; lds_mem =
// 2 * kWideLdsBuf bytes of LDS, free on entry.  With nparts == 1 and H given it writes H
// (bias and activation applied), else partial[part][row][col].
template <bool HB>
__device__ __forceinline__ void gate_wide_tile(const void* __restrict__ h, const uint16_t* __restrict__ w,
                                               const float* __restrict__ bias, int rows, int hidden, int dim, int act,
                                               int mg, int ct, int part, int nparts, unsigned char* lds_mem,
                                               float* __restrict__ H, float* __restrict__ partial) {
  constexpr int kThreads = 512;                        // eight waves of 32 columns
  unsigned char* lds[2] = {lds_mem, lds_mem + kWideLdsBuf};
  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const int g = lane >> 4, i16 = lane & 15;
  const int nst = hidden / kWideStage;
  const int s0 = (int)((long long)nst * part / nparts), s1 = (int)((long long)nst * (part + 1) / nparts);
  const int row0 = mg * kWideRows;

  // this wave's W rows (columns 256 ct + 32 wv + 16 nt + i16), 16 bytes at dims 8 g of
  // each 32-wide step
  const uint16_t* wr[2];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) wr[nt] = w + (size_t)(ct * kWideCols + 32 * wv + 16 * nt + i16) * hidden + 8 * g;
  auto load_b = [&](int st, u32x4 (&b)[4][2]) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) b[q][nt] = *reinterpret_cast<const u32x4*>(wr[nt] + (size_t)st * kWideStage + 32 * q);
  };

  // staging: thread slot e (0, 1) covers row (tid + 512 e) / 16, 16-byte slot
  // (tid + 512 e) % 16 of the stage.  A row past the input repeats the last row (loaded
  // on every path, so that the compiler's wait counts stay exact); its accumulator rows
  // are never stored, and MFMA rows do not mix.
  f32x4 xa[2][2];
  u32x4 xb[2];
  auto load_a = [&](int st) {
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int idx = tid + kThreads * e;
      const int r = idx / kWideSlots, c = idx % kWideSlots;
      const int grow = row0 + r;
      const size_t off = (size_t)(grow < rows ? grow : rows - 1) * hidden + (size_t)st * kWideStage + 8 * c;
      if constexpr (HB) {
        xb[e] = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(h) + off);
      } else {
        xa[e][0] = *reinterpret_cast<const f32x4*>(static_cast<const float*>(h) + off);
        xa[e][1] = *reinterpret_cast<const f32x4*>(static_cast<const float*>(h) + off + 4);
      }
    }
  };
  auto store_a = [&](unsigned char* buf) {
    // row tid / 16 + 32 e has the swizzle of row tid / 16: one offset, plus 32 e rows
    const int base = wide_lds_off(tid / kWideSlots, tid % kWideSlots);
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      u32x4 a;
      if constexpr (HB) {
        a = xb[e];
      } else {
        a.x = pack_bf16x2(xa[e][0].x, xa[e][0].y);
        a.y = pack_bf16x2(xa[e][0].z, xa[e][0].w);
        a.z = pack_bf16x2(xa[e][1].x, xa[e][1].y);
        a.w = pack_bf16x2(xa[e][1].z, xa[e][1].w);
      }
      *reinterpret_cast<u32x4*>(buf + base + e * (kThreads / kWideSlots) * kWideSlots * 16) = a;
    }
  };

  f32x4 acc[4][2];
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) acc[m][nt] = (f32x4){0.f, 0.f, 0.f, 0.f};

  // stage st on LDS buffer cur and W slot wb; meanwhile the next stage's hidden rows are
  // loaded (and stored to nxt at the end) and this W slot is refilled with the stage
  // after next (the part's last stage again past its end: valid, unused, so that every
  // path issues the same loads; staging the rows two stages ahead measured no faster)
  u32x4 wb0[4][2], wb1[4][2];
  auto stage = [&](int st, unsigned char* cur, unsigned char* nxt, u32x4 (&wb)[4][2]) {
    load_a(st + 1 < s1 ? st + 1 : st);
    __builtin_amdgcn_sched_barrier(0);                // issued before the stage's MFMAs
#pragma unroll
    for (int q = 0; q < 4; ++q) {
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(cur + wide_lds_off(16 * m + i16, 4 * q + g));
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
          acc[m][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                               __builtin_bit_cast(bf16x8, wb[q][nt]), acc[m][nt], 0,
                                                               0, 0);
      }
    }
    load_b(st + 2 < s1 ? st + 2 : s1 - 1, wb);
    __builtin_amdgcn_sched_barrier(0);
    store_a(nxt);
    __syncthreads();
  };
  load_b(s0, wb0);
  load_b(s0 + 1 < s1 ? s0 + 1 : s0, wb1);
  load_a(s0);
  store_a(lds[0]);
  __syncthreads();
  int st = s0;
  for (; st + 1 < s1; st += 2) {
    stage(st, lds[0], lds[1], wb0);
    stage(st + 1, lds[1], lds[0], wb1);
  }
  if (st < s1) stage(st, lds[0], lds[1], wb0);

  // D layout: lane (g, i16), register r -> row 16 m + 4 g + r, column 16 nt + i16 of
  // this wave's 32
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = row0 + 16 * m + 4 * g + r;
        const int col = ct * kWideCols + 32 * wv + 16 * nt + i16;
        if (row < rows) {
          if (H != nullptr && nparts == 1)
            H[(size_t)row * dim + col] = gate_act(acc[m][nt][r] + (bias ? bias[col] : 0.f), act);
          else
            partial[((size_t)part * rows + row) * dim + col] = acc[m][nt][r];
        }
      }
}

}  // namespace df2
