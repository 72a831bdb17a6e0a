// Pair scores S_t(a, b) = U_t(b) + <A(a) (.) H(h_t), B(b)> for the 16 x 16 adjacent
// candidate pairs of one draft position, and the walk over them (pegainfer issue
// "DFlash 2 proposer", section "What upstream shipped", item 1, and section
// "Proposal", phase 1: block_size x 16 predecessors x 16 candidates x 256 dims, then
// a <= block_size-step argmax walk).
#pragma once

#include "device_common.h"

namespace df2 {

constexpr int kPairThreads = 256;   // 4 waves; each wave owns a quarter of the selector dims

struct PairShared {
  float red[4][kNC][kNC];
  float S[kNC][kNC];
  int prev[kNC];
  int cur[kNC];
  float U[kNC];
  int flags;
};

struct WalkShared {
  int next[64 * kNC];
  int tok[64 * kNC];
  int path[64];
};

__device__ __forceinline__ int clamp_id(int id, int V, int* bad) {
  if (id < 0 || id >= V) {
    *bad = 1;
    return id < 0 ? 0 : V - 1;
  }
  return id;
}

// One position's 16 x 16 scores from sm.prev (predecessor ids), sm.cur (candidate ids)
// and sm.U (candidate logits), all set by the caller and visible to the block (all 256
// threads call it).  Writes the tile to sm.S and to S_out[256]; returns the row-status
// bits (block-uniform): 2 = an id outside [0, V) (clamped), 1 = a non-finite score.
//
// MFMA mapping (v_mfma_f32_16x16x4_f32, wave64): lane l feeds A[i = l % 16][k = l / 16]
// and B[k = l / 16][j = l % 16]; step s of wave w uses, for k-group g = l / 16, the
// selector dim d = w * DIM/4 + g * DIM/16 + s, so each lane reads one contiguous
// DIM/16-wide slice of its table rows.  The product over d is order-free, so this
// permutation of the contraction is exact up to fp32 rounding order.  A scheduling
// barrier keeps every gather ahead of the first MFMA (one memory round trip), and the
// four waves' partial tiles are summed in a fixed order.
template <int DIM, bool BF16>
__device__ __forceinline__ int pair_tile(const void* __restrict__ emb_a, const void* __restrict__ emb_b, int V,
                                         const float* __restrict__ Hrow, float* __restrict__ S_out, PairShared& sm) {
  constexpr int ND = DIM / 16;                       // dims per lane
  constexpr int NV = BF16 ? (ND + 7) / 8 : ND / 4;   // 16-byte loads per table slice (ND >= 4)
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int g = lane >> 4;
  const int r16 = lane & 15;
  const int d0 = w * (DIM / 4) + g * ND;

  int bad = 0;
  const int prev = clamp_id(sm.prev[r16], V, &bad);
  const int cur = clamp_id(sm.cur[r16], V, &bad);
  if (tid == 0) sm.flags = 0;

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  f32x4 hq[ND / 4];
#pragma unroll
  for (int i = 0; i < ND / 4; ++i) hq[i] = *reinterpret_cast<const f32x4*>(Hrow + d0 + 4 * i);
  if constexpr (BF16) {
    // table slices stay packed (two bf16 per register) until their MFMA step
    uint32_t aw[ND / 2], bw[ND / 2];
    const uint16_t* ap = static_cast<const uint16_t*>(emb_a) + (size_t)prev * DIM + d0;
    const uint16_t* bp = static_cast<const uint16_t*>(emb_b) + (size_t)cur * DIM + d0;
    if constexpr (ND >= 8) {
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const u32x4 x = *reinterpret_cast<const u32x4*>(ap + 8 * i);
        const u32x4 y = *reinterpret_cast<const u32x4*>(bp + 8 * i);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          aw[4 * i + c] = x[c];
          bw[4 * i + c] = y[c];
        }
      }
    } else {
      typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
      const u32x2 x = *reinterpret_cast<const u32x2*>(ap);
      const u32x2 y = *reinterpret_cast<const u32x2*>(bp);
      aw[0] = x.x;
      aw[1] = x.y;
      bw[0] = y.x;
      bw[1] = y.y;
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < ND; ++s) {
      const float a = (s & 1) ? bf16_hi(aw[s >> 1]) : bf16_lo(aw[s >> 1]);
      const float bb = (s & 1) ? bf16_hi(bw[s >> 1]) : bf16_lo(bw[s >> 1]);
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a * hq[s >> 2][s & 3], bb, acc, 0, 0, 0);
    }
  } else {
    f32x4 x[NV], y[NV];
    const float* ap = static_cast<const float*>(emb_a) + (size_t)prev * DIM + d0;
    const float* bp = static_cast<const float*>(emb_b) + (size_t)cur * DIM + d0;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      x[i] = *reinterpret_cast<const f32x4*>(ap + 4 * i);
      y[i] = *reinterpret_cast<const f32x4*>(bp + 4 * i);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < ND; ++s)
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(x[s >> 2][s & 3] * hq[s >> 2][s & 3], y[s >> 2][s & 3], acc, 0, 0, 0);
  }

  // D layout: lane l, register r holds D[4 * (l / 16) + r][l % 16]
#pragma unroll
  for (int r = 0; r < 4; ++r) sm.red[w][4 * g + r][r16] = acc[r];
  __syncthreads();
  if (bad) atomicOr(&sm.flags, 2);
  {
    const int i = tid >> 4, j = tid & 15;
    const float s = sm.U[j] + (((sm.red[0][i][j] + sm.red[1][i][j]) + sm.red[2][i][j]) + sm.red[3][i][j]);
    sm.S[i][j] = s;
    S_out[tid] = s;
    if (!__builtin_isfinite(s)) atomicOr(&sm.flags, 1);
  }
  __syncthreads();
  return sm.flags;
}

// Successor table of a position: next[i] = the slot taken from row i of the tile in
// sm.S, and (when qrows is not null) qrows[i][j] = that row's distribution (all 256
// threads; thread i * 16 + j holds slot j of row i).
__device__ __forceinline__ void tile_successors(const PairShared& sm, float inv_t, float u, int* __restrict__ next,
                                                float* __restrict__ qrows) {
  const int i = threadIdx.x >> 4, j = threadIdx.x & 15;
  float qj;
  const int pick = row16_pick(sm.S[i][j], inv_t, u, &qj);
  if (j == 0) next[i] = pick;
  if (qrows) qrows[threadIdx.x] = qj;
}

}  // namespace df2
