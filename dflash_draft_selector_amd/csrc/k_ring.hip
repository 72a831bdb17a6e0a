// Draft-block attention over each request's K/V ring ([FT] "Details": sliding-window
// attention with window 2048; runtime: the draft's K/V lives in a ring of 2112 rows per
// request, the window plus room for a verify's rejected rows; the draft forward over
// [last token, mask x 7] reads it; a causal draft is refused, so the block's rows see
// each other).
//
// Keys of request b: its last min(ctx_len, window - 1) context positions p0 .. L - 1
// (position p in ring row p mod ring), then the block's own nq rows.  Every query row of
// the block attends to all of them; query head h uses K/V head h / (Hq / Hkv).
//
// Ring layouts, chosen for this read (the hot one: every draft step reads the whole
// window, a verify writes a few rows): K head-major [B][Hkv][ring][Dh]; V transposed
// [B][Hkv][Dh][ring], so the P V product's V^T fragments (one dim, 8 consecutive
// positions) are single 16-byte loads.  ring % 8 == 0, and positions are walked in
// 8-aligned groups, so a group never wraps.  The context splits start on multiples of
// kRingAlign positions: with ring % 64 == 0 (2112 = 33 x 64) a split's 128 positions
// of one V^T row are two whole 128-byte lines instead of three partial ones.
//
// k_ring_partial: one 256-thread work-group per (request, K/V head, split).  Split s <
// nctx_splits takes the 128 positions pa + 128 s .. (pa = p0 rounded down to kRingAlign) of the
// context, masked to [p0, L); the last split takes the block's keys.  The rows are the
// nq x G query rows of the K/V head, in MT 16-row tiles.  Wave w computes S for keys
// 32w .. 32w+31 on v_mfma_f32_16x16x32_bf16 (Q and K fragments straight from memory);
// row maxima and sums go through LDS; P = exp(S - m) is split into bf16 hi + lo parts
// (relative error <= 2^-16) and stored row-major in LDS; wave w accumulates O^T for dims
// 32w .. 32w+31 as V^T x P^T (hi and lo), its V^T fragments loaded at the start.  Each
// work-group stores its rows' (max, sum, O); k_ring_combine merges the splits.
#include "dflash2_internal.h"
#include "device_common.h"
#include "topk_dev.h"

namespace df2 {

constexpr int kRingThreads = 256;            // 4 waves
constexpr int kRingDh = 128;                 // head dim
constexpr int kRingC = 128;                  // keys per work-group
constexpr int kRingPPitch = kRingC + 8;      // bf16 elements per staged P row (16-byte aligned rows)
#ifndef DF2_RING_ALIGN
#define DF2_RING_ALIGN 64
#endif
constexpr int kRingAlign = DF2_RING_ALIGN;   // context splits start on multiples of this many positions
static_assert(kRingAlign % 8 == 0 && kRingC % kRingAlign == 0, "split starts keep 8-aligned groups");

RingWs carve_ring(Carver& c, int64_t batch, int64_t hkv, int nsplit, int rows_pad) {
  RingWs w;
  const size_t units = (size_t)batch * hkv * nsplit;
  w.ml = c.take<float>(units * rows_pad * 2);
  w.o = c.take<float>(units * rows_pad * kRingDh);
  return w;
}

template <int MT>
struct RingShared {
  uint16_t p_hi[MT * 16][kRingPPitch];       // P rows, bf16 high part
  uint16_t p_lo[MT * 16][kRingPPitch];       // P rows, bf16 low part
  float red_max[4][MT * 16];                 // per-wave row maxima
  float red_sum[4][MT * 16];                 // per-wave row sums
};

// sum over the 16 lanes of the row, every lane gets it (the reduction order of row16_max)
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f<0xb1>(v);              // quad_perm [1,0,3,2]
  v += dpp_f<0x4e>(v);              // quad_perm [2,3,0,1]
  v += dpp_f<0x141>(v);             // row_half_mirror
  v += dpp_f<0x140>(v);             // row_mirror
  return v;
}

// The work of one non-empty split (BLK: the block's keys; else 128 context positions
// from base; EDGE: some of its keys lie outside [lo, hi) and are masked).  Templated so
// that each form's loads are straight-line code (the waits on them then count
// outstanding loads exactly instead of draining them) and interior splits skip the
// masking.
template <int MT, bool BLK, bool EDGE>
__device__ __forceinline__ void ring_split(RingShared<MT>& sm, const uint16_t* __restrict__ q,
                                           const uint16_t* __restrict__ k_blk, const uint16_t* __restrict__ v_blk,
                                           const uint16_t* __restrict__ k_ring, const uint16_t* __restrict__ v_ring,
                                           int b, int kvh, int nq, int hq, int hkv, int ring, int base, int lo, int hi,
                                           float scale_log2, float* __restrict__ ml, float* __restrict__ os) {
  constexpr int kRows = MT * 16;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int g = lane >> 4, i16 = lane & 15;
  const int G = hq / hkv;
  const int nrows = nq * G;
  const size_t head = (size_t)b * hkv + kvh;

  // ---- loads: Q, K and V^T fragments --------------------------------------------------
  u32x4 qf[MT][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int r = 16 * mt + i16;
    const int rr = r < nrows ? r : 0;
    const uint16_t* qp = q + ((size_t)(b * nq + rr / G) * hq + kvh * G + rr % G) * kRingDh + 8 * g;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(qp + 32 * s);
      qf[mt][s] = r < nrows ? v : (u32x4){0u, 0u, 0u, 0u};
    }
  }
  u32x4 kf[2][4];
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    const int key = base + 32 * wv + 16 * n + i16;
    const uint16_t* kp = BLK ? k_blk + ((size_t)(b * nq + (key < nq ? key : 0)) * hkv + kvh) * kRingDh
                             : k_ring + (head * ring + key % ring) * kRingDh;
#pragma unroll
    for (int s = 0; s < 4; ++s) kf[n][s] = *reinterpret_cast<const u32x4*>(kp + 8 * g + 32 * s);
  }
  // V^T fragment (dt, ks): dim 32 wv + 16 dt + i16, keys base + 32 ks + 8 g .. + 7, keys
  // outside [lo, hi) zeroed (a stale row never enters, not even times zero)
  u32x4 vf[2][kRingC / 32];
#pragma unroll
  for (int dt = 0; dt < 2; ++dt) {
    const int d = 32 * wv + 16 * dt + i16;
#pragma unroll
    for (int ks = 0; ks < kRingC / 32; ++ks) {
      const int k0 = base + 32 * ks + 8 * g;
      uint32_t w[4];
      if constexpr (!BLK) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(v_ring + (head * kRingDh + d) * ring + k0 % ring);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          if constexpr (EDGE) {
            const bool e0 = k0 + 2 * c >= lo && k0 + 2 * c < hi;
            const bool e1 = k0 + 2 * c + 1 >= lo && k0 + 2 * c + 1 < hi;
            w[c] = (e0 ? (v[c] & 0xffffu) : 0u) | (e1 ? (v[c] & 0xffff0000u) : 0u);
          } else {
            w[c] = v[c];
          }
        }
      } else {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int j0 = k0 + 2 * c, j1 = j0 + 1;
          const uint32_t a = v_blk[((size_t)(b * nq + (j0 < nq ? j0 : 0)) * hkv + kvh) * kRingDh + d];
          const uint32_t bb = v_blk[((size_t)(b * nq + (j1 < nq ? j1 : 0)) * hkv + kvh) * kRingDh + d];
          w[c] = (j0 < nq ? a : 0u) | (j1 < nq ? (bb << 16) : 0u);
        }
      }
      vf[dt][ks] = (u32x4){w[0], w[1], w[2], w[3]};
    }
  }

  // ---- S = Q K^T for keys base + 32 wv + 16 n + i16, scaled to log2 units, masked -----
  f32x4 sacc[2][MT];
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    const int key = base + 32 * wv + 16 * n + i16;
    const bool valid = key >= lo && key < hi;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      sacc[n][mt] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s)
        sacc[n][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, qf[mt][s]),
                                                             __builtin_bit_cast(bf16x8, kf[n][s]), sacc[n][mt], 0, 0, 0);
#pragma unroll
      for (int r = 0; r < 4; ++r)
        sacc[n][mt][r] = (!EDGE || valid) ? sacc[n][mt][r] * scale_log2 : -__builtin_inff();
    }
  }
  // ---- row maxima (every row has a valid key in a non-empty split) ------------------
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float x = row16_max(fmaxf(sacc[0][mt][r], sacc[1][mt][r]));
      if (i16 == 0) sm.red_max[wv][16 * mt + 4 * g + r] = x;
    }
  __syncthreads();
  // ---- P = exp2(S - m): bf16 hi / lo parts into LDS, row sums -----------------------
  float mrow[MT][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 16 * mt + 4 * g + r;
      const float m = fmaxf(fmaxf(sm.red_max[0][row], sm.red_max[1][row]),
                            fmaxf(sm.red_max[2][row], sm.red_max[3][row]));
      mrow[mt][r] = m;
      float sum = 0.f;
#pragma unroll
      for (int n = 0; n < 2; ++n) {
        const float p = __builtin_amdgcn_exp2f(sacc[n][mt][r] - m);   // v_exp_f32; 2^-inf = 0
        sum += p;
        const __bf16 hb = static_cast<__bf16>(p);                      // v_cvt_pk_bf16_f32, nearest even
        const uint32_t ph = __builtin_bit_cast(uint16_t, hb);
        const uint32_t pl = __builtin_bit_cast(uint16_t, static_cast<__bf16>(p - static_cast<float>(hb)));
        const int col = 32 * wv + 16 * n + i16;
        sm.p_hi[row][col] = (uint16_t)ph;
        sm.p_lo[row][col] = (uint16_t)pl;
      }
      sum = row16_sum(sum);
      if (i16 == 0) sm.red_sum[wv][row] = sum;
    }
  __syncthreads();
  // ---- O^T = V^T x P^T (hi, then lo) --------------------------------------------------
  f32x4 o[2][MT];
#pragma unroll
  for (int dt = 0; dt < 2; ++dt)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) o[dt][mt] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < kRingC / 32; ++ks)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const u32x4 ph = *reinterpret_cast<const u32x4*>(&sm.p_hi[16 * mt + i16][32 * ks + 8 * g]);
      const u32x4 pl = *reinterpret_cast<const u32x4*>(&sm.p_lo[16 * mt + i16][32 * ks + 8 * g]);
#pragma unroll
      for (int dt = 0; dt < 2; ++dt) {
        o[dt][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, vf[dt][ks]),
                                                            __builtin_bit_cast(bf16x8, ph), o[dt][mt], 0, 0, 0);
        o[dt][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, vf[dt][ks]),
                                                            __builtin_bit_cast(bf16x8, pl), o[dt][mt], 0, 0, 0);
      }
    }

  // ---- the split's state: (max, sum) per row, and O (rows x 128 dims) --------------
  if (wv == 0 && i16 == 0) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 16 * mt + 4 * g + r;
        ml[2 * row] = mrow[mt][r];
        ml[2 * row + 1] = (sm.red_sum[0][row] + sm.red_sum[1][row]) + (sm.red_sum[2][row] + sm.red_sum[3][row]);
      }
  }
  // O^T tile (dims 32 wv + 16 dt + 4 g + r, row 16 mt + i16) -> O[row][dims .. + 3]
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
      *reinterpret_cast<f32x4*>(os + (size_t)(16 * mt + i16) * kRingDh + 32 * wv + 16 * dt + 4 * g) = o[dt][mt];
}

template <int MT>
__global__ void __launch_bounds__(kRingThreads) k_ring_partial(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_blk, const uint16_t* __restrict__ v_blk,
    const uint16_t* __restrict__ k_ring, const uint16_t* __restrict__ v_ring, const int32_t* __restrict__ ctx_len,
    int nq, int hq, int hkv, int ring, int window, float scale_log2, int nctx_splits, float* __restrict__ ws_ml,
    float* __restrict__ ws_o) {
  __shared__ RingShared<MT> sm;
  constexpr int kRows = MT * 16;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int g = lane >> 4, i16 = lane & 15;
  const int nsplit = nctx_splits + 1;
  const int unit = blockIdx.x;                              // (b * hkv + kvh) * nsplit + split
  const int split = unit % nsplit;
  const int bk = unit / nsplit;
  const int kvh = bk % hkv, b = bk / hkv;
  const int G = hq / hkv;
  const int nrows = nq * G;

  const int L = ctx_len[b] > 0 ? ctx_len[b] : 0;
  const int nctx = L < window - 1 ? L : window - 1;
  const int p0 = L - nctx;
  const bool blk = split == nctx_splits;
  const int base = blk ? 0 : (p0 & ~(kRingAlign - 1)) + kRingC * split;  // first key: a position, or block row 0
  const int lo = blk ? 0 : p0;                              // keys [lo, hi) are read
  const int hi = blk ? nq : L;
  float* ml = ws_ml + (size_t)unit * kRows * 2;
  float* os = ws_o + (size_t)unit * kRows * kRingDh;
  if (base >= hi || (!blk && nctx == 0)) {                 // a context split past the window: empty
    for (int e = tid; e < kRows; e += kRingThreads) {
      ml[2 * e] = -__builtin_inff();
      ml[2 * e + 1] = 0.f;
    }
    for (int e = tid; e < kRows * kRingDh / 4; e += kRingThreads)
      reinterpret_cast<f32x4*>(os)[e] = (f32x4){0.f, 0.f, 0.f, 0.f};
    return;
  }
  if (blk)
    ring_split<MT, true, true>(sm, q, k_blk, v_blk, k_ring, v_ring, b, kvh, nq, hq, hkv, ring, base, lo, hi,
                               scale_log2, ml, os);
  else if (base >= lo && base + kRingC <= hi)
    ring_split<MT, false, false>(sm, q, k_blk, v_blk, k_ring, v_ring, b, kvh, nq, hq, hkv, ring, base, lo, hi,
                                 scale_log2, ml, os);
  else
    ring_split<MT, false, true>(sm, q, k_blk, v_blk, k_ring, v_ring, b, kvh, nq, hq, hkv, ring, base, lo, hi,
                                scale_log2, ml, os);
}

// One work-group per (request, K/V head, 2 query rows): out = sum_s w_s O_s with
// w_s = e^(m_s - M) / sum_s' e^(m_s' - M) l_s' (M the rows' maximum over the splits);
// the weights of a row are formed once, then every output adds its splits' values with
// all loads in flight.
constexpr int kRingCombRows = 2;                // query rows per combine work-group: one output per thread
constexpr int kRingMaxSplits = 32;

template <int MT, int NSP>
__global__ void __launch_bounds__(kRingThreads) k_ring_combine(const float* __restrict__ ws_ml,
                                                                const float* __restrict__ ws_o, int nq, int hq,
                                                                int hkv, int nsplit, float* __restrict__ out) {
  constexpr int kRows = MT * 16;
  __shared__ float msh[kRingCombRows][NSP], lsh[kRingCombRows][NSP];
  __shared__ float wsh[kRingCombRows][NSP];
  const int groups = (kRows + kRingCombRows - 1) / kRingCombRows;
  const int bk = (int)blockIdx.x / groups;
  const int r0 = ((int)blockIdx.x % groups) * kRingCombRows;
  const int kvh = bk % hkv, b = bk / hkv;
  const int G = hq / hkv;
  const int nrows = nq * G;
  const size_t u0 = (size_t)bk * nsplit;
  // every (row, split) statistic loaded at once
  for (int e = threadIdx.x; e < kRingCombRows * nsplit; e += kRingThreads) {
    const int rl = e / nsplit, sp = e - rl * nsplit;
    const float* p = ws_ml + (u0 + sp) * kRows * 2 + 2 * (r0 + rl);
    msh[rl][sp] = p[0];
    lsh[rl][sp] = p[1];
  }
  __syncthreads();
  if (threadIdx.x < kRingCombRows) {
    const int rl = threadIdx.x;
    float M = -__builtin_inff();
    for (int sp = 0; sp < nsplit; ++sp) M = fmaxf(M, msh[rl][sp]);
    float den = 0.f;
    for (int sp = 0; sp < nsplit; ++sp) {
      const float w = msh[rl][sp] == -__builtin_inff() ? 0.f : exp2f(msh[rl][sp] - M);
      wsh[rl][sp] = w;
      den += w * lsh[rl][sp];
    }
    for (int sp = 0; sp < nsplit; ++sp) wsh[rl][sp] /= den;
    for (int sp = nsplit; sp < NSP; ++sp) wsh[rl][sp] = 0.f;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < kRingCombRows * kRingDh; e += kRingThreads) {
    const int rl = e / kRingDh, d = e - rl * kRingDh;
    const int row = r0 + rl;
    // every split's value in flight at once (past the last split: reread it, weight 0)
    float v[NSP];
#pragma unroll
    for (int sp = 0; sp < NSP; ++sp) v[sp] = ws_o[((u0 + (sp < nsplit ? sp : nsplit - 1)) * kRows + row) * kRingDh + d];
    float num = 0.f;
#pragma unroll
    for (int sp = 0; sp < NSP; ++sp) num += wsh[rl][sp] * v[sp];
    if (row < nrows) {
      const int i = row / G, h = kvh * G + row % G;
      out[((size_t)(b * nq + i) * hq + h) * kRingDh + d] = num;
    }
  }
}

int ring_rows_pad(int nq, int hq, int hkv) {
  const int rows = nq * (hq / hkv);
  return rows <= 16 ? 16 : rows <= 32 ? 32 : 48;
}

// Context splits of 128 positions covering window - 1 positions from a kRingAlign-aligned
// start, plus one split for the block's keys.
int ring_splits(int nq, int window) {
  (void)nq;
  return (window - 1 + kRingAlign - 1 + kRingC - 1) / kRingC + 1;
}

template <int MT>
static void ring_launch(hipStream_t s, const uint16_t* q, const uint16_t* kb, const uint16_t* vb, const uint16_t* kr,
                        const uint16_t* vr, const int32_t* ctx, int B, int nq, int hq, int hkv, int ring, int window,
                        float scale_log2, int nsplit, const RingWs& ws, float* out) {
  hipLaunchKernelGGL((k_ring_partial<MT>), dim3((unsigned)(B * hkv * nsplit)), dim3(kRingThreads), 0, s, q, kb, vb, kr,
                     vr, ctx, nq, hq, hkv, ring, window, scale_log2, nsplit - 1, ws.ml, ws.o);
  const int groups = (MT * 16 + kRingCombRows - 1) / kRingCombRows;
  const dim3 grid((unsigned)(B * hkv * groups));
  if (nsplit <= 8)
    hipLaunchKernelGGL((k_ring_combine<MT, 8>), grid, dim3(kRingThreads), 0, s, ws.ml, ws.o, nq, hq, hkv, nsplit, out);
  else if (nsplit <= 16)
    hipLaunchKernelGGL((k_ring_combine<MT, 16>), grid, dim3(kRingThreads), 0, s, ws.ml, ws.o, nq, hq, hkv, nsplit, out);
  else if (nsplit <= 24)
    hipLaunchKernelGGL((k_ring_combine<MT, 24>), grid, dim3(kRingThreads), 0, s, ws.ml, ws.o, nq, hq, hkv, nsplit, out);
  else
    hipLaunchKernelGGL((k_ring_combine<MT, 32>), grid, dim3(kRingThreads), 0, s, ws.ml, ws.o, nq, hq, hkv, nsplit, out);
}

hipError_t launch_ring_attention(const uint16_t* q, const uint16_t* k_blk, const uint16_t* v_blk,
                                 const uint16_t* k_ring, const uint16_t* v_ring, const int32_t* ctx_len, int batch,
                                 int nq, int hq, int hkv, int ring, int window, float scale, int nsplit, RingWs ws,
                                 float* out, hipStream_t s) {
  const float scale_log2 = scale * 1.4426950408889634f;
  switch (ring_rows_pad(nq, hq, hkv) / 16) {
    case 1: ring_launch<1>(s, q, k_blk, v_blk, k_ring, v_ring, ctx_len, batch, nq, hq, hkv, ring, window, scale_log2, nsplit, ws, out); break;
    case 2: ring_launch<2>(s, q, k_blk, v_blk, k_ring, v_ring, ctx_len, batch, nq, hq, hkv, ring, window, scale_log2, nsplit, ws, out); break;
    default: ring_launch<3>(s, q, k_blk, v_blk, k_ring, v_ring, ctx_len, batch, nq, hq, hkv, ring, window, scale_log2, nsplit, ws, out); break;
  }
  return hipGetLastError();
}

}  // namespace df2
