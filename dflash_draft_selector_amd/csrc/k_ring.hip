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
// window, a verify writes a few rows), both in tiles of 32 positions per (request, K/V
// head), ring % 32 == 0:
//   K [B][Hkv][ring / 32][2][4][4][16][8]: tile position p, dim d at [(p / 4) % 2]
//     [d / 32][(d % 32) / 8][4 (p / 8) + p % 4][d % 8], the order in which the MFMA
//     A-operand slices of a step are read, so each slice is one contiguous 1 KB;
//   V [B][Hkv][ring / 32][Dh][32]: transposed within the tile.
// The keys of a (request, K/V head) are cut into steps of 32: context step j covers
// positions pa + 32 j .. (pa = p0 rounded down to 32), masked to [p0, L), and is one
// whole tile of each ring (8 KB each); the block's keys follow as ceil(nq / 32) more
// steps.
//
// k_ring_split: one work-group of 8 waves per (request, K/V head, 16 query rows, key
// split).  The row tiles of a (request, K/V head) run side by side on one XCD and read
// the same tiles, so HBM delivers each tile once and L2 the rest; key splits are added
// only when the row tiles alone leave compute units idle.  A split takes an equal share
// of the steps and wave w every 8th of those.  A wave folds its steps on its own, with
// no LDS traffic but the Q^T slices and no barrier: S^T = K Q^T on
// v_mfma_f32_16x16x32_bf16 (K rows as the A operand, in an order chosen so that each lane
// ends up holding the scores of 8 consecutive keys of one query row: exactly the lane
// layout of the B operand of the next product), an online softmax per query row
// (maximum across the row's four lanes with two permlane swaps), P = 2^(S - m) split
// into bf16 high and low parts, and O^T += V^T P^T on the same MFMA with V^T straight
// from the tile.  Two fragment sets per wave: the next step's loads are in flight while
// a step is folded.  At the end the waves' (max, sum, O) are merged through LDS and the
// work-group writes the normalised output, or its rows' state when there are several
// splits, which k_ring_combine then merges.
#include "dflash2_internal.h"
#include "device_common.h"

namespace df2 {

constexpr int kRingWaves = 8;                // waves of a split work-group
constexpr int kRingThreads = 64 * kRingWaves;
constexpr int kCombThreads = 256;
constexpr int kRingDh = 128;                 // head dim
constexpr int kRingStep = 32;                // keys per wave step
constexpr int kRingTargetGroups = 256;       // work-groups aimed for: one per compute unit
constexpr int kRingMaxSplits = 32;
constexpr int kRingRedPitch = 64 + 4;        // floats per staged half row of O (dims 64 at a time)

RingWs carve_ring(Carver& c, int64_t batch, int64_t hkv, int nsplit, int rows_pad) {
  RingWs w;
  const size_t units = (size_t)batch * hkv * nsplit;
  w.ml = c.take<float>(units * rows_pad * 2);
  w.o = c.take<float>(units * rows_pad * kRingDh);
  return w;
}

template <int MT, int W = kRingWaves>
struct RingShared {
  u32x4 q[MT][4][64];                        // Q^T B-operand slices in lane order (read each step)
  float m[W][MT * 16];                       // per-wave row maxima (log2 units)
  float l[W][MT * 16];                       // per-wave row sums
  float lt[MT * 16];                         // the work-group's row sums
  float red[W][MT * 16][kRingRedPitch];      // per-wave O, half the dims at a time
};

// max / sum over the four 16-lane rows of the wave (lanes l, l ^ 16, l ^ 32, l ^ 48);
// every lane gets the same value
__device__ __forceinline__ float quad_row_max(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float quad_row_sum(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Operands of one 32-key step as the MFMAs take them.  S^T tile t (16 keys x 16 rows):
// A-operand row m is key 8 (m / 4) + 4 t + m % 4, so the result's lane (row, g) holds in
// register r the score of key 8 g + 4 t + r; over t = 0, 1 that is keys 8 g .. 8 g + 7,
// the B-operand slice of P^T for the O^T product.  k[t][s]: dims 32 s + 8 g .. + 7 of the
// lane's key; v[dt]: V^T dim 16 dt + i16 over keys 8 g .. 8 g + 7.
struct RingFrag {
  u32x4 k[2][4];
  u32x4 v[kRingDh / 16];
};

// Buffer resource over `bytes` bytes from p (raw, offsets in bytes; reads past the end
// return zero).  Every per-lane offset below is a 32-bit byte offset into one head's
// part of a ring or of the block, so a lane needs one VGPR per address instead of two.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t ring_rsrc(const void* p, uint64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0,
                                           (int)(bytes > 0xffffffffull ? 0xffffffffu : (uint32_t)bytes), 0x00020000);
}

// The resources of one (request, K/V head): its K and V tiles (ring * Dh elements each),
// and its rows of the block's K and V ([nq] rows, hkv * Dh elements apart).
struct RingRes {
  __amdgpu_buffer_rsrc_t kr, vr, kb, vb;
};

constexpr int kRingAux = 0;                  // cache policy of the ring reads (non-temporal re-fetched half lines)

// This lane's byte offsets within a step's tiles: its 16 bytes of every K slice (k), and
// V^T dim i16 at positions 8 g .. 8 g + 7 (v); the tile and the slice or 16-dim group
// come in as scalar or immediate offsets.
struct RingLane {
  uint32_t k;
  uint32_t v;
};

__device__ __forceinline__ RingLane ring_lane() {
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4, i16 = lane & 15;
  RingLane l;
  l.k = (uint32_t)lane * 16;
  l.v = (uint32_t)i16 * (kRingStep * 2) + 16 * g;
  return l;
}

// Context step whose tile starts at ring row rb (a multiple of 32): both tiles are
// kRingStep * Dh * 2 = 8 KB from byte rb * Dh * 2; K slice (t, s) is the tile's 1 KB
// number 4 t + s.
__device__ __forceinline__ void ring_load_step(RingFrag& f, const RingRes& rr, const RingLane& ln, int rb) {
  const uint32_t tile = (uint32_t)rb * (kRingDh * 2);
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int s = 0; s < 4; ++s)
      f.k[t][s] = __builtin_amdgcn_raw_buffer_load_b128(rr.kr, ln.k + (4 * t + s) * 1024, tile, kRingAux);
#pragma unroll
  for (int dt = 0; dt < kRingDh / 16; ++dt)
    f.v[dt] = __builtin_amdgcn_raw_buffer_load_b128(rr.vr, ln.v + dt * 16 * kRingStep * 2, tile, kRingAux);
}

// The block's keys kb0 .. kb0 + 31; keys past nq read row 0 and are masked when folded.
__device__ __forceinline__ void ring_load_blk(RingFrag& f, const RingRes& rr, int nq, int hkv, int kb0) {
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4, i16 = lane & 15;
  const int koff = 8 * (i16 >> 2) + (i16 & 3);
  const uint32_t rowb = (uint32_t)hkv * (kRingDh * 2);       // bytes between the block's rows
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int key = kb0 + koff + 4 * t;
    const uint32_t o = (uint32_t)(key < nq ? key : 0) * rowb + 16 * g;
#pragma unroll
    for (int s = 0; s < 4; ++s) f.k[t][s] = __builtin_amdgcn_raw_buffer_load_b128(rr.kb, o + 64 * s, 0, 0);
  }
  uint32_t w[kRingDh / 16][4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int j0 = kb0 + 8 * g + 2 * c, j1 = j0 + 1;
    const uint32_t o0 = (uint32_t)(j0 < nq ? j0 : 0) * rowb + 2 * i16;
    const uint32_t o1 = (uint32_t)(j1 < nq ? j1 : 0) * rowb + 2 * i16;
#pragma unroll
    for (int dt = 0; dt < kRingDh / 16; ++dt) {
      const uint32_t a = __builtin_amdgcn_raw_buffer_load_b16(rr.vb, o0 + 32 * dt, 0, 0);
      const uint32_t bb = __builtin_amdgcn_raw_buffer_load_b16(rr.vb, o1 + 32 * dt, 0, 0);
      w[dt][c] = a | (bb << 16);
    }
  }
#pragma unroll
  for (int dt = 0; dt < kRingDh / 16; ++dt) f.v[dt] = (u32x4){w[dt][0], w[dt][1], w[dt][2], w[dt][3]};
}

// A wave's running softmax state for its rows: the maximum m (log2 units; the same in
// the four lanes of a row), this lane's share of the row sum, and O^T (lane (row, g)
// holds dims 16 dt + 4 g .. + 3).
template <int MT>
struct RingState {
  float m[MT];
  float l[MT];
  f32x4 o[kRingDh / 16][MT];
};

// One step (keys base + 0 .. 31, valid where lo <= key < hi) is folded into the state:
// ring_scores takes S^T = K Q^T (keys outside [lo, hi) get -inf), ring_accum the online
// softmax and O^T += V^T P^T (keys outside get zero V^T words: a stale row never enters,
// not even times zero).  The masks are computed on every step, without a branch.
template <int MT>
__device__ __forceinline__ void ring_scores(const RingShared<MT>& sm, const u32x4 (&k)[2][4], int base, int lo, int hi,
                                            float scale_log2, float (&x)[MT][8]) {
  const int lane = threadIdx.x & 63;
  const int kl = base + 8 * (lane >> 4);       // this lane's keys: kl + 0 .. 7
  // Q^T slices come from LDS each step: the address goes through an empty asm, so the
  // reads cannot be hoisted out of the step loop into registers
  typedef __attribute__((address_space(3))) const u32x4 lds_u32x4;
  lds_u32x4* qs = (lds_u32x4*)&sm.q[0][0][lane];
  asm volatile("" : "+v"(qs));
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    f32x4 sacc[2] = {(f32x4){0.f, 0.f, 0.f, 0.f}, (f32x4){0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const u32x4 qv = qs[(mt * 4 + s) * 64];
#pragma unroll
      for (int t = 0; t < 2; ++t)
        sacc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, k[t][s]),
                                                         __builtin_bit_cast(bf16x8, qv), sacc[t], 0, 0, 0);
    }
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int jj = 4 * t + r;
        const float v = sacc[t][r] * scale_log2;
        x[mt][jj] = (unsigned)(kl + jj - lo) < (unsigned)(hi - lo) ? v : -__builtin_inff();
      }
  }
}

template <int MT>
__device__ __forceinline__ void ring_accum(u32x4 (&v)[kRingDh / 16], const float (&x)[MT][8], int base, int lo, int hi,
                                           RingState<MT>& st) {
  const int lane = threadIdx.x & 63;
  const int kl = base + 8 * (lane >> 4);
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const bool v0 = (unsigned)(kl + 2 * c - lo) < (unsigned)(hi - lo);
    const bool v1 = (unsigned)(kl + 2 * c + 1 - lo) < (unsigned)(hi - lo);
    const uint32_t keep = (v0 ? 0xffffu : 0u) | (v1 ? 0xffff0000u : 0u);
#pragma unroll
    for (int dt = 0; dt < kRingDh / 16; ++dt) v[dt][c] &= keep;
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    float mloc = -__builtin_inff();
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) mloc = fmaxf(mloc, x[mt][jj]);
    const float mn = fmaxf(st.m[mt], quad_row_max(mloc));   // finite: every step holds a valid key
    const float alpha = st.m[mt] == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(st.m[mt] - mn);
    st.m[mt] = mn;
    float sum = 0.f;
    uint32_t ph[4], pl[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const float p0 = __builtin_amdgcn_exp2f(x[mt][2 * c] - mn);   // v_exp_f32; 2^-inf = 0
      const float p1 = __builtin_amdgcn_exp2f(x[mt][2 * c + 1] - mn);
      sum += p0;
      sum += p1;
      const bf16x2 h = __builtin_convertvector((f32x2){p0, p1}, bf16x2);   // nearest even
      const f32x2 hf = __builtin_convertvector(h, f32x2);
      const bf16x2 lw = __builtin_convertvector((f32x2){p0 - hf[0], p1 - hf[1]}, bf16x2);
      ph[c] = __builtin_bit_cast(uint32_t, h);
      pl[c] = __builtin_bit_cast(uint32_t, lw);
    }
    st.l[mt] = st.l[mt] * alpha + sum;
#pragma unroll
    for (int dt = 0; dt < kRingDh / 16; ++dt) st.o[dt][mt] *= alpha;
    const bf16x8 bh = __builtin_bit_cast(bf16x8, (u32x4){ph[0], ph[1], ph[2], ph[3]});
    const bf16x8 bl = __builtin_bit_cast(bf16x8, (u32x4){pl[0], pl[1], pl[2], pl[3]});
#pragma unroll
    for (int dt = 0; dt < kRingDh / 16; ++dt) {
      st.o[dt][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, v[dt]), bh, st.o[dt][mt], 0, 0,
                                                             0);
      st.o[dt][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, v[dt]), bl, st.o[dt][mt], 0, 0,
                                                             0);
    }
  }
}

template <int MT>
__device__ __forceinline__ void ring_fold(const RingShared<MT>& sm, RingFrag& f, int base, int lo, int hi,
                                          float scale_log2, RingState<MT>& st) {
  float x[MT][8];
  ring_scores<MT>(sm, f.k, base, lo, hi, scale_log2, x);
  ring_accum<MT>(f.v, x, base, lo, hi, st);
}

// Steps of a request: context steps covering [pa, L) (none when the window is empty),
// then the block's.
struct RingSteps {
  int L, p0, pa, nsc, total;
};

__device__ __forceinline__ RingSteps ring_steps(int ctx, int window, int nq) {
  RingSteps r;
  r.L = ctx > 0 ? ctx : 0;
  const int nctx = r.L < window - 1 ? r.L : window - 1;
  r.p0 = r.L - nctx;
  r.pa = r.p0 & ~(kRingStep - 1);
  r.nsc = nctx > 0 ? (r.L - r.pa + kRingStep - 1) / kRingStep : 0;
  r.total = r.nsc + (nq + kRingStep - 1) / kRingStep;
  return r;
}

template <int MT>
__global__ void __launch_bounds__(kRingThreads, 8 / kRingWaves) k_ring_split(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_blk, const uint16_t* __restrict__ v_blk,
    const uint16_t* __restrict__ k_ring, const uint16_t* __restrict__ v_ring, const int32_t* __restrict__ ctx_len,
    int nq, int hq, int hkv, int ring, int window, float scale_log2, int nsplit, int ntile, int nunits,
    float* __restrict__ ws_ml, float* __restrict__ ws_o, float* __restrict__ out) {
  __shared__ RingShared<MT> sm;
  constexpr int kRows = MT * 16;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int g = lane >> 4, i16 = lane & 15;
  // work-group id -> (request, K/V head, split) unit u and row tile rt; the ntile row
  // tiles of a unit get ids 8 apart, so they run on one XCD and share its L2 copy of the
  // unit's K/V tiles (the ring is read from HBM once)
  const int id = blockIdx.x;
  const int u = ((id >> 3) / ntile) * 8 + (id & 7);
  const int rt = (id >> 3) % ntile;
  if (u >= nunits) return;                                  // padding work-groups
  const int split = u % nsplit;
  const int bk = u / nsplit;
  const int unit = (bk * ntile + rt) * nsplit + split;      // this work-group's partial-sum slot
  const int row0 = kRows * rt;                              // its first query row
  const int kvh = bk % hkv, b = bk / hkv;
  const int G = hq / hkv;
  const int nrows = nq * G;
  const size_t head = (size_t)b * hkv + kvh;

  const RingSteps rs = ring_steps(ctx_len[b], window, nq);
  const int c0 = (int)((long long)split * rs.total / nsplit);
  const int c1 = (int)((long long)(split + 1) * rs.total / nsplit);

  // the wave's steps (wave-uniform: the loop and its branches stay scalar); the first
  // step's loads are issued before Q is staged, so that the two latencies overlap
  RingRes rr;
  rr.kr = ring_rsrc(k_ring + head * ring * kRingDh, (uint64_t)ring * kRingDh * 2);
  rr.vr = ring_rsrc(v_ring + head * kRingDh * ring, (uint64_t)ring * kRingDh * 2);
  const size_t blk0 = ((size_t)b * nq * hkv + kvh) * kRingDh;
  const uint64_t blk_bytes = ((uint64_t)(nq - 1) * hkv + 1) * kRingDh * 2;
  rr.kb = ring_rsrc(k_blk + blk0, blk_bytes);
  rr.vb = ring_rsrc(v_blk + blk0, blk_bytes);
  RingFrag f;
  int j = c0 + __builtin_amdgcn_readfirstlane(wv);
  const int jend = c1 < rs.nsc ? c1 : rs.nsc;   // the wave's context steps: j, j + W, .. < jend
  const RingLane ln = ring_lane();
  const int jlast = j + kRingWaves * ((jend - 1 - j) / kRingWaves);
  const int rstep = kRingStep * kRingWaves;     // ring rows between the wave's steps
  // positions relative to pa from here on (a context length near INT_MAX stays in range)
  const int ra = rs.pa % ring;                  // ring row of position pa
  const int lo = rs.p0 - rs.pa, hi = rs.L - rs.pa;
  int rb = (ra + kRingStep * j) % ring;
  const int rlast = (ra + kRingStep * jlast) % ring;
  if (j < jend) ring_load_step(f, rr, ln, rb);

  // Q^T as the B operand, staged in LDS: entry [mt][s][lane] is row 16 mt + lane % 16,
  // dims 32 s + 8 (lane / 16) .. + 7 (zero for padding rows)
  for (int e = tid; e < MT * 4 * 64; e += kRingThreads) {
    const int mt = e >> 8, s4 = (e >> 6) & 3, l = e & 63;
    const int r = row0 + 16 * mt + (l & 15);
    u32x4 v = (u32x4){0u, 0u, 0u, 0u};
    if (r < nrows)
      v = *reinterpret_cast<const u32x4*>(q + ((size_t)(b * nq + r / G) * hq + kvh * G + r % G) * kRingDh + 32 * s4 +
                                          8 * (l >> 4));
    sm.q[mt][s4][l] = v;
  }
  __syncthreads();
  RingState<MT> st;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    st.m[mt] = -__builtin_inff();
    st.l[mt] = 0.f;
#pragma unroll
    for (int dt = 0; dt < kRingDh / 16; ++dt) st.o[dt][mt] = (f32x4){0.f, 0.f, 0.f, 0.f};
  }

  if (j < jend) {
    // two fragment sets, the next step's loads issued before this one is folded (past the
    // wave's last step its last one is loaded again, from cache)
    RingFrag fb;
    for (;;) {
      {
        int rn = rb + rstep;
        rn = rn >= ring ? rn % ring : rn;
        ring_load_step(fb, rr, ln, j + kRingWaves < jend ? rn : rlast);
        ring_fold<MT>(sm, f, kRingStep * j, lo, hi, scale_log2, st);
        j += kRingWaves;
        rb = rn;
        if (j >= jend) break;
      }
      {
        int rn = rb + rstep;
        rn = rn >= ring ? rn % ring : rn;
        ring_load_step(f, rr, ln, j + kRingWaves < jend ? rn : rlast);
        ring_fold<MT>(sm, fb, kRingStep * j, lo, hi, scale_log2, st);
        j += kRingWaves;
        rb = rn;
        if (j >= jend) break;
      }
    }
  }
  for (; j < c1; j += kRingWaves) {             // steps of the block's keys
    const int kb0 = kRingStep * (j - rs.nsc);
    ring_load_blk(f, rr, nq, hkv, kb0);
    ring_fold<MT>(sm, f, kb0, 0, nq, scale_log2, st);
  }

  // ---- merge the waves: row maxima and sums, then O half the dims at a time -----------
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const float lw = quad_row_sum(st.l[mt]);
    if (g == 0) {
      sm.m[wv][16 * mt + i16] = st.m[mt];
      sm.l[wv][16 * mt + i16] = lw;
    }
  }
  __syncthreads();
  float aself[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int row = 16 * mt + i16;
    float M = -__builtin_inff();
#pragma unroll
    for (int w = 0; w < kRingWaves; ++w) M = fmaxf(M, sm.m[w][row]);
    float lt = 0.f;
#pragma unroll
    for (int w = 0; w < kRingWaves; ++w)
      lt += (sm.m[w][row] == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(sm.m[w][row] - M)) * sm.l[w][row];
    aself[mt] = st.m[mt] == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(st.m[mt] - M);
    if (wv == 0 && g == 0) {
      sm.lt[row] = lt;
      if (nsplit > 1) {
        ws_ml[((size_t)unit * kRows + row) * 2] = M;
        ws_ml[((size_t)unit * kRows + row) * 2 + 1] = lt;
      }
    }
  }
  float* os = ws_o + (size_t)unit * kRows * kRingDh;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int d4 = 0; d4 < 4; ++d4)
        *reinterpret_cast<f32x4*>(&sm.red[wv][16 * mt + i16][16 * d4 + 4 * g]) = st.o[4 * half + d4][mt] * aself[mt];
    __syncthreads();
    for (int e = tid; e < kRows * 16; e += kRingThreads) {
      const int row = e >> 4, c4 = e & 15;
      f32x4 v = *reinterpret_cast<const f32x4*>(&sm.red[0][row][4 * c4]);
#pragma unroll
      for (int w = 1; w < kRingWaves; ++w) v += *reinterpret_cast<const f32x4*>(&sm.red[w][row][4 * c4]);
      const int d = 64 * half + 4 * c4;
      if (nsplit > 1) {
        *reinterpret_cast<f32x4*>(os + (size_t)row * kRingDh + d) = v;
      } else if (row0 + row < nrows) {
        const float inv = 1.f / sm.lt[row];
        const int i = (row0 + row) / G, h = kvh * G + (row0 + row) % G;
        *reinterpret_cast<f32x4*>(out + ((size_t)(b * nq + i) * hq + h) * kRingDh + d) = v * inv;
      }
    }
    __syncthreads();
  }
}

// One wave per (request, K/V head, query row): out = sum_s w_s O_s / sum_s w_s l_s with
// w_s = 2^(m_s - M) (M the row's maximum over the splits).  Every split's (max, sum) and
// the lane's two dims of every split's O are loaded at once; the splits are added in
// order.
template <int MT, int NSP>
__global__ void __launch_bounds__(kCombThreads) k_ring_combine(const float* __restrict__ ws_ml,
                                                                const float* __restrict__ ws_o, int nq, int hq,
                                                                int hkv, int nsplit, int ntile, int nunits,
                                                                float* __restrict__ out) {
  constexpr int kRows = MT * 16;
  const int lane = threadIdx.x & 63;
  const int wid = (int)blockIdx.x * (kCombThreads / 64) + (int)(threadIdx.x >> 6);
  if (wid >= nunits) return;                       // whole waves
  const int G = hq / hkv;
  const int nrows = nq * G;
  const int bk = wid / nrows, row = wid - bk * nrows;
  const int rt = row / kRows, rl = row - rt * kRows;      // row tile and row within it
  const size_t u0 = ((size_t)bk * ntile + rt) * nsplit;
  float m = -__builtin_inff(), l = 0.f;
  if (lane < nsplit) {
    m = ws_ml[((u0 + lane) * kRows + rl) * 2];
    l = ws_ml[((u0 + lane) * kRows + rl) * 2 + 1];
  }
  f32x2 o[NSP];
#pragma unroll
  for (int sp = 0; sp < NSP; ++sp)
    o[sp] = *reinterpret_cast<const f32x2*>(ws_o + ((u0 + (sp < nsplit ? sp : 0)) * kRows + rl) * kRingDh + 2 * lane);
  float M = m;
#pragma unroll
  for (int x = 1; x < 64; x <<= 1) M = fmaxf(M, __shfl_xor(M, x));
  const float w = m == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(m - M);
  float den = w * l;
#pragma unroll
  for (int x = 1; x < 64; x <<= 1) den += __shfl_xor(den, x);
  f32x2 num = (f32x2){0.f, 0.f};
#pragma unroll
  for (int sp = 0; sp < NSP; ++sp) {
    const float ws = __shfl(w, sp);                // zero past the last split
    num += ws * o[sp];
  }
  const int i = row / G, h = (bk % hkv) * G + row % G;
  const int b = bk / hkv;
  *reinterpret_cast<f32x2*>(out + ((size_t)(b * nq + i) * hq + h) * kRingDh + 2 * lane) = num * (1.f / den);
}

int ring_rows_pad(int nq, int hq, int hkv) {
  const int rows = nq * (hq / hkv);
  return rows <= 16 ? 16 : rows <= 32 ? 32 : 48;
}

// The most steps a request can have: window - 1 context positions from a 32-aligned
// start, then the block's.
static int ring_max_steps(int nq, int window) {
  return (window - 1 + 2 * (kRingStep - 1)) / kRingStep + (nq + kRingStep - 1) / kRingStep;
}

// Row tiles of 16 query rows per (request, K/V head); each is its own work-group.
static int ring_tiles(int nq, int hq, int hkv) { return ring_rows_pad(nq, hq, hkv) / 16; }

// Key splits per (request, K/V head): enough work-groups (row tiles x splits) for one per
// compute unit, at least one step per wave of the longest request, at most kRingMaxSplits.
int ring_splits(int64_t batch, int64_t hkv, int nq, int hq, int window) {
  const int64_t groups = batch * hkv * ring_tiles(nq, hq, (int)hkv);
  int64_t n = kRingTargetGroups / groups;
  const int most = (ring_max_steps(nq, window) + kRingWaves - 1) / kRingWaves;
  if (n > most) n = most;
  if (n > kRingMaxSplits) n = kRingMaxSplits;
  return n < 1 ? 1 : (int)n;
}

hipError_t launch_ring_attention(const uint16_t* q, const uint16_t* k_blk, const uint16_t* v_blk,
                                 const uint16_t* k_ring, const uint16_t* v_ring, const int32_t* ctx_len, int batch,
                                 int nq, int hq, int hkv, int ring, int window, float scale, int nsplit, RingWs ws,
                                 float* out, hipStream_t s) {
  if (nsplit < 1 || nsplit > kRingMaxSplits) return hipErrorInvalidValue;
  const float scale_log2 = scale * 1.4426950408889634f;
  const int ntile = ring_tiles(nq, hq, hkv);
  const int nunits = batch * hkv * nsplit;                 // (request, K/V head, split)
  const unsigned groups = (unsigned)((nunits + 7) / 8 * 8 * ntile);
  hipLaunchKernelGGL((k_ring_split<1>), dim3(groups), dim3(kRingThreads), 0, s, q, k_blk, v_blk, k_ring, v_ring,
                     ctx_len, nq, hq, hkv, ring, window, scale_log2, nsplit, ntile, nunits, ws.ml, ws.o, out);
  if (nsplit > 1) {
    const int nrows_all = batch * hkv * nq * (hq / hkv);
    const dim3 grid((unsigned)((nrows_all + kCombThreads / 64 - 1) / (kCombThreads / 64)));
    if (nsplit <= 4)
      hipLaunchKernelGGL((k_ring_combine<1, 4>), grid, dim3(kCombThreads), 0, s, ws.ml, ws.o, nq, hq, hkv, nsplit, ntile, nrows_all, out);
    else if (nsplit <= 8)
      hipLaunchKernelGGL((k_ring_combine<1, 8>), grid, dim3(kCombThreads), 0, s, ws.ml, ws.o, nq, hq, hkv, nsplit, ntile, nrows_all, out);
    else if (nsplit <= 16)
      hipLaunchKernelGGL((k_ring_combine<1, 16>), grid, dim3(kCombThreads), 0, s, ws.ml, ws.o, nq, hq, hkv, nsplit, ntile, nrows_all, out);
    else
      hipLaunchKernelGGL((k_ring_combine<1, 32>), grid, dim3(kCombThreads), 0, s, ws.ml, ws.o, nq, hq, hkv, nsplit, ntile, nrows_all, out);
  }
  return hipGetLastError();
}

}  // namespace df2
