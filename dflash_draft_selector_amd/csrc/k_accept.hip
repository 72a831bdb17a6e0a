// Lossless verify (FreeToken PR "Adds DFlash 2", section "Details", sampled verify:
// accept with min(1, p/q), on a reject resample from max(0, p - q); all-greedy keeps
// the prefix match.  pegainfer issue "DFlash 2 proposer", "Proposal", phase 3).
//
// Pass 1 streams every target row once, split like the top-16 stream (512-thread
// work-groups, 19 loads of 16 bytes in flight per lane).  T > 0 (k_accept_stats): each
// wave owns a contiguous sub-chunk of its work-group's vectors and writes the sub-chunk's
// max and sum of exp((l - max)/T).  T == 0 (k_greedy_argmax): the chunk argmax.
// Pass 2, one work-group per request.  Greedy (k_greedy_decide, one wave): the row
// argmaxes and the prefix match.  Sampled (k_accept_decide): one wave merges the rows'
// statistics (fixed sub-chunk order), runs the accept tests and finds the sub-chunk in
// which the inverse-CDF draw lands (sub-chunk masses minus the draft's mass at its
// candidates); the whole work-group then rescans that one sub-chunk.
#include "device_common.h"
#include "dflash2.h"
#include "dflash2_internal.h"
#include "topk_dev.h"
#include "verify_dev.h"

namespace df2 {

AcceptWs carve_accept(Carver& c, int64_t nrows, int64_t vocab) {
  AcceptWs w;
  const size_t n = (size_t)nrows * topk_num_chunks(vocab);
  w.chunk_max = c.take<float>(n * kSubPerChunk);
  w.chunk_sum = c.take<float>(n * kSubPerChunk);
  w.chunk_arg = c.take<unsigned long long>(n);
  return w;
}

__device__ __forceinline__ float order_to_float(int s) { return bf16_to_f32(order_to_bits(s)); }

// ---- sampled pass 1: max and sum of weights of every sub-chunk ------------------------
// Wave j of work-group (row, c) reads sub-chunk 8c + j: lane l holds its vectors l,
// l + 64, ... (each load instruction covers 1 KB of the row).  Missing logits read as
// -inf (weight 0).  Each lane folds every vector in as soon as its load lands: a running
// max m and the sum of weights relative to it (rescaled when m grows), so the weights are
// formed while the rest of the row is still streaming in.  A sub-chunk holding +inf or
// NaN (a raw half >= 0x7f80 read as signed, or > 0xff80 read as unsigned) gets a NaN max.
// No LDS and no barrier: each wave writes its own pair.

__device__ __forceinline__ int float_order(float f) {
  const int b = __float_as_int(f);
  return b ^ ((b >> 31) & 0x7fffffff);
}
__device__ __forceinline__ float order_float(int o) { return __int_as_float(o ^ ((o >> 31) & 0x7fffffff)); }

__global__ void __launch_bounds__(kTopkThreads) k_accept_stats(const uint16_t* __restrict__ target, int64_t ld,
                                                               int64_t batch_stride, int K, int V, int nchunks,
                                                               float inv_t, AcceptWs ws, int batch) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
  // per-request rows: request b's blocks on the XCD of its decide work-group
  const int blk = batch_stride == 0 ? (int)blockIdx.x : xcd_chunk_block((int)blockIdx.x, batch, K + 1, nchunks);
  if (blk < 0) return;                            // padding ids (the whole work-group)
  const int r = blk / nchunks;
  const int c = blk - r * nchunks;
  const int b = batch_stride == 0 ? 0 : r / (K + 1);
  const int t = batch_stride == 0 ? r : r - b * (K + 1);
  const uint16_t* rowp = target + (size_t)b * batch_stride + (size_t)t * ld;
  const u32x4* __restrict__ rowv = reinterpret_cast<const u32x4*>(rowp);
  const int s = c * kSubPerChunk + wave;
  const int s0 = sub_begin(V, nchunks, s), s1 = sub_begin(V, nchunks, s + 1);
  const int safe = sub_begin(V, nchunks, c * kSubPerChunk);   // the chunk's first vector: whole
  const int nfull = V >> 3;

  u32x4 d[kTopkVecPerThread];
  unsigned whole = 0u;
#pragma unroll
  for (int k = 0; k < kTopkVecPerThread; ++k) {
    const int v = s0 + lane + k * kWave;
    const bool w = v < s1 && v < nfull;
    d[k] = __builtin_nontemporal_load(rowv + (w ? v : safe));
    whole |= (w ? 1u : 0u) << k;
  }
  // every load is issued before any is used: the fold below consumes the vectors in
  // order (a slot that is not whole as -inf), and without this fence the scheduler
  // trades loads in flight for registers
  __builtin_amdgcn_sched_barrier(0);
  // the row's ragged last vector (V % 8 != 0), in the one lane that owns it
  const int vr = nfull - s0;
  if ((V & 7) != 0 && nfull < s1 && vr >= 0 && lane == (vr & (kWave - 1))) {
    uint32_t w4[4] = {0xff80ff80u, 0xff80ff80u, 0xff80ff80u, 0xff80ff80u};
#pragma unroll 1
    for (int e = 0; e < (V & 7); ++e) {
      const uint32_t bb = rowp[8 * nfull + e];
      w4[e >> 1] = (e & 1) ? ((w4[e >> 1] & 0xffffu) | (bb << 16)) : ((w4[e >> 1] & 0xffff0000u) | bb);
    }
    const u32x4 x = (u32x4){w4[0], w4[1], w4[2], w4[3]};
    const int kr = vr / kWave;
#pragma unroll
    for (int k = 0; k < kTopkVecPerThread; ++k)
      if (k == kr) d[k] = x;
    whole |= 1u << kr;
  }

  const float c2 = inv_t * kLog2e;
  float m = -__builtin_inff(), S = 0.f;
  s16x2 hs = (s16x2){-32768, -32768};
  u16x2 hu = (u16x2){0, 0};
#pragma unroll
  for (int k = 0; k < kTopkVecPerThread; ++k) {
    const u32x4 x = ((whole >> k) & 1u) ? d[k] : (u32x4){0xff80ff80u, 0xff80ff80u, 0xff80ff80u, 0xff80ff80u};
    const s16x2 a0 = __builtin_bit_cast(s16x2, x.x), a1 = __builtin_bit_cast(s16x2, x.y);
    const s16x2 a2 = __builtin_bit_cast(s16x2, x.z), a3 = __builtin_bit_cast(s16x2, x.w);
    hs = __builtin_elementwise_max(hs, __builtin_elementwise_max(__builtin_elementwise_max(a0, a1),
                                                                 __builtin_elementwise_max(a2, a3)));
    const u16x2 b0 = __builtin_bit_cast(u16x2, x.x), b1 = __builtin_bit_cast(u16x2, x.y);
    const u16x2 b2 = __builtin_bit_cast(u16x2, x.z), b3 = __builtin_bit_cast(u16x2, x.w);
    hu = __builtin_elementwise_max(hu, __builtin_elementwise_max(__builtin_elementwise_max(b0, b1),
                                                                 __builtin_elementwise_max(b2, b3)));
    float f[8];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      f[2 * w] = bf16_lo(x[w]);
      f[2 * w + 1] = bf16_hi(x[w]);
    }
    // (NaN is ignored by the max; its sub-chunk is marked non-finite below)
    const float vm = fmaxf(fmaxf(fmaxf(f[0], f[1]), fmaxf(f[2], f[3])), fmaxf(fmaxf(f[4], f[5]), fmaxf(f[6], f[7])));
    const float mn = fmaxf(m, vm);
    const float mref = mn == -__builtin_inff() ? 0.f : mn;   // every logit so far -inf: weights 0
    S *= mn == m ? 1.f : tweight(m, mref, c2);
#pragma unroll
    for (int e = 0; e < 8; ++e) S += tweight(f[e], mref, c2);
    m = mn;
  }
  // the wave's pair: its max, and the lanes' sums rescaled to it
  const int hmax = hs.x > hs.y ? (int)hs.x : (int)hs.y;
  const int umax = hu.x > hu.y ? (int)hu.x : (int)hu.y;
  const bool nonfinite = __ballot(hmax >= 0x7f80 || umax > 0xff80) != 0ull;
  const float mw = order_float(wave_max_i32(float_order(m)));
  const float sum = wave_total(m == -__builtin_inff() ? 0.f : S * tweight(m, mw, c2));
  if (lane == 0) {
    const size_t si = (size_t)r * (nchunks * kSubPerChunk) + s;
    ws.chunk_max[si] = nonfinite ? __builtin_nanf("") : mw;
    ws.chunk_sum[si] = sum;
  }
}

// ---- greedy pass 1: the argmax of every target row -----------------------------------
// Rows are split like the top-16 chunks (two 512-thread blocks per row at V = 151936,
// 19 loads of 16 bytes in flight per lane).  A block's chunk argmax: the maximum of
// the packed signed-order halves (+NaN clamped to +inf), reduced over the block; then
// the lowest id whose key equals it, searched only in vectors whose maximum reaches it
// (-0 sits one order below +0 and shares its key).  A chunk whose only maxima were
// +NaN finds none and takes the exact composite maximum.
__global__ void __launch_bounds__(kTopkThreads) k_greedy_argmax(const uint16_t* __restrict__ target, int64_t ld,
                                                                int64_t batch_stride, int K, int V, int nchunks,
                                                                unsigned long long* __restrict__ chunk_arg) {
  __shared__ int s_red[kTopkWaves];
  __shared__ unsigned long long s_redu[kTopkWaves];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1), wave = tid >> 6;
  // (no XCD placement here: the greedy decide reads 8 bytes per chunk, and placing the
  // blocks measured 0.07 us slower)
  const int r = blockIdx.x / nchunks;
  const int c = blockIdx.x - r * nchunks;
  const int b = batch_stride == 0 ? 0 : r / (K + 1);
  const int t = batch_stride == 0 ? r : r - b * (K + 1);
  const uint16_t* rowp = target + (size_t)b * batch_stride + (size_t)t * ld;
  const int v0 = chunk_begin(V, nchunks, c), v1 = chunk_begin(V, nchunks, c + 1);

  u32x4 d[kTopkVecPerThread];
  load_chunk(rowp, V, v0, v1, d);                  // missing logits read as -NaN (lowest)
  int vmax[kTopkVecPerThread];
  int lmax = vector_maxima<true>(d, vmax);
  lmax = lmax > 0x7f80 ? 0x7f80 : lmax;
  lmax = wave_max_i32(lmax);
  if (lane == 0) s_red[wave] = lmax;
  __syncthreads();
  int M = s_red[0];
#pragma unroll
  for (int w = 1; w < kTopkWaves; ++w) M = max(M, s_red[w]);
  const uint32_t mbits = order_to_bits(M);
  const uint32_t mkey = bf16_key(mbits);
  // Only the vectors holding the maximum reach M - 1: usually one lane of one wave.
  // Each lane marks its own on the vector unit; a wave with none skips the search.
  const int nfull = V >> 3;
  uint32_t q = 0;
#pragma unroll
  for (int k = 0; k < kTopkVecPerThread; ++k) {
    const int v = v0 + tid + k * kTopkThreads;
    q |= (v < v1 && (vmax[k] > 0x7f80 ? 0x7f80 : vmax[k]) >= M - 1) ? (1u << k) : 0u;
  }
  int best = 0x7fffffff;
  if (__ballot(q != 0u) != 0ull) {
#pragma unroll
    for (int k = 0; k < kTopkVecPerThread; ++k) {
      if ((q >> k) & 1u) {
        const int v = v0 + tid + k * kTopkThreads;
        const int lim = v < nfull ? 8 : V - 8 * v;     // logits of the vector that exist
        int e_hit = 8;
#pragma unroll
        for (int e = 7; e >= 0; --e) {
          const int hit = (int)(e < lim) & (int)(bf16_key(elem_bits(d[k], e)) == mkey);   // no short circuit
          e_hit = hit ? e : e_hit;
        }
        if (e_hit < 8) best = min(best, 8 * v + e_hit);
      }
    }
  }
  best = -wave_max_i32(-best);
  __syncthreads();                                 // every wave has read s_red
  if (lane == 0) s_red[wave] = best;
  __syncthreads();
  best = s_red[0];
#pragma unroll
  for (int w = 1; w < kTopkWaves; ++w) best = min(best, s_red[w]);
  const size_t ci = (size_t)r * nchunks + c;
  if (best != 0x7fffffff) {
    if (tid == 0) chunk_arg[ci] = make_rc(mkey, (unsigned)best, mbits);
    return;
  }
  // exact composite maximum (only when the block maximum was +NaN): a rolled loop that
  // re-reads the chunk, to keep the common path's code small
  unsigned long long comp = 0ull;
#pragma unroll 1
  for (int k = 0; k < kTopkVecPerThread; ++k) {
    const int v = v0 + tid + k * kTopkThreads;
    if (v >= v1) break;
#pragma unroll 1
    for (int e = 0; e < 8; ++e) {
      const int id = 8 * v + e;
      if (id < V) {
        const uint32_t bits = rowp[id];
        const unsigned long long x = make_rc(bf16_key(bits), (unsigned)id, bits);
        comp = x > comp ? x : comp;
      }
    }
  }
  comp = wave_max_u64(comp);
  if (lane == 0) s_redu[wave] = comp;
  __syncthreads();
  if (tid == 0) {
    unsigned long long m = s_redu[0];
    for (int w = 1; w < kTopkWaves; ++w) m = s_redu[w] > m ? s_redu[w] : m;
    chunk_arg[ci] = m;
  }
}

// ---- greedy pass 2: one wave per request ----------------------------------------------
// Lane t takes the argmax of row t (and lane 0 that of row 64 when K = 64): the maximum
// of its chunks' composites.  The first position whose draft differs from the argmax
// ends the prefix; the row argmax there is the committed token.
__global__ void __launch_bounds__(kWave) k_greedy_decide(const int32_t* __restrict__ tokens,
                                                         const int32_t* __restrict__ cand_idx, int64_t batch_stride,
                                                         int K, int V, int nchunks,
                                                         const unsigned long long* __restrict__ chunk_arg,
                                                         int32_t* __restrict__ out_tokens,
                                                         int32_t* __restrict__ n_accepted,
                                                         int32_t* __restrict__ row_status) {
  const int lane = threadIdx.x;
  const int b = blockIdx.x;
  const int rbase = batch_stride == 0 ? 0 : b * (K + 1);
  int32_t* out_b = out_tokens + (size_t)b * (K + 1);
  int g[2] = {0, 0};
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int row = lane + i * kWave;
    if (row <= K) {
      const unsigned long long* a = chunk_arg + (size_t)(rbase + row) * nchunks;
      unsigned long long mx = 0ull;
#pragma unroll
      for (int j = 0; j < kMaxChunks; ++j) {
        const unsigned long long x = j < nchunks ? a[j] : 0ull;
        mx = x > mx ? x : mx;
      }
      g[i] = rc_id(mx);
    }
  }
  bool bad = false;
  int x = 0;
  if (lane < K) {
    x = tokens[(size_t)b * K + lane];
    bad = x < 0 || x >= V;
    const int32_t* cb = cand_idx + ((size_t)b * K + lane) * kNC;
#pragma unroll
    for (int j = 0; j < kNC; ++j) {
      const int id = cb[j];
      bad |= id < 0 || id >= V;
    }
  }
  const bool ids_bad = __ballot(bad) != 0ull;
  const unsigned long long miss = __ballot(lane < K && x != g[0]);
  const int tstar = miss != 0ull ? __builtin_ctzll(miss) : K;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int row = lane + i * kWave;
    if (row <= K) out_b[row] = row <= tstar ? g[i] : -1;
  }
  if (lane == 0) {
    n_accepted[b] = tstar;
    if (row_status) row_status[b] = ids_bad ? 2 : 0;
  }
}

// ---- sampled pass 2 -------------------------------------------------------------------
constexpr int kAccThreads = 512;
constexpr int kAccWaves = kAccThreads / kWave;
constexpr int kFineVec = (kSubVec + kAccThreads - 1) / kAccThreads;   // 16-byte vectors per thread of a rescan
constexpr int kFineLen = 8 * kFineVec;                                // logits per thread
constexpr int kMaxStatRows = DFLASH2_MAX_K + 1;
constexpr int kNCP = kNC + 1;            // LDS pitch of a position's candidates (odd: lanes
constexpr int kSubP = kMaxSub + 1;       // reading one position or row each hit distinct banks)

struct DecideShared {
  // the request's inputs, loaded once at entry
  int tok[DFLASH2_MAX_K];
  int cand[DFLASH2_MAX_K * kNCP];
  float q[DFLASH2_MAX_K * kNCP];
  uint32_t xbits[DFLASH2_MAX_K];          // target logit (bits) of each drafted token
  uint32_t cbits[DFLASH2_MAX_K * kNCP];   // target logit (bits) of each candidate
  float smax[kMaxStatRows * kSubP];       // sub-chunk j of row r at r * (nsub + 1) + j
  float ssum[kMaxStatRows * kSubP];
  // the draw, as the deciding wave leaves it
  int done;                               // the request is finished (a non-finite row)
  int trow;                               // the row drawn from
  int e0, e1;                             // the logits [e0, e1) to rescan
  float rem;                              // the draw's target minus the mass before e0
  float m, invZ;                          // the drawn row's max and 1 / sum of weights
  int residual;                           // draw from max(0, p - q) (else from p)
  int cl_id[kNC];                         // the drawn position's candidates: an id at its
  float cl_qf[kNC];                       // first slot (else -1) and its total draft mass
  float wtot[kAccWaves];                  // rescan: the weight of each wave's logits
  int pick;
};

// Merged statistics of one row from its sub-chunks, in sub-chunk order: the max, and the
// sum of weights relative to it (NaN when a sub-chunk is non-finite or no logit is
// finite).  nsub is a multiple of 8; the loads of 8 sub-chunks go out together.
__device__ __forceinline__ void merge_row(const float* mx, const float* sx, int nsub, float c2, float& m_out,
                                          float& z_out) {
  float mm = -__builtin_inff();
  bool bad = false;
#pragma unroll 1
  for (int j0 = 0; j0 < nsub; j0 += kSubPerChunk) {
#pragma unroll
    for (int u = 0; u < kSubPerChunk; ++u) {
      const float v = mx[j0 + u];
      bad |= v != v;
      mm = fmaxf(mm, v);                  // a NaN is skipped (and flagged)
    }
  }
  float Z = 0.f;
#pragma unroll 1
  for (int j0 = 0; j0 < nsub; j0 += kSubPerChunk) {
#pragma unroll
    for (int u = 0; u < kSubPerChunk; ++u) Z += sx[j0 + u] * tweight(mx[j0 + u], mm, c2);   // -inf max: 0 * 0
  }
  m_out = mm;
  z_out = (bad || mm == -__builtin_inff()) ? __builtin_nanf("") : Z;
}

struct CoarsePick {
  int sub;      // -1: no mass
  float rem;
};

// The deciding wave's step over the sub-chunks of row `trow` (lane s owns sub-chunk s,
// whose logits are [e0, e1)): each sub-chunk's mass, less the draft's mass min(p, q) at
// the candidates it holds when `residual` (cid / csub: lane j < 16 holds slot j, an id at
// its first slot else -1), then the sub-chunk whose running sum first exceeds u times the
// total.
__device__ __forceinline__ CoarsePick coarse_pick(const DecideShared& sm, int trow, int nsub, int e0, int e1,
                                                  float m, float invZ, float c2, float u, bool residual, int cid,
                                                  float csub) {
  const int lane = threadIdx.x & (kWave - 1);
  float P = 0.f;
  if (lane < nsub) {
    const float mc = sm.smax[trow * (nsub + 1) + lane];
    P = mc == -__builtin_inff() ? 0.f : sm.ssum[trow * (nsub + 1) + lane] * tweight(mc, m, c2) * invZ;
  }
  if (residual) {
#pragma unroll
    for (int i = 0; i < kNC; ++i) {
      const int id = __builtin_amdgcn_readlane(cid, i);
      const float x = readlane_f(csub, i);
      P -= (id >= e0 && id < e1) ? x : 0.f;
    }
  }
  const float R = lane < nsub ? fmaxf(P, 0.f) : 0.f;
  const float incl = wave_incl_scan(R);
  const float excl = wave_excl_from_incl(incl);
  const float target = u * readlane_f(incl, kWave - 1);
  CoarsePick cp;
  cp.sub = wave_pick_lane(R, incl, target);
  cp.rem = target - readlane_f(excl, cp.sub < 0 ? 0 : cp.sub);
  return cp;
}

// The draw inside logits [sm.e0, sm.e1) of row rowp, by the whole work-group: thread i
// owns a contiguous run of L <= kFineLen logits; every load goes out at once (a vector not
// wholly inside the range reads the row's first vector and is replaced) and the weights
// stay in registers.  Returns the token id (the same in every thread), -1 if no weight is
// positive.
__device__ __forceinline__ int fine_pick(const uint16_t* __restrict__ rowp, float c2, DecideShared& sm) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
  const int e0 = sm.e0, e1 = sm.e1;
  const float m = sm.m, invZ = sm.invZ, rem = sm.rem;
  const bool residual = sm.residual != 0;
  const int L = (((e1 - e0) + kAccThreads * 8 - 1) / (kAccThreads * 8)) * 8;
  const int a0 = e0 + tid * L;
  u32x4 raw[kFineVec];
#pragma unroll
  for (int k = 0; k < kFineVec; ++k) {
    const int base = a0 + 8 * k;
    const bool full = 8 * k < L && base + 8 <= e1;
    raw[k] = *reinterpret_cast<const u32x4*>(rowp + (full ? base : 0));
    if (!full) raw[k] = (u32x4){0u, 0u, 0u, 0u};
  }
#pragma unroll
  for (int k = 0; k < kFineVec; ++k) {
    const int base = a0 + 8 * k;
    if (8 * k < L && base < e1 && base + 8 > e1) {     // the row's ragged last vector
      uint32_t w4[4] = {0u, 0u, 0u, 0u};
      for (int e = 0; e < 8 && base + e < e1; ++e) w4[e >> 1] |= (uint32_t)rowp[base + e] << ((e & 1) * 16);
      raw[k] = (u32x4){w4[0], w4[1], w4[2], w4[3]};
    }
  }
  // which of this thread's logits are candidates (bit = offset from a0)
  unsigned cmask = 0u;
  if (residual) {
#pragma unroll
    for (int i = 0; i < kNC; ++i) {
      const int off = sm.cl_id[i] - a0;               // an unused slot holds -1: off < 0
      if (off >= 0 && off < L) cmask |= 1u << off;
    }
  }
  // weights p of every logit, branch-free; then, only in the threads that need it, zero
  // the logits outside the range and replace candidates' weights by max(0, p - q)
  float w[kFineLen];
#pragma unroll
  for (int k = 0; k < kFineVec; ++k)
#pragma unroll
    for (int e = 0; e < 8; ++e) w[8 * k + e] = tweight(bf16_to_f32(elem_bits(raw[k], e)), m, c2) * invZ;
  if (!(L == kFineLen && a0 + kFineLen <= e1)) {
#pragma unroll
    for (int off = 0; off < kFineLen; ++off)
      if (!(off < L && a0 + off < e1)) w[off] = 0.f;
  }
  if (cmask != 0u) {
#pragma unroll
    for (int off = 0; off < kFineLen; ++off)
      if ((cmask >> off) & 1u) {
        float qf = 0.f;
        for (int i = 0; i < kNC; ++i) qf = sm.cl_id[i] == a0 + off ? sm.cl_qf[i] : qf;
        w[off] = fmaxf(w[off] - qf, 0.f);
      }
  }
  float tsum = 0.f;
#pragma unroll
  for (int off = 0; off < kFineLen; ++off) tsum += w[off];
  const float incl = wave_incl_scan(tsum);
  const float excl = wave_excl_from_incl(incl);
  if (lane == kWave - 1) sm.wtot[wave] = incl;
  __syncthreads();
  // the wave whose logits hold the crossing (the same in every thread)
  float off = 0.f, offw = 0.f, offlast = 0.f;
  int W = -1, wlast = -1;
#pragma unroll
  for (int i = 0; i < kAccWaves; ++i) {
    const float t = sm.wtot[i];
    if (W < 0 && t > 0.f && rem < off + t) {
      W = i;
      offw = off;
    }
    if (t > 0.f) {
      wlast = i;
      offlast = off;
    }
    off += t;
  }
  const bool take_last = W < 0;               // rounding left the target past the total
  if (take_last) {
    W = wlast;
    offw = offlast;
  }
  if (W < 0) return -1;                       // no positive weight (uniform)
  if (wave == W) {
    const float local = rem - offw;
    const int l = wave_pick_lane(tsum, incl, take_last ? __builtin_inff() : local);
    if (lane == l) {
      // the same weights, in the same order, now with the running sum
      float run = excl;
      int pick = -1, lastp = -1;
#pragma unroll
      for (int o = 0; o < kFineLen; ++o) {
        run += w[o];
        if (pick < 0 && !take_last && local < run) pick = a0 + o;
        if (w[o] > 0.f) lastp = a0 + o;
      }
      sm.pick = pick >= 0 ? pick : lastp;     // the lane holds a positive weight
    }
  }
  __syncthreads();
  return sm.pick;
}

__global__ void __launch_bounds__(kAccThreads) k_accept_decide(const uint16_t* __restrict__ target, int64_t ld,
                                                               int64_t batch_stride, const int32_t* __restrict__ tokens,
                                                               const int32_t* __restrict__ cand_idx,
                                                               const float* __restrict__ q, int K, int V, int nchunks,
                                                               float inv_t, uint64_t seed, int32_t* __restrict__ out_tokens,
                                                               int32_t* __restrict__ n_accepted,
                                                               int32_t* __restrict__ row_status, AcceptWs ws) {
  __shared__ DecideShared sm;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
  const int b = blockIdx.x;
  const int32_t* tok_b = tokens + (size_t)b * K;
  const int32_t* cand_b = cand_idx + (size_t)b * K * kNC;
  const uint16_t* tb = target + (size_t)b * batch_stride;
  const int rbase = batch_stride == 0 ? 0 : b * (K + 1);
  int32_t* out_b = out_tokens + (size_t)b * (K + 1);
  const float c2 = inv_t * kLog2e;
  const int nsub = nchunks * kSubPerChunk;
  const int pitch = nsub + 1;

  // ---- everything the decision reads, in two dependent memory round trips ------------
  for (int e = tid; e < K * kNC; e += kAccThreads) {
    const int t = e >> 4, j = e & (kNC - 1);
    const int id = cand_b[e];
    sm.cand[t * kNCP + j] = id;
    sm.q[t * kNCP + j] = q[(size_t)b * K * kNC + e];
    const int idc = id < 0 ? 0 : (id >= V ? V - 1 : id);          // read in bounds; flagged below
    sm.cbits[t * kNCP + j] = tb[(size_t)t * ld + idc];
  }
  for (int e = tid; e < K; e += kAccThreads) {
    const int x = tok_b[e];
    sm.tok[e] = x;
    sm.xbits[e] = tb[(size_t)e * ld + (x < 0 ? 0 : (x >= V ? V - 1 : x))];
  }
  const int nst = (K + 1) * nsub;
  const size_t s0 = (size_t)rbase * nsub;
  for (int e = tid; e < nst; e += kAccThreads) {
    const int row = (int)((unsigned)e / (unsigned)nsub);
    const int at = e + row;                                     // row * pitch + (e - row * nsub)
    sm.smax[at] = ws.chunk_max[s0 + e];
    sm.ssum[at] = ws.chunk_sum[s0 + e];
  }
  __syncthreads();

  // ---- the decision, in wave 0 alone: lane t owns position t and row t (lane 0 also
  // row 64 when K = 64); flags and the first reject come from ballots
  int tstar = 0, trow = 0, status = 0;
  bool fault = false;
  float m = 0.f, invZ = 0.f, u_res = 0.f;
  int se0 = 0, se1 = 0;
  if (wave == 0) {
    // the logits of sub-chunk `lane`
    se0 = 8 * sub_begin(V, nchunks, lane);
    se1 = min(8 * sub_begin(V, nchunks, lane + 1), V);
    float mr0 = 0.f, zr0 = 1.f, mr1 = 0.f, zr1 = 1.f;
    bool nonfinite = false;
#pragma unroll 1
    for (int i = 0; i < (K >= kWave ? 2 : 1); ++i) {
      const int row = lane + i * kWave;
      if (row <= K) {
        float mm, zz;
        merge_row(sm.smax + row * pitch, sm.ssum + row * pitch, nsub, c2, mm, zz);
        nonfinite |= !__builtin_isfinite(zz);
        if (i == 0) {
          mr0 = mm;
          zr0 = zz;
        } else {
          mr1 = mm;
          zr1 = zz;
        }
      }
    }
    // ids in range, and a valid draft distribution at every position
    bool bad = false, qok = true;
    float qx = 0.f;
    if (lane < K) {
      const int x = sm.tok[lane];
      bad = x < 0 || x >= V;
      float sq = 0.f;
#pragma unroll
      for (int j = 0; j < kNC; ++j) {
        const int id = sm.cand[lane * kNCP + j];
        const float v = sm.q[lane * kNCP + j];
        bad |= id < 0 || id >= V;
        qok &= __builtin_isfinite(v) && v >= 0.f;
        sq += v;
        qx += id == x ? v : 0.f;
      }
      qok &= fabsf(sq - 1.f) <= 1e-3f;
    }
    const bool ids_bad = __ballot(bad) != 0ull;
    const bool q_bad = __ballot(lane < K && !(qok && (ids_bad || qx > 0.f))) != 0ull;
    status = (ids_bad ? 2 : 0) | (q_bad ? 4 : 0);
    fault = ids_bad || q_bad;
    if (__ballot(nonfinite) != 0ull) {
      // a non-finite target row: commit nothing
      if (lane <= K) out_b[lane] = -1;
      if (lane == 0) {
        if (K >= kWave) out_b[kWave] = -1;
        n_accepted[b] = 0;
        if (row_status) row_status[b] = 1;
        sm.done = 1;
      }
    } else {
      // accept tests at every position (the first reject decides); skipped when the ids
      // or the draft distributions are invalid, which commits one token from p_0
      const uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
      bool rej = false;
      if (!fault && lane < K) {
        const float px = tweight(bf16_to_f32(sm.xbits[lane]), mr0, c2) / zr0;
        const float u_acc = word_to_uniform(philox4x32_10((uint32_t)lane, (uint32_t)b, 1u, 0u, k0, k1).x0);
        rej = !(u_acc * qx < px);
      }
      const unsigned long long rejm = __ballot(rej);
      tstar = fault ? 0 : (rejm != 0ull ? __builtin_ctzll(rejm) : K);
      if (lane <= K && lane != tstar) out_b[lane] = lane < tstar ? sm.tok[lane] : -1;
      if (lane == 0 && K >= kWave && tstar != kWave) out_b[kWave] = -1;      // row 64 lies past tstar
      u_res = word_to_uniform(philox4x32_10((uint32_t)tstar, (uint32_t)b, 1u, 0u, k0, k1).x1);
      // the residual max(0, p - q) at a reject (p instead when it has no mass), else p of
      // the bonus row (or of row 0 after a fault)
      trow = fault ? 0 : tstar;
      bool residual = !fault && tstar < K;
      const bool hi = trow >= kWave;
      const int src = trow & (kWave - 1);
      m = readlane_f(hi ? mr1 : mr0, src);
      invZ = 1.f / readlane_f(hi ? zr1 : zr0, src);
      // the drawn position's distinct candidates, their total draft mass (slot order)
      int cid = -1;
      float cqf = 0.f, csub = 0.f;
      if (residual) {
        const int j = lane & (kNC - 1);
        const int id = sm.cand[trow * kNCP + j];
        const float qv = sm.q[trow * kNCP + j];
        const float pv = tweight(bf16_to_f32(sm.cbits[trow * kNCP + j]), m, c2) * invZ;
        bool first = true;
#pragma unroll
        for (int i = 0; i < kNC; ++i) {
          const int oi = __builtin_amdgcn_readlane(id, i);
          const float qi = readlane_f(qv, i);
          if (oi == id) {
            cqf += qi;
            if (i < j) first = false;
          }
        }
        cid = first ? id : -1;
        csub = first ? fminf(pv, cqf) : 0.f;
      }
      CoarsePick cp = coarse_pick(sm, trow, nsub, se0, se1, m, invZ, c2, u_res, residual, cid, csub);
      if (cp.sub < 0 && residual) {           // the residual has no mass: draw from p
        status |= 8;
        residual = false;
        cp = coarse_pick(sm, trow, nsub, se0, se1, m, invZ, c2, u_res, false, -1, 0.f);
      }
      if (lane < kNC) {
        sm.cl_id[lane] = cid;
        sm.cl_qf[lane] = cqf;
      }
      // (no mass at all cannot happen for p of a finite row; an empty range then draws -1)
      const int ce0 = cp.sub < 0 ? 0 : __builtin_amdgcn_readlane(se0, cp.sub);
      const int ce1 = cp.sub < 0 ? 0 : __builtin_amdgcn_readlane(se1, cp.sub);
      if (lane == 0) {
        sm.done = 0;
        sm.trow = trow;
        sm.e0 = ce0;
        sm.e1 = ce1;
        sm.rem = cp.rem;
        sm.m = m;
        sm.invZ = invZ;
        sm.residual = residual ? 1 : 0;
      }
    }
  }
  __syncthreads();
  if (sm.done) return;

  // ---- the rescan of one sub-chunk by the whole work-group --------------------------
  const uint16_t* rowp = tb + (size_t)sm.trow * ld;
  bool res = sm.residual != 0;
  int v;
  for (;;) {
    v = fine_pick(rowp, c2, sm);
    if (v >= 0 || !res) break;
    // the residual had mass in the sub-chunk sums but none in the rescan: draw from p
    res = false;
    if (wave == 0) {
      status |= 8;
      const CoarsePick cp = coarse_pick(sm, trow, nsub, se0, se1, m, invZ, c2, u_res, false, -1, 0.f);
      const int ce0 = cp.sub < 0 ? 0 : __builtin_amdgcn_readlane(se0, cp.sub);
      const int ce1 = cp.sub < 0 ? 0 : __builtin_amdgcn_readlane(se1, cp.sub);
      if (lane == 0) {
        sm.e0 = ce0;
        sm.e1 = ce1;
        sm.rem = cp.rem;
        sm.residual = 0;
      }
    }
    __syncthreads();
  }
  if (tid == 0) {
    out_b[tstar] = v;
    n_accepted[b] = fault ? 0 : tstar;
    if (row_status) row_status[b] = status;
  }
}

hipError_t launch_spec_accept(const uint16_t* target, int64_t ld, int64_t batch_stride, const int32_t* tokens,
                              const int32_t* cand_idx, const float* q, int batch, int K, int vocab, float temperature,
                              uint64_t seed, int32_t* out_tokens, int32_t* n_accepted, int32_t* row_status, AcceptWs ws,
                              hipStream_t s) {
  const float inv_t = temperature == 0.f ? 0.f : 1.f / temperature;
  const int nchunks = topk_num_chunks(vocab);
  const int nrows = batch_stride == 0 ? K + 1 : batch * (K + 1);
  const dim3 grid((unsigned)(batch_stride == 0 ? (long long)(K + 1) * nchunks : xcd_chunk_grid(batch, K + 1, nchunks)));
  if (inv_t == 0.f) {
    hipLaunchKernelGGL(k_greedy_argmax, dim3((unsigned)(nrows * nchunks)), dim3(kTopkThreads), 0, s, target, ld,
                       batch_stride, K, vocab, nchunks, ws.chunk_arg);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_greedy_decide, dim3((unsigned)batch), dim3(kWave), 0, s, tokens, cand_idx, batch_stride, K,
                       vocab, nchunks, ws.chunk_arg, out_tokens, n_accepted, row_status);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(k_accept_stats, grid, dim3(kTopkThreads), 0, s, target, ld, batch_stride, K, vocab, nchunks, inv_t,
                     ws, batch);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_accept_decide, dim3((unsigned)batch), dim3(kAccThreads), 0, s, target, ld, batch_stride, tokens,
                     cand_idx, q, K, vocab, nchunks, inv_t, seed, out_tokens, n_accepted, row_status, ws);
  return hipGetLastError();
}

}  // namespace df2
