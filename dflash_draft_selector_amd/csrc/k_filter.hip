// Filtered-target verify (FreeToken PR "Adds DFlash 2": "Speed" and "All settings" sample
// with temperature 1.0, top_p 0.95 and top_k 20; "Details", sampled verify: accept with
// min(1, p/q), on a reject resample from max(0, p - q); "Known gaps": one sparse-q verify
// with top-k + top-p).
//
// p_t is the target distribution after the filters: the top_k largest logits of row t
// (value desc, id asc), softmax(l / T) over them, then the shortest prefix of that order
// whose mass reaches top_p, renormalised.  Only a row's top_k logits enter it, so:
// Pass 1 (k_filter_topk) streams every target row once in the top-16 stream shape; each
// wave owns one contiguous sub-chunk and writes that sub-chunk's top_k, best first, and
// whether it holds +inf or NaN.  The wave's bound is the top_k-th largest of its 64 lane
// maxima (at least top_k logits reach it); it gathers the logits at or above the bound
// and ranks them.  No LDS is shared between waves and there is no barrier.
// Pass 2 (k_filter_decide), one work-group per request: each wave merges one row's
// sub-chunk lists into the row's top_k (pruned by a bound from the lists' heads),
// forms the filtered p over them; wave 0 runs the accept tests and the draw over at most
// top_k tokens, in token-id order.
#include "dflash2.h"
#include "dflash2_internal.h"
#include "filter.h"
#include "topk_dev.h"
#include "verify_dev.h"

namespace df2 {

constexpr int kFiltCap = 128;                  // logits a wave gathers before its exact path
constexpr int kFiltVecCap = 64;                // candidate vectors a wave stages
constexpr int kFiltThreads = 512;              // pass 2
constexpr int kFiltWaves = kFiltThreads / kWave;
constexpr int kFiltRowCap = 256;               // pruned list entries a deciding wave keeps
constexpr int kFiltMaxEnt = kMaxSub * DFLASH2_MAX_TOPK / kWave;   // list entries per lane of a row
constexpr int kFiltRows = DFLASH2_MAX_K + 1;
constexpr int kFiltNCP = kNC + 1;              // LDS pitches: odd, so lanes reading one row
constexpr int kFiltKP = DFLASH2_MAX_TOPK + 1;  // each hit distinct banks
static_assert(DFLASH2_MAX_TOPK <= kWave && DFLASH2_MAX_TOPK <= kFiltCap, "top_k fits a wave");

FilterWs carve_filter(Carver& c, int64_t nrows, int64_t vocab) {
  FilterWs w;
  const size_t n = (size_t)nrows * topk_num_chunks(vocab) * kSubPerChunk;
  w.lists = c.take<unsigned long long>(n * DFLASH2_MAX_TOPK);
  w.flags = c.take<int>(n);
  return w;
}

// ---- a full bitonic sort of the wave's 64 lane values, largest first ----------------
// Batcher's network: blocks of SIZE lanes run descending where lane bit SIZE is clear
// (every block at SIZE = 64), partners at distance J (DPP inside a row, ds_bpermute
// across rows).
template <int SIZE, int J>
__device__ __forceinline__ int wave_bitonic_step(int x) {
  const int lane = threadIdx.x & (kWave - 1);
  const bool desc = SIZE >= kWave || (lane & SIZE) == 0;
  int p;
  if constexpr (J >= 16)
    p = xor_lane_i32(x, J);
  else
    p = row_partner_i32<J>(x);
  return cmpx_i32(x, p, ((lane & J) == 0) == desc);
}

__device__ __forceinline__ int wave_sort64_desc(int x) {
  x = wave_bitonic_step<2, 1>(x);
  x = wave_bitonic_step<4, 2>(x);
  x = wave_bitonic_step<4, 1>(x);
  x = wave_bitonic_step<8, 4>(x);
  x = wave_bitonic_step<8, 2>(x);
  x = wave_bitonic_step<8, 1>(x);
  x = wave_bitonic_step<16, 8>(x);
  x = wave_bitonic_step<16, 4>(x);
  x = wave_bitonic_step<16, 2>(x);
  x = wave_bitonic_step<16, 1>(x);
  x = wave_bitonic_step<32, 16>(x);
  x = wave_bitonic_step<32, 8>(x);
  x = wave_bitonic_step<32, 4>(x);
  x = wave_bitonic_step<32, 2>(x);
  x = wave_bitonic_step<32, 1>(x);
  x = wave_bitonic_step<64, 32>(x);
  x = wave_bitonic_step<64, 16>(x);
  x = wave_bitonic_step<64, 8>(x);
  x = wave_bitonic_step<64, 4>(x);
  x = wave_bitonic_step<64, 2>(x);
  return wave_bitonic_step<64, 1>(x);
}

// Appends the logits of vector v marked in m8 (this lane's) to the wave's list cw, in
// lane order then element order; stores those below `limit`.  Returns the new count
// (the same in every lane).  The whole wave calls it.
__device__ __forceinline__ int gather_vector(unsigned long long* cw, int n, unsigned m8, const u32x4& x, int v,
                                             int limit) {
  const int cnt = __popc(m8);
  const int incl = wave_incl_scan_i32(cnt);
  int at = n + incl - cnt;
#pragma unroll
  for (int e = 0; e < 8; ++e)
    if ((m8 >> e) & 1u) {
      if (at < limit) {
        const uint32_t bits = elem_bits(x, e);
        cw[at] = make_rc(bf16_key(bits), (uint32_t)(8 * v + e), bits);
      }
      ++at;
    }
  return n + __builtin_amdgcn_readlane(incl, kWave - 1);
}

// Rare sub-chunks with more than kFiltCap logits at or above the bound (ties at it): the
// bound rises to the top_k-th best of the kFiltCap logits kept, which at least top_k
// logits still reach, and the sub-chunk is gathered again from memory; each round leaves
// out the kFiltCap - top_k kept logits below the new bound.  With `regather` (more
// candidate vectors than were staged) the first round gathers at `thr` itself.  Rolled
// and out of line, to keep the common path small.  Returns the count gathered
// (<= kFiltCap).
__device__ __noinline__ int gather_raised(const uint16_t* __restrict__ rowp, int V, int s0, int s1, int top_k,
                                          unsigned long long thr, bool regather, unsigned long long* cw,
                                          unsigned long long* thr_slot) {
  const int lane = threadIdx.x & (kWave - 1);
  const int nfull = V >> 3;
  int n;
#pragma unroll 1
  for (;;) {
    if (!regather) {
      wave_lds_sync();
      for (int i = lane; i < kFiltCap; i += kWave) {
        const unsigned long long x = cw[i];
        int rank = 0;
        for (int j = 0; j < kFiltCap; ++j) rank += cw[j] > x ? 1 : 0;
        if (rank == top_k - 1) *thr_slot = x;
      }
      wave_lds_sync();
      thr = *thr_slot;
      wave_lds_sync();
    }
    regather = false;
    n = 0;
#pragma unroll 1
    for (int k = 0; k < kTopkVecPerThread; ++k) {
      const int v = s0 + lane + k * kWave;
      uint32_t w4[4] = {0u, 0u, 0u, 0u};
      unsigned m8 = 0u;
      if (v < s1) {
        const int lim = v < nfull ? 8 : V - 8 * v;
#pragma unroll 1
        for (int e = 0; e < lim; ++e) {
          const uint32_t bits = rowp[8 * v + e];
          w4[e >> 1] |= bits << ((e & 1) * 16);
          m8 |= (make_rc(bf16_key(bits), (uint32_t)(8 * v + e), bits) >= thr ? 1u : 0u) << e;
        }
      }
      n = gather_vector(cw, n, m8, (u32x4){w4[0], w4[1], w4[2], w4[3]}, v, kFiltCap);
    }
    if (n <= kFiltCap) return n;
  }
}

__global__ void __launch_bounds__(kTopkThreads) k_filter_topk(const uint16_t* __restrict__ target, int64_t ld,
                                                              int64_t batch_stride, int K, int V, int nchunks,
                                                              int top_k, unsigned long long* __restrict__ lists,
                                                              int* __restrict__ flags, int batch) {
  __shared__ unsigned long long s_cand[kTopkWaves][kFiltCap];
  __shared__ unsigned long long s_thr[kTopkWaves];
  __shared__ u32x4 s_vec[kTopkWaves][kFiltVecCap];
  __shared__ int s_vpos[kTopkWaves][kFiltVecCap];
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
  const int nsub = nchunks * kSubPerChunk;
  const int s = c * kSubPerChunk + wave;
  const int s0 = sub_begin(V, nchunks, s), s1 = sub_begin(V, nchunks, s + 1);
  const int safe = sub_begin(V, nchunks, c * kSubPerChunk);   // the chunk's first vector: whole
  const int nfull = V >> 3;

  // ---- the sub-chunk, every load in flight before any is used; missing logits -inf --
  u32x4 d[kTopkVecPerThread];
  unsigned whole = 0u;
#pragma unroll
  for (int k = 0; k < kTopkVecPerThread; ++k) {
    const int v = s0 + lane + k * kWave;
    const bool w = v < s1 && v < nfull;
    d[k] = __builtin_nontemporal_load(rowv + (w ? v : safe));
    whole |= (w ? 1u : 0u) << k;
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int k = 0; k < kTopkVecPerThread; ++k)
    if (!((whole >> k) & 1u)) d[k] = (u32x4){0xff80ff80u, 0xff80ff80u, 0xff80ff80u, 0xff80ff80u};
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
  }

  // ---- +inf / NaN (a raw half >= 0x7f80 as signed, or > 0xff80 as unsigned) -------
  s16x2 hs = (s16x2){-32768, -32768};
  u16x2 hu = (u16x2){0, 0};
#pragma unroll
  for (int k = 0; k < kTopkVecPerThread; ++k) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      hs = __builtin_elementwise_max(hs, __builtin_bit_cast(s16x2, (uint32_t)d[k][w]));
      hu = __builtin_elementwise_max(hu, __builtin_bit_cast(u16x2, (uint32_t)d[k][w]));
    }
  }
  const bool nonfinite = __ballot(max_halves(hs) >= 0x7f80 || (hu.x > hu.y ? hu.x : hu.y) > 0xff80) != 0ull;

  // ---- the bound: the top_k-th largest lane maximum (signed order) ------------------
  int vmax[kTopkVecPerThread];
  const int lmax = vector_maxima<true>(d, vmax);
  int tau = __builtin_amdgcn_readlane(wave_sort64_desc(lmax), top_k - 1);
  tau = tau > 0x7f80 ? 0x7f80 : tau;                           // never above +inf
  const int tkey = (int)bf16_key(order_to_bits(tau));

  // ---- gather every logit whose key reaches the bound (the sub-chunk's top_k all do):
  // first the vectors that can hold one (signed maximum >= tau - 1: -0 sits one below
  // +0 and shares its key) are staged in LDS, a few instructions per slot; then each
  // lane tests the elements of one staged vector
  unsigned long long* cw = s_cand[wave];
  int nv = 0;
#pragma unroll
  for (int k = 0; k < kTopkVecPerThread; ++k) {
    const int v = s0 + lane + k * kWave;
    const bool f = v < s1 && vmax[k] >= tau - 1;
    const unsigned long long bal = __ballot(f);
    if (bal != 0ull) {
      const int at = nv + (int)__builtin_amdgcn_mbcnt_hi((unsigned)(bal >> 32),
                                                         __builtin_amdgcn_mbcnt_lo((unsigned)bal, 0u));
      if (f && at < kFiltVecCap) {
        s_vec[wave][at] = d[k];
        s_vpos[wave][at] = v;
      }
      nv += __popcll(bal);
    }
  }
  int n;
  if (nv <= kFiltVecCap) {
    wave_lds_sync();
    n = 0;
    for (int i0 = 0; i0 < nv; i0 += kWave) {          // uniform trip count
      const int i = i0 + lane;
      unsigned m8 = 0u;
      u32x4 x = (u32x4){0u, 0u, 0u, 0u};
      int v = 0;
      if (i < nv) {
        x = s_vec[wave][i];
        v = s_vpos[wave][i];
        const int lim = v < nfull ? 8 : V - 8 * v;
#pragma unroll
        for (int e = 0; e < 8; ++e) m8 |= (unsigned)((e < lim) & ((int)bf16_key(elem_bits(x, e)) >= tkey)) << e;
      }
      n = gather_vector(cw, n, m8, x, v, kFiltCap);
    }
  } else {
    n = kFiltCap + 1;                                 // more vectors than staged: gather from memory
    s_thr[wave] = 0ull;
  }
  if (n > kFiltCap) n = gather_raised(rowp, V, s0, s1, top_k, (unsigned long long)tkey << 48, nv > kFiltVecCap, cw,
                                      &s_thr[wave]);
  wave_lds_sync();

  // ---- rank the gathered logits (distinct composites); the best top_k, best first ---
  unsigned long long* out = lists + ((size_t)r * nsub + s) * top_k;
  for (int i = lane; i < n; i += kWave) {
    const unsigned long long x = cw[i];
    int rank = 0;
    for (int j = 0; j < n; ++j) rank += cw[j] > x ? 1 : 0;
    if (rank < top_k) out[rank] = x;
  }
  for (int i = n + lane; i < top_k; i += kWave) out[i] = 0ull;
  if (lane == 0) flags[(size_t)r * nsub + s] = nonfinite ? 1 : 0;
}

// ---- pass 2 -------------------------------------------------------------------------
struct FilterShared {
  int tok[DFLASH2_MAX_K];
  int cand[DFLASH2_MAX_K * kFiltNCP];
  float q[DFLASH2_MAX_K * kFiltNCP];
  int nkeep[kFiltRows];                          // kept tokens of each row (a prefix of its top_k)
  int keep_id[kFiltRows * kFiltKP];              // their ids and filtered p, best first
  float keep_p[kFiltRows * kFiltKP];
  unsigned long long pool[kFiltWaves][kFiltRowCap];
  unsigned long long top[kFiltWaves][DFLASH2_MAX_TOPK];
  unsigned long long thr[kFiltWaves];
  int draw_id[DFLASH2_MAX_TOPK];
  float draw_w[DFLASH2_MAX_TOPK];
  int nonfinite_w[kFiltWaves];                   // each wave: one of its rows holds +inf or NaN
};

// Row `row` of the request: merge its sub-chunk lists into the row's top_k (by one wave),
// then the filtered p over them into sm.keep_*.  Returns whether the row holds +inf/NaN.
__device__ __forceinline__ bool filter_row(const unsigned long long* __restrict__ L, const int* __restrict__ F,
                                           int nsub, int top_k, float top_p, float c2, int row, FilterShared& sm) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
  const int nent = nsub * top_k;
  wave_lds_sync();                               // the previous row's reads of pool / top are done
  // the sub-chunk flags, the list heads and every list entry (at most kFiltMaxEnt per
  // lane), all in flight at once
  const int per = kWave / nsub;
  const int ls = lane / per, lj = lane - ls * per;
  const bool head = ls < nsub && lj < top_k;
  const int fl = F[lane < nsub ? lane : 0];
  const unsigned long long hx = L[head ? ls * top_k + lj : 0];
  unsigned long long e[kFiltMaxEnt];
#pragma unroll
  for (int j = 0; j < kFiltMaxEnt; ++j) {
    const int i = lane + j * kWave;
    e[j] = L[i < nent ? i : 0];
  }
  __builtin_amdgcn_sched_barrier(0);                 // every load issued before any is used
#pragma unroll
  for (int j = 0; j < kFiltMaxEnt; ++j)
    if (lane + j * kWave >= nent) e[j] = 0ull;
  const bool nonfinite = __ballot(lane < nsub && fl != 0) != 0ull;
  // the bound: the top_k-th largest key among the best 64 / nsub entries of every
  // list (at least top_k of the row's logits reach it, so its top_k all do; the
  // row's best logits sit near the heads of the lists, so few others do)
  const int hk = head ? (int)(hx >> 48) : 0;
  unsigned long long lb = (unsigned long long)__builtin_amdgcn_readlane(wave_sort64_desc(hk), top_k - 1) << 48;
  unsigned long long* pool = sm.pool[wave];
  unsigned long long* top = sm.top[wave];
  for (;;) {
    int np = 0;
#pragma unroll
    for (int j = 0; j < kFiltMaxEnt; ++j) {
      const bool keep = e[j] != 0ull && e[j] >= lb;
      const unsigned long long bal = __ballot(keep);
      if (bal == 0ull) continue;
      const int at = np + (int)__builtin_amdgcn_mbcnt_hi((unsigned)(bal >> 32),
                                                         __builtin_amdgcn_mbcnt_lo((unsigned)bal, 0u));
      if (keep && at < kFiltRowCap) pool[at] = e[j];
      np += __popcll(bal);
    }
    wave_lds_sync();
    if (np <= kWave) {
      // the usual case: one pooled entry per lane, ranked against the others through
      // readlane (no LDS round trip per comparison)
      const unsigned long long x = lane < np ? pool[lane] : 0ull;
      const uint32_t xl = (uint32_t)x, xh = (uint32_t)(x >> 32);
      int rank = 0;
      for (int j = 0; j < np; ++j) {
        const uint32_t yl = __builtin_amdgcn_readlane(xl, j), yh = __builtin_amdgcn_readlane(xh, j);
        rank += (yh > xh || (yh == xh && yl > xl)) ? 1 : 0;
      }
      if (lane < np && rank < top_k) top[rank] = x;
      for (int i = np + lane; i < top_k; i += kWave) top[i] = 0ull;
      break;
    }
    const int ns = np < kFiltRowCap ? np : kFiltRowCap;
    for (int i = lane; i < ns; i += kWave) {
      const unsigned long long x = pool[i];
      int rank = 0;
      for (int j = 0; j < ns; ++j) rank += pool[j] > x ? 1 : 0;
      if (np <= kFiltRowCap) {
        if (rank < top_k) top[rank] = x;
      } else if (rank == top_k - 1) {
        sm.thr[wave] = x;
      }
    }
    if (np <= kFiltRowCap) {
      for (int i = np + lane; i < top_k; i += kWave) top[i] = 0ull;
      break;
    }
    // more entries reach the bound than the pool holds (adversarial rows): raise it to
    // the top_k-th best of the entries kept, which at least top_k entries still reach
    wave_lds_sync();
    lb = sm.thr[wave];
    wave_lds_sync();
  }
  wave_lds_sync();
  // the filtered p over the top_k (lane i holds the i-th best)
  const unsigned long long x = lane < top_k ? top[lane] : 0ull;
  const bool valid = x != 0ull;
  const float l = bf16_to_f32(rc_bits(x));
  const float m = readlane_f(l, 0);
  const float w = valid ? tweight(l, m, c2) : 0.f;
  const float Z = wave_total(w);
  const float incl = wave_incl_scan(w / Z);
  const float before = wave_excl_from_incl(incl);
  const bool keep = valid && (top_p >= 1.f || before < top_p);
  const unsigned long long kb = __ballot(keep);
  const int nk = (~kb) == 0ull ? kWave : __builtin_ctzll(~kb);   // kept tokens: a prefix
  const float Zk = wave_total(lane < nk ? w : 0.f);
  if (lane < nk) {
    sm.keep_id[row * kFiltKP + lane] = rc_id(x);
    sm.keep_p[row * kFiltKP + lane] = w / Zk;
  }
  if (lane == 0) sm.nkeep[row] = nk;
  return nonfinite;
}

__global__ void __launch_bounds__(kFiltThreads) k_filter_decide(const int32_t* __restrict__ tokens,
                                                                const int32_t* __restrict__ cand_idx,
                                                                const float* __restrict__ q, int64_t batch_stride,
                                                                int K, int V, int nchunks, int top_k, float top_p,
                                                                float inv_t, uint64_t seed,
                                                                const unsigned long long* __restrict__ lists,
                                                                const int* __restrict__ flags,
                                                                int32_t* __restrict__ out_tokens,
                                                                int32_t* __restrict__ n_accepted,
                                                                int32_t* __restrict__ row_status) {
  __shared__ FilterShared sm;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
  const int b = blockIdx.x;
  const int rbase = batch_stride == 0 ? 0 : b * (K + 1);
  int32_t* out_b = out_tokens + (size_t)b * (K + 1);
  const float c2 = inv_t * kLog2e;
  const int nsub = nchunks * kSubPerChunk;

  // the drafts, loaded into registers first so that their loads overlap the rows' list
  // loads, and stored to LDS after
  constexpr int kPer = DFLASH2_MAX_K * kNC / kFiltThreads;
  int cv[kPer];
  float qv[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int e = tid + j * kFiltThreads;
    const int ec = e < K * kNC ? e : 0;
    cv[j] = cand_idx[(size_t)b * K * kNC + ec];
    qv[j] = q[(size_t)b * K * kNC + ec];
  }
  const int tv = tokens[(size_t)b * K + (tid < K ? tid : 0)];
  bool nf = false;
  for (int row = wave; row <= K; row += kFiltWaves) {
    const size_t at = (size_t)(rbase + row) * nsub;
    nf |= filter_row(lists + at * top_k, flags + at, nsub, top_k, top_p, c2, row, sm);
  }
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int e = tid + j * kFiltThreads;
    if (e < K * kNC) {
      sm.cand[(e >> 4) * kFiltNCP + (e & (kNC - 1))] = cv[j];
      sm.q[(e >> 4) * kFiltNCP + (e & (kNC - 1))] = qv[j];
    }
  }
  if (tid < K) sm.tok[tid] = tv;
  if (lane == 0) sm.nonfinite_w[wave] = nf ? 1 : 0;
  __syncthreads();
  if (wave != 0) return;

  // ---- the decision, in wave 0: lane t owns position t -------------------------------
  if (__ballot(lane < kFiltWaves && sm.nonfinite_w[lane < kFiltWaves ? lane : 0] != 0) != 0ull) {
    // a target row holds +inf or NaN: commit nothing
    for (int t = lane; t <= K; t += kWave) out_b[t] = -1;
    if (lane == 0) {
      n_accepted[b] = 0;
      if (row_status) row_status[b] = 1;
    }
    return;
  }
  bool bad = false, qok = true;
  float qx = 0.f, px = 0.f;
  if (lane < K) {
    const int x = sm.tok[lane];
    bad = x < 0 || x >= V;
    float sq = 0.f;
#pragma unroll
    for (int j = 0; j < kNC; ++j) {
      const int id = sm.cand[lane * kFiltNCP + j];
      const float v = sm.q[lane * kFiltNCP + j];
      bad |= id < 0 || id >= V;
      qok &= __builtin_isfinite(v) && v >= 0.f;
      sq += v;
      qx += id == x ? v : 0.f;
    }
    qok &= fabsf(sq - 1.f) <= 1e-3f;
    const int nk = sm.nkeep[lane];
#pragma unroll
    for (int i = 0; i < DFLASH2_MAX_TOPK; ++i)
      px = (i < nk && sm.keep_id[lane * kFiltKP + i] == x) ? sm.keep_p[lane * kFiltKP + i] : px;
  }
  const bool ids_bad = __ballot(bad) != 0ull;
  const bool q_bad = __ballot(lane < K && !(qok && (ids_bad || qx > 0.f))) != 0ull;
  int status = (ids_bad ? 2 : 0) | (q_bad ? 4 : 0);
  const bool fault = ids_bad || q_bad;
  const uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
  bool rej = false;
  if (!fault && lane < K) {
    const float u_acc = word_to_uniform(philox4x32_10((uint32_t)lane, (uint32_t)b, 1u, 0u, k0, k1).x0);
    rej = !(u_acc * qx < px);
  }
  const unsigned long long rejm = __ballot(rej);
  const int tstar = fault ? 0 : (rejm != 0ull ? __builtin_ctzll(rejm) : K);
  const float u_res = word_to_uniform(philox4x32_10((uint32_t)tstar, (uint32_t)b, 1u, 0u, k0, k1).x1);
  const int trow = fault ? 0 : tstar;
  bool residual = !fault && tstar < K;
  // the drawn row's kept tokens (lane i), their p, and max(0, p - q) at a reject
  const int nk = sm.nkeep[trow];
  const int id = lane < nk ? sm.keep_id[trow * kFiltKP + lane] : 0x7fffffff;
  const float pv = lane < nk ? sm.keep_p[trow * kFiltKP + lane] : 0.f;
  float rv = pv;
  if (residual) {
    float qf = 0.f;
#pragma unroll
    for (int j = 0; j < kNC; ++j) qf += sm.cand[trow * kFiltNCP + j] == id ? sm.q[trow * kFiltNCP + j] : 0.f;
    rv = fmaxf(pv - qf, 0.f);
    if (!(wave_total(rv) > 0.f)) {              // the residual has no mass: draw from p
      status |= 8;
      rv = pv;
    }
  }
  // token-id order: lane i's rank among the kept ids, then the weights in that order
  int rank = 0;
#pragma unroll
  for (int j = 0; j < DFLASH2_MAX_TOPK; ++j) rank += (j < nk && __builtin_amdgcn_readlane(id, j) < id) ? 1 : 0;
  if (lane < nk) {
    sm.draw_id[rank] = id;
    sm.draw_w[rank] = rv;
  }
  wave_lds_sync();
  const float wv = lane < nk ? sm.draw_w[lane] : 0.f;
  const int did = lane < nk ? sm.draw_id[lane] : -1;
  const float incl = wave_incl_scan(wv);
  const int l = wave_pick_lane(wv, incl, u_res * readlane_f(incl, kWave - 1));
  const int v = l < 0 ? -1 : __builtin_amdgcn_readlane(did, l);
  for (int t = lane; t <= K; t += kWave) out_b[t] = t < tstar ? sm.tok[t] : (t == tstar ? v : -1);
  if (lane == 0) {
    n_accepted[b] = fault ? 0 : tstar;
    if (row_status) row_status[b] = status;
  }
}

hipError_t launch_spec_accept_filtered(const uint16_t* target, int64_t ld, int64_t batch_stride,
                                       const int32_t* tokens, const int32_t* cand_idx, const float* q, int batch,
                                       int K, int vocab, float temperature, int top_k, float top_p, uint64_t seed,
                                       int32_t* out_tokens, int32_t* n_accepted, int32_t* row_status, FilterWs ws,
                                       hipStream_t s) {
  const int nchunks = topk_num_chunks(vocab);
  const dim3 grid((unsigned)(batch_stride == 0 ? (long long)(K + 1) * nchunks : xcd_chunk_grid(batch, K + 1, nchunks)));
  hipLaunchKernelGGL(k_filter_topk, grid, dim3(kTopkThreads), 0, s, target, ld, batch_stride, K, vocab, nchunks, top_k,
                     ws.lists, ws.flags, batch);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_filter_decide, dim3((unsigned)batch), dim3(kFiltThreads), 0, s, tokens, cand_idx, q,
                     batch_stride, K, vocab, nchunks, top_k, top_p, 1.f / temperature, seed, ws.lists, ws.flags,
                     out_tokens, n_accepted, row_status);
  return hipGetLastError();
}

}  // namespace df2
