// Lossless verify (FreeToken PR "Adds DFlash 2", section "Details", sampled verify:
// accept with min(1, p/q), on a reject resample from max(0, p - q); all-greedy keeps
// the prefix match.  pegainfer issue "DFlash 2 proposer", "Proposal", phase 3).
//
// Pass 1: split-vocabulary statistics of every target row -- per chunk the max and
// the sum of exp((l - max)/T) (k_accept_stats), or the chunk argmax when T == 0
// (k_greedy_argmax).
// Pass 2 (k_accept_decide): one block per request merges its rows' chunk statistics
// (fixed chunk order), runs the accept tests, then draws the committed token by
// inverse CDF: the chunk is found from the chunk masses (minus the draft's mass at its
// candidates), and only that chunk is rescanned.
#include "device_common.h"
#include "dflash2.h"
#include "dflash2_internal.h"
#include "topk_dev.h"

namespace df2 {

constexpr int kAccThreads = 256;
constexpr int kAccVecPerThread = 8;                          // 8 x 16 B loads in flight per lane
constexpr int kAccChunkVec = kAccThreads * kAccVecPerThread;  // 2048 vectors = 16384 logits
constexpr int kAccMaxChunks = 32;                            // vocab <= 2^19

__host__ __device__ __forceinline__ int acc_num_chunks(long long vocab) {
  const long long nvec = (vocab + 7) / 8;
  return (int)((nvec + kAccChunkVec - 1) / kAccChunkVec);
}

int64_t accept_stats_blocks(int64_t nrows, int64_t vocab) { return nrows * acc_num_chunks(vocab); }

AcceptWs carve_accept(Carver& c, int64_t nrows, int64_t vocab) {
  AcceptWs w;
  const size_t n = (size_t)nrows * acc_num_chunks(vocab);
  w.chunk_max = c.take<float>(n);
  w.chunk_sum = c.take<float>(n);
  w.chunk_arg = c.take<unsigned long long>(n);
  return w;
}

__device__ __forceinline__ float order_to_float(int s) { return bf16_to_f32(order_to_bits(s)); }

constexpr float kLog2e = 1.44269504088896341f;

// exp((l - m) / T) formed as 2^((l - m) * c2) with c2 = log2(e) / T: one v_exp_f32 per
// weight.  Every weight of the target distribution (chunk sums, the accept test and
// the draws) is formed this one way.
__device__ __forceinline__ float tweight(float l, float m, float c2) { return __builtin_amdgcn_exp2f((l - m) * c2); }

template <typename T>
__device__ __forceinline__ T block_reduce(T v, T* red, bool is_max) {
  // fixed-order block reduction over 4 waves (deterministic)
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const T other = __shfl_xor(v, o);
    v = is_max ? (other > v ? other : v) : v + other;
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  T r = red[0];
  for (int w = 1; w < kAccThreads / 64; ++w) r = is_max ? (red[w] > r ? red[w] : r) : r + red[w];
  return r;
}

// Sampled statistics (T > 0) of one chunk of a target row.
__global__ void __launch_bounds__(kAccThreads) k_accept_stats(const uint16_t* __restrict__ target, int64_t ld,
                                                              int64_t batch_stride, int K, int V, int nchunks,
                                                              float inv_t, AcceptWs ws) {
  __shared__ float s_redf[4];
  __shared__ int s_redi[4];
  const int tid = threadIdx.x;
  const int r = blockIdx.x / nchunks;
  const int c = blockIdx.x - r * nchunks;
  const int b = batch_stride == 0 ? 0 : r / (K + 1);
  const int t = batch_stride == 0 ? r : r - b * (K + 1);
  const uint16_t* rowp = target + (size_t)b * batch_stride + (size_t)t * ld;
  const u32x4* rowv = reinterpret_cast<const u32x4*>(rowp);
  const int v0 = chunk_begin(V, nchunks, c), v1 = chunk_begin(V, nchunks, c + 1);
  const int nfull = V >> 3;

  u32x4 d[kAccVecPerThread];
#pragma unroll
  for (int k = 0; k < kAccVecPerThread; ++k) {
    const int v = v0 + tid + k * kAccThreads;
    if (v < v1 && v < nfull) {
      d[k] = __builtin_nontemporal_load(rowv + v);
    } else {
      uint32_t wds[4] = {0xff80ff80u, 0xff80ff80u, 0xff80ff80u, 0xff80ff80u};   // -inf padding
      if (v < v1) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          if (8 * v + e < V) {
            const uint32_t bb = rowp[8 * v + e];
            wds[e >> 1] = (e & 1) ? ((wds[e >> 1] & 0xffffu) | (bb << 16)) : ((wds[e >> 1] & 0xffff0000u) | bb);
          }
        }
      }
      d[k] = (u32x4){wds[0], wds[1], wds[2], wds[3]};
    }
  }

  const size_t ci = (size_t)r * nchunks + c;
  // signed-order max / min (to find +inf and NaN) and the chunk maximum
  int smax = -32768, smin = 32767;
#pragma unroll
  for (int k = 0; k < kAccVecPerThread; ++k) {
    const s16x2 a = signed_order2(d[k].x), bq = signed_order2(d[k].y);
    const s16x2 cq = signed_order2(d[k].z), dq = signed_order2(d[k].w);
    const s16x2 mx = __builtin_elementwise_max(__builtin_elementwise_max(a, bq), __builtin_elementwise_max(cq, dq));
    const s16x2 mn = __builtin_elementwise_min(__builtin_elementwise_min(a, bq), __builtin_elementwise_min(cq, dq));
    smax = max_halves(mx) > smax ? max_halves(mx) : smax;
    const int lo = mn.x < mn.y ? (int)mn.x : (int)mn.y;
    smin = lo < smin ? lo : smin;
  }
  smax = block_reduce<int>(smax, s_redi, true);
  smin = -block_reduce<int>(-smin, s_redi, true);
  const bool nonfinite = smax >= 32640 || smin < -32641;       // +inf / +NaN, or -NaN
  const float m_c = order_to_float(smax > 32640 ? 32640 : smax);
  float sum = 0.f;
  if (!nonfinite && m_c != -__builtin_inff()) {
    const float c2 = inv_t * kLog2e;
#pragma unroll
    for (int k = 0; k < kAccVecPerThread; ++k) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        sum += tweight(bf16_lo(d[k][w]), m_c, c2);
        sum += tweight(bf16_hi(d[k][w]), m_c, c2);
      }
    }
  }
  sum = block_reduce<float>(sum, s_redf, false);
  if (tid == 0) {
    ws.chunk_max[ci] = nonfinite ? __builtin_nanf("") : m_c;
    ws.chunk_sum[ci] = sum;
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

constexpr int kMaxStatRows = DFLASH2_MAX_K + 1;

struct DecideShared {
  // the request's inputs, loaded once at entry
  int tok[DFLASH2_MAX_K];
  int cand[DFLASH2_MAX_K * kNC];
  float q[DFLASH2_MAX_K * kNC];
  uint32_t xbits[DFLASH2_MAX_K];          // target logit (bits) of each drafted token
  uint32_t cbits[DFLASH2_MAX_K * kNC];    // target logit (bits) of each candidate
  union {
    struct {
      float max[kMaxStatRows * kAccMaxChunks];
      float sum[kMaxStatRows * kAccMaxChunks];
    } st;                                 // sampled: chunk statistics of the request's rows
    unsigned long long arg[kMaxStatRows * kMaxChunks];   // greedy: chunk argmax composites
  } cs;
  float row_max[kMaxStatRows];            // merged statistics of the request's rows
  float row_sum[kMaxStatRows];            // NaN: a non-finite row
  int row_arg[kMaxStatRows];              // greedy: the row argmax
  int tstar;
  int ids_bad;
  int q_bad;
  int pick;
  int chunk;
  int who;
  int last;
  float rem;
  float before;
  int ncl;
  int cl_id[kNC];
  float cl_qf[kNC];
  float cl_p[kNC];
  float R[kAccMaxChunks];
  float tsum[kAccThreads];
};

// Result of wave_find_crossing, the same in every lane of the wave.
struct Crossing {
  int idx;        // first index whose running sum exceeds the target, -1 if none
  float before;   // the running sum before idx
  int last;       // last index holding a positive value, -1 if none
};

// One whole wave over vals[0 .. n) (LDS, non-negative, n <= 256).  Lane l owns
// vals[4l .. 4l + 3]; its offset is an inclusive scan of the lane sums over lanes, and
// within the lane the sums run in index order.
__device__ __forceinline__ Crossing wave_find_crossing(const float* vals, int n, float target) {
  const int lane = threadIdx.x & 63;
  float v[4], part[4];
  float run = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int i = 4 * lane + j;
    v[j] = i < n ? vals[i] : 0.f;
    run += v[j];
    part[j] = run;
  }
  float inc = part[3];
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const float y = __shfl_up(inc, o);
    if (lane >= o) inc += y;
  }
  float excl = __shfl_up(inc, 1);
  if (lane == 0) excl = 0.f;
  int jhit = 0;
  while (jhit < 3 && !(target < excl + part[jhit])) ++jhit;
  const float bef = jhit == 0 ? excl : excl + part[jhit - 1];
  int jlast = 3;
  while (jlast > 0 && !(v[jlast] > 0.f)) --jlast;
  const unsigned long long hit = __ballot(target < excl + part[3]);
  const unsigned long long pos = __ballot(part[3] > 0.f);
  Crossing cr = {-1, 0.f, -1};
  if (hit) {
    const int src = __builtin_ctzll(hit);
    cr.idx = 4 * src + __builtin_amdgcn_readlane(jhit, src);
    cr.before = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(bef), src));
  }
  if (pos) {
    const int src = 63 - __builtin_clzll(pos);
    cr.last = 4 * src + __builtin_amdgcn_readlane(jlast, src);
  }
  return cr;
}

// Inverse-CDF draw from target row t of the request (row pointer rowp), whose merged
// max and sum are m and Z: weights p (residual == false) or max(0, p - q) with q
// supported on the request's candidates of position t (in LDS).  Block-wide; returns
// the token id (valid in every thread), or -1 for a residual without mass.  Inlined
// at a single call site, so that `sm` stays a known LDS object (ds_* accesses).
constexpr int kFineVec = kAccChunkVec / kAccThreads;    // 16-byte vectors per thread of a chunk rescan
constexpr int kFineLen = 8 * kFineVec;                  // logits per thread

__device__ __forceinline__ int draw_from_row(const uint16_t* __restrict__ rowp, int t, float m, float Z,
                                                       int V, int nchunks, float c2, float u, bool residual,
                                                       DecideShared& sm) {
  const int tid = threadIdx.x;
  const float invZ = 1.f / Z;
  // residual: the distinct candidate ids with their total draft mass (summed in slot
  // order) and their p, sorted by id -- lane j of wave 0 owns slot j & 15
  if (tid < kWave) {
    int ncl = 0;
    if (residual) {
      const int j = tid & (kNC - 1);
      const int id = sm.cand[t * kNC + j];
      const float qv = sm.q[t * kNC + j];
      const float pv = tweight(bf16_to_f32(sm.cbits[t * kNC + j]), m, c2) * invZ;
      bool first = true;
      float qf = 0.f;
#pragma unroll
      for (int i = 0; i < kNC; ++i) {
        const int oi = __shfl(id, i);
        const float qi = __shfl(qv, i);
        if (oi == id) {
          qf += qi;
          if (i < j) first = false;
        }
      }
      int smaller = 0;
#pragma unroll
      for (int i = 0; i < kNC; ++i) {
        const int oi = __shfl(id, i);
        const int fi = __shfl(first ? 1 : 0, i);
        if (fi && oi < id) ++smaller;
      }
      const unsigned long long fm = __ballot(tid < kNC && first);
      if (tid < kNC && first) {
        sm.cl_id[smaller] = id;
        sm.cl_qf[smaller] = qf;
        sm.cl_p[smaller] = pv;
      }
      ncl = __popcll(fm);
    }
    if (tid == 0) sm.ncl = ncl;
  }
  __syncthreads();
  // coarse: mass of every chunk, minus the draft's mass at the candidates it holds
  for (int c = tid; c < nchunks; c += kAccThreads) {
    const float mc = sm.cs.st.max[t * nchunks + c];
    float P = mc == -__builtin_inff() ? 0.f : sm.cs.st.sum[t * nchunks + c] * tweight(mc, m, c2) * invZ;
    const int e0 = 8 * chunk_begin(V, nchunks, c);
    const int e1 = min(8 * chunk_begin(V, nchunks, c + 1), V);
    for (int i = 0; i < sm.ncl; ++i) {
      const int id = sm.cl_id[i];
      if (id >= e0 && id < e1) P -= fminf(sm.cl_p[i], sm.cl_qf[i]);
    }
    sm.R[c] = fmaxf(P, 0.f);
  }
  __syncthreads();
  if (tid < kWave) {
    float Zr = 0.f;
    for (int c = tid; c < nchunks; c += kWave) Zr += sm.R[c];
    Zr = wave_sum(Zr);
    const float target = u * Zr;
    const Crossing cr = wave_find_crossing(sm.R, nchunks, target);
    int idx = cr.idx;
    float before = cr.before;
    const int last = cr.last;
    if (tid == 0) {
      if (idx < 0) {                       // rounding left the target past the total
        idx = last;
        before = 0.f;
        for (int c = 0; c < last; ++c) before += sm.R[c];
      }
      sm.chunk = (residual && !(Zr > 0.f)) || idx < 0 ? -1 : idx;   // a residual without mass
      sm.rem = target - before;
      sm.pick = -1;
    }
  }
  __syncthreads();
  if (sm.chunk < 0) return -1;
  // fine: rescan the chosen chunk; thread i owns a contiguous run of L <= kFineLen
  // logits.  All its loads go out at once (a vector not wholly inside the chunk reads
  // the chunk's first vector and is replaced), and its weights stay in registers.
  const int c = sm.chunk;
  const int e0 = 8 * chunk_begin(V, nchunks, c);
  const int e1 = min(8 * chunk_begin(V, nchunks, c + 1), V);
  const int L = (((e1 - e0) + kAccThreads * 8 - 1) / (kAccThreads * 8)) * 8;
  const int a0 = e0 + tid * L;
  u32x4 raw[kFineVec];
#pragma unroll
  for (int k = 0; k < kFineVec; ++k) {
    const int base = a0 + 8 * k;
    const bool full = 8 * k < L && base + 8 <= e1;
    raw[k] = *reinterpret_cast<const u32x4*>(rowp + (full ? base : e0));
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
  unsigned long long cmask = 0ull;
  for (int i = 0; i < sm.ncl; ++i) {
    const int off = sm.cl_id[i] - a0;
    if (off >= 0 && off < L) cmask |= 1ull << off;
  }
  // weights p of every logit, branch-free; then, only in the threads that need it,
  // zero the logits outside the chunk and replace candidates' weights by max(0, p - q)
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
  if (cmask != 0ull) {
#pragma unroll
    for (int off = 0; off < kFineLen; ++off)
      if ((cmask >> off) & 1ull) {
        float qf = 0.f;
        for (int i = 0; i < sm.ncl; ++i) qf = sm.cl_id[i] == a0 + off ? sm.cl_qf[i] : qf;
        w[off] = fmaxf(w[off] - qf, 0.f);
      }
  }
  float tsum = 0.f;
#pragma unroll
  for (int off = 0; off < kFineLen; ++off) tsum += w[off];
  sm.tsum[tid] = tsum;
  __syncthreads();
  if (tid < kWave) {
    const Crossing cr = wave_find_crossing(sm.tsum, kAccThreads, sm.rem);
    if (tid == 0) {
      sm.who = cr.idx >= 0 ? cr.idx : cr.last;
      sm.before = cr.idx >= 0 ? cr.before : 0.f;
      sm.last = cr.idx < 0 ? 1 : 0;        // no crossing: take the last positive weight
    }
  }
  __syncthreads();
  if (tid == sm.who) {
    // the same weights, in the same order, now with the running sum
    float run = sm.before;
    int pick = -1, lastp = -1;
    const bool take_last = sm.last != 0;
    const float rem = sm.rem;
    // (weights outside the chunk are 0: they neither cross nor count as positive)
#pragma unroll
    for (int off = 0; off < kFineLen; ++off) {
      run += w[off];
      if (pick < 0 && !take_last && rem < run) pick = a0 + off;
      if (w[off] > 0.f) lastp = a0 + off;
    }
    sm.pick = pick >= 0 ? pick : lastp;
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
  const int tid = threadIdx.x;
  const int b = blockIdx.x;
  const int32_t* tok_b = tokens + (size_t)b * K;
  const int32_t* cand_b = cand_idx + (size_t)b * K * kNC;
  const uint16_t* tb = target + (size_t)b * batch_stride;
  const int rbase = batch_stride == 0 ? 0 : b * (K + 1);
  int32_t* out_b = out_tokens + (size_t)b * (K + 1);
  const uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
  const float c2 = inv_t * kLog2e;
  const bool sampled = inv_t != 0.f;

  // ---- everything the decision reads, in at most two dependent memory round trips ----
  for (int e = tid; e < K * kNC; e += kAccThreads) {
    const int id = cand_b[e];
    sm.cand[e] = id;
    if (sampled) {
      sm.q[e] = q[(size_t)b * K * kNC + e];
      const int idc = id < 0 ? 0 : (id >= V ? V - 1 : id);          // read in bounds; flagged below
      sm.cbits[e] = tb[(size_t)(e / kNC) * ld + idc];
    }
  }
  for (int e = tid; e < K; e += kAccThreads) {
    const int x = tok_b[e];
    sm.tok[e] = x;
    if (sampled) sm.xbits[e] = tb[(size_t)e * ld + (x < 0 ? 0 : (x >= V ? V - 1 : x))];
  }
  const int nst = (K + 1) * nchunks;
  const size_t s0 = (size_t)rbase * nchunks;
  for (int e = tid; e < nst; e += kAccThreads) {
    if (sampled) {
      sm.cs.st.max[e] = ws.chunk_max[s0 + e];
      sm.cs.st.sum[e] = ws.chunk_sum[s0 + e];
    } else {
      sm.cs.arg[e] = ws.chunk_arg[s0 + e];
    }
  }
  if (tid == 0) {
    sm.ids_bad = 0;
    sm.q_bad = 0;
    sm.tstar = K;
  }
  __syncthreads();

  // ---- merge the chunk statistics of the request's rows (one thread per row, chunk order)
  if (tid <= K) {
    const int c0 = tid * nchunks;
    if (!sampled) {
      unsigned long long a = 0ull;
      for (int j = 0; j < nchunks; ++j) {
        const unsigned long long x = sm.cs.arg[c0 + j];
        a = x > a ? x : a;
      }
      sm.row_arg[tid] = rc_id(a);
    } else {
      float m = -__builtin_inff();
      bool bad = false;
      for (int j = 0; j < nchunks; ++j) {
        const float mj = sm.cs.st.max[c0 + j];
        if (__builtin_isnan(mj)) bad = true;
        else m = fmaxf(m, mj);
      }
      float Z = 0.f;
      for (int j = 0; j < nchunks; ++j) {
        const float mj = sm.cs.st.max[c0 + j];
        if (!__builtin_isnan(mj) && mj != -__builtin_inff()) Z += sm.cs.st.sum[c0 + j] * tweight(mj, m, c2);
      }
      sm.row_max[tid] = m;
      sm.row_sum[tid] = (bad || m == -__builtin_inff()) ? __builtin_nanf("") : Z;
    }
  }
  for (int e = tid; e < K * (kNC + 1); e += kAccThreads) {
    const int id = e < K ? sm.tok[e] : sm.cand[e - K];
    if (id < 0 || id >= V) atomicOr(&sm.ids_bad, 1);
  }
  for (int e = tid; e <= K; e += kAccThreads) out_b[e] = -1;
  __syncthreads();
  const bool ids_bad = sm.ids_bad != 0;

  if (!sampled) {
    if (tid == 0) {
      int t = 0;
      while (t < K) {
        const int g = sm.row_arg[t];
        if (sm.tok[t] != g) break;
        out_b[t] = g;
        ++t;
      }
      out_b[t] = sm.row_arg[t];
      n_accepted[b] = t;
      if (row_status) row_status[b] = ids_bad ? 2 : 0;
    }
    return;
  }

  // non-finite target rows: commit nothing
  int nonfinite = 0;
  for (int t = 0; t <= K; ++t) nonfinite |= !__builtin_isfinite(sm.row_sum[t]);
  if (nonfinite) {
    if (tid == 0) {
      n_accepted[b] = 0;
      if (row_status) row_status[b] = 1;
    }
    return;
  }

  // validity of the draft distributions
  if (tid < K) {
    float s = 0.f, qx = 0.f;
    bool ok = true;
    for (int j = 0; j < kNC; ++j) {
      const float v = sm.q[tid * kNC + j];
      ok &= __builtin_isfinite(v) && v >= 0.f;
      s += v;
      qx += sm.cand[tid * kNC + j] == sm.tok[tid] ? v : 0.f;
    }
    ok &= fabsf(s - 1.f) <= 1e-3f;
    if (!ids_bad) ok &= qx > 0.f;
    if (!ok) atomicOr(&sm.q_bad, 1);
  }
  __syncthreads();
  const bool q_bad = sm.q_bad != 0;
  int status = (ids_bad ? 2 : 0) | (q_bad ? 4 : 0);

  // accept tests (all positions at once; the first reject decides); skipped when the
  // ids or the draft distributions are invalid, which commits one token from p_0
  const bool fault = ids_bad || q_bad;
  if (!fault && tid < K) {
    const int t = tid;
    const int x = sm.tok[t];
    float qx = 0.f;
    for (int j = 0; j < kNC; ++j) qx += sm.cand[t * kNC + j] == x ? sm.q[t * kNC + j] : 0.f;
    const float px = tweight(bf16_to_f32(sm.xbits[t]), sm.row_max[t], c2) / sm.row_sum[t];
    const float u_acc = word_to_uniform(philox4x32_10((uint32_t)t, (uint32_t)b, 1u, 0u, k0, k1).x0);
    if (!(u_acc * qx < px)) atomicMin(&sm.tstar, t);
  }
  __syncthreads();
  const int tstar = fault ? 0 : sm.tstar;
  if (!fault)
    for (int t = tid; t < tstar; t += kAccThreads) out_b[t] = sm.tok[t];
  const float u_res = word_to_uniform(philox4x32_10((uint32_t)tstar, (uint32_t)b, 1u, 0u, k0, k1).x1);
  // the residual max(0, p - q) at a reject (p instead when it has no mass), else p of
  // the bonus row (or of row 0 after a fault)
  const int trow = fault ? 0 : tstar;
  bool residual = !fault && tstar < K;
  const uint16_t* rowp = tb + (size_t)trow * ld;
  int v = -1;
  for (int pass = 0; pass < 2; ++pass) {
    v = draw_from_row(rowp, trow, sm.row_max[trow], sm.row_sum[trow], V, nchunks, c2, u_res, residual, sm);
    if (v >= 0 || !residual) break;
    status |= 8;
    residual = false;
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
  const int nrows = batch_stride == 0 ? K + 1 : batch * (K + 1);
  const float inv_t = temperature == 0.f ? 0.f : 1.f / temperature;
  int nchunks;
  if (inv_t == 0.f) {
    nchunks = topk_num_chunks(vocab);          // <= acc_num_chunks(vocab): fits the workspace
    hipLaunchKernelGGL(k_greedy_argmax, dim3((unsigned)(nrows * nchunks)), dim3(kTopkThreads), 0, s, target, ld,
                       batch_stride, K, vocab, nchunks, ws.chunk_arg);
  } else {
    nchunks = acc_num_chunks(vocab);
    hipLaunchKernelGGL(k_accept_stats, dim3((unsigned)(nrows * nchunks)), dim3(kAccThreads), 0, s, target, ld,
                       batch_stride, K, vocab, nchunks, inv_t, ws);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_accept_decide, dim3((unsigned)batch), dim3(kAccThreads), 0, s, target, ld, batch_stride, tokens,
                     cand_idx, q, K, vocab, nchunks, inv_t, seed, out_tokens, n_accepted, row_status, ws);
  return hipGetLastError();
}

}  // namespace df2
