// Top-16, pair-score and walk kernels, and the proposer step built from them.
//
// The proposer step (dflash2_select) runs as two back-to-back kernels on one stream:
//   1. k_chunk_lists  streams the logits (two 512-thread blocks per row at V = 151936)
//                     and writes each chunk's sorted top-16; it also zeroes one ticket
//                     per request for stage 2;
//   2. k_positions    one 4-wave block per draft position: merges the chunk top-16s of
//                     rows t - 1 and t, writes row t's candidates, gathers the table rows
//                     of the 16 x 16 adjacent pairs, computes the scores of t (the
//                     selector dims split over the waves) and the successor table (the
//                     slot taken from each predecessor slot); the block that completes
//                     its request's last table (counted on the request's ticket) then
//                     follows the tables from the verified row and writes tokens, slots
//                     and q.
// The gated step (dflash2_select_gated) launches k_chunk_gate in place of stage 1 (the
// same blocks plus the context gate's tiles as extra work-groups), and its stage 2
// adds each row's gate slices before the scores.
// A kernel boundary hands the chunk lists to stage 2; inside stage 2 the tables reach the
// walking block through agent-scope stores and loads and the ticket, so no work-group
// ever waits for another (the walk this way costs less than a third kernel's boundary
// and launch; the chunk lists' hand-off measured no cheaper than the boundary).  Stage 2
// runs one block per position rather than one per request so that each request's table
// rows (about 107 KB at K = 7) are gathered by K compute units instead of one.  Every
// entry point computes a tile with the same block routine (pair_dev.h), so all of them
// give bit-identical scores.
#include "dflash2_internal.h"
#include "gate_dev.h"
#include "pair_dev.h"
#include "topk_dev.h"

namespace df2 {

TopkWs carve_topk(Carver& c, int64_t rows, int64_t vocab) {
  TopkWs w;
  w.partials = c.take<unsigned long long>((size_t)rows * topk_num_chunks(vocab) * kNC);
  return w;
}

SelectWs carve_select(Carver& c, int64_t batch, int64_t K, int64_t vocab) {
  SelectWs w;
  w.topk = carve_topk(c, batch * K, vocab);
  w.next = c.take<int>((size_t)(batch * K * kNC));
  w.qtab = c.take<float>((size_t)(batch * K * kNC * kNC));
  w.tickets = c.take<unsigned>((size_t)batch * kWalkTicketStride);
  return w;
}

// The gate of the gated select: tiles of 16 rows x 64 columns, eight waves per
// work-group with kFusedGateSteps 32-wide steps each, so a slice spans
// 8 * kFusedGateSteps steps of the hidden dimension.
constexpr int kFusedGateSteps = 2;
constexpr int kFusedGateCols = 64;

int fused_gate_splits(int64_t hidden) {
  const int64_t steps = (hidden + 31) / 32;
  const int64_t per = (int64_t)kTopkWaves * kFusedGateSteps;
  return (int)((steps + per - 1) / per);
}

int64_t fused_gate_blocks(int64_t rows, int64_t hidden, int64_t dim) {
  return ((rows + 15) / 16) * (dim / kFusedGateCols) * fused_gate_splits(hidden);
}

SelectGatedWs carve_select_gated(Carver& c, int64_t batch, int64_t K, int64_t vocab, int64_t hidden, int64_t dim) {
  SelectGatedWs w;
  w.sel = carve_select(c, batch, K, vocab);
  w.nsplit = fused_gate_splits(hidden);
  w.partial = c.take<float>((size_t)w.nsplit * batch * K * dim);
  return w;
}

// ---- stage 1: chunk top-16s ---------------------------------------------------------------

// Block (row, chunk) writes list row * nchunks + chunk.
__device__ __forceinline__ void chunk_block(const uint16_t* __restrict__ logits, int64_t ld, int V, int nchunks,
                                            int blk, ChunkShared& sm, unsigned long long* __restrict__ partials) {
  const int row = blk / nchunks;
  const int chunk = blk - row * nchunks;
  chunk_top16(logits + (size_t)row * ld, V, chunk_begin(V, nchunks, chunk), chunk_begin(V, nchunks, chunk + 1), sm,
              partials + (size_t)blk * kNC);
}

__global__ void __launch_bounds__(kTopkThreads) k_chunk_lists(const uint16_t* __restrict__ logits, int64_t ld, int V,
                                                              int nchunks, unsigned long long* __restrict__ partials,
                                                              int batch, int K, unsigned* __restrict__ tickets) {
  args_in_sgprs(logits, ld, V, nchunks, partials, batch, K, tickets);
  __shared__ ChunkShared sm;
  // the next kernel's per-request tickets start at zero (written here, read after the
  // kernel boundary)
  if (tickets && blockIdx.x == 0)
    for (int b = (int)threadIdx.x; b < batch; b += kTopkThreads) tickets[(size_t)b * kWalkTicketStride] = 0u;
  // a request's chunk blocks on the XCD of its position blocks (k_positions), so the
  // chunk lists are read back from the L2 they were written to
  const int blk = xcd_chunk_block((int)blockIdx.x, batch, K, nchunks);
  if (blk < 0) return;                            // padding ids (the whole work-group)
  chunk_block(logits, ld, V, nchunks, blk, sm, partials);
}

// ---- stage 1 of the gated select: chunk top-16s and gate tiles in one launch ---------
// Blocks [0, nchunk_blocks) stream the logits as k_chunk_lists does; the rest compute
// the context gate's partial sums (gate_dev.h tiles, 8 waves) on the compute units the
// stream leaves idle or shares.

union ChunkGateShared {
  ChunkShared c;
  float red[kTopkWaves * 16 * kFusedGateCols];
};

template <bool HB>
__global__ void __launch_bounds__(kTopkThreads) k_chunk_gate(const uint16_t* __restrict__ logits, int64_t ld, int V,
                                                             int nchunks, int nchunk_blocks,
                                                             unsigned long long* __restrict__ partials,
                                                             const void* __restrict__ h,
                                                             const uint16_t* __restrict__ w_h, int rows, int hidden,
                                                             int dim, int ntiles, int nsplit,
                                                             float* __restrict__ gate_partial,
                                                             unsigned* __restrict__ tickets, int batch) {
  args_in_sgprs(logits, ld, V, nchunks, nchunk_blocks, partials);
  __shared__ ChunkGateShared sm;
  if (blockIdx.x == 0)
    for (int b = (int)threadIdx.x; b < batch; b += kTopkThreads) tickets[(size_t)b * kWalkTicketStride] = 0u;
  if ((int)blockIdx.x < nchunk_blocks) {
    chunk_block(logits, ld, V, nchunks, (int)blockIdx.x, sm.c, partials);
    return;
  }
  const int gb = (int)blockIdx.x - nchunk_blocks;
  const int per = ntiles * nsplit;
  const int mt = gb / per;
  const int rem = gb - mt * per;
  const int nt = rem / nsplit;
  const int split = rem - nt * nsplit;
  gate_tile<kFusedGateCols / 16, kTopkWaves, kFusedGateSteps, HB>(h, w_h, nullptr, rows, hidden, dim, 0, mt, nt, split,
                                                              nsplit, sm.red, nullptr, gate_partial);
}

// ---- top-16: merge each row's chunk lists (one wave per logits row) ---------------------

constexpr int kMergeWaves = 4;                    // rows per block of the standalone merge

__global__ void __launch_bounds__(kMergeWaves * kWave) k_merge_lists(const unsigned long long* __restrict__ partials,
                                                                     int rows, int nlists,
                                                                     int32_t* __restrict__ cand_idx,
                                                                     float* __restrict__ cand_val,
                                                                     int32_t* __restrict__ row_status) {
  args_in_sgprs(partials, rows, nlists, cand_idx, cand_val, row_status);
  const int row = blockIdx.x * kMergeWaves + (int)(threadIdx.x >> 6);
  if (row >= rows) return;                        // the whole wave
  const int lane = threadIdx.x & 63;
  const unsigned long long rc = wave_merge_lists(partials + (size_t)row * nlists * kNC, nlists);
  const float v = bf16_to_f32(rc_bits(rc));
  const bool bad = __ballot(lane < kNC && !__builtin_isfinite(v)) != 0ull;
  if (lane < kNC) {
    cand_idx[(size_t)row * kNC + lane] = rc ? rc_id(rc) : 0;
    cand_val[(size_t)row * kNC + lane] = v;
  }
  if (row_status && lane == 0) row_status[row] = bad ? 1 : 0;
}

// ---- pair scores ------------------------------------------------------------------------

template <int DIM, bool BF16>
__global__ void __launch_bounds__(kTileThreads) k_pair_score(const int32_t* __restrict__ cand_idx,
                                                             const float* __restrict__ cand_val,
                                                             const int32_t* __restrict__ verified,
                                                             const void* __restrict__ emb_a,
                                                             const void* __restrict__ emb_b, int V,
                                                             const float* __restrict__ H, int K, float* __restrict__ S,
                                                             int32_t* __restrict__ row_status) {
  args_in_sgprs(cand_idx, cand_val, verified, emb_a, emb_b, V, H, K, S, row_status);
  __shared__ TileShared sm;
  const int pos = blockIdx.x;
  const int b = pos / K, t = pos - b * K;
  const int tid = threadIdx.x, r = tid & 15;
  int bad = 0;
  const int prev = clamp_id(t == 0 ? verified[b] : cand_idx[((size_t)pos - 1) * kNC + r], V, &bad);
  const int cur = clamp_id(cand_idx[(size_t)pos * kNC + r], V, &bad);
  const float s = block_pair_tile<DIM, BF16>(emb_a, emb_b, prev, cur, H + (size_t)pos * DIM,
                                             cand_val[(size_t)pos * kNC + r], sm);
  const bool nonfin = block_any(!__builtin_isfinite(s), sm);
  S[(size_t)pos * kNC * kNC + tid] = s;
  const bool any_bad = __ballot(bad != 0) != 0ull;             // wave 0 holds every id
  if (row_status && tid == 0) row_status[pos] = (any_bad ? 2 : 0) | (nonfin ? 1 : 0);
}

// ---- walk ------------------------------------------------------------------------------

// From scores alone: position by position, build the successor table, follow it from
// the slot taken at the previous position, and emit that row's distribution.
__global__ void __launch_bounds__(256) k_walk(const float* __restrict__ S, const int32_t* __restrict__ cand_idx, int K,
                                              float inv_t, uint64_t seed, int32_t* __restrict__ tokens,
                                              int32_t* __restrict__ slots, float* __restrict__ q) {
  args_in_sgprs(S, cand_idx, K, inv_t, seed, tokens, slots, q);
  __shared__ int s_next[kNC];
  const int b = blockIdx.x;
  const int i = threadIdx.x >> 4, j = threadIdx.x & 15;
  const float* S_b = S + (size_t)b * K * kNC * kNC;
  int from = 0;                                       // slot taken at the previous position
  for (int t = 0; t < K; ++t) {
    const float u = inv_t == 0.f ? 0.f : walk_uniform(seed, (uint32_t)b, (uint32_t)t);
    float qj;
    const int pick = row16_pick(S_b[((size_t)t * kNC + i) * kNC + j], inv_t, u, &qj);
    if (j == 0) s_next[i] = pick;
    if (i == from) q[((size_t)b * K + t) * kNC + j] = qj;
    __syncthreads();
    const int to = s_next[from];
    if (threadIdx.x == 0) {
      slots[(size_t)b * K + t] = to;
      tokens[(size_t)b * K + t] = cand_idx[((size_t)b * K + t) * kNC + to];
    }
    __syncthreads();
    from = to;
  }
}

constexpr int kMaxK = 64;               // draft positions per request (the ABI's limit)
constexpr int kStagedK = 16;            // distributions staged in LDS up to this many positions

struct WalkShared {
  int tok[kMaxK * kNC];                 // the request's candidates
  float qtab[kStagedK * kNC * kNC];     // each predecessor row's distribution (sampled)
  int path[kMaxK];
};

// The walk of request b from the successor tables its position blocks built: next[t][i]
// (slot taken at t after slot i at t - 1) and, when sampling, qtab[t][i][.] (that row's
// distribution), stored at agent scope by the request's other blocks.  Wave 0 follows
// the tables (lane r holds next[t][r]; each step reads the lane of the previous slot)
// while waves 1-3 stage the candidates and distributions, so nothing read after the
// walk depends on it through global memory (the distributions of a request longer than
// kStagedK positions are read after the walk).  All 256 threads of the block call it.
__device__ __forceinline__ void walk_tables(int b, int K, bool sampled, const int* __restrict__ next,
                                            const float* __restrict__ qtab, const int32_t* __restrict__ cand_idx,
                                            int32_t* __restrict__ tokens, int32_t* __restrict__ slots,
                                            float* __restrict__ q, WalkShared& sm) {
  const int tid = threadIdx.x;
  const size_t base = (size_t)b * K * kNC;
  if (tid < kWave) {
    const int r = tid & 15;
    int from = 0;
    for (int t0 = 0; t0 < K; t0 += 16) {
      int nt[16];
#pragma unroll
      for (int k = 0; k < 16; ++k) nt[k] = t0 + k < K ? load_agent(next + base + (size_t)(t0 + k) * kNC + r) : 0;
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        if (t0 + k < K) {
          from = __builtin_amdgcn_readlane(nt[k], from);
          if (tid == 0) sm.path[t0 + k] = from;
        }
      }
    }
  } else {
    // every load of a thread's share issued before its first LDS store
    constexpr int kStagers = kTileThreads - kWave;
    constexpr int kTokPer = (kMaxK * kNC + kStagers - 1) / kStagers;
    constexpr int kQPer = (kStagedK * kNC * kNC + kStagers - 1) / kStagers;
    const int ti = tid - kWave;
    int tv[kTokPer];
#pragma unroll
    for (int k = 0; k < kTokPer; ++k)
      tv[k] = ti + k * kStagers < K * kNC ? load_agent(cand_idx + base + ti + k * kStagers) : 0;
    if (sampled && K <= kStagedK) {
      float qv[kQPer];
#pragma unroll
      for (int k = 0; k < kQPer; ++k) {
        const int e = ti + k * kStagers;
        qv[k] = e < K * kNC * kNC ? load_agent(qtab + base * kNC + e) : 0.f;
      }
#pragma unroll
      for (int k = 0; k < kQPer; ++k)
        if (ti + k * kStagers < K * kNC * kNC) sm.qtab[ti + k * kStagers] = qv[k];
    }
#pragma unroll
    for (int k = 0; k < kTokPer; ++k)
      if (ti + k * kStagers < K * kNC) sm.tok[ti + k * kStagers] = tv[k];
  }
  __syncthreads();
  const bool staged = K <= kStagedK;
  for (int e = tid; e < K * kNC; e += kTileThreads) {
    const int t = e >> 4, j = e & 15;
    const int to = sm.path[t];
    const int from = t == 0 ? 0 : sm.path[t - 1];
    const int qi = (t * kNC + from) * kNC + j;
    q[base + e] = sampled ? (staged ? sm.qtab[qi] : load_agent(qtab + base * kNC + qi)) : (j == to ? 1.f : 0.f);
    if (j == 0) {
      slots[(size_t)b * K + t] = to;
      tokens[(size_t)b * K + t] = sm.tok[t * kNC + to];
    }
  }
}

// ---- the gate rows of the gated step -----------------------------------------------------

struct GateArgs {
  const float* partial = nullptr;    // [nsplit][rows][dim] slice sums of the fused gate tiles
  const float* bias = nullptr;
  int nsplit = 0;
  int act = 0;
  float* H_out = nullptr;
};

// H[e] for the n = nrows * DIM gate values of rows row0.. (e = t * DIM + d): the slice sums
// added in slice order, then the bias and the activation (as gate_finish), written to dst
// (LDS) and to H_out when given.  The first nthreads threads of the block (index ti) call
// it; each thread's loads of kE values x kS slices are in flight together (kE values per
// thread cover DIM with 128 threads; 16 slices when kE <= 2, so the ten slices of a
// 5120-wide hidden cost one memory round trip).
template <int DIM>
__device__ __forceinline__ void gated_rows(const GateArgs& ga, int rows, int row0, int n, int ti, int nthreads,
                                           float* dst) {
  constexpr int kE = DIM >= 1024 ? 8 : (DIM + 127) / 128;
  constexpr int kS = kE <= 2 ? 16 : 8;
  const size_t stride = (size_t)rows * DIM;
  for (int e0 = ti; e0 < n; e0 += kE * nthreads) {
    float sum[kE];
#pragma unroll
    for (int k = 0; k < kE; ++k) sum[k] = 0.f;
    for (int s0 = 0; s0 < ga.nsplit; s0 += kS) {
      float v[kS][kE];
#pragma unroll
      for (int sp = 0; sp < kS; ++sp)
#pragma unroll
        for (int k = 0; k < kE; ++k) {
          const int e = e0 + k * nthreads;
          v[sp][k] = (s0 + sp < ga.nsplit && e < n)
                         ? ga.partial[(size_t)(s0 + sp) * stride + (size_t)row0 * DIM + e]
                         : 0.f;
        }
#pragma unroll
      for (int sp = 0; sp < kS; ++sp)
#pragma unroll
        for (int k = 0; k < kE; ++k)
          if (s0 + sp < ga.nsplit) sum[k] += v[sp][k];
    }
#pragma unroll
    for (int k = 0; k < kE; ++k) {
      const int e = e0 + k * nthreads;
      if (e < n) {
        const int d = e & (DIM - 1);
        const float h = gate_act(sum[k] + (ga.bias ? ga.bias[d] : 0.f), ga.act);
        dst[e] = h;
        if (ga.H_out) ga.H_out[(size_t)row0 * DIM + e] = h;
      }
    }
  }
}

struct SelectOut {
  int32_t* cand_idx;
  float* cand_val;
  float* S;
  int32_t* tokens;
  int32_t* slots;
  float* q;
  int32_t* row_status;
};

// ---- stage 2 of the proposer step: one block per draft position ------------------------

// GATED: H is not given; waves 1-3 add the row's gate slices, apply the bias and the
// activation, keep the row in LDS and write it to H_out when given.
template <int DIM, bool BF16, bool GATED>
__global__ void __launch_bounds__(kTileThreads) k_positions(const unsigned long long* __restrict__ partials,
                                                            int nchunks, int K, int rows,
                                                            const int32_t* __restrict__ verified,
                                                            const void* __restrict__ emb_a,
                                                            const void* __restrict__ emb_b, int V,
                                                            const float* __restrict__ H, GateArgs ga, float inv_t,
                                                            uint64_t seed, int32_t* __restrict__ cand_idx,
                                                            float* __restrict__ cand_val, float* __restrict__ S,
                                                            int* __restrict__ next, float* __restrict__ qtab,
                                                            int32_t* __restrict__ row_status,
                                                            unsigned* __restrict__ tickets,
                                                            int32_t* __restrict__ tokens, int32_t* __restrict__ slots,
                                                            float* __restrict__ q) {
  args_in_sgprs(partials, nchunks, K, rows, verified, emb_a, emb_b, V, H, inv_t, seed, cand_idx, cand_val, S, next, qtab,
                row_status);
  if constexpr (GATED) args_in_sgprs(ga.partial, ga.bias, ga.nsplit, ga.act, ga.H_out);
  __shared__ union {
    TileShared tile;
    WalkShared walk;
  } shm;
  TileShared& sm = shm.tile;
  __shared__ float s_H[GATED ? DIM : 1];
  __shared__ int s_walker;
  __shared__ int s_prev[kNC], s_cur[kNC];
  __shared__ float s_U[kNC];
  __shared__ int s_bits;
  // placement as in k_chunk_lists: the K blocks of request b on the XCD of b % 8
  const int pos = xcd_chunk_block((int)blockIdx.x, rows / K, K, 1);
  if (pos < 0) return;                            // padding ids (the whole block)
  const int b = pos / K, t = pos - b * K;
  const int tid = threadIdx.x, w = tid >> 6, r = tid & 15;
  const int nlists = nchunks;
  if (w == 0) {
    // wave 0 merges row pos
    const unsigned long long rc = wave_merge_lists(partials + (size_t)pos * nlists * kNC, nlists);
    const float v = bf16_to_f32(rc_bits(rc));
    const bool nf = __ballot(tid < kNC && !__builtin_isfinite(v)) != 0ull;
    if (tid < kNC) {
      s_cur[tid] = rc ? rc_id(rc) : 0;
      s_U[tid] = v;
    }
    if (tid == 0) s_bits = nf ? 1 : 0;
  } else if (w == 1) {
    // wave 1 merges row pos - 1 (the predecessors)
    if (t == 0) {
      if (tid < kWave + kNC) s_prev[tid - kWave] = verified[b];
    } else {
      const unsigned long long rc = wave_merge_lists(partials + (size_t)(pos - 1) * nlists * kNC, nlists);
      if (tid < kWave + kNC) s_prev[tid - kWave] = rc ? rc_id(rc) : 0;
    }
  } else if constexpr (GATED) {
    gated_rows<DIM>(ga, rows, pos, DIM, tid - 2 * kWave, kTileThreads - 2 * kWave, s_H);
  }
  __syncthreads();
  int bad = 0;
  const int prev = clamp_id(s_prev[r], V, &bad);
  const int cur = clamp_id(s_cur[r], V, &bad);
  float s;
  if constexpr (GATED)
    s = block_pair_tile<DIM, BF16>(emb_a, emb_b, prev, cur, s_H, s_U[r], sm);
  else
    s = block_pair_tile<DIM, BF16>(emb_a, emb_b, prev, cur, H + (size_t)pos * DIM, s_U[r], sm);
  const bool nonfin = block_any(!__builtin_isfinite(s), sm);
  // thread 16 i + j holds S[i][j]: its 16-lane group decides row i
  const float u = inv_t == 0.f ? 0.f : walk_uniform(seed, (uint32_t)b, (uint32_t)t);
  float qj;
  const int pick = row16_pick(s, inv_t, u, &qj);
  S[(size_t)pos * kNC * kNC + tid] = s;
  // what the request's walk reads goes out at agent scope (another block may walk)
  if (inv_t != 0.f) store_agent(qtab + (size_t)pos * kNC * kNC + tid, qj);
  if (r == 0) store_agent(next + (size_t)pos * kNC + (tid >> 4), pick);
  if (tid < kNC) {
    store_agent(cand_idx + (size_t)pos * kNC + tid, s_cur[tid]);
    cand_val[(size_t)pos * kNC + tid] = s_U[tid];
  }
  const bool any_bad = __ballot(bad != 0) != 0ull;             // wave 0 holds every id
  if (row_status && tid == 0) row_status[pos] = s_bits | (any_bad ? 2 : 0) | (nonfin ? 1 : 0);
  if constexpr (GATED) {
    if (ga.H_out)
      for (int d = tid; d < DIM; d += kTileThreads) ga.H_out[(size_t)pos * DIM + d] = s_H[d];
  }
  // the block that builds its request's last position walks the request: a ticket per
  // request (zeroed by the stream kernel) counts the positions whose tables are out
  drain_memory();
  __syncthreads();
  if (tid == 0)
    s_walker = __hip_atomic_fetch_add(tickets + (size_t)b * kWalkTicketStride, 1u, __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT) + 1u == (unsigned)K;
  __syncthreads();
  if (s_walker) walk_tables(b, K, inv_t != 0.f, next, qtab, cand_idx, tokens, slots, q, shm.walk);
}

// ---- launchers -----------------------------------------------------------------------

hipError_t launch_topk16(const uint16_t* logits, int rows, int vocab, int64_t ld, int32_t* cand_idx, float* cand_val,
                         int32_t* row_status, TopkWs ws, hipStream_t s) {
  const int nchunks = topk_num_chunks(vocab);
  hipLaunchKernelGGL(k_chunk_lists, dim3((unsigned)xcd_chunk_grid(rows, 1, nchunks)), dim3(kTopkThreads), 0, s, logits,
                     ld, vocab, nchunks, ws.partials, rows, 1, (unsigned*)nullptr);
  hipLaunchKernelGGL(k_merge_lists, dim3((unsigned)((rows + kMergeWaves - 1) / kMergeWaves)), dim3(kMergeWaves * kWave),
                     0, s, ws.partials, rows, nchunks, cand_idx, cand_val, row_status);
  return hipGetLastError();
}

// Calls f.template operator()<DIM>() for the selector width dim (a power of two in
// [16, 1024]); returns false for any other width.
template <typename F>
static bool with_dim(int dim, F&& f) {
  switch (dim) {
    case 16: f.template operator()<16>(); return true;
    case 32: f.template operator()<32>(); return true;
    case 64: f.template operator()<64>(); return true;
    case 128: f.template operator()<128>(); return true;
    case 256: f.template operator()<256>(); return true;
    case 512: f.template operator()<512>(); return true;
    case 1024: f.template operator()<1024>(); return true;
    default: return false;
  }
}

hipError_t launch_pair_score(const int32_t* cand_idx, const float* cand_val, const int32_t* verified, const void* emb_a,
                             const void* emb_b, bool bf16, int vocab, int dim, const float* H, int batch, int K,
                             float* S, int32_t* row_status, hipStream_t s) {
  const dim3 grid((unsigned)(batch * K));
  const bool ok = with_dim(dim, [&]<int D>() {
    if (bf16)
      hipLaunchKernelGGL((k_pair_score<D, true>), grid, dim3(kTileThreads), 0, s, cand_idx, cand_val, verified, emb_a,
                         emb_b, vocab, H, K, S, row_status);
    else
      hipLaunchKernelGGL((k_pair_score<D, false>), grid, dim3(kTileThreads), 0, s, cand_idx, cand_val, verified, emb_a,
                         emb_b, vocab, H, K, S, row_status);
  });
  return ok ? hipGetLastError() : hipErrorInvalidValue;
}

hipError_t launch_walk(const float* S, const int32_t* cand_idx, int batch, int K, float temperature, uint64_t seed,
                       int32_t* tokens, int32_t* slots, float* q, hipStream_t s) {
  const float inv_t = temperature == 0.f ? 0.f : 1.f / temperature;
  hipLaunchKernelGGL(k_walk, dim3((unsigned)batch), dim3(256), 0, s, S, cand_idx, K, inv_t, seed, tokens, slots, q);
  return hipGetLastError();
}

// Stages 2 and 3 of the select; stage 1 has filled ws.topk.partials.
template <bool GATED>
static hipError_t select_tail(int nchunks, const int32_t* verified, const void* emb_a, const void* emb_b, bool bf16,
                              int vocab, int dim, const float* H, const GateArgs& ga, int batch, int K, float inv_t,
                              uint64_t seed, const SelectOut& out, const SelectWs& ws, hipStream_t s) {
  const int rows = batch * K;
  const dim3 grid((unsigned)xcd_chunk_grid(batch, K, 1));      // placed as k_chunk_lists
  const bool ok = with_dim(dim, [&]<int D>() {
    if (bf16)
      hipLaunchKernelGGL((k_positions<D, true, GATED>), grid, dim3(kTileThreads), 0, s,
                         ws.topk.partials, nchunks, K, rows, verified, emb_a, emb_b, vocab, H, ga, inv_t, seed,
                         out.cand_idx, out.cand_val, out.S, ws.next, ws.qtab, out.row_status, ws.tickets, out.tokens,
                         out.slots, out.q);
    else
      hipLaunchKernelGGL((k_positions<D, false, GATED>), grid, dim3(kTileThreads), 0, s,
                         ws.topk.partials, nchunks, K, rows, verified, emb_a, emb_b, vocab, H, ga, inv_t, seed,
                         out.cand_idx, out.cand_val, out.S, ws.next, ws.qtab, out.row_status, ws.tickets, out.tokens,
                         out.slots, out.q);
  });
  if (!ok) return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_select(const uint16_t* logits, int64_t ld, const int32_t* verified, const void* emb_a,
                         const void* emb_b, bool bf16, int vocab, int dim, const float* H, int batch, int K,
                         float temperature, uint64_t seed, int32_t* cand_idx, float* cand_val, float* S,
                         int32_t* tokens, int32_t* slots, float* q, int32_t* row_status, SelectWs ws, hipStream_t s) {
  const int nchunks = topk_num_chunks(vocab);
  const float inv_t = temperature == 0.f ? 0.f : 1.f / temperature;
  hipLaunchKernelGGL(k_chunk_lists, dim3((unsigned)xcd_chunk_grid(batch, K, nchunks)), dim3(kTopkThreads), 0, s,
                     logits, ld, vocab, nchunks, ws.topk.partials, batch, K, ws.tickets);
  const SelectOut out{cand_idx, cand_val, S, tokens, slots, q, row_status};
  return select_tail<false>(nchunks, verified, emb_a, emb_b, bf16, vocab, dim, H, GateArgs{}, batch, K, inv_t, seed,
                            out, ws, s);
}

hipError_t launch_select_gated(const uint16_t* logits, int64_t ld, const int32_t* verified, const void* emb_a,
                               const void* emb_b, bool bf16, int vocab, int dim, const void* h, bool h_bf16,
                               const uint16_t* w_h, const float* bias, int hidden, int act, int batch, int K,
                               float temperature, uint64_t seed, float* H_out, int32_t* cand_idx, float* cand_val,
                               float* S, int32_t* tokens, int32_t* slots, float* q, int32_t* row_status,
                               SelectGatedWs ws, hipStream_t s) {
  const int nchunks = topk_num_chunks(vocab);
  const float inv_t = temperature == 0.f ? 0.f : 1.f / temperature;
  const int rows = batch * K;
  const int nchunk_blocks = rows * nchunks;
  const int ntiles = dim / kFusedGateCols;
  const long long blocks = (long long)nchunk_blocks + fused_gate_blocks(rows, hidden, dim);
  hipLaunchKernelGGL(h_bf16 ? k_chunk_gate<true> : k_chunk_gate<false>, dim3((unsigned)blocks), dim3(kTopkThreads), 0,
                     s, logits, ld, vocab, nchunks, nchunk_blocks, ws.sel.topk.partials, h, w_h, rows, hidden, dim,
                     ntiles, ws.nsplit, ws.partial, ws.sel.tickets, batch);
  GateArgs ga;
  ga.partial = ws.partial;
  ga.bias = bias;
  ga.nsplit = ws.nsplit;
  ga.act = act;
  ga.H_out = H_out;
  const SelectOut out{cand_idx, cand_val, S, tokens, slots, q, row_status};
  return select_tail<true>(nchunks, verified, emb_a, emb_b, bf16, vocab, dim, nullptr, ga, batch, K, inv_t, seed, out,
                           ws.sel, s);
}

}  // namespace df2
