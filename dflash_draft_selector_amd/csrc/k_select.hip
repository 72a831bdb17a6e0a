// Top-16, pair-score and walk kernels, and the proposer step built from them.
//
// The proposer step (dflash2_select) runs as three back-to-back kernels on one stream:
//   1. k_chunk_lists  streams the logits (two 512-thread blocks per row at V = 151936)
//                     and writes each chunk's sorted top-16;
//   2. k_positions    one block per draft position: merges the chunk top-16s of rows
//                     t - 1 and t, writes row t's candidates, computes the 16 x 16
//                     scores of t and the successor table (the slot taken from each
//                     predecessor slot);
//   3. k_walk_tables  one block per request: chases the tables from the verified row
//                     and writes tokens, slots and q.
// The gated step (dflash2_select_gated) launches k_chunk_gate in place of stage 1 (the
// same blocks plus the context gate's tiles as extra work-groups), and its stage 2
// adds each row's gate slices before the scores.
// Kernel boundaries replace every cross-work-group hand-off, so no work-group ever
// waits for another and no workspace counter exists.
#include "dflash2_internal.h"
#include "gate_dev.h"
#include "pair_dev.h"
#include "topk_dev.h"

namespace df2 {

constexpr int kMergeRows = 16;                    // rows per block of the standalone top-16 merge

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

__global__ void __launch_bounds__(kTopkThreads) k_chunk_lists(const uint16_t* __restrict__ logits, int64_t ld, int V,
                                                              int nchunks, unsigned long long* __restrict__ partials) {
  __shared__ ChunkShared sm;
  const int row = blockIdx.x / nchunks;
  const int chunk = blockIdx.x - row * nchunks;
  chunk_top16(logits + (size_t)row * ld, V, chunk_begin(V, nchunks, chunk), chunk_begin(V, nchunks, chunk + 1), sm,
              partials + ((size_t)row * nchunks + chunk) * kNC);
}

// ---- stage 1 of the gated select: chunk top-16s and gate tiles in one launch ---------
// Blocks [0, nchunk_blocks) stream the logits as k_chunk_lists does; the rest compute
// the context gate's partial sums (gate_dev.h tiles, 8 waves) on the compute units the
// stream leaves idle or shares.

union ChunkGateShared {
  ChunkShared c;
  float red[kTopkWaves * 16 * kFusedGateCols];
};

__global__ void __launch_bounds__(kTopkThreads) k_chunk_gate(const uint16_t* __restrict__ logits, int64_t ld, int V,
                                                             int nchunks, int nchunk_blocks,
                                                             unsigned long long* __restrict__ partials,
                                                             const float* __restrict__ h,
                                                             const uint16_t* __restrict__ w_h, int rows, int hidden,
                                                             int dim, int ntiles, int nsplit,
                                                             float* __restrict__ gate_partial) {
  __shared__ ChunkGateShared sm;
  if ((int)blockIdx.x < nchunk_blocks) {
    const int row = blockIdx.x / nchunks;
    const int chunk = blockIdx.x - row * nchunks;
    chunk_top16(logits + (size_t)row * ld, V, chunk_begin(V, nchunks, chunk), chunk_begin(V, nchunks, chunk + 1), sm.c,
                partials + ((size_t)row * nchunks + chunk) * kNC);
    return;
  }
  const int gb = (int)blockIdx.x - nchunk_blocks;
  const int per = ntiles * nsplit;
  const int mt = gb / per;
  const int rem = gb - mt * per;
  const int nt = rem / nsplit;
  const int split = rem - nt * nsplit;
  gate_tile<kFusedGateCols / 16, kTopkWaves, kFusedGateSteps>(h, w_h, nullptr, rows, hidden, dim, 0, mt, nt, split,
                                                              nsplit, sm.red, nullptr, gate_partial);
}

// ---- top-16: merge each row's chunk top-16s (one 16-lane row per logits row) ----------

__global__ void __launch_bounds__(kMergeRows * kNC) k_merge_lists(const unsigned long long* __restrict__ partials,
                                                                  int rows, int nchunks,
                                                                  int32_t* __restrict__ cand_idx,
                                                                  float* __restrict__ cand_val,
                                                                  int32_t* __restrict__ row_status) {
  const int i = threadIdx.x & 15;
  const int row_raw = blockIdx.x * kMergeRows + (threadIdx.x >> 4);
  const int row = row_raw < rows ? row_raw : rows - 1;   // spare lanes redo the last row, every lane merges
  const unsigned long long rc = row16_merge_chunks(partials + (size_t)row * nchunks * kNC, nchunks);
  const float v = bf16_to_f32(rc_bits(rc));
  const unsigned long long bad = __ballot(!__builtin_isfinite(v));
  if (row_raw < rows) {
    cand_idx[(size_t)row * kNC + i] = rc ? rc_id(rc) : 0;
    cand_val[(size_t)row * kNC + i] = v;
    const int sh = (threadIdx.x & 63) & ~15;
    if (row_status && i == 0) row_status[row] = ((bad >> sh) & 0xffffull) ? 1 : 0;
  }
}

// ---- pair scores ------------------------------------------------------------------------

template <int DIM, bool BF16>
__global__ void __launch_bounds__(kPairThreads) k_pair_score(const int32_t* __restrict__ cand_idx,
                                                             const float* __restrict__ cand_val,
                                                             const int32_t* __restrict__ verified,
                                                             const void* __restrict__ emb_a,
                                                             const void* __restrict__ emb_b, int V,
                                                             const float* __restrict__ H, int K, float* __restrict__ S,
                                                             int32_t* __restrict__ row_status) {
  __shared__ PairShared sm;
  const int pos = blockIdx.x;
  const int b = pos / K, p = pos - b * K;
  const int tid = threadIdx.x;
  if (tid < kNC) {
    sm.prev[tid] = p == 0 ? verified[b] : cand_idx[((size_t)pos - 1) * kNC + tid];
    sm.cur[tid] = cand_idx[(size_t)pos * kNC + tid];
    sm.U[tid] = cand_val[(size_t)pos * kNC + tid];
  }
  __syncthreads();
  const int bits = pair_tile<DIM, BF16>(emb_a, emb_b, V, H + (size_t)pos * DIM, S + (size_t)pos * kNC * kNC, sm);
  if (row_status && tid == 0) row_status[pos] = bits;
}

// ---- walk ------------------------------------------------------------------------------

// From scores alone: position by position, build the successor table, follow it from
// the slot taken at the previous position, and emit that row's distribution.
__global__ void __launch_bounds__(256) k_walk(const float* __restrict__ S, const int32_t* __restrict__ cand_idx, int K,
                                              float inv_t, uint64_t seed, int32_t* __restrict__ tokens,
                                              int32_t* __restrict__ slots, float* __restrict__ q) {
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

// From the successor tables stage 2 built: next[t][i] (slot taken at t after slot i at
// t - 1) and, when sampling, qtab[t][i][.] (that row's distribution).
__global__ void __launch_bounds__(256) k_walk_tables(const int* __restrict__ next, const float* __restrict__ qtab,
                                                     const int32_t* __restrict__ cand_idx, int K, bool sampled,
                                                     int32_t* __restrict__ tokens, int32_t* __restrict__ slots,
                                                     float* __restrict__ q) {
  __shared__ WalkShared sm;
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const size_t base = (size_t)b * K * kNC;
  for (int e = tid; e < K * kNC; e += blockDim.x) {
    sm.next[e] = next[base + e];
    sm.tok[e] = cand_idx[base + e];
  }
  __syncthreads();
  if (tid == 0) {
    int i = 0;
    for (int t = 0; t < K; ++t) {
      i = sm.next[t * kNC + i];
      sm.path[t] = i;
    }
  }
  __syncthreads();
  for (int e = tid; e < K * kNC; e += blockDim.x) {
    const int t = e >> 4, j = e & 15;
    const int from = t == 0 ? 0 : sm.path[t - 1];
    q[base + e] = sampled ? qtab[(base + (size_t)t * kNC + from) * kNC + j] : (j == sm.path[t] ? 1.f : 0.f);
    if (j == 0) {
      slots[(size_t)b * K + t] = sm.path[t];
      tokens[(size_t)b * K + t] = sm.tok[t * kNC + sm.path[t]];
    }
  }
}

// ---- stage 2 of the proposer step -------------------------------------------------------

// GATED: H is not given; the block adds its row's gate slices (gate_partial, nsplit of
// them) in slice order, applies the bias and the activation, keeps the row in LDS and
// writes it to H_out when given.
template <int DIM, bool BF16, bool GATED>
__global__ void __launch_bounds__(kPairThreads) k_positions(const unsigned long long* __restrict__ partials,
                                                            int nchunks, int K, const int32_t* __restrict__ verified,
                                                            const void* __restrict__ emb_a,
                                                            const void* __restrict__ emb_b, int V,
                                                            const float* __restrict__ H,
                                                            const float* __restrict__ gate_partial,
                                                            const float* __restrict__ gate_bias, int gate_nsplit,
                                                            int gate_act_id, float* __restrict__ H_out, float inv_t,
                                                            uint64_t seed,
                                                            int32_t* __restrict__ cand_idx,
                                                            float* __restrict__ cand_val, float* __restrict__ S,
                                                            int* __restrict__ next, float* __restrict__ qtab,
                                                            int32_t* __restrict__ row_status) {
  __shared__ PairShared ps;
  __shared__ int s_bits;
  __shared__ float s_H[GATED ? DIM : 1];
  const int pos = blockIdx.x;
  const int b = pos / K, p = pos - b * K;
  const int tid = threadIdx.x;
  if constexpr (GATED) {
    const int rows = (int)gridDim.x;
    for (int d = tid; d < DIM; d += kPairThreads) {
      const float v = gate_finish(gate_partial, gate_bias, rows, DIM, gate_nsplit, gate_act_id, pos, d);
      s_H[d] = v;
      if (H_out) H_out[(size_t)pos * DIM + d] = v;
    }
  }
  if (tid < kWave) {
    // rows 0 and 2 of wave 0 merge row pos, rows 1 and 3 row pos - 1 (the predecessors)
    const int i = tid & 15;
    const bool pred = (tid & 16) != 0;
    const int r = pred && p > 0 ? pos - 1 : pos;
    const unsigned long long rc = row16_merge_chunks(partials + (size_t)r * nchunks * kNC, nchunks);
    const float v = bf16_to_f32(rc_bits(rc));
    const bool bad = __ballot(tid < kNC && !__builtin_isfinite(v)) != 0ull;
    if (tid < kNC) {
      cand_idx[(size_t)pos * kNC + i] = rc ? rc_id(rc) : 0;
      cand_val[(size_t)pos * kNC + i] = v;
      ps.cur[i] = rc ? rc_id(rc) : 0;
      ps.U[i] = v;
    } else if (tid < 2 * kNC) {
      ps.prev[i] = p == 0 ? verified[b] : (rc ? rc_id(rc) : 0);
    }
    if (tid == 0) s_bits = bad ? 1 : 0;
  }
  __syncthreads();
  const float* Hrow = GATED ? s_H : H + (size_t)pos * DIM;
  const int pbits = pair_tile<DIM, BF16>(emb_a, emb_b, V, Hrow, S + (size_t)pos * kNC * kNC, ps);
  const float u = inv_t == 0.f ? 0.f : walk_uniform(seed, (uint32_t)b, (uint32_t)p);
  tile_successors(ps, inv_t, u, next + (size_t)pos * kNC, inv_t == 0.f ? nullptr : qtab + (size_t)pos * kNC * kNC);
  if (row_status && tid == 0) row_status[pos] = s_bits | pbits;
}

// ---- launchers -----------------------------------------------------------------------

hipError_t launch_topk16(const uint16_t* logits, int rows, int vocab, int64_t ld, int32_t* cand_idx, float* cand_val,
                         int32_t* row_status, TopkWs ws, hipStream_t s) {
  const int nchunks = topk_num_chunks(vocab);
  hipLaunchKernelGGL(k_chunk_lists, dim3((unsigned)(rows * nchunks)), dim3(kTopkThreads), 0, s, logits, ld, vocab,
                     nchunks, ws.partials);
  hipLaunchKernelGGL(k_merge_lists, dim3((unsigned)((rows + kMergeRows - 1) / kMergeRows)), dim3(kMergeRows * kNC),
                     0, s, ws.partials, rows, nchunks, cand_idx, cand_val, row_status);
  return hipGetLastError();
}

template <int DIM, bool BF16>
static void pair_launch(dim3 grid, hipStream_t s, const int32_t* cand_idx, const float* cand_val,
                        const int32_t* verified, const void* a, const void* b, int V, const float* H, int K, float* S,
                        int32_t* st) {
  hipLaunchKernelGGL((k_pair_score<DIM, BF16>), grid, dim3(kPairThreads), 0, s, cand_idx, cand_val, verified, a, b, V,
                     H, K, S, st);
}

hipError_t launch_pair_score(const int32_t* cand_idx, const float* cand_val, const int32_t* verified, const void* emb_a,
                             const void* emb_b, bool bf16, int vocab, int dim, const float* H, int batch, int K,
                             float* S, int32_t* row_status, hipStream_t s) {
  const dim3 grid((unsigned)(batch * K));
#define DF2_PAIR(D)                                                                                           \
  case D:                                                                                                     \
    if (bf16)                                                                                                 \
      pair_launch<D, true>(grid, s, cand_idx, cand_val, verified, emb_a, emb_b, vocab, H, K, S, row_status);  \
    else                                                                                                      \
      pair_launch<D, false>(grid, s, cand_idx, cand_val, verified, emb_a, emb_b, vocab, H, K, S, row_status); \
    break;
  switch (dim) {
    DF2_PAIR(64)
    DF2_PAIR(128)
    DF2_PAIR(256)
    DF2_PAIR(512)
    default:
      return hipErrorInvalidValue;
  }
#undef DF2_PAIR
  return hipGetLastError();
}

hipError_t launch_walk(const float* S, const int32_t* cand_idx, int batch, int K, float temperature, uint64_t seed,
                       int32_t* tokens, int32_t* slots, float* q, hipStream_t s) {
  const float inv_t = temperature == 0.f ? 0.f : 1.f / temperature;
  hipLaunchKernelGGL(k_walk, dim3((unsigned)batch), dim3(256), 0, s, S, cand_idx, K, inv_t, seed, tokens, slots, q);
  return hipGetLastError();
}

struct GateArgs {
  const float* partial = nullptr;
  const float* bias = nullptr;
  int nsplit = 0;
  int act = 0;
  float* H_out = nullptr;
};

template <int DIM, bool BF16, bool GATED>
static void positions_launch(dim3 grid, hipStream_t s, const unsigned long long* partials, int nchunks, int K,
                             const int32_t* verified, const void* a, const void* b, int V, const float* H,
                             const GateArgs& ga, float inv_t, uint64_t seed, int32_t* ci, float* cv, float* S,
                             int* next, float* qtab, int32_t* st) {
  hipLaunchKernelGGL((k_positions<DIM, BF16, GATED>), grid, dim3(kPairThreads), 0, s, partials, nchunks, K, verified,
                     a, b, V, H, ga.partial, ga.bias, ga.nsplit, ga.act, ga.H_out, inv_t, seed, ci, cv, S, next,
                     qtab, st);
}

// Stages 2 and 3 of the select (stage 1 has filled ws.topk.partials).
template <bool GATED>
static hipError_t select_tail(const uint16_t* /*logits*/, int nchunks, const int32_t* verified, const void* emb_a,
                              const void* emb_b, bool bf16, int vocab, int dim, const float* H, const GateArgs& ga,
                              int batch, int K, float inv_t, uint64_t seed, int32_t* cand_idx, float* cand_val,
                              float* S, int32_t* tokens, int32_t* slots, float* q, int32_t* row_status,
                              const SelectWs& ws, hipStream_t s) {
  const dim3 grid((unsigned)(batch * K));
#define DF2_POS(D)                                                                                                   \
  case D:                                                                                                            \
    if (bf16)                                                                                                        \
      positions_launch<D, true, GATED>(grid, s, ws.topk.partials, nchunks, K, verified, emb_a, emb_b, vocab, H, ga,  \
                                       inv_t, seed, cand_idx, cand_val, S, ws.next, ws.qtab, row_status);            \
    else                                                                                                             \
      positions_launch<D, false, GATED>(grid, s, ws.topk.partials, nchunks, K, verified, emb_a, emb_b, vocab, H, ga, \
                                        inv_t, seed, cand_idx, cand_val, S, ws.next, ws.qtab, row_status);           \
    break;
  switch (dim) {
    DF2_POS(64)
    DF2_POS(128)
    DF2_POS(256)
    DF2_POS(512)
    default:
      return hipErrorInvalidValue;
  }
#undef DF2_POS
  hipLaunchKernelGGL(k_walk_tables, dim3((unsigned)batch), dim3(256), 0, s, ws.next, ws.qtab, cand_idx, K,
                     inv_t != 0.f, tokens, slots, q);
  return hipGetLastError();
}

hipError_t launch_select(const uint16_t* logits, int64_t ld, const int32_t* verified, const void* emb_a,
                         const void* emb_b, bool bf16, int vocab, int dim, const float* H, int batch, int K,
                         float temperature, uint64_t seed, int32_t* cand_idx, float* cand_val, float* S,
                         int32_t* tokens, int32_t* slots, float* q, int32_t* row_status, SelectWs ws, hipStream_t s) {
  const int nchunks = topk_num_chunks(vocab);
  const float inv_t = temperature == 0.f ? 0.f : 1.f / temperature;
  hipLaunchKernelGGL(k_chunk_lists, dim3((unsigned)(batch * K * nchunks)), dim3(kTopkThreads), 0, s, logits, ld, vocab,
                     nchunks, ws.topk.partials);
  return select_tail<false>(logits, nchunks, verified, emb_a, emb_b, bf16, vocab, dim, H, GateArgs{}, batch, K, inv_t,
                            seed, cand_idx, cand_val, S, tokens, slots, q, row_status, ws, s);
}

hipError_t launch_select_gated(const uint16_t* logits, int64_t ld, const int32_t* verified, const void* emb_a,
                               const void* emb_b, bool bf16, int vocab, int dim, const float* h,
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
  hipLaunchKernelGGL(k_chunk_gate, dim3((unsigned)blocks), dim3(kTopkThreads), 0, s, logits, ld, vocab, nchunks,
                     nchunk_blocks, ws.sel.topk.partials, h, w_h, rows, hidden, dim, ntiles, ws.nsplit, ws.partial);
  GateArgs ga;
  ga.partial = ws.partial;
  ga.bias = bias;
  ga.nsplit = ws.nsplit;
  ga.act = act;
  ga.H_out = H_out;
  return select_tail<true>(logits, nchunks, verified, emb_a, emb_b, bf16, vocab, dim, nullptr, ga, batch, K, inv_t,
                           seed, cand_idx, cand_val, S, tokens, slots, q, row_status, ws.sel, s);
}

}  // namespace df2
