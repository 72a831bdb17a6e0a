// Internal interface between the C-ABI entry points and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace df2 {

// Carves aligned sub-buffers out of a caller workspace (or only sizes them when the
// base is null).
struct Carver {
  char* base;
  size_t off = 0;
  explicit Carver(void* b) : base(static_cast<char*>(b)) {}
  template <typename T>
  T* take(size_t count) {
    off = (off + 255) & ~size_t(255);
    T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
    off += count * sizeof(T);
    return p;
  }
};

struct TopkWs {
  unsigned long long* partials;   // [rows][nchunks][16] chunk top-16s, best first
};
TopkWs carve_topk(Carver& c, int64_t rows, int64_t vocab);

struct SelectWs {
  TopkWs topk;
  int* next;                      // [rows][16] successor slot per predecessor slot
  float* qtab;                    // [rows][16][16] distribution of each predecessor's row
  unsigned* tickets;              // [batch] x kWalkTicketStride: positions built per request
};
constexpr int kWalkTicketStride = 64;   // 256 bytes apart: concurrent atomics on one line serialise
SelectWs carve_select(Carver& c, int64_t batch, int64_t K, int64_t vocab);

struct SelectGatedWs {
  SelectWs sel;
  float* partial;                 // [nsplit][rows][dim] gate partial sums
  int nsplit;
};
SelectGatedWs carve_select_gated(Carver& c, int64_t batch, int64_t K, int64_t vocab, int64_t hidden, int64_t dim);
int64_t fused_gate_blocks(int64_t rows, int64_t hidden, int64_t dim);

struct LmheadWs {
  unsigned long long* partials;   // [rows][tiles][16] per 256-column tile top-16s, best first
  unsigned char* tail;            // fp32 partial tiles of a split last round
  size_t tail_bytes;
};
constexpr int kLmMaxRows = 128;   // rows per LM-head tile launch (eight 16-row MFMA tiles)
int lmhead_tiles(int64_t vocab);
LmheadWs carve_lmhead(Carver& c, int64_t rows, int64_t vocab);

struct RingWs {
  float* ml;                      // [batch][hkv][nsplit][rows_pad][2] per-split row max (log2 units) and sum
  float* o;                       // [batch][hkv][nsplit][rows_pad][128] per-split unnormalised outputs
};
constexpr int kRingMaxRows = 48;  // query rows (block positions x query heads per K/V head)
int ring_rows_pad(int nq, int hq, int hkv);
int ring_splits(int64_t batch, int64_t hkv, int nq, int hq, int window);
RingWs carve_ring(Carver& c, int64_t batch, int64_t hkv, int nsplit, int rows_pad);

struct GateWs {
  float* partial;                 // [nsplit][rows][dim] slice sums (nsplit > 1)
  int nsplit;                     // slices of the hidden dimension
};
int gate_splits(int64_t rows, int64_t hidden, int64_t dim);
bool gate_wide(int64_t rows, int64_t hidden, int64_t dim);        // wide gate tiles (bf16 weight)
int gate_wide_parts(int64_t rows, int64_t hidden, int64_t dim);
GateWs carve_gate(Carver& c, int64_t rows, int64_t hidden, int64_t dim);
constexpr int kGateBlockThreads = 512;    // threads of a standalone gate work-group
int64_t gate_grid_blocks(int64_t rows, int64_t hidden, int64_t dim);

struct AcceptWs {
  float* chunk_max;               // [nrows][8 * nchunks] sub-chunk max; NaN: non-finite
  float* chunk_sum;               // [nrows][8 * nchunks] sub-chunk sum of weights
  unsigned long long* chunk_arg;  // [nrows][nchunks] (greedy)
};
AcceptWs carve_accept(Carver& c, int64_t nrows, int64_t vocab);

hipError_t launch_topk16(const uint16_t* logits, int rows, int vocab, int64_t ld, int32_t* cand_idx,
                         float* cand_val, int32_t* row_status, TopkWs ws, hipStream_t s);

hipError_t launch_pair_score(const int32_t* cand_idx, const float* cand_val, const int32_t* verified,
                             const void* emb_a, const void* emb_b, bool bf16, int vocab, int dim, const float* H,
                             int batch, int K, float* S, int32_t* row_status, hipStream_t s);

hipError_t launch_walk(const float* S, const int32_t* cand_idx, int batch, int K, float temperature,
                       uint64_t seed, int32_t* tokens, int32_t* slots, float* q, hipStream_t s);

hipError_t launch_select(const uint16_t* logits, int64_t ld, const int32_t* verified, const void* emb_a,
                         const void* emb_b, bool bf16, int vocab, int dim, const float* H, int batch, int K,
                         float temperature, uint64_t seed, int32_t* cand_idx, float* cand_val, float* S,
                         int32_t* tokens, int32_t* slots, float* q, int32_t* row_status, SelectWs ws,
                         hipStream_t s);

hipError_t launch_select_gated(const uint16_t* logits, int64_t ld, const int32_t* verified, const void* emb_a,
                               const void* emb_b, bool bf16, int vocab, int dim, const void* h, bool h_bf16,
                               const uint16_t* w_h, const float* bias, int hidden, int act, int batch, int K,
                               float temperature, uint64_t seed, float* H_out, int32_t* cand_idx, float* cand_val,
                               float* S, int32_t* tokens, int32_t* slots, float* q, int32_t* row_status,
                               SelectGatedWs ws, hipStream_t s);

size_t lmhead_packed_elems(int64_t vocab, int64_t hidden);
hipError_t launch_lmhead_pack(const uint16_t* w, int vocab, int hidden, uint16_t* w_packed, hipStream_t s);
hipError_t launch_lmhead_topk16(const uint16_t* h, const uint16_t* w, bool packed, int rows, int hidden, int vocab,
                                int32_t* cand_idx, float* cand_val, int32_t* row_status, LmheadWs ws,
                                hipStream_t s);

hipError_t launch_ring_attention(const uint16_t* q, const uint16_t* k_blk, const uint16_t* v_blk,
                                 const uint16_t* k_ring, const uint16_t* v_ring, const int32_t* ctx_len, int batch,
                                 int nq, int hq, int hkv, int ring, int window, float scale, int nsplit, RingWs ws,
                                 float* out, hipStream_t s);

hipError_t launch_gate(const void* h, bool h_bf16, const void* w_h, bool w_bf16, const float* bias, int rows,
                       int hidden, int dim, int act, float* H, GateWs ws, hipStream_t s);

hipError_t launch_conv2tap(const float* x, const float* x_prev, const float* taps, int64_t sites, int64_t batch,
                           int K, int64_t hidden, int64_t group, float* y, hipStream_t s);

hipError_t launch_spec_accept(const uint16_t* target, int64_t ld, int64_t batch_stride, const int32_t* tokens,
                              const int32_t* cand_idx, const float* q, int batch, int K, int vocab,
                              float temperature, uint64_t seed, int32_t* out_tokens, int32_t* n_accepted,
                              int32_t* row_status, AcceptWs ws, hipStream_t s);

}  // namespace df2
