// C-ABI entry points of libdflash2: argument checks (before any HIP call), workspace
// sizing, and dispatch to the kernel launchers.
#include <math.h>

#include <mutex>
#include <new>

#include "dflash2.h"
#include "dflash2_internal.h"
#include "filter.h"
#include "topk_dev.h"

using namespace df2;

// Scratch of dflash2_select_noalloc: one array per GPU, in the library's own device
// memory (resident from the code object's load on that GPU to the end of the process),
// shared by every call on that GPU.  Host code uses the address hipGetSymbolAddress
// gives for the current device, never the array's name.
constexpr size_t kNoallocScratchBytes = (size_t)4 << 20;
static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

namespace {

constexpr int64_t kMaxVocab = (int64_t)1 << 19;
static_assert((int64_t)kMaxChunks * kChunkVec * 8 >= kMaxVocab, "top-16 chunking must cover the vocabulary limit");
// An AQL dispatch packet carries the grid size as a 32-bit count of work-items.
constexpr int64_t kMaxItems = 0xffffffffLL;

bool items_ok(int64_t blocks, int64_t threads) { return blocks >= 1 && blocks <= kMaxItems / threads; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool pow2_in(int64_t v, int64_t lo, int64_t hi) { return v >= lo && v <= hi && (v & (v - 1)) == 0; }

dflash2_status hip_status(hipError_t e) { return e == hipSuccess ? DFLASH2_OK : DFLASH2_ERR_HIP; }

dflash2_status check_logits(const uint16_t* logits, int64_t rows, int64_t vocab, int64_t ld) {
  if (!logits) return DFLASH2_ERR_NULL;
  if (rows < 1 || vocab < DFLASH2_NCAND || vocab > kMaxVocab || ld < vocab) return DFLASH2_ERR_SHAPE;
  // the stream grids pad the rows (or requests) to a multiple of 8, one lane per XCD
  if (rows > kMaxItems || !items_ok((rows + 7) / 8 * 8 * topk_num_chunks(vocab), kTopkThreads)) return DFLASH2_ERR_SHAPE;
  if (!aligned16(logits) || (ld % 8) != 0) return DFLASH2_ERR_ALIGN;
  return DFLASH2_OK;
}

dflash2_status check_emb(const void* a, const void* b, dflash2_dtype dt, int64_t vocab, int64_t dim) {
  if (!a || !b) return DFLASH2_ERR_NULL;
  if (dt != DFLASH2_F32 && dt != DFLASH2_BF16) return DFLASH2_ERR_DTYPE;
  if (vocab < DFLASH2_NCAND || vocab > kMaxVocab) return DFLASH2_ERR_SHAPE;
  if (!pow2_in(dim, 16, 1024)) return DFLASH2_ERR_SHAPE;
  if (!aligned16(a) || !aligned16(b)) return DFLASH2_ERR_ALIGN;
  return DFLASH2_OK;
}

dflash2_status check_bk(int64_t batch, int64_t K) {
  if (batch < 1 || batch >= ((int64_t)1 << 31) || K < 1 || K > DFLASH2_MAX_K) return DFLASH2_ERR_SHAPE;
  if (!items_ok((batch + 7) / 8 * 8 * K, 256)) return DFLASH2_ERR_SHAPE;
  return DFLASH2_OK;
}

// A temperature is 0 (greedy) or a finite value of at least FLT_MIN (2^-126): the
// kernels scale scores by 1/T (and by log2(e)/T), which overflows to +inf for the
// subnormal temperatures below it.
dflash2_status check_temp(float t) {
  if (isnan(t) || isinf(t) || t < 0.f) return DFLASH2_ERR_VALUE;
  if (t > 0.f && t < 1.17549435e-38f) return DFLASH2_ERR_VALUE;
  return DFLASH2_OK;
}

// The argument checks of dflash2_select (and of its variant without workspace).
dflash2_status check_select(const uint16_t* logits, int64_t ld, const int32_t* verified, const void* emb_a,
                            const void* emb_b, dflash2_dtype emb_dtype, int64_t vocab, int64_t dim, const float* H,
                            int64_t batch, int64_t K, float temperature, const int32_t* cand_idx,
                            const float* cand_val, const float* S, const int32_t* tokens, const int32_t* slots,
                            const float* q) {
  dflash2_status st = check_bk(batch, K);
  if (st != DFLASH2_OK) return st;
  st = check_logits(logits, batch * K, vocab, ld);
  if (st != DFLASH2_OK) return st;
  if (!items_ok((batch + 7) / 8 * 8 * K * topk_num_chunks(vocab), kTopkThreads)) return DFLASH2_ERR_SHAPE;
  st = check_emb(emb_a, emb_b, emb_dtype, vocab, dim);
  if (st != DFLASH2_OK) return st;
  if (!verified || !H || !cand_idx || !cand_val || !S || !tokens || !slots || !q) return DFLASH2_ERR_NULL;
  if (!aligned16(H) || !aligned16(S)) return DFLASH2_ERR_ALIGN;
  return check_temp(temperature);
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_addr[kMaxDevices] = {};

// This GPU's scratch address, looked up on the first call on each device.
dflash2_status noalloc_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return DFLASH2_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_addr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return DFLASH2_ERR_HIP;
    g_scratch_addr[dev] = p;
  }
  *out = g_scratch_addr[dev];
  return DFLASH2_OK;
}

struct FilteredWs {
  AcceptWs acc;      // the greedy path (temperature 0)
  FilterWs filt;
};
FilteredWs carve_filtered(Carver& c, int64_t nrows, int64_t vocab) {
  FilteredWs w;
  w.acc = carve_accept(c, nrows, vocab);
  w.filt = carve_filter(c, nrows, vocab);
  return w;
}

template <typename WsT, typename F>
dflash2_status carve_checked(void* ws, size_t bytes, F&& carve, WsT* out) {
  Carver sizing(nullptr);
  carve(sizing);
  if (!ws) return DFLASH2_ERR_WORKSPACE;
  if (bytes < sizing.off) return DFLASH2_ERR_WORKSPACE;
  if (!aligned16(ws)) return DFLASH2_ERR_ALIGN;
  Carver c(ws);
  *out = carve(c);
  return DFLASH2_OK;
}

}  // namespace

extern "C" {

int dflash2_abi_version(void) { return DFLASH2_ABI_VERSION; }

const char* dflash2_status_str(int status) {
  switch (status) {
    case DFLASH2_OK: return "DFLASH2_OK";
    case DFLASH2_ERR_NULL: return "DFLASH2_ERR_NULL";
    case DFLASH2_ERR_SHAPE: return "DFLASH2_ERR_SHAPE";
    case DFLASH2_ERR_ALIGN: return "DFLASH2_ERR_ALIGN";
    case DFLASH2_ERR_DTYPE: return "DFLASH2_ERR_DTYPE";
    case DFLASH2_ERR_WORKSPACE: return "DFLASH2_ERR_WORKSPACE";
    case DFLASH2_ERR_VALUE: return "DFLASH2_ERR_VALUE";
    case DFLASH2_ERR_HIP: return "DFLASH2_ERR_HIP";
    default: return "DFLASH2_UNKNOWN_STATUS";
  }
}

size_t dflash2_topk16_workspace(int64_t rows, int64_t vocab) {
  if (rows < 1 || vocab < 1) return 0;
  Carver c(nullptr);
  carve_topk(c, rows, vocab);
  return c.off + 256;
}

dflash2_status dflash2_topk16(const uint16_t* logits, int64_t rows, int64_t vocab, int64_t ld, int32_t* cand_idx,
                              float* cand_val, int32_t* row_status, void* workspace, size_t workspace_bytes,
                              hipStream_t stream) {
  dflash2_status st = check_logits(logits, rows, vocab, ld);
  if (st != DFLASH2_OK) return st;
  if (!cand_idx || !cand_val) return DFLASH2_ERR_NULL;
  TopkWs ws;
  st = carve_checked(workspace, workspace_bytes, [&](Carver& c) { return carve_topk(c, rows, vocab); }, &ws);
  if (st != DFLASH2_OK) return st;
  return hip_status(launch_topk16(logits, (int)rows, (int)vocab, ld, cand_idx, cand_val, row_status, ws, stream));
}

size_t dflash2_lmhead_topk16_workspace(int64_t rows, int64_t vocab) {
  if (rows < 1 || vocab < 1) return 0;
  Carver c(nullptr);
  carve_lmhead(c, rows, vocab);
  return c.off + 256;
}

dflash2_status dflash2_lmhead_topk16(const uint16_t* h, const uint16_t* w, int64_t rows, int64_t hidden,
                                     int64_t vocab, int32_t* cand_idx, float* cand_val, int32_t* row_status,
                                     void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!h || !w || !cand_idx || !cand_val) return DFLASH2_ERR_NULL;
  if (rows < 1 || rows > kMaxItems / 1024 || hidden < 256 || hidden % 256 != 0 || hidden > ((int64_t)1 << 20) ||
      vocab < DFLASH2_NCAND || vocab > kMaxVocab)
    return DFLASH2_ERR_SHAPE;
  if (!aligned16(h) || !aligned16(w)) return DFLASH2_ERR_ALIGN;
  LmheadWs ws;
  dflash2_status st =
      carve_checked(workspace, workspace_bytes, [&](Carver& c) { return carve_lmhead(c, rows, vocab); }, &ws);
  if (st != DFLASH2_OK) return st;
  return hip_status(launch_lmhead_topk16(h, w, false, (int)rows, (int)hidden, (int)vocab, cand_idx, cand_val,
                                         row_status, ws, stream));
}

size_t dflash2_lmhead_packed_bytes(int64_t vocab, int64_t hidden) {
  if (vocab < DFLASH2_NCAND || vocab > kMaxVocab || hidden < 256 || hidden % 256 != 0 || hidden > ((int64_t)1 << 20))
    return 0;
  return lmhead_packed_elems(vocab, hidden) * sizeof(uint16_t);
}

dflash2_status dflash2_lmhead_pack(const uint16_t* w, int64_t vocab, int64_t hidden, uint16_t* w_packed,
                                   hipStream_t stream) {
  if (!w || !w_packed) return DFLASH2_ERR_NULL;
  if (vocab < DFLASH2_NCAND || vocab > kMaxVocab || hidden < 256 || hidden % 256 != 0 || hidden > ((int64_t)1 << 20))
    return DFLASH2_ERR_SHAPE;
  if (!aligned16(w) || !aligned16(w_packed)) return DFLASH2_ERR_ALIGN;
  return hip_status(launch_lmhead_pack(w, (int)vocab, (int)hidden, w_packed, stream));
}

dflash2_status dflash2_lmhead_topk16_packed(const uint16_t* h, const uint16_t* w_packed, int64_t rows,
                                            int64_t hidden, int64_t vocab, int32_t* cand_idx, float* cand_val,
                                            int32_t* row_status, void* workspace, size_t workspace_bytes,
                                            hipStream_t stream) {
  if (!h || !w_packed || !cand_idx || !cand_val) return DFLASH2_ERR_NULL;
  if (rows < 1 || rows > kMaxItems / 1024 || hidden < 256 || hidden % 256 != 0 || hidden > ((int64_t)1 << 20) ||
      vocab < DFLASH2_NCAND || vocab > kMaxVocab)
    return DFLASH2_ERR_SHAPE;
  if (!aligned16(h) || !aligned16(w_packed)) return DFLASH2_ERR_ALIGN;
  LmheadWs ws;
  dflash2_status st =
      carve_checked(workspace, workspace_bytes, [&](Carver& c) { return carve_lmhead(c, rows, vocab); }, &ws);
  if (st != DFLASH2_OK) return st;
  return hip_status(launch_lmhead_topk16(h, w_packed, true, (int)rows, (int)hidden, (int)vocab, cand_idx, cand_val,
                                         row_status, ws, stream));
}

size_t dflash2_ring_attention_workspace(int64_t batch, int64_t nq, int64_t hq, int64_t hkv, int64_t window) {
  if (batch < 1 || batch > (1 << 20) || nq < 1 || nq > 128 || hkv < 1 || hq < hkv || hq % hkv != 0 || window < 1 ||
      window > (1 << 24))
    return 0;
  Carver c(nullptr);
  carve_ring(c, batch, hkv, ring_splits(batch, hkv, (int)nq, (int)hq, (int)window), ring_rows_pad((int)nq, (int)hq, (int)hkv));
  return c.off + 256;
}

dflash2_status dflash2_ring_attention(const uint16_t* q, const uint16_t* k_blk, const uint16_t* v_blk,
                                      const uint16_t* k_ring, const uint16_t* v_ring, const int32_t* ctx_len,
                                      int64_t batch, int64_t nq, int64_t hq, int64_t hkv, int64_t head_dim,
                                      int64_t ring, int64_t window, float scale, float* out, void* workspace,
                                      size_t workspace_bytes, hipStream_t stream) {
  if (!q || !k_blk || !v_blk || !k_ring || !v_ring || !ctx_len || !out) return DFLASH2_ERR_NULL;
  if (batch < 1 || batch > (1 << 20) || nq < 1 || hkv < 1 || hq < hkv || hq % hkv != 0 || head_dim != 128 ||
      nq * (hq / hkv) > kRingMaxRows || nq > 128 || ring < 32 || ring % 32 != 0 || ring > (1 << 24) || window < 1 ||
      window > ring)
    return DFLASH2_ERR_SHAPE;
  if (isnan(scale) || isinf(scale) || scale < 0.f) return DFLASH2_ERR_VALUE;
  if (!aligned16(q) || !aligned16(k_blk) || !aligned16(v_blk) || !aligned16(k_ring) || !aligned16(v_ring) ||
      !aligned16(out))
    return DFLASH2_ERR_ALIGN;
  const int nsplit = ring_splits(batch, hkv, (int)nq, (int)hq, (int)window);
  const int rows_pad = ring_rows_pad((int)nq, (int)hq, (int)hkv);
  RingWs ws;
  dflash2_status st = carve_checked(
      workspace, workspace_bytes, [&](Carver& c) { return carve_ring(c, batch, hkv, nsplit, rows_pad); }, &ws);
  if (st != DFLASH2_OK) return st;
  const float sc = scale > 0.f ? scale : 1.f / sqrtf((float)head_dim);
  return hip_status(launch_ring_attention(q, k_blk, v_blk, k_ring, v_ring, ctx_len, (int)batch, (int)nq, (int)hq,
                                          (int)hkv, (int)ring, (int)window, sc, nsplit, ws, out, stream));
}

size_t dflash2_context_gate_workspace(int64_t rows, int64_t hidden, int64_t dim) {
  if (rows < 1 || hidden < 1 || dim < 1) return 0;
  Carver c(nullptr);
  carve_gate(c, rows, hidden, dim);
  return c.off + 256;
}

dflash2_status dflash2_context_gate(const void* h, dflash2_dtype h_dtype, const void* w_h, dflash2_dtype w_dtype,
                                    const float* bias, int64_t rows, int64_t hidden, int64_t dim, dflash2_gate_act act,
                                    float* H, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!h || !w_h || !H) return DFLASH2_ERR_NULL;
  if (h_dtype != DFLASH2_F32 && h_dtype != DFLASH2_BF16) return DFLASH2_ERR_DTYPE;
  if (w_dtype != DFLASH2_F32 && w_dtype != DFLASH2_BF16) return DFLASH2_ERR_DTYPE;
  if (act != DFLASH2_GATE_SIGMOID && act != DFLASH2_GATE_IDENTITY) return DFLASH2_ERR_DTYPE;
  if (rows < 1 || rows > ((int64_t)1 << 30) || hidden < 8 || hidden % 8 != 0 || hidden > ((int64_t)1 << 24) ||
      !pow2_in(dim, 16, 1024))
    return DFLASH2_ERR_SHAPE;
  if (!items_ok((rows * dim + 255) / 256, 256) || !items_ok(gate_grid_blocks(rows, hidden, dim), kGateBlockThreads))
    return DFLASH2_ERR_SHAPE;
  if (!aligned16(h) || !aligned16(w_h)) return DFLASH2_ERR_ALIGN;
  GateWs ws;
  dflash2_status st =
      carve_checked(workspace, workspace_bytes, [&](Carver& c) { return carve_gate(c, rows, hidden, dim); }, &ws);
  if (st != DFLASH2_OK) return st;
  return hip_status(launch_gate(h, h_dtype == DFLASH2_BF16, w_h, w_dtype == DFLASH2_BF16, bias, (int)rows,
                                (int)hidden, (int)dim, (int)act, H, ws, stream));
}

dflash2_status dflash2_pair_score(const int32_t* cand_idx, const float* cand_val, const int32_t* verified,
                                  const void* emb_a, const void* emb_b, dflash2_dtype emb_dtype, int64_t vocab,
                                  int64_t dim, const float* H, int64_t batch, int64_t K, float* S, int32_t* row_status,
                                  hipStream_t stream) {
  if (!cand_idx || !cand_val || !verified || !H || !S) return DFLASH2_ERR_NULL;
  dflash2_status st = check_emb(emb_a, emb_b, emb_dtype, vocab, dim);
  if (st != DFLASH2_OK) return st;
  st = check_bk(batch, K);
  if (st != DFLASH2_OK) return st;
  if (!aligned16(H)) return DFLASH2_ERR_ALIGN;
  return hip_status(launch_pair_score(cand_idx, cand_val, verified, emb_a, emb_b, emb_dtype == DFLASH2_BF16, (int)vocab,
                                      (int)dim, H, (int)batch, (int)K, S, row_status, stream));
}

dflash2_status dflash2_walk(const float* S, const int32_t* cand_idx, int64_t batch, int64_t K, float temperature,
                            uint64_t seed, int32_t* tokens, int32_t* slots, float* q, hipStream_t stream) {
  if (!S || !cand_idx || !tokens || !slots || !q) return DFLASH2_ERR_NULL;
  dflash2_status st = check_bk(batch, K);
  if (st != DFLASH2_OK) return st;
  st = check_temp(temperature);
  if (st != DFLASH2_OK) return st;
  return hip_status(launch_walk(S, cand_idx, (int)batch, (int)K, temperature, seed, tokens, slots, q, stream));
}

size_t dflash2_select_workspace(int64_t batch, int64_t K, int64_t vocab) {
  if (batch < 1 || K < 1 || vocab < 1) return 0;
  Carver c(nullptr);
  carve_select(c, batch, K, vocab);
  return c.off + 256;
}

dflash2_status dflash2_select(const uint16_t* logits, int64_t ld, const int32_t* verified, const void* emb_a,
                              const void* emb_b, dflash2_dtype emb_dtype, int64_t vocab, int64_t dim, const float* H,
                              int64_t batch, int64_t K, float temperature, uint64_t seed, int32_t* cand_idx,
                              float* cand_val, float* S, int32_t* tokens, int32_t* slots, float* q,
                              int32_t* row_status, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  dflash2_status st = check_select(logits, ld, verified, emb_a, emb_b, emb_dtype, vocab, dim, H, batch, K, temperature,
                                   cand_idx, cand_val, S, tokens, slots, q);
  if (st != DFLASH2_OK) return st;
  SelectWs ws;
  st = carve_checked(workspace, workspace_bytes, [&](Carver& c) { return carve_select(c, batch, K, vocab); }, &ws);
  if (st != DFLASH2_OK) return st;
  return hip_status(launch_select(logits, ld, verified, emb_a, emb_b, emb_dtype == DFLASH2_BF16, (int)vocab, (int)dim,
                                  H, (int)batch, (int)K, temperature, seed, cand_idx, cand_val, S, tokens, slots, q,
                                  row_status, ws, stream));
}

dflash2_status dflash2_select_noalloc(const uint16_t* logits, int64_t ld, const int32_t* verified, const void* emb_a,
                                      const void* emb_b, dflash2_dtype emb_dtype, int64_t vocab, int64_t dim,
                                      const float* H, int64_t batch, int64_t K, float temperature, uint64_t seed,
                                      int32_t* cand_idx, float* cand_val, float* S, int32_t* tokens, int32_t* slots,
                                      float* q, int32_t* row_status, hipStream_t stream) {
  dflash2_status st = check_select(logits, ld, verified, emb_a, emb_b, emb_dtype, vocab, dim, H, batch, K, temperature,
                                   cand_idx, cand_val, S, tokens, slots, q);
  if (st != DFLASH2_OK) return st;
  const size_t need = dflash2_select_workspace(batch, K, vocab);
  if (need == 0 || need > kNoallocScratchBytes) return DFLASH2_ERR_WORKSPACE;
  void* ws_base = nullptr;
  st = noalloc_scratch(&ws_base);
  if (st != DFLASH2_OK) return st;
  Carver c(ws_base);
  const SelectWs ws = carve_select(c, batch, K, vocab);
  return hip_status(launch_select(logits, ld, verified, emb_a, emb_b, emb_dtype == DFLASH2_BF16, (int)vocab, (int)dim,
                                  H, (int)batch, (int)K, temperature, seed, cand_idx, cand_val, S, tokens, slots, q,
                                  row_status, ws, stream));
}

size_t dflash2_select_gated_workspace(int64_t batch, int64_t K, int64_t vocab, int64_t hidden, int64_t dim) {
  if (batch < 1 || K < 1 || vocab < 1 || hidden < 1 || dim < 1) return 0;
  Carver c(nullptr);
  carve_select_gated(c, batch, K, vocab, hidden, dim);
  return c.off + 256;
}

dflash2_status dflash2_select_gated(const uint16_t* logits, int64_t ld, const int32_t* verified, const void* emb_a,
                                    const void* emb_b, dflash2_dtype emb_dtype, int64_t vocab, int64_t dim,
                                    const void* h, dflash2_dtype h_dtype, const void* w_h, dflash2_dtype w_dtype,
                                    const float* bias, int64_t hidden, dflash2_gate_act act, int64_t batch, int64_t K,
                                    float temperature, uint64_t seed, float* H_out, int32_t* cand_idx,
                                    float* cand_val, float* S, int32_t* tokens, int32_t* slots, float* q,
                                    int32_t* row_status, void* workspace, size_t workspace_bytes,
                                    hipStream_t stream) {
  dflash2_status st = check_bk(batch, K);
  if (st != DFLASH2_OK) return st;
  st = check_logits(logits, batch * K, vocab, ld);
  if (st != DFLASH2_OK) return st;
  st = check_emb(emb_a, emb_b, emb_dtype, vocab, dim);
  if (st != DFLASH2_OK) return st;
  if (!verified || !h || !w_h || !cand_idx || !cand_val || !S || !tokens || !slots || !q) return DFLASH2_ERR_NULL;
  if (w_dtype != DFLASH2_BF16 || (h_dtype != DFLASH2_F32 && h_dtype != DFLASH2_BF16)) return DFLASH2_ERR_DTYPE;
  if (act != DFLASH2_GATE_SIGMOID && act != DFLASH2_GATE_IDENTITY) return DFLASH2_ERR_DTYPE;
  // the fused gate tiles are 64 columns wide
  if (dim < 64 || hidden < 8 || hidden % 8 != 0 || hidden > ((int64_t)1 << 24)) return DFLASH2_ERR_SHAPE;
  const int64_t rows = batch * K;
  if (!items_ok(rows * topk_num_chunks(vocab) + fused_gate_blocks(rows, hidden, dim), kTopkThreads))
    return DFLASH2_ERR_SHAPE;
  if (!aligned16(h) || !aligned16(w_h) || !aligned16(S) || (H_out && !aligned16(H_out))) return DFLASH2_ERR_ALIGN;
  st = check_temp(temperature);
  if (st != DFLASH2_OK) return st;
  SelectGatedWs ws;
  st = carve_checked(workspace, workspace_bytes,
                     [&](Carver& c) { return carve_select_gated(c, batch, K, vocab, hidden, dim); }, &ws);
  if (st != DFLASH2_OK) return st;
  return hip_status(launch_select_gated(logits, ld, verified, emb_a, emb_b, emb_dtype == DFLASH2_BF16, (int)vocab,
                                        (int)dim, h, h_dtype == DFLASH2_BF16, static_cast<const uint16_t*>(w_h), bias,
                                        (int)hidden, (int)act, (int)batch, (int)K, temperature, seed, H_out, cand_idx,
                                        cand_val, S, tokens, slots, q, row_status, ws, stream));
}

dflash2_status dflash2_conv2tap(const float* x, const float* x_prev, const float* taps, int64_t sites, int64_t batch,
                                int64_t K, int64_t hidden, int64_t group, float* y, hipStream_t stream) {
  if (!x || !x_prev || !taps || !y) return DFLASH2_ERR_NULL;
  if (sites < 1 || batch < 1 || K < 1 || K > DFLASH2_MAX_K || hidden < 1 || group < 1 || hidden % group != 0)
    return DFLASH2_ERR_SHAPE;
  if (sites > kMaxItems || batch > kMaxItems / sites) return DFLASH2_ERR_SHAPE;
  const int64_t rows = sites * batch * K;                 // one thread per channel and row at most
  if (rows > kMaxItems || hidden > (kMaxItems - 255) / rows) return DFLASH2_ERR_SHAPE;
  return hip_status(launch_conv2tap(x, x_prev, taps, sites, batch, (int)K, hidden, group, y, stream));
}

size_t dflash2_spec_accept_workspace(int64_t batch, int64_t K, int64_t vocab) {
  if (batch < 1 || K < 1 || vocab < 1) return 0;
  Carver c(nullptr);
  carve_accept(c, batch * (K + 1), vocab);
  return c.off + 256;
}

dflash2_status dflash2_spec_accept(const uint16_t* target_logits, int64_t ld, int64_t batch_stride,
                                   const int32_t* tokens, const int32_t* cand_idx, const float* q, int64_t batch,
                                   int64_t K, int64_t vocab, float temperature, uint64_t seed, int32_t* out_tokens,
                                   int32_t* n_accepted, int32_t* row_status, void* workspace, size_t workspace_bytes,
                                   hipStream_t stream) {
  dflash2_status st = check_bk(batch, K);
  if (st != DFLASH2_OK) return st;
  const int64_t nrows = batch_stride == 0 ? K + 1 : batch * (K + 1);
  st = check_logits(target_logits, nrows, vocab, ld);
  if (st != DFLASH2_OK) return st;
  if (batch_stride < 0 || (batch_stride > 0 && batch_stride < (K + 1) * ld)) return DFLASH2_ERR_SHAPE;
  if (batch_stride % 8 != 0) return DFLASH2_ERR_ALIGN;
  if (!items_ok(xcd_chunk_grid(batch, K + 1, topk_num_chunks(vocab)), kTopkThreads)) return DFLASH2_ERR_SHAPE;
  if (!tokens || !cand_idx || !out_tokens || !n_accepted) return DFLASH2_ERR_NULL;
  st = check_temp(temperature);
  if (st != DFLASH2_OK) return st;
  if (temperature > 0.f && !q) return DFLASH2_ERR_NULL;
  AcceptWs ws;
  st = carve_checked(workspace, workspace_bytes, [&](Carver& c) { return carve_accept(c, nrows, vocab); }, &ws);
  if (st != DFLASH2_OK) return st;
  return hip_status(launch_spec_accept(target_logits, ld, batch_stride, tokens, cand_idx, q, (int)batch, (int)K,
                                       (int)vocab, temperature, seed, out_tokens, n_accepted, row_status, ws, stream));
}

size_t dflash2_spec_accept_filtered_workspace(int64_t batch, int64_t K, int64_t vocab) {
  if (batch < 1 || K < 1 || vocab < 1) return 0;
  Carver c(nullptr);
  carve_filtered(c, batch * (K + 1), vocab);
  return c.off + 256;
}

dflash2_status dflash2_spec_accept_filtered(const uint16_t* target_logits, int64_t ld, int64_t batch_stride,
                                            const int32_t* tokens, const int32_t* cand_idx, const float* q,
                                            int64_t batch, int64_t K, int64_t vocab, float temperature,
                                            int32_t top_k, float top_p, uint64_t seed, int32_t* out_tokens,
                                            int32_t* n_accepted, int32_t* row_status, void* workspace,
                                            size_t workspace_bytes, hipStream_t stream) {
  dflash2_status st = check_bk(batch, K);
  if (st != DFLASH2_OK) return st;
  const int64_t nrows = batch_stride == 0 ? K + 1 : batch * (K + 1);
  st = check_logits(target_logits, nrows, vocab, ld);
  if (st != DFLASH2_OK) return st;
  if (batch_stride < 0 || (batch_stride > 0 && batch_stride < (K + 1) * ld)) return DFLASH2_ERR_SHAPE;
  if (batch_stride % 8 != 0) return DFLASH2_ERR_ALIGN;
  if (!items_ok(xcd_chunk_grid(batch, K + 1, topk_num_chunks(vocab)), kTopkThreads)) return DFLASH2_ERR_SHAPE;
  if (!tokens || !cand_idx || !out_tokens || !n_accepted) return DFLASH2_ERR_NULL;
  st = check_temp(temperature);
  if (st != DFLASH2_OK) return st;
  if (top_k < 1 || top_k > DFLASH2_MAX_TOPK || !(top_p > 0.f && top_p <= 1.f)) return DFLASH2_ERR_VALUE;
  if (temperature > 0.f && !q) return DFLASH2_ERR_NULL;
  FilteredWs ws;
  st = carve_checked(workspace, workspace_bytes, [&](Carver& c) { return carve_filtered(c, nrows, vocab); }, &ws);
  if (st != DFLASH2_OK) return st;
  if (temperature == 0.f)
    return hip_status(launch_spec_accept(target_logits, ld, batch_stride, tokens, cand_idx, q, (int)batch, (int)K,
                                         (int)vocab, 0.f, seed, out_tokens, n_accepted, row_status, ws.acc, stream));
  return hip_status(launch_spec_accept_filtered(target_logits, ld, batch_stride, tokens, cand_idx, q, (int)batch,
                                                (int)K, (int)vocab, temperature, top_k, top_p, seed, out_tokens,
                                                n_accepted, row_status, ws.filt, stream));
}


struct dflash2_graph_s {
  hipGraph_t graph;
  hipGraphExec_t exec;
};

dflash2_status dflash2_graph_begin(hipStream_t stream) {
  if (!stream) return DFLASH2_ERR_NULL;
  return hip_status(hipStreamBeginCapture(stream, hipStreamCaptureModeThreadLocal));
}

dflash2_status dflash2_graph_end(hipStream_t stream, dflash2_graph* graph) {
  if (!stream || !graph) return DFLASH2_ERR_NULL;
  *graph = nullptr;
  hipGraph_t g = nullptr;
  if (hipStreamEndCapture(stream, &g) != hipSuccess || !g) return DFLASH2_ERR_HIP;
  hipGraphExec_t x = nullptr;
  if (hipGraphInstantiate(&x, g, nullptr, nullptr, 0) != hipSuccess) {
    (void)hipGraphDestroy(g);
    return DFLASH2_ERR_HIP;
  }
  dflash2_graph h = new (std::nothrow) dflash2_graph_s{g, x};
  if (!h) {
    (void)hipGraphExecDestroy(x);
    (void)hipGraphDestroy(g);
    return DFLASH2_ERR_HIP;
  }
  *graph = h;
  return DFLASH2_OK;
}

dflash2_status dflash2_graph_launch(dflash2_graph graph, hipStream_t stream) {
  if (!graph) return DFLASH2_ERR_NULL;
  return hip_status(hipGraphLaunch(graph->exec, stream));
}

dflash2_status dflash2_graph_destroy(dflash2_graph graph) {
  if (!graph) return DFLASH2_ERR_NULL;
  const hipError_t a = hipGraphExecDestroy(graph->exec);
  const hipError_t b = hipGraphDestroy(graph->graph);
  delete graph;
  return (a == hipSuccess && b == hipSuccess) ? DFLASH2_OK : DFLASH2_ERR_HIP;
}

}  // extern "C"
