/*
 * libdflash2 -- the DFlash 2 proposer hot path on AMD Instinct MI355X (gfx950).
 *
 * Sources: the pegainfer issue "qwen3/dflash: DFlash 2 proposer -- top-16 path
 * selector + two-tap dynamic convolution" (cited as [PEGA]) and the FreeToken pull
 * request "Adds DFlash 2 as a second speculative decoding method" (cited as [FT]).
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Pointers are DEVICE pointers unless stated otherwise; tensors are row-major and
 *    contiguous, except that logits rows may be strided (`ld`, in elements).
 *  - bf16 data is passed as its uint16_t bit pattern.
 *  - The caller owns every buffer.  The library allocates no device memory and keeps
 *    no state between calls.  Scratch memory comes only from a caller-provided
 *    workspace sized by the matching *_workspace() query.  A workspace needs no
 *    initialisation: a call writes every workspace byte it reads before reading it,
 *    so a buffer may serve any later call whose query returns no more than its size.
 *    Calls that overlap in time must not share a workspace.
 *  - Every call validates its arguments on the host, enqueues its kernels on `stream`
 *    and returns without synchronising.  Host-detectable errors are returned before
 *    anything is enqueued; nothing aborts, prints or reads the environment.
 *  - Sizes whose kernels would need more than 2^32 - 1 work-items in one launch (the
 *    limit of a dispatch packet) are rejected with DFLASH2_ERR_SHAPE.
 *  - Results are deterministic: bit-identical across runs for the same inputs.
 *  - Outputs must not alias inputs.
 *  - Per-row data faults are reported in optional int32 `row_status` arrays (pass
 *    NULL to drop them):
 *      bit 0  non-finite value (a selected logit, a score, or a target row)
 *      bit 1  a token id outside [0, vocab) (clamped for reading, never dereferenced
 *             out of bounds)
 *      bit 2  an invalid draft distribution q (speculative accept)
 *      bit 3  a residual distribution without mass (speculative accept)
 */
#ifndef DFLASH2_H
#define DFLASH2_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DFLASH2_ABI_VERSION 3
#define DFLASH2_NCAND 16       /* candidates per draft position */
#define DFLASH2_MAX_K 64       /* draft positions per request */
#define DFLASH2_MAX_TOPK 32    /* largest top_k of the filtered verify */

typedef enum dflash2_status {
  DFLASH2_OK = 0,
  DFLASH2_ERR_NULL = 1,       /* a required pointer is NULL */
  DFLASH2_ERR_SHAPE = 2,      /* a size is out of range or inconsistent */
  DFLASH2_ERR_ALIGN = 3,      /* a pointer or row stride breaks the 16-byte alignment rule */
  DFLASH2_ERR_DTYPE = 4,      /* an unknown dtype or activation enum */
  DFLASH2_ERR_WORKSPACE = 5,  /* workspace NULL or smaller than the query returned */
  DFLASH2_ERR_VALUE = 6,      /* a value out of range: a temperature that is negative, NaN,
                                 infinite or positive below FLT_MIN = 2^-126 (whose reciprocal
                                 overflows); a bad top_p or scale where a call takes one */
  DFLASH2_ERR_HIP = 7         /* a HIP launch failed */
} dflash2_status;

typedef enum dflash2_dtype { DFLASH2_F32 = 0, DFLASH2_BF16 = 1 } dflash2_dtype;

typedef enum dflash2_gate_act { DFLASH2_GATE_SIGMOID = 0, DFLASH2_GATE_IDENTITY = 1 } dflash2_gate_act;

/* ABI version of the loaded library (DFLASH2_ABI_VERSION it was built with). */
int dflash2_abi_version(void);

/* Static, NUL-terminated name of a status code (host memory owned by the library). */
const char* dflash2_status_str(int status);

/* ---------------------------------------------------------------------------------
 * Top-16 candidates per draft position.
 * [PEGA] "What upstream shipped", item 1: keep the top-16 candidates per position;
 * [FT] "Details", runtime: the target LM head gives 16 candidates per slot.
 *
 * logits     bf16 bits [rows, ld]; element (r, v) at logits[r*ld + v], v < vocab.
 *            The base pointer and ld*2 bytes must be 16-byte aligned (ld % 8 == 0).
 * cand_idx   int32 [rows, 16]: token ids sorted by (logit desc, id asc).
 *            -0 equals +0; NaN ranks below -inf.
 * cand_val   float [rows, 16]: the selected logits widened exactly to fp32.
 * row_status int32 [rows] or NULL: bit 0 if a selected value is not finite.
 * Errors: NULL pointers, rows < 1, vocab < 16 or > 2^19, ld < vocab, alignment,
 *         workspace.
 * ------------------------------------------------------------------------------- */
size_t dflash2_topk16_workspace(int64_t rows, int64_t vocab);
dflash2_status dflash2_topk16(const uint16_t* logits, int64_t rows, int64_t vocab, int64_t ld,
                              int32_t* cand_idx, float* cand_val, int32_t* row_status,
                              void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------------
 * LM head with the top-16 fused in: the candidates of dflash2_topk16 taken straight
 * from the draft hidden rows and the (shared target) LM-head weight, without writing
 * the logits.  [FT] "Details", runtime (the target LM head gives 16 candidates per
 * slot); [RFC] "Questions", item 4 (the draft shares the target's LM head).
 *
 * logit[r, v] = bf16( sum_d h[r, d] * W[v, d] ): bf16 products accumulated in fp32 on
 * the matrix cores, then rounded to bf16 (nearest even), the precision of the draft
 * logits dflash2_topk16 reads.  The top-16 of each row is then taken in the order of
 * dflash2_topk16 (value desc, id asc, NaN lowest).  Values near a bf16 rounding
 * boundary may round either way against an exact sum (fp32 accumulation order).
 *
 * h          bf16 bits [rows, hidden], row-major, 16-byte aligned.
 * w          bf16 bits [vocab, hidden], row-major, 16-byte aligned (read once per
 *            group of up to 128 rows: a larger batch streams it once per 128 rows).
 * cand_idx   int32 [rows, 16]; cand_val float [rows, 16] (the bf16 logits widened);
 * row_status int32 [rows] or NULL: bit 0 if a selected value is not finite.
 * Workspace: dflash2_lmhead_topk16_workspace bytes, any contents (every call writes
 * what it reads): one sorted 16-list per row and 256-column tile.
 * Errors: NULL pointers, rows < 1, hidden < 256 or hidden % 256 != 0, vocab < 16 or
 *         > 2^19, alignment, workspace.
 * ------------------------------------------------------------------------------- */
size_t dflash2_lmhead_topk16_workspace(int64_t rows, int64_t vocab);
dflash2_status dflash2_lmhead_topk16(const uint16_t* h, const uint16_t* w, int64_t rows, int64_t hidden,
                                     int64_t vocab, int32_t* cand_idx, float* cand_val, int32_t* row_status,
                                     void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------------
 * The same LM head on a weight packed once for the matrix cores.  The weight is
 * constant (the target's LM head, [RFC] "Questions", item 4), so it can be re-laid once
 * at load time in the order the tile kernel reads it: every load instruction then reads
 * one contiguous 1 KB instead of 64 bytes of 16 rows.  Results are bit-identical to
 * dflash2_lmhead_topk16 on the unpacked weight.
 *
 * Packed layout (bf16 bits, dflash2_lmhead_packed_bytes bytes): tiles of 256 vocabulary
 * columns; tile T, hidden step k (32 dims) is 16 KB laid out
 * [nt (2)][wave (8)][g (4)][i (16)][8 dims], column 256 T + 32 wave + 16 nt + i, dims
 * 32 k + 8 g .. + 7; columns past the vocabulary are zero.  Element (v, d) sits at
 * ((((T * hidden / 32 + d / 32) * 2 + nt) * 8 + wave) * 64 + 16 ((d % 32) / 8) + i) * 8
 * + d % 8 with T = v / 256, wave = (v % 256) / 32, nt = (v % 32) / 16, i = v % 16.
 *
 * dflash2_lmhead_pack: w bf16 bits [vocab, hidden] row-major -> w_packed (16-byte
 *   aligned, dflash2_lmhead_packed_bytes; 0 on a bad shape); enqueued on `stream`.
 * dflash2_lmhead_topk16_packed: as dflash2_lmhead_topk16 with w_packed in place of w.
 * Errors: as dflash2_lmhead_topk16.
 * ------------------------------------------------------------------------------- */
size_t dflash2_lmhead_packed_bytes(int64_t vocab, int64_t hidden);
dflash2_status dflash2_lmhead_pack(const uint16_t* w, int64_t vocab, int64_t hidden, uint16_t* w_packed,
                                   hipStream_t stream);
dflash2_status dflash2_lmhead_topk16_packed(const uint16_t* h, const uint16_t* w_packed, int64_t rows,
                                            int64_t hidden, int64_t vocab, int32_t* cand_idx, float* cand_val,
                                            int32_t* row_status, void* workspace, size_t workspace_bytes,
                                            hipStream_t stream);

/* ---------------------------------------------------------------------------------
 * Draft-block attention over each request's K/V ring.  [FT] "Details": the released
 * drafts use sliding-window attention (window 2048); runtime: the draft's K/V lives in
 * a ring of 2112 positions per request (the window plus 64 rows of room for a verify's
 * rejected rows and for prefill rows past a snapshot boundary), and the draft forward
 * over [last token, mask x 7] reads it; prefix cache: the ring is rebuilt from the
 * last 2047 context rows; a causal draft is refused at startup.
 *
 * Keys of request b: its last n = min(ctx_len[b], window - 1) context positions p
 * (ring row p mod ring), then the block's nq rows.  Every query row attends to all of
 * them (non-causal); query head h uses K/V head h / (hq / hkv);
 * out = softmax(q k^T * scale) v, scale = 1/sqrt(head_dim) when 0 is passed.  Rows of
 * positions >= ctx_len (rejected or unwritten) and older than the window are never read.
 * q k^T: bf16 products accumulated in fp32 on the matrix cores; p = exp(s - max) in
 * fp32, carried into the p v product as two bf16 parts (relative error <= 2^-16);
 * accumulation in fp32.  Rotary embedding is applied before (the ring holds rotated
 * keys).
 *
 * q bf16 [batch, nq, hq, head_dim]; k_blk, v_blk bf16 [batch, nq, hkv, head_dim];
 * Both rings are kept in tiles of 32 positions per (request, K/V head), the layouts that
 * let every draft step read the window as contiguous 8 KB tiles (a verify writes a few
 * rows); position p, dim d of tile p / 32 (pp = p % 32):
 *   k_ring bf16 [batch, hkv, ring / 32, 2, 4, 4, 16, 8] at
 *     [(pp / 4) % 2][d / 32][(d % 32) / 8][4 (pp / 8) + pp % 4][d % 8]
 *     (the order in which the matrix cores read a tile);
 *   v_ring bf16 [batch, hkv, ring / 32, head_dim, 32] at [d][pp] (transposed).
 * ctx_len int32 [batch] (values < 0 read as 0); out float [batch, nq, hq, head_dim].
 * Other arrays row-major; all 16-byte aligned.  Workspace:
 * dflash2_ring_attention_workspace bytes, any contents.
 * Errors: NULL pointers; head_dim != 128, hq % hkv != 0, nq * hq / hkv > 48, ring < 32
 *         or ring % 32 != 0, window < 1 or window > ring -> DFLASH2_ERR_SHAPE;
 *         scale < 0 or not finite -> DFLASH2_ERR_VALUE; alignment; workspace.
 * ------------------------------------------------------------------------------- */
size_t dflash2_ring_attention_workspace(int64_t batch, int64_t nq, int64_t hq, int64_t hkv, int64_t window);
dflash2_status dflash2_ring_attention(const uint16_t* q, const uint16_t* k_blk, const uint16_t* v_blk,
                                      const uint16_t* k_ring, const uint16_t* v_ring, const int32_t* ctx_len,
                                      int64_t batch, int64_t nq, int64_t hq, int64_t hkv, int64_t head_dim,
                                      int64_t ring, int64_t window, float scale, float* out, void* workspace,
                                      size_t workspace_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------------
 * Context gate H = act(W_H h + b), one `dim`-wide gate per draft position.
 * [PEGA] "What upstream shipped", item 1 (256-dim token embeddings + context gate).
 * The gate is read as a logistic sigmoid of an affine map (DFLASH2_GATE_SIGMOID);
 * DFLASH2_GATE_IDENTITY returns the affine map.
 *
 * h        [rows, hidden] in h_dtype (DFLASH2_F32 or DFLASH2_BF16).
 * w_h      [dim, hidden] in w_dtype.  With DFLASH2_BF16 each fp32 h value is first
 *          rounded to bf16 (nearest, ties to even; bf16 h is used as it is) and the
 *          product runs on bf16 MFMA with fp32 accumulation; with DFLASH2_F32 it runs
 *          on fp32 MFMA (bf16 h widened exactly to fp32).
 * bias     float [dim] or NULL (= 0).
 * H        float [rows, dim].
 * Errors: NULL pointers, rows < 1, hidden < 8 or hidden % 8 != 0, dim not a power of
 *         two in [16, 1024], bad h_dtype, w_dtype or act, h / w_h not 16-byte
 *         aligned, workspace.
 * ------------------------------------------------------------------------------- */
size_t dflash2_context_gate_workspace(int64_t rows, int64_t hidden, int64_t dim);
dflash2_status dflash2_context_gate(const void* h, dflash2_dtype h_dtype, const void* w_h,
                                    dflash2_dtype w_dtype, const float* bias, int64_t rows,
                                    int64_t hidden, int64_t dim, dflash2_gate_act act, float* H,
                                    void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------------
 * Pair scores S_t(a, b) = U_t(b) + <A(a) (.) H(h_t), B(b)> for every adjacent pair.
 * [PEGA] "What upstream shipped", item 1, and "Proposal", phase 1
 * (block_size x 16 predecessors x 16 candidates x 256 dims).
 *
 * S[b,t,i,j] = cand_val[b,t,j] + sum_d A[prev_i, d] * H[b,t,d] * B[cand_idx[b,t,j], d]
 * with prev_i = verified[b] at t = 0 (all 16 rows) and cand_idx[b,t-1,i] at t >= 1.
 *
 * cand_idx int32 [batch, K, 16], cand_val float [batch, K, 16], verified int32 [batch],
 * emb_a, emb_b [vocab, dim] in emb_dtype (16-byte aligned), H float [batch, K, dim],
 * S float [batch, K, 16, 16], row_status int32 [batch, K] or NULL: bit 0 non-finite
 * score, bit 1 id out of range (clamped to [0, vocab), never read out of bounds).
 * Arithmetic: fp32 tables run on fp32 MFMA (fp32 products, fp32 sums).  bf16 tables
 * run on bf16 MFMA: each A[prev_i, d] * H[d] is split into a nearest-bf16 part and the
 * bf16 of its remainder (taken with a fused multiply-add), both multiplied exactly by
 * the bf16 B value and summed in fp32, so each term is within about 2^-18 of its fp32
 * value.  Every entry point that computes scores uses this arithmetic, bit for bit.
 * Errors: NULL pointers, batch < 1, K not in [1, 64], vocab < 16, dim not a power of
 *         two in [16, 1024] (DFLASH2_ERR_SHAPE), dtype, alignment.
 * ------------------------------------------------------------------------------- */
dflash2_status dflash2_pair_score(const int32_t* cand_idx, const float* cand_val,
                                  const int32_t* verified, const void* emb_a, const void* emb_b,
                                  dflash2_dtype emb_dtype, int64_t vocab, int64_t dim,
                                  const float* H, int64_t batch, int64_t K, float* S,
                                  int32_t* row_status, hipStream_t stream);

/* ---------------------------------------------------------------------------------
 * Walk over the precomputed scores: the proposed path.
 * [PEGA] "What upstream shipped", item 1 (a single greedy/sampled walk over the
 * precomputed scores) and "Proposal", phase 1 (<= block_size argmax steps);
 * [FT] "Details", runtime (sampled from q, or argmax when greedy) and shared changes
 * (the proposer returns tokens, candidates and q).
 *
 * Step t reads row i_{t-1} of S[b,t] (i_{-1} = 0, the verified token's row).
 * temperature == 0: greedy, slot = lowest j of the row maximum, q one-hot.
 * temperature  > 0: q = softmax(row / T) over the 16 slots; slot = the first j whose
 *                   prefix weight exceeds u * total, u from Philox4x32-10 with key
 *                   (lo32(seed), hi32(seed)) and counter (t, b, 0, 0), word 0,
 *                   u = (word >> 8) * 2^-24.
 * Non-finite scores never win (weight 0); an all-non-finite row picks slot 0.
 *
 * S float [batch, K, 16, 16]; cand_idx int32 [batch, K, 16];
 * tokens, slots int32 [batch, K]; q float [batch, K, 16].
 * Errors: NULL pointers, batch < 1, batch >= 2^31, K not in [1, 64], temperature.
 * ------------------------------------------------------------------------------- */
dflash2_status dflash2_walk(const float* S, const int32_t* cand_idx, int64_t batch, int64_t K,
                            float temperature, uint64_t seed, int32_t* tokens, int32_t* slots,
                            float* q, hipStream_t stream);

/* ---------------------------------------------------------------------------------
 * Fused proposer step: topk16 -> pair_score -> walk in one call (no host
 * synchronisation).  Same passages as the three calls above; the outputs are
 * bit-identical to calling dflash2_topk16 on every position's logits row, then
 * dflash2_pair_score, then dflash2_walk.  logits rows are addressed as
 * logits[(b*K + t)*ld + v].  Two kernels on `stream`: one streams the logits, then one
 * block per draft position merges its candidates and scores its row, and the block that
 * finishes a request's last row walks that request.
 *
 * S must be 16-byte aligned.  row_status int32 [batch, K] or NULL (the union of the
 * top-16 and pair-score bits).
 * Errors: the union of the three calls' checks, S alignment, plus workspace.
 * ------------------------------------------------------------------------------- */
size_t dflash2_select_workspace(int64_t batch, int64_t K, int64_t vocab);
dflash2_status dflash2_select(const uint16_t* logits, int64_t ld, const int32_t* verified,
                              const void* emb_a, const void* emb_b, dflash2_dtype emb_dtype,
                              int64_t vocab, int64_t dim, const float* H, int64_t batch, int64_t K,
                              float temperature, uint64_t seed, int32_t* cand_idx, float* cand_val,
                              float* S, int32_t* tokens, int32_t* slots, float* q,
                              int32_t* row_status, void* workspace, size_t workspace_bytes,
                              hipStream_t stream);

/* ---------------------------------------------------------------------------------
 * dflash2_select without a workspace argument, for callers that cannot allocate device
 * memory (code recorded under graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Same arguments (minus workspace and workspace_bytes), same outputs, bit
 * for bit, and the same kernels as dflash2_select.
 *
 * Its scratch is a 4 MiB array in the library's own device memory, one per GPU, held
 * from the library's load on that GPU until the process ends; the call allocates
 * nothing (no hipMalloc, hipFree or allocating library routine).  Every call on a GPU
 * shares that GPU's array, so calls that overlap on one GPU (other streams, other host
 * threads) race: the caller serialises them.  The array needs no initialisation (every
 * call writes the scratch it reads).
 * Errors: those of dflash2_select; a request whose dflash2_select_workspace exceeds
 *         4 MiB (above about 2000 draft positions, batch x K, at the largest vocabulary)
 *         -> DFLASH2_ERR_WORKSPACE; the scratch address not obtainable -> DFLASH2_ERR_HIP.
 * ------------------------------------------------------------------------------- */
dflash2_status dflash2_select_noalloc(const uint16_t* logits, int64_t ld, const int32_t* verified,
                                      const void* emb_a, const void* emb_b, dflash2_dtype emb_dtype,
                                      int64_t vocab, int64_t dim, const float* H, int64_t batch,
                                      int64_t K, float temperature, uint64_t seed, int32_t* cand_idx,
                                      float* cand_val, float* S, int32_t* tokens, int32_t* slots,
                                      float* q, int32_t* row_status, hipStream_t stream);

/* ---------------------------------------------------------------------------------
 * Gated proposer step: context gate -> topk16 -> pair_score -> walk in one call.
 * The passages of dflash2_context_gate and dflash2_select.  The gate's bf16 matrix
 * product runs inside the launch that streams the logits (on compute units the stream
 * leaves idle or shares), and each draft position adds its own row's gate slices, so
 * H never makes a separate round trip.
 *
 * h [batch, K, hidden] in h_dtype (DFLASH2_F32 or DFLASH2_BF16); w_h [dim, hidden] in
 * w_dtype, which must be DFLASH2_BF16 (fp32 h rounded to bf16 as in
 * dflash2_context_gate); bias float [dim] or
 * NULL; act as in dflash2_context_gate.  H_out float [batch, K, dim] or NULL: the gate
 * values the scores used.  They equal dflash2_context_gate's up to the fp32 summation
 * order over `hidden` (deterministic, not bit-identical to it); every other output is
 * bit-identical to dflash2_select called with H = H_out.
 * Errors: the checks of dflash2_select and dflash2_context_gate, w_dtype other than
 *         DFLASH2_BF16 or a bad h_dtype (DFLASH2_ERR_DTYPE), dim < 64 (the fused gate
 *         tiles are 64 columns wide; DFLASH2_ERR_SHAPE), H_out not 16-byte aligned,
 *         workspace.
 * ------------------------------------------------------------------------------- */
size_t dflash2_select_gated_workspace(int64_t batch, int64_t K, int64_t vocab, int64_t hidden,
                                      int64_t dim);
dflash2_status dflash2_select_gated(const uint16_t* logits, int64_t ld, const int32_t* verified,
                                    const void* emb_a, const void* emb_b, dflash2_dtype emb_dtype,
                                    int64_t vocab, int64_t dim, const void* h, dflash2_dtype h_dtype,
                                    const void* w_h, dflash2_dtype w_dtype, const float* bias,
                                    int64_t hidden, dflash2_gate_act act, int64_t batch, int64_t K,
                                    float temperature, uint64_t seed, float* H_out,
                                    int32_t* cand_idx, float* cand_val, float* S, int32_t* tokens,
                                    int32_t* slots, float* q, int32_t* row_status, void* workspace,
                                    size_t workspace_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------------
 * Two-tap dynamic depthwise convolution, at `sites` independent sublayer sites.
 * [PEGA] "What upstream shipped", item 2:
 *   Conv(x)_t = k_{t,0} (.) x_t + k_{t,1} (.) x_{t-1},  x_{-1} = the last verified
 *   token's hidden.
 * [FT] "Tests added or changed" / "Details": taps are shared by `group` adjacent
 * channels (conv_group_size must divide hidden); channel d uses tap d / group.
 *
 * x float [sites, batch, K, hidden]; x_prev float [sites, batch, hidden];
 * taps float [sites, batch, K, 2, hidden/group]; y float [sites, batch, K, hidden].
 * Errors: NULL pointers, sizes < 1, K > 64, hidden % group != 0.
 * ------------------------------------------------------------------------------- */
dflash2_status dflash2_conv2tap(const float* x, const float* x_prev, const float* taps,
                                int64_t sites, int64_t batch, int64_t K, int64_t hidden,
                                int64_t group, float* y, hipStream_t stream);

/* ---------------------------------------------------------------------------------
 * Lossless verify of K drafted tokens against the target.
 * [FT] "Details", sampled verify: accept with min(1, p/q); on a reject resample from
 * max(0, p - q), so the output follows the target distribution; all-greedy keeps the
 * prefix match.  [PEGA] "Proposal", phase 3.
 *
 * target_logits bf16 bits; row (b, t) for t in [0, K] at
 *   target_logits[b*batch_stride + t*ld], ld % 8 == 0, 16-byte aligned base.
 *   batch_stride may be 0 (every request verifies against the same K+1 rows).
 * tokens int32 [batch, K]; cand_idx int32 [batch, K, 16]; q float [batch, K, 16]
 *   (q may be NULL when temperature == 0).
 * temperature > 0, per request b, with p_t = softmax(target row t / T):
 *   step t accepts x_t iff u_acc * q_t(x_t) < p_t(x_t), q_t(v) = sum of q[b,t,j] over
 *   slots j with cand_idx[b,t,j] == v; at the first reject it commits
 *   v ~ max(0, p_t - q_t) (inverse CDF in token-id order with u_res) and stops; if all
 *   K are accepted it commits a bonus token from p_K.  (u_acc, u_res) are words 0 and
 *   1 of Philox4x32-10 at counter (t, b, 1, 0) under key (lo32(seed), hi32(seed)).
 * temperature == 0: g_t = argmax of target row t (lowest id); accept while
 *   tokens[b,t] == g_t; commit g at the first mismatch, or the bonus g_K.
 * Outputs: out_tokens int32 [batch, K+1] (committed ids, then -1), n_accepted int32
 *   [batch], row_status int32 [batch] or NULL:
 *   bit 0 (T > 0) a target row holds NaN or +inf: nothing is committed;
 *   bit 1 a token or candidate id outside [0, vocab): (T > 0) commit one token from p_0;
 *   bit 2 (T > 0) a q row has NaN / negative entries, a sum off 1 by > 1e-3, or
 *         q_t(x_t) <= 0: commit one token drawn from p_0;
 *   bit 3 (T > 0) the residual has no mass: draw from p_t instead.
 * Errors: NULL pointers, batch < 1, K not in [1, 64], vocab < 16 or > 2^19,
 *         ld < vocab, alignment, temperature, workspace.
 * ------------------------------------------------------------------------------- */
size_t dflash2_spec_accept_workspace(int64_t batch, int64_t K, int64_t vocab);
dflash2_status dflash2_spec_accept(const uint16_t* target_logits, int64_t ld, int64_t batch_stride,
                                   const int32_t* tokens, const int32_t* cand_idx, const float* q,
                                   int64_t batch, int64_t K, int64_t vocab, float temperature,
                                   uint64_t seed, int32_t* out_tokens, int32_t* n_accepted,
                                   int32_t* row_status, void* workspace, size_t workspace_bytes,
                                   hipStream_t stream);

/* ---- dflash2_spec_accept_filtered ---------------------------------------------
 * The verify of dflash2_spec_accept against the filtered target distribution of the
 * FreeToken runs' sampling settings (FreeToken PR "Adds DFlash 2", "Speed" and "All
 * settings": temperature 1.0, top_p 0.95, top_k 20; "Known gaps": the sparse-q verify
 * with top-k + top-p).  For temperature > 0, p_t of target row t is:
 *   the top_k largest logits of the row (value desc, lowest id first on ties), exactly
 *   top_k of them; softmax(l / T) over those; then, walking them in that order, every
 *   token whose preceding mass is below top_p (the token reaching top_p is kept;
 *   top_p >= 1 cuts nothing); renormalised.  Every other token has p = 0.
 * That p replaces softmax(l / T) everywhere in the rule of dflash2_spec_accept: the
 * accept test, the residual max(0, p - q), the bonus token and the fallbacks, with the
 * same Philox counters, status bits and outputs.  temperature == 0 is the greedy
 * prefix match of dflash2_spec_accept (the filters keep the argmax).
 * Arguments and layouts as dflash2_spec_accept, plus top_k in [1, DFLASH2_MAX_TOPK] and
 * top_p in (0, 1].  The workspace (dflash2_spec_accept_filtered_workspace bytes, any
 * contents) holds each 1/8 chunk's top_k and is rewritten by every call.
 * Errors: as dflash2_spec_accept; top_k or top_p out of range -> DFLASH2_ERR_VALUE.
 * ------------------------------------------------------------------------------- */
size_t dflash2_spec_accept_filtered_workspace(int64_t batch, int64_t K, int64_t vocab);
dflash2_status dflash2_spec_accept_filtered(const uint16_t* target_logits, int64_t ld, int64_t batch_stride,
                                            const int32_t* tokens, const int32_t* cand_idx, const float* q,
                                            int64_t batch, int64_t K, int64_t vocab, float temperature,
                                            int32_t top_k, float top_p, uint64_t seed, int32_t* out_tokens,
                                            int32_t* n_accepted, int32_t* row_status, void* workspace,
                                            size_t workspace_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------------
 * One launch per proposer step: HIP graphs of library calls.  [RFC] "Questions",
 * item 5 (greedy-only CUDA-graph capture; a single active speculative generation
 * graph) and [PEGA] "Proposal", phase 1 (the walk as a launch-floor candidate, under
 * the same graph treatment).
 *
 * dflash2_graph_begin starts recording the work enqueued on `stream` (HIP stream
 * capture, thread-local mode): the dflash2_* calls made on it until dflash2_graph_end
 * are recorded, not run.  dflash2_graph_end instantiates them into *graph; each
 * dflash2_graph_launch replays the whole sequence with one launch, on the buffers the
 * calls were given (callers refresh inputs in place between launches).  The calls
 * recorded must not need new workspace or outputs while recording (make each call once
 * before, so its buffers exist); none of them records a memset.  The graph and its
 * executable are host objects of the HIP runtime, owned by the caller until
 * dflash2_graph_destroy.  `stream` must not be the legacy default stream.
 * Errors: NULL stream or handle -> DFLASH2_ERR_NULL; a failed capture, instantiation
 * or launch -> DFLASH2_ERR_HIP (a failed capture leaves no graph).
 * ------------------------------------------------------------------------------- */
typedef struct dflash2_graph_s* dflash2_graph;
dflash2_status dflash2_graph_begin(hipStream_t stream);
dflash2_status dflash2_graph_end(hipStream_t stream, dflash2_graph* graph);
dflash2_status dflash2_graph_launch(dflash2_graph graph, hipStream_t stream);
dflash2_status dflash2_graph_destroy(dflash2_graph graph);

#ifdef __cplusplus
}
#endif

#endif /* DFLASH2_H */
