"""CPU oracle for the DFlash 2 proposer hot path -- TEST INFRASTRUCTURE ONLY.

Plain, slow, float64 numpy code that states what each step of the path computes.
Only the tests, the package's smoke check and the benchmark's CPU-baseline leg may
import it; the library path never does.  It shares no code with the HIP library.

Sources (the three pages this method is described on):
  [RFC]  TensorRT-LLM issue "[RFC] DFlash2 for Qwen3.8 on consumer Blackwell:
         integration boundary before we propose a PR"
  [PEGA] pegainfer issue "qwen3/dflash: DFlash 2 proposer -- top-16 path selector +
         two-tap dynamic convolution"
  [FT]   FreeToken pull request "Adds DFlash 2 as a second speculative decoding method"
Each function cites the section it follows.  Where the pages leave a step open,
the docstring says which reading is taken.

Every function here is pinned by CPU tests against brute force, closed forms,
hand-worked fixtures, an independent Philox implementation, or the
speculative-sampling theorem; none is "parity unpinned".
"""

from __future__ import annotations

import numpy as np

NCAND = 16

# ----------------------------------------------------------------------------------
# bf16 helpers
# ----------------------------------------------------------------------------------


def bf16_to_f64(bits) -> np.ndarray:
    """Value of bf16 bit patterns: the top half of an IEEE binary32 word (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def round_to_bf16(x) -> np.ndarray:
    """Round finite float32 values to the nearest bf16 value (ties to even), as float64.

    bf16 keeps 8 significant bits, so the spacing of bf16 values around x is
    2^(e-8) for x = m * 2^e with 0.5 <= |m| < 1, and never finer than the
    subnormal spacing 2^-133.  np.rint rounds halves to even.
    """
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    quantum = np.ldexp(1.0, np.maximum(e - 8, -133))
    y = np.rint(x / quantum) * quantum
    return np.where(np.abs(y) >= 2.0 ** 128, np.copysign(np.inf, x), y)


# ----------------------------------------------------------------------------------
# Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy as
# 1, 2, 3", SC'11), vectorised over counters with numpy uint64 arithmetic.
# ----------------------------------------------------------------------------------

_PHILOX_M0 = np.uint64(0xD2511F53)
_PHILOX_M1 = np.uint64(0xCD9E8D57)
_PHILOX_W0 = np.uint64(0x9E3779B9)
_PHILOX_W1 = np.uint64(0xBB67AE85)
_MASK32 = np.uint64(0xFFFFFFFF)


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Ten Philox-4x32 rounds on counter (c0..c3) under key (k0, k1).

    One round multiplies words 0 and 2 by the two round multipliers, keeps the
    64-bit products as (hi, lo) halves, and outputs
    (hi(M1*c2) ^ c1 ^ k0, lo(M1*c2), hi(M0*c0) ^ c3 ^ k1, lo(M0*c0));
    between rounds the key is advanced by the two Weyl constants.
    Inputs broadcast; returns four uint64 arrays holding 32-bit words.
    """
    c0, c1, c2, c3, k0, k1 = np.broadcast_arrays(*[np.asarray(v, dtype=np.uint64) & _MASK32
                                                   for v in (c0, c1, c2, c3, k0, k1)])
    c0, c1, c2, c3, k0, k1 = (a.copy() for a in (c0, c1, c2, c3, k0, k1))
    for rnd in range(10):
        p0 = _PHILOX_M0 * c0
        p1 = _PHILOX_M1 * c2
        n0 = (p1 >> np.uint64(32)) ^ c1 ^ k0
        n1 = p1 & _MASK32
        n2 = (p0 >> np.uint64(32)) ^ c3 ^ k1
        n3 = p0 & _MASK32
        c0, c1, c2, c3 = n0, n1, n2, n3
        if rnd < 9:
            k0 = (k0 + _PHILOX_W0) & _MASK32
            k1 = (k1 + _PHILOX_W1) & _MASK32
    return c0, c1, c2, c3


def word_to_uniform(x) -> np.ndarray:
    """Uniform in [0, 1) from a 32-bit word: its top 24 bits times 2^-24 (exact)."""
    return (np.asarray(x, dtype=np.uint64) >> np.uint64(8)).astype(np.float64) * 2.0 ** -24


def _key(seed: int):
    seed = int(seed) & 0xFFFFFFFFFFFFFFFF
    return seed & 0xFFFFFFFF, seed >> 32


def walk_uniform(seed: int, b, t) -> np.ndarray:
    """Uniform of the sampled walk for (request b, position t): counter (t, b, 0, 0), word 0.

    The synthetic workload keys the draws by (seed, request, position); the
    counter layout is this oracle's reading of that phrase.
    """
    k0, k1 = _key(seed)
    x0, _, _, _ = philox4x32_10(t, b, 0, 0, k0, k1)
    return word_to_uniform(x0)


def verify_uniforms(seed: int, b, t):
    """(u_accept, u_resample) of the verify for (request b, position t): counter (t, b, 1, 0)."""
    k0, k1 = _key(seed)
    x0, x1, _, _ = philox4x32_10(t, b, 1, 0, k0, k1)
    return word_to_uniform(x0), word_to_uniform(x1)


# ----------------------------------------------------------------------------------
# Top-16 candidates
# ----------------------------------------------------------------------------------


def topk16(logits_bits, k: int = NCAND):
    """The k largest draft logits of every row, by (value desc, token id asc).

    [PEGA] "What upstream shipped", item 1: keep the top-16 candidates per draft
    position.  [FT] "Details", runtime: the target LM head gives 16 candidates per
    slot.  Ties break toward the lowest token id; -0 equals +0; NaN ranks below
    -inf.  Implemented as the definition: a stable full sort of the row.

    logits_bits: uint16 [..., V].  Returns (idx int64 [..., k], val float64 [..., k]).
    """
    bits = np.asarray(logits_bits, dtype=np.uint16)
    lead = bits.shape[:-1]
    V = bits.shape[-1]
    rows = bits.reshape(-1, V)
    idx = np.empty((rows.shape[0], k), dtype=np.int64)
    val = np.empty((rows.shape[0], k), dtype=np.float64)
    ids = np.arange(V)
    for r in range(rows.shape[0]):
        v = bf16_to_f64(rows[r])
        isnan = np.isnan(v)
        neg = np.where(isnan, 0.0, -v) + 0.0          # + 0.0 turns -0.0 into +0.0
        order = np.lexsort((ids, neg, isnan))          # last key is the primary key
        idx[r] = order[:k]
        val[r] = v[order[:k]]
    return idx.reshape(lead + (k,)), val.reshape(lead + (k,))


# ----------------------------------------------------------------------------------
# Context gate H(h_t)
# ----------------------------------------------------------------------------------


def context_gate(h, w, bias, w_is_bf16: bool, act: str = "sigmoid"):
    """H = act(W_H . h_hat + b), one 256-wide gate per draft position.

    [PEGA] "What upstream shipped", item 1: 256-dim token embeddings plus a
    context gate.  Reading taken: a gate multiplies elementwise, so it is the
    logistic sigmoid of an affine map (act="sigmoid"); act="identity" returns the
    affine map.  When W_H is bf16, h is rounded to bf16 first (h_hat), as a bf16
    matrix product would consume it; otherwise h_hat = h.

    h: float32 [R, D]; w: float64-convertible [dim, D] (decode bf16 first);
    bias: [dim].  Returns (H, pre, pre_abs) with pre_abs = sum |W h_hat| + |b|,
    the scale the floating-point tolerance is relative to.
    """
    h = np.asarray(h, dtype=np.float64)
    h_hat = round_to_bf16(h) if w_is_bf16 else h
    w = np.asarray(w, dtype=np.float64)
    b = np.asarray(bias, dtype=np.float64)
    pre = h_hat @ w.T + b
    pre_abs = np.abs(h_hat) @ np.abs(w).T + np.abs(b)
    if act == "sigmoid":
        H = 1.0 / (1.0 + np.exp(-pre))
    elif act == "identity":
        H = pre
    else:
        raise ValueError(act)
    return H, pre, pre_abs


# ----------------------------------------------------------------------------------
# Pair scores S_t(a, b)
# ----------------------------------------------------------------------------------


def pair_score(cand_idx, cand_val, verified, emb_a, emb_b, H):
    """S[b,t,i,j] = U_t(c_j) + sum_d A(prev_i)_d * H(h_t)_d * B(c_j)_d.

    [PEGA] "What upstream shipped", item 1: score every adjacent pair with
    S_t(a,b) = U_t(b) + <A(a) (.) H(h_t), B(b)>, a low-rank bilinear form; and
    "Proposal", phase 1: block_size x 16 predecessors x 16 candidates x 256 dims.
    U_t(b) is the candidate's own draft logit.  Reading taken for the first
    position: its only predecessor is the last verified token, so all 16 rows of
    S[b,0] use verified[b].  Ids outside [0, V) are clamped and flagged (bit 1).

    cand_idx int [B,K,16], cand_val [B,K,16], verified int [B], emb_a / emb_b
    float [V, dim], H [B,K,dim].  Returns (S, S_abs, status) where S_abs is
    |U| + sum_d |A H B| and status is int32 [B,K].
    """
    cand_idx = np.asarray(cand_idx, dtype=np.int64)
    U = np.asarray(cand_val, dtype=np.float64)
    A = np.asarray(emb_a, dtype=np.float64)
    Bt = np.asarray(emb_b, dtype=np.float64)
    H = np.asarray(H, dtype=np.float64)
    B_, K = cand_idx.shape[:2]
    V = A.shape[0]
    S = np.empty((B_, K, NCAND, NCAND))
    S_abs = np.empty_like(S)
    status = np.zeros((B_, K), dtype=np.int32)
    for b in range(B_):
        for t in range(K):
            prev = np.full(NCAND, int(verified[b])) if t == 0 else cand_idx[b, t - 1]
            cur = cand_idx[b, t]
            if np.any((prev < 0) | (prev >= V)) or np.any((cur < 0) | (cur >= V)):
                status[b, t] |= 2
            prev = np.clip(prev, 0, V - 1)
            cur = np.clip(cur, 0, V - 1)
            G = A[prev] * H[b, t][None, :]
            S[b, t] = U[b, t][None, :] + G @ Bt[cur].T
            S_abs[b, t] = np.abs(U[b, t])[None, :] + np.abs(G) @ np.abs(Bt[cur]).T
            if not np.all(np.isfinite(S[b, t])):
                status[b, t] |= 1
    return S, S_abs, status


# ----------------------------------------------------------------------------------
# Walk over the precomputed scores
# ----------------------------------------------------------------------------------


def greedy_pick(row) -> int:
    """Lowest slot j holding the maximum of a 16-score row; non-finite scores never
    win (an all-non-finite row picks slot 0)."""
    row = np.asarray(row, dtype=np.float64)
    fin = np.isfinite(row)
    if not fin.any():
        return 0
    return int(np.argmax(np.where(fin, row, -np.inf)))


def sample_pick(row, temperature: float, u: float):
    """Inverse-CDF draw from softmax(row / T) over the 16 slots, in slot order.

    w_j = exp((s_j - max)/T) (0 for non-finite s_j), W = sum_j w_j,
    j = min { j : u * W < w_0 + ... + w_j }.  Returns (j, q) with q = w / W.
    An all-non-finite row returns slot 0 with a one-hot q.
    """
    row = np.asarray(row, dtype=np.float64)
    fin = np.isfinite(row)
    q = np.zeros(NCAND)
    if not fin.any():
        q[0] = 1.0
        return 0, q
    m = row[fin].max()
    w = np.where(fin, np.exp((np.where(fin, row, m) - m) / temperature), 0.0)
    W = w.sum()
    P = np.cumsum(w)
    hit = np.nonzero(u * W < P)[0]
    j = int(hit[0]) if hit.size else int(np.nonzero(w > 0)[0][-1])
    return j, w / W


def walk(S, cand_idx, temperature: float = 0.0, seed: int = 0):
    """The proposed path: one greedy or sampled step per draft position.

    [PEGA] "What upstream shipped", item 1: a single greedy/sampled walk over the
    precomputed scores picks the proposed path; "Proposal", phase 1: at most
    block_size argmax steps.  [FT] "Details", runtime: sampled from the
    selector's distribution q, or argmax when greedy; the proposer returns
    (tokens, cand, q).  The walk starts on row 0 of S[b,0] (the verified token);
    at step t it uses row i = the slot chosen at t-1.  T = 0 is greedy (q is
    one-hot); T > 0 samples with the uniform of (seed, b, t).

    Returns (tokens int64 [B,K], slots int64 [B,K], q float64 [B,K,16]).
    """
    S = np.asarray(S, dtype=np.float64)
    cand_idx = np.asarray(cand_idx)
    B_, K = S.shape[:2]
    tokens = np.empty((B_, K), dtype=np.int64)
    slots = np.empty((B_, K), dtype=np.int64)
    q = np.zeros((B_, K, NCAND))
    if temperature != 0.0:
        u_walk = walk_uniform(seed, np.arange(B_)[:, None], np.arange(K)[None, :])
    for b in range(B_):
        i = 0
        for t in range(K):
            row = S[b, t, i]
            if temperature == 0.0:
                j = greedy_pick(row)
                q[b, t, j] = 1.0
            else:
                j, q[b, t] = sample_pick(row, temperature, float(u_walk[b, t]))
            slots[b, t] = j
            tokens[b, t] = cand_idx[b, t, j]
            i = j
    return tokens, slots, q


# ----------------------------------------------------------------------------------
# Two-tap dynamic depthwise convolution
# ----------------------------------------------------------------------------------


def conv2tap(x, prev, taps, group: int = 1):
    """Conv(x)_t = k_{t,0} (.) x_t + k_{t,1} (.) x_{t-1}; x_{-1} is the last verified
    token's hidden.

    [PEGA] "What upstream shipped", item 2 (two-tap dynamic depthwise conv).
    [FT] "Details" and "Tests added or changed" (grouped conv; conv_group_size
    divides hidden): channel d uses tap d // group.

    x [S,B,K,D], prev [S,B,D], taps [S,B,K,2,D/group].  Returns (y, y_abs) with
    y_abs = |k0 x_t| + |k1 x_{t-1}|.
    """
    x = np.asarray(x, dtype=np.float64)
    prev = np.asarray(prev, dtype=np.float64)
    taps = np.asarray(taps, dtype=np.float64)
    D = x.shape[-1]
    k = np.repeat(taps, group, axis=-1)[..., :D]     # tap of channel d is taps[..., d // group]
    xm1 = np.concatenate([prev[:, :, None, :], x[:, :, :-1, :]], axis=2)
    t0 = k[..., 0, :] * x
    t1 = k[..., 1, :] * xm1
    return t0 + t1, np.abs(t0) + np.abs(t1)


# ----------------------------------------------------------------------------------
# Speculative-sampling verify
# ----------------------------------------------------------------------------------


def _inverse_cdf(weights, u: float) -> int:
    """min { v : u * sum(w) < w_0 + ... + w_v } in token-id order (last positive
    weight if rounding leaves none)."""
    P = np.cumsum(weights)
    hit = np.nonzero(u * P[-1] < P)[0]
    return int(hit[0]) if hit.size else int(np.nonzero(weights > 0)[0][-1])


def target_probs(bits_row, temperature: float) -> np.ndarray:
    """p = softmax(l / T) over the vocabulary (float64)."""
    l = bf16_to_f64(bits_row)
    m = l.max()
    w = np.exp((l - m) / temperature)
    return w / w.sum()


def filtered_target_probs(bits_row, temperature: float, top_k: int = 0, top_p: float = 1.0,
                          margin: list | None = None) -> np.ndarray:
    """p after the sampling filters, applied in the order the [FT] runs name them
    ("Speed" and "All settings": temperature, then top_p = 0.95 and top_k = 20).

    Readings (the pages name the settings, not their tie or boundary rules):
      - top-k keeps exactly top_k tokens, the largest logits by (value desc, token id
        asc), the candidate order used everywhere else on this path; top_k = 0 keeps all;
      - p over the kept tokens is softmax(l / T) renormalised over them;
      - top-p walks the kept tokens in that same order and keeps each one whose
        preceding cumulative mass is below top_p (the token that reaches top_p is
        kept, so at least one token is); top_p >= 1 cuts nothing (no rounding of the
        running sum up to 1 may drop the tail);
      - the surviving masses are renormalised; every other token has p = 0.
    `margin`, when given, receives |cumulative mass before a token - top_p| at the two
    tokens on either side of the top-p cut (how close the cut is to moving).
    """
    l = bf16_to_f64(bits_row)
    V = l.size
    order = np.lexsort((np.arange(V), -l))            # value desc, id asc
    kept = order[:top_k] if top_k > 0 else order
    z = l[kept] / temperature
    w = np.exp(z - z.max())
    pk = w / w.sum()
    before = np.concatenate([[0.0], np.cumsum(pk)[:-1]])
    keep = before < top_p if top_p < 1.0 else np.ones(before.size, dtype=bool)   # top_p >= 1: no cut
    n = int(keep.sum())
    if margin is not None:
        margin.append(min(abs(before[i] - top_p) for i in (n - 1, n) if i < before.size))
    p = np.zeros(V)
    p[kept[:n]] = pk[:n] / pk[:n].sum()
    return p


def bf16_argmax(bits_row) -> int:
    """Lowest token id holding the largest bf16 logit.  NaN ranks below every number,
    -inf included (the candidate order's reading); an all-NaN row gives token 0."""
    l = bf16_to_f64(bits_row)
    ok = ~np.isnan(l)
    if not ok.any():
        return 0
    m = l[ok].max()
    return int(np.flatnonzero(ok & (l == m))[0])


def spec_accept(target_bits, tokens, cand_idx, q, temperature: float, seed: int = 0,
                return_trace: bool = False, top_k: int = 0, top_p: float = 1.0):
    """Lossless verify of K drafted tokens against target logits [B, K+1, V].

    [FT] "Details", sampled verify: accept with min(1, p/q); on a reject resample
    from max(0, p - q), so the output follows the target distribution.  [PEGA]
    "Proposal", phase 3 (rejection sampling restores the target distribution;
    greedy stays longest-prefix).  [FT] "Tests added or changed": trusted, NaN,
    wrong-total and greedy rows.

    T > 0, per request b:
      p_t = softmax(l_t / T); q_t(v) = sum of q[b,t,j] over slots with cand = v.
      Step t accepts x_t iff u_acc * q_t(x_t) < p_t(x_t)  (so with prob min(1, p/q)).
      At the first reject, commit v ~ max(0, p_t - q_t) (inverse CDF with u_res,
      token-id order) and stop.  If all K are accepted, commit a bonus token from
      p_K with u_res of position K.
    T = 0: g_t = argmax l_t; accept while tokens[t] == g_t; commit g at the first
    mismatch, or the bonus g_K.
    With top_k > 0 or top_p < 1 (T > 0 only), p_t is the filtered target distribution
    of `filtered_target_probs` throughout: the accept test, the residual max(0, p - q),
    the bonus and the fallbacks.  Without them the rule is the one above unchanged.

    Readings taken for malformed rows (status bits):
      bit 0  a target row of the request holds NaN or +inf (T > 0): nothing is committed.
      bit 1  a draft token or candidate id outside [0, V): T > 0 falls back to
             one token drawn from p_0; T = 0 keeps the prefix rule.
      bit 2  a q row with a NaN or negative entry, a sum off 1 by more than 1e-3,
             or q_t(x_t) <= 0: falls back to one token drawn from p_0.
      bit 3  the residual has no mass (rounding only): draw from p_t instead.

    Returns (out_tokens int64 [B,K+1] padded with -1, n_accepted int64 [B],
    status int32 [B]) and, with return_trace, per-request dicts of the decisions.
    """
    target_bits = np.asarray(target_bits, dtype=np.uint16)
    tokens = np.asarray(tokens, dtype=np.int64)
    cand_idx = np.asarray(cand_idx, dtype=np.int64)
    B_, K = tokens.shape
    V = target_bits.shape[-1]
    out = np.full((B_, K + 1), -1, dtype=np.int64)
    n_acc = np.zeros(B_, dtype=np.int64)
    status = np.zeros(B_, dtype=np.int32)
    traces = []
    if temperature != 0.0:
        U_acc, U_res = verify_uniforms(seed, np.arange(B_)[:, None], np.arange(K + 1)[None, :])
    for b in range(B_):
        tr = {"accepts": [], "resample": None, "topp_margin": []}
        traces.append(tr)
        ids_bad = np.any((tokens[b] < 0) | (tokens[b] >= V)) or np.any((cand_idx[b] < 0) | (cand_idx[b] >= V))
        if temperature == 0.0:
            if ids_bad:
                status[b] |= 2
            t = 0
            while t < K:
                g = bf16_argmax(target_bits[b, t])
                if tokens[b, t] != g:
                    break
                out[b, t] = g
                t += 1
            out[b, t] = bf16_argmax(target_bits[b, t])
            n_acc[b] = t
            continue
        logits = bf16_to_f64(target_bits[b])
        if np.any(np.isnan(logits) | (logits == np.inf)):
            status[b] |= 1
            continue
        if top_k > 0 or top_p < 1.0:
            p = np.stack([filtered_target_probs(target_bits[b, t], temperature, top_k, top_p, tr["topp_margin"])
                          for t in range(K + 1)])
        else:
            p = np.stack([target_probs(target_bits[b, t], temperature) for t in range(K + 1)])
        qb = np.asarray(q[b], dtype=np.float64)
        q_bad = False
        for t in range(K):
            qt = qb[t]
            if not np.all(np.isfinite(qt)) or np.any(qt < 0) or abs(qt.sum() - 1.0) > 1e-3:
                q_bad = True
            elif not ids_bad and qt[cand_idx[b, t] == tokens[b, t]].sum() <= 0:
                q_bad = True
        if ids_bad:
            status[b] |= 2
        if q_bad:
            status[b] |= 4
        if ids_bad or q_bad:
            u_res = U_res[b, 0]
            out[b, 0] = _inverse_cdf(p[0], float(u_res))
            tr["resample"] = (0, "p", float(u_res))
            continue
        t = 0
        while t < K:
            u_acc, u_res = U_acc[b, t], U_res[b, t]
            x = tokens[b, t]
            qx = qb[t][cand_idx[b, t] == x].sum()
            accept = float(u_acc) * qx < p[t, x]
            tr["accepts"].append((t, float(u_acc), float(qx), float(p[t, x]), bool(accept)))
            if not accept:
                qfull = np.zeros(V)
                np.add.at(qfull, cand_idx[b, t], qb[t])
                r = np.maximum(0.0, p[t] - qfull)
                if r.sum() > 0:
                    out[b, t] = _inverse_cdf(r, float(u_res))
                    tr["resample"] = (t, "residual", float(u_res))
                else:
                    status[b] |= 8
                    out[b, t] = _inverse_cdf(p[t], float(u_res))
                    tr["resample"] = (t, "p", float(u_res))
                break
            out[b, t] = x
            t += 1
        if t == K:
            u_res = U_res[b, K]
            out[b, K] = _inverse_cdf(p[K], float(u_res))
            tr["resample"] = (K, "bonus", float(u_res))
        n_acc[b] = t
    if return_trace:
        return out, n_acc, status, traces
    return out, n_acc, status


# ----------------------------------------------------------------------------------
# LM head with the top-16 taken from its output (the draft side's adjacent step)
# ----------------------------------------------------------------------------------


def bf16_bits_of(values) -> np.ndarray:
    """bf16 bit patterns of values that are already bf16 numbers (exact, no rounding)."""
    v = np.asarray(values, dtype=np.float64).astype(np.float32)
    return (v.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def lmhead_logits(h_bits, w_bits):
    """Draft logits of a shared LM head: l[r, v] = bf16( sum_d h[r, d] * W[v, d] ).

    [FT] "Details", runtime: one draft forward over the block, then the target's LM
    head gives the 16 candidates of every slot; [RFC] "Questions", item 4: the draft
    shares the target's embedding and LM head.  The pages do not state the head's
    arithmetic.  Reading: the product of bf16 hidden rows and a bf16 weight [V, D],
    and logits stored as bf16, as the draft's logits are everywhere else on this
    path.  The oracle rounds the exact dot product once (float64 sums of exact bf16
    products are exact to about 1e-12 relative here), ties to even.

    h_bits uint16 [R, D], w_bits uint16 [V, D].  Returns (exact float64 [R, V],
    logit bits uint16 [R, V]).
    """
    h = bf16_to_f64(h_bits)
    w = bf16_to_f64(w_bits)
    exact = h @ w.T
    return exact, bf16_bits_of(round_to_bf16(exact))


def lmhead_topk16(h_bits, w_bits):
    """The top-16 candidates of every draft slot straight from the LM head's inputs:
    topk16 of lmhead_logits (same order: value desc, token id asc)."""
    _, bits = lmhead_logits(h_bits, w_bits)
    return topk16(bits)


# ----------------------------------------------------------------------------------
# Draft attention over the per-request K/V ring (sliding window)
# ----------------------------------------------------------------------------------


def ring_window_keys(ctx_len: int, window: int, ring: int):
    """Ring rows of the context keys one draft block reads, oldest first.

    [FT] "Details", runtime: the draft's K/V lives in a ring of 2112 positions per
    request (the 2048-token window plus 64 rows of room for a verify's rejected rows
    and for prefill rows past a snapshot boundary); prefix cache: the ring is rebuilt
    from the last 2047 context rows.  Reading: context position j sits in ring row
    j mod ring; the block reads the last min(ctx_len, window - 1) committed positions,
    so the window holds those plus the block's own first row, and no row of a position
    >= ctx_len (a rejected or not yet committed row) is ever read.
    """
    n = min(int(ctx_len), window - 1)
    return [(p % ring) for p in range(int(ctx_len) - n, int(ctx_len))]


def ring_attention(q, k_blk, v_blk, k_ring, v_ring, ctx_len, window: int = 2048, scale=None):
    """Non-causal draft-block attention over the window of each request's K/V ring.

    [FT] "Details": the released drafts use sliding-window attention (window 2048);
    the draft forward over [last token, mask x 7] reads the ring; a causal draft is
    refused at startup, so the block's rows see each other.  Reading: every query row
    of the block attends to the window's context keys (ring_window_keys) and to all
    block keys, softmax(q . k * scale) with scale = 1/sqrt(head_dim), grouped heads
    (query head h uses K/V head h // (Hq / Hkv)).  Rotary embedding is applied before
    (the ring holds rotated keys).  The oracle gathers the window into a dense key list
    and applies the definition in float64.

    q [B, nq, Hq, Dh], k_blk / v_blk [B, nq, Hkv, Dh], k_ring / v_ring
    [B, ring, Hkv, Dh] (float values; bf16 inputs are passed decoded), ctx_len [B].
    Returns (out float64 [B, nq, Hq, Dh], pv_abs [B, nq, Hq, Dh] = sum_k p_k |v_k| with
    normalised p, smax [B, nq, Hq] = max_k sum_d |q_d k_d| * scale).
    """
    q = np.asarray(q, dtype=np.float64)
    B, nq, Hq, Dh = q.shape
    Hkv = k_blk.shape[2]
    G = Hq // Hkv
    ring = k_ring.shape[1]
    scale = 1.0 / np.sqrt(Dh) if scale is None else scale
    out = np.zeros((B, nq, Hq, Dh))
    pv_abs = np.zeros((B, nq, Hq, Dh))
    smax = np.zeros((B, nq, Hq))
    for b in range(B):
        rows = ring_window_keys(ctx_len[b], window, ring)
        for hk in range(Hkv):
            K = np.concatenate([np.asarray(k_ring[b, rows, hk], dtype=np.float64),
                                np.asarray(k_blk[b, :, hk], dtype=np.float64)], axis=0)
            V = np.concatenate([np.asarray(v_ring[b, rows, hk], dtype=np.float64),
                                np.asarray(v_blk[b, :, hk], dtype=np.float64)], axis=0)
            for hq in range(hk * G, (hk + 1) * G):
                Q = q[b, :, hq]                             # [nq, Dh]
                s = Q @ K.T * scale                         # [nq, nkeys]
                p = np.exp(s - s.max(axis=1, keepdims=True))
                p /= p.sum(axis=1, keepdims=True)
                out[b, :, hq] = p @ V
                pv_abs[b, :, hq] = p @ np.abs(V)
                smax[b, :, hq] = (np.abs(Q) @ np.abs(K).T * scale).max(axis=1)
    return out, pv_abs, smax
