"""Comparison rules between libdflash2 and the CPU oracle.

  * integer / index outputs (candidates, slots, tokens): bit-exact, except walk steps
    and verify draws whose decision the oracle itself places within a relative 1e-5
    of a tie or a CDF boundary; those are counted and reported, never silently passed.
  * floating point: |got - ref| <= 1e-4 * (sum of the magnitudes of the terms), which
    is the plain relative error when nothing cancels (scores, gate, conv).
"""

from __future__ import annotations

import numpy as np

import oracle

REL = 1e-4          # floating-point tolerance, relative to the term-magnitude sum
BAND = 1e-5         # decision band (near ties / near CDF boundaries)


def to_gpu_bits(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda()


def to_gpu(a, dtype=None):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def cpu(t):
    return t.detach().cpu().numpy()


def assert_close_scaled(got, ref, scale, rel=REL, what=""):
    got = np.asarray(got, dtype=np.float64)
    err = np.abs(got - ref)
    lim = rel * np.asarray(scale) + 1e-30
    bad = err > lim
    if bad.any():
        i = np.unravel_index(np.argmax(err / lim), err.shape)
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} outside tolerance; worst at {i}: "
                             f"got {got[i]!r} ref {ref[i]!r} scale {np.asarray(scale)[i]!r}")


# Decision counts of every check in this process; the test session prints them and
# writes them to parity_counts.json in the run's output folder (tests/conftest.py).
COUNTS = {"walk_steps": 0, "walk_near_ties": 0, "walk_band": 0, "verify_requests": 0, "verify_band": 0}


def check_walk(S_ref, cand_idx, tokens, slots, q, temperature, seed):
    """Teacher-forced check of a walk: every step is re-decided by the oracle on the
    predecessor slot the library chose.  Returns counts {steps, near_ties, band}."""
    S_ref = np.asarray(S_ref, dtype=np.float64)
    B, K = slots.shape
    stats = {"steps": 0, "near_ties": 0, "band": 0}
    for b in range(B):
        for t in range(K):
            stats["steps"] += 1
            i = 0 if t == 0 else int(slots[b, t - 1])
            row = S_ref[b, t, i]
            j = int(slots[b, t])
            assert tokens[b, t] == cand_idx[b, t, j], (b, t)
            if temperature == 0.0:
                jr = oracle.greedy_pick(row)
                srt = np.sort(row[np.isfinite(row)])[::-1]
                if srt.size > 1 and srt[0] - srt[1] <= BAND * max(abs(srt[0]), abs(srt[1])):
                    stats["near_ties"] += 1
                if j != jr:
                    s1, sg = row[jr], row[j]
                    assert s1 - sg <= BAND * max(abs(s1), abs(sg)), ("greedy step differs outside the tie band", b, t, j, jr)
                    stats["band"] += 1
                qref = np.zeros(16)
                qref[j] = 1.0
                assert np.array_equal(q[b, t], qref), (b, t)
            else:
                u = float(oracle.walk_uniform(seed, b, t))
                jr, qref = oracle.sample_pick(row, temperature, u)
                if j != jr:
                    fin = np.isfinite(row)
                    w = np.where(fin, np.exp((np.where(fin, row, 0) - row[fin].max()) / temperature), 0.0)
                    P = np.concatenate([[0.0], np.cumsum(w)])
                    W = P[-1]
                    near = any(abs(u * W - P[k]) <= BAND * W for k in {j, j + 1, jr, jr + 1} if 0 <= k < P.size)
                    assert near, ("sampled step differs outside the boundary band", b, t, j, jr)
                    stats["band"] += 1
                assert np.abs(q[b, t] - qref).max() <= REL, (b, t)
    COUNTS["walk_steps"] += stats["steps"]
    COUNTS["walk_near_ties"] += stats["near_ties"]
    COUNTS["walk_band"] += stats["band"]
    return stats


def _draw_near(weights, u, picks):
    """Whether u * Z lies within BAND * Z of the inverse-CDF boundary below or above any
    of the picked tokens (Z = total weight, boundaries in token-id order)."""
    P = np.concatenate([[0.0], np.cumsum(weights)])
    Z = P[-1]
    return any(0 <= k < P.size and abs(u * Z - P[k]) <= BAND * Z for v in picks for k in (v, v + 1))


def check_accept(target_bits, tokens, cand_idx, q, temperature, seed, out, n_acc, status, top_k=0, top_p=1.0):
    """Compare a verify with the oracle.  A request may differ only at its first
    divergent position t, and only where the oracle's decision at t lies within BAND of
    a boundary: the accept test at t (the library took the other branch), the inverse-CDF
    draw at t (both rejected, or both reached the bonus, and drew different tokens), or
    the top-p cut of target row t (the filtered p of that row moved).  Greedy verifies
    (integer argmax over bf16 keys) must match exactly."""
    ref_out, ref_n, ref_st, traces = oracle.spec_accept(target_bits, tokens, cand_idx, q, temperature, seed,
                                                        return_trace=True, top_k=top_k, top_p=top_p)
    stats = {"requests": int(tokens.shape[0]), "band": 0}
    np.testing.assert_array_equal(status, ref_st)
    K = tokens.shape[1]
    for b in range(tokens.shape[0]):
        if np.array_equal(out[b], ref_out[b]) and n_acc[b] == ref_n[b]:
            continue
        assert temperature != 0.0, ("greedy verify differs", b, out[b].tolist(), ref_out[b].tolist())
        diff = np.flatnonzero(out[b] != ref_out[b])
        assert diff.size, ("same tokens, different accepted counts", b, int(n_acc[b]), int(ref_n[b]))
        t = int(diff[0])
        tr = traces[b]
        margins = tr.get("topp_margin", [])
        near = bool(margins) and t < len(margins) and margins[t] <= BAND
        accepts = {a[0]: a for a in tr["accepts"]}
        took_draft = t < K and out[b, t] == tokens[b, t]
        if not near and t in accepts:
            _, u, qx, px, acc = accepts[t]
            # the oracle accepted and the library did not, or the reverse
            if acc != took_draft and abs(u * qx - px) <= BAND * max(px, u * qx):
                near = True
        if not near and tr["resample"] is not None and tr["resample"][0] == t and not took_draft:
            _, kind, u = tr["resample"]
            bits = np.asarray(target_bits[b, t])
            p = (oracle.filtered_target_probs(bits, temperature, top_k, top_p) if top_k > 0 or top_p < 1.0
                 else oracle.target_probs(bits, temperature))
            if kind == "residual":
                qfull = np.zeros(p.size)
                np.add.at(qfull, cand_idx[b, t], q[b, t])
                w = np.maximum(0.0, p - qfull)
            else:
                w = p
            near = _draw_near(w, u, (int(ref_out[b, t]), int(out[b, t])))
        assert near, ("verify differs outside the decision band at its first divergent position", b, t,
                      out[b].tolist(), ref_out[b].tolist())
        stats["band"] += 1
    COUNTS["verify_requests"] += stats["requests"]
    COUNTS["verify_band"] += stats["band"]
    return stats
