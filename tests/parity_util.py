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
    return stats


def check_accept(target_bits, tokens, cand_idx, q, temperature, seed, out, n_acc, status, top_k=0, top_p=1.0):
    """Compare a verify with the oracle; differences are allowed only where the oracle's
    own accept test, inverse-CDF draw or top-p cut lies within BAND of a boundary."""
    ref_out, ref_n, ref_st, traces = oracle.spec_accept(target_bits, tokens, cand_idx, q, temperature, seed,
                                                        return_trace=True, top_k=top_k, top_p=top_p)
    stats = {"requests": int(tokens.shape[0]), "band": 0}
    np.testing.assert_array_equal(status, ref_st)
    for b in range(tokens.shape[0]):
        if np.array_equal(out[b], ref_out[b]) and n_acc[b] == ref_n[b]:
            continue
        tr = traces[b]
        near = False
        for (t, u, qx, px, acc) in tr["accepts"]:
            if abs(u * qx - px) <= BAND * max(px, u * qx):
                near = True
        if any(m <= BAND for m in tr.get("topp_margin", [])):
            near = True
        if tr["resample"] is not None and not near:
            t, kind, u = tr["resample"]
            bits = np.asarray(target_bits[b, t])
            p = (oracle.filtered_target_probs(bits, temperature, top_k, top_p) if top_k > 0 or top_p < 1.0
                 else oracle.target_probs(bits, temperature))
            if kind == "residual":
                qfull = np.zeros(p.size)
                np.add.at(qfull, cand_idx[b, t], q[b, t])
                w = np.maximum(0.0, p - qfull)
            else:
                w = p
            P = np.concatenate([[0.0], np.cumsum(w)])
            Z = P[-1]
            for k in (ref_out[b, t], ref_out[b, t] + 1, out[b, t], out[b, t] + 1):
                if 0 <= k < P.size and abs(u * Z - P[k]) <= BAND * Z:
                    near = True
        assert near, ("verify differs outside the decision band", b, out[b].tolist(), ref_out[b].tolist())
        stats["band"] += 1
    return stats
