"""Filtered-target verify (top-k then top-p on the target distribution) of libdflash2
against the CPU oracle, through the C ABI.

The FreeToken runs sample with temperature 1.0, top_p 0.95 and top_k 20 (FreeToken PR
"Adds DFlash 2", "Speed"); these tests use that setting on the c4 shapes, other
settings on ragged and degenerate rows, and a Monte Carlo of the lossless property
with the filtered target.
"""

import numpy as np
import pytest

import oracle
from dflash_draft_selector_amd import synth
from parity_util import check_accept, cpu, to_gpu, to_gpu_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def d2():
    import torch
    from dflash_draft_selector_amd import dflash2
    dflash2.load_library()
    torch.cuda.init()
    return dflash2


_C4 = {}


def _c4(d2):
    if "x" not in _C4:
        w = synth.workload(4)
        inp = synth.make_inputs(w)
        A, B = to_gpu_bits(inp["emb_a_bits"]), to_gpu_bits(inp["emb_b_bits"])
        Hg = d2.context_gate(to_gpu(inp["h"]), to_gpu_bits(inp["w_h_bits"]), to_gpu(inp["bias"]))
        out = d2.select(to_gpu_bits(inp["logits_bits"]), to_gpu(inp["verified"]), A, B, Hg, w.temperature,
                        w.walk_seed)
        _C4["x"] = (w, inp, cpu(out["tokens"]), cpu(out["cand_idx"]), cpu(out["q"]))
    return _C4["x"]


def _padded(tb):
    """Rows padded to the 16-byte row stride; returns the [..., :V] view on the GPU."""
    V = tb.shape[-1]
    ld = (V + 7) // 8 * 8
    buf = np.zeros(tb.shape[:-1] + (ld,), np.uint16)
    buf[..., :V] = tb
    return to_gpu_bits(buf)[..., :V]


def _verify(d2, tb, tokens, cand, q, T, top_k, top_p, seed, **kw):
    o, n, st = d2.spec_accept_filtered(_padded(tb), to_gpu(tokens), to_gpu(cand), to_gpu(q.astype(np.float32)), T,
                                       top_k, top_p, seed=seed, **kw)
    return cpu(o), cpu(n), cpu(st)


@pytest.mark.parametrize("T,top_k,top_p", [(1.0, 20, 0.95), (0.6, 32, 0.8), (1.0, 7, 1.0), (1.5, 32, 0.5)])
def test_filtered_c4(d2, T, top_k, top_p):
    w, inp, tokens, cand, q = _c4(d2)
    tb = inp["target_bits"]
    print(f"filtered verify c4 T={T} top_k={top_k} top_p={top_p}", flush=True)
    o, n, st = _verify(d2, tb, tokens, cand, q, T, top_k, top_p, 11)
    stats = check_accept(tb, tokens, cand, q, T, 11, o, n, st, top_k=top_k, top_p=top_p)
    print("filtered verify stats", stats, "accepted", n.tolist(), flush=True)


def test_filtered_correlated_target_reaches_every_branch(d2):
    # target = a sharpened draft: drafts are often accepted, rejects resample from the
    # residual over the kept set, and requests that accept everything draw a bonus
    w, inp, tokens, cand, q = _c4(d2)
    rng = np.random.default_rng(8)
    draft = synth.bf16_bits_as_f32(inp["logits_bits"])
    tgt = 4.0 * np.concatenate([draft, draft[:, -1:]], axis=1) + rng.standard_normal((w.B, w.K + 1, w.V)).astype(
        np.float32) * 0.3
    tb = synth.f32_to_bf16_bits(tgt)
    o, n, st = _verify(d2, tb, tokens, cand, q, 1.0, 20, 0.95, 12)
    stats = check_accept(tb, tokens, cand, q, 1.0, 12, o, n, st, top_k=20, top_p=0.95)
    print("correlated filtered verify stats", stats, "accepted", n.tolist(), flush=True)
    assert n.max() > 0


def test_filtered_greedy_is_the_prefix_match(d2):
    w, inp, tokens, cand, q = _c4(d2)
    tb = inp["target_bits"]
    g = np.argmax(oracle.bf16_to_f64(tb), axis=-1)
    tokens = tokens.copy()
    for b in range(w.B):
        tokens[b, :b % (w.K + 1)] = g[b, :b % (w.K + 1)]
    o, n, st = _verify(d2, tb, tokens, cand, q, 0.0, 20, 0.95, 1)
    check_accept(tb, tokens, cand, q, 0.0, 1, o, n, st)


def test_filtered_top1_equals_greedy(d2):
    # top-k 1 leaves a one-hot p at the argmax: the result is the greedy prefix match
    w, inp, tokens, cand, q = _c4(d2)
    rng = np.random.default_rng(5)
    tb = inp["target_bits"].copy()
    g = np.argmax(oracle.bf16_to_f64(tb), axis=-1)
    tokens = tokens.copy()
    cand = cand.copy()
    for b in range(w.B):
        for t in range(b % (w.K + 1)):
            cand[b, t, 0] = g[b, t] if g[b, t] not in cand[b, t, 1:] else cand[b, t, 0]
            tokens[b, t] = cand[b, t, 0]
    qq = rng.dirichlet(np.ones(16), size=(w.B, w.K)).astype(np.float32)
    o1, n1, s1 = _verify(d2, tb, tokens, cand, qq, 1.0, 1, 1.0, 3)
    og, ng, sg = _verify(d2, tb, tokens, cand, qq, 0.0, 1, 1.0, 3)
    np.testing.assert_array_equal(o1, og)
    np.testing.assert_array_equal(n1, ng)
    assert np.all(s1 == 0)


@pytest.mark.parametrize("V", [16, 23, 77, 1003, 9729, 40000])
@pytest.mark.parametrize("top_k,top_p", [(1, 1.0), (5, 0.9), (20, 0.95), (32, 0.7)])
def test_filtered_small_and_ragged_vocab(d2, V, top_k, top_p):
    rng = np.random.default_rng(V + top_k)
    B, K, T = 6, 4, 0.8
    vals = rng.standard_normal((B, K + 1, V)).astype(np.float32) * 2.0
    tb = synth.f32_to_bf16_bits(vals)
    pf = np.stack([[oracle.filtered_target_probs(tb[b, t], T, top_k, top_p) for t in range(K + 1)] for b in range(B)])
    p = np.stack([[oracle.target_probs(tb[b, t], T) for t in range(K + 1)] for b in range(B)])
    cand = np.argsort(-p[:, :K], axis=-1, kind="stable")[..., :16].astype(np.int32)
    qq = np.take_along_axis(pf[:, :K] + 1e-3, cand.astype(np.int64), axis=-1)
    qq = 0.5 * qq / qq.sum(-1, keepdims=True) + 0.5 * rng.dirichlet(np.ones(16), size=(B, K))
    qq = (qq / qq.sum(-1, keepdims=True)).astype(np.float32)
    tokens = cand[:, :, 0].copy()
    print(f"filtered verify V={V} top_k={top_k} top_p={top_p}", flush=True)
    o, n, st = _verify(d2, tb, tokens, cand, qq, T, top_k, top_p, V)
    check_accept(tb, tokens, cand, qq, T, V, o, n, st, top_k=top_k, top_p=top_p)


def test_filtered_ties_and_degenerate_rows(d2):
    """Rows whose top_k is decided by ties: a constant row (every sub-chunk gathers far
    more than its capacity and raises its bound), a row of few distinct values, +0 and
    -0 mixed, and a row whose best values sit in its last, ragged vector."""
    B, K, V = 4, 3, 40003
    rng = np.random.default_rng(61)
    tb = synth.f32_to_bf16_bits(rng.standard_normal((B, K + 1, V)).astype(np.float32))
    tb[0, 0, :] = 0x3F80                                       # all 1.0
    tb[0, 1, :] = synth.f32_to_bf16_bits(rng.integers(0, 3, V).astype(np.float32))   # values 0, 1, 2
    tb[1, 0, :] = np.where(rng.random(V) < 0.5, 0x0000, 0x8000)                      # +0 / -0
    tb[1, 1, V - 5:] = 0x4200                                  # 32.0 in the ragged tail
    tb[2, 2, ::97] = 0x4100                                    # 8.0 at every 97th id
    cand = np.stack([np.stack([rng.choice(V, 16, replace=False) for _ in range(K)]) for _ in range(B)]).astype(np.int32)
    cand[0, 0, :5] = [0, 1, 2, 3, 4]
    qq = rng.dirichlet(np.ones(16), size=(B, K)).astype(np.float32)
    tokens = cand[:, :, 0].copy()
    for T, top_k, top_p in ((1.0, 20, 0.95), (0.5, 32, 1.0), (2.0, 3, 0.6)):
        print(f"filtered verify ties T={T} top_k={top_k} top_p={top_p}", flush=True)
        o, n, st = _verify(d2, tb, tokens, cand, qq, T, top_k, top_p, 17)
        check_accept(tb, tokens, cand, qq, T, 17, o, n, st, top_k=top_k, top_p=top_p)


def test_filtered_fault_rows(d2):
    rng = np.random.default_rng(14)
    B, K, V = 6, 3, 5000
    tb = synth.f32_to_bf16_bits(rng.standard_normal((B, K + 1, V)).astype(np.float32))
    cand = np.stack([np.stack([rng.choice(V, 16, replace=False) for _ in range(K)]) for _ in range(B)]).astype(np.int32)
    qq = np.full((B, K, 16), 1.0 / 16, np.float32)
    tokens = cand[:, :, 0].copy()
    tb[0, 1, 77] = 0x7FC0                 # NaN target -> bit 0
    qq[1, 0, 3] = np.nan                  # NaN q -> bit 2
    qq[2, 2] *= 0.5                       # wrong total -> bit 2
    tokens[3, 1] = V + 4                  # out-of-range draft -> bit 1
    qq[4, 1, :] = 0.0                     # q(x) = 0 -> bit 2
    qq[4, 1, 5] = 1.0
    tb[5, 0, 4999] = 0x7F80               # +inf in the last logit -> bit 0
    o, n, st = _verify(d2, tb, tokens, cand, qq, 1.0, 20, 0.95, 3)
    check_accept(tb, tokens, cand, qq, 1.0, 3, o, n, st, top_k=20, top_p=0.95)
    assert st.tolist() == [1, 4, 4, 2, 4, 1]


def test_filtered_shared_target_and_k64(d2):
    rng = np.random.default_rng(71)
    B, K, V = 3, 64, 5000
    tb = synth.f32_to_bf16_bits(rng.standard_normal((K + 1, V)).astype(np.float32) * 3.0)
    cand = np.stack([np.stack([rng.choice(V, 16, replace=False) for _ in range(K)]) for _ in range(B)]).astype(np.int32)
    qq = rng.dirichlet(np.ones(16), size=(B, K)).astype(np.float32)
    tokens = cand[:, :, 0].copy()
    # request 2's drafts carry almost all of the target's mass: all 64 are accepted and
    # the bonus comes from row 64
    full = np.broadcast_to(tb, (B, K + 1, V)).copy()
    for t in range(K):
        full[2, t, tokens[2, t]] = synth.f32_to_bf16_bits(np.float32(60.0))[0]
    o, n, st = _verify(d2, full, tokens, cand, qq, 0.9, 20, 0.95, 9)
    check_accept(full, tokens, cand, qq, 0.9, 9, o, n, st, top_k=20, top_p=0.95)
    assert n[2] == K
    o1, n1, s1 = d2.spec_accept_filtered(_padded(tb), to_gpu(tokens), to_gpu(cand), to_gpu(qq), 0.9, 20, 0.95, seed=4,
                                         shared_target=True)
    o2, n2, s2 = _verify(d2, np.broadcast_to(tb, (B, K + 1, V)), tokens, cand, qq, 0.9, 20, 0.95, 4)
    np.testing.assert_array_equal(cpu(o1), o2)
    np.testing.assert_array_equal(cpu(n1), n2)


def test_filtered_monte_carlo_marginals(d2):
    # the lossless property with the filtered target: conditional on reaching position
    # t, the committed token follows the filtered p_t (zero outside its kept set);
    # 10^6 requests of one c4 request's drafts against a correlated target
    import torch
    w, inp, tokens, cand, q = _c4(d2)
    A, B = to_gpu_bits(inp["emb_a_bits"]), to_gpu_bits(inp["emb_b_bits"])
    Hg = d2.context_gate(to_gpu(inp["h"]), to_gpu_bits(inp["w_h_bits"]), to_gpu(inp["bias"]))
    out = d2.select(to_gpu_bits(inp["logits_bits"]), to_gpu(inp["verified"]), A, B, Hg, w.temperature, w.walk_seed)
    S0, cand0 = out["S"][0:1].contiguous(), out["cand_idx"][0:1].contiguous()
    rng = np.random.default_rng(45)
    draft0 = synth.bf16_bits_as_f32(inp["logits_bits"][0])
    tgt = 1.5 * np.concatenate([draft0, draft0[-1:]], axis=0) + 0.5 * rng.standard_normal((w.K + 1, w.V)).astype(
        np.float32)
    tb0 = synth.f32_to_bf16_bits(tgt)
    T, top_k, top_p, chunk, total = 1.0, 20, 0.95, 10 ** 5, 10 ** 6
    K, V = w.K, w.V
    counts = torch.zeros((K + 1, V), dtype=torch.int64, device="cuda")
    reach = np.zeros(K + 1, dtype=np.int64)
    S_rep = S0.expand(chunk, -1, -1, -1).contiguous()
    cand_rep = cand0.expand(chunk, -1, -1).contiguous()
    tgt_g = _padded(tb0)
    for c in range(total // chunk):
        tok, slots, qg = d2.walk(S_rep, cand_rep, T, seed=3000 + c)
        o, n, st = d2.spec_accept_filtered(tgt_g, tok, cand_rep, qg, T, top_k, top_p, seed=4000 + c,
                                           shared_target=True)
        assert int(st.abs().sum()) == 0
        for t in range(K + 1):
            col = o[:, t]
            m = col >= 0
            reach[t] += int(m.sum())
            counts[t] += torch.bincount(col[m].long(), minlength=V)
        if c == 0:
            nreq = 150
            check_accept(np.broadcast_to(tb0, (nreq, K + 1, V)), cpu(tok[:nreq]), cpu(cand_rep[:nreq]),
                         cpu(qg[:nreq]), T, 4000, cpu(o[:nreq]), cpu(n[:nreq]), cpu(st[:nreq]), top_k=top_k,
                         top_p=top_p)
    counts = cpu(counts)
    worst = []
    for t in range(K + 1):
        if reach[t] < 10 ** 5:
            continue
        p = oracle.filtered_target_probs(tb0[t], T, top_k, top_p)
        freq = counts[t] / reach[t]
        assert np.all(freq[p == 0] == 0), t
        dev = np.abs(freq - p).max()
        worst.append((t, int(reach[t]), float(dev)))
        assert dev <= 5e-3, (t, dev)
    print("filtered MC (t, rows, max |freq - p|):", worst, "reach:", reach.tolist(), flush=True)
    assert len(worst) >= 2
