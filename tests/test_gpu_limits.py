"""Parity at the limits of the C ABI: the largest draft block (K = 64), every selector
width the pair kernels are built for (the powers of two from 16 to 1024), both sides of
the walk's staging limit (the step distributions of up to 16 positions staged in LDS),
fp32 and bf16 tables, the largest vocabulary (2^19) and a ragged one, batches at and past
whole lanes of 8 requests, through the C ABI against the oracle."""

import numpy as np
import pytest

import oracle
from dflash_draft_selector_amd import synth
from parity_util import assert_close_scaled, check_accept, check_walk, cpu, to_gpu, to_gpu_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def d2():
    import torch
    from dflash_draft_selector_amd import dflash2
    dflash2.load_library()
    torch.cuda.init()
    return dflash2


def _tables(inp):
    if "emb_a_bits" in inp:
        return (oracle.bf16_to_f64(inp["emb_a_bits"]), oracle.bf16_to_f64(inp["emb_b_bits"]),
                to_gpu_bits(inp["emb_a_bits"]), to_gpu_bits(inp["emb_b_bits"]),
                oracle.bf16_to_f64(inp["w_h_bits"]), to_gpu_bits(inp["w_h_bits"]), True)
    return (inp["emb_a"], inp["emb_b"], to_gpu(inp["emb_a"]), to_gpu(inp["emb_b"]), inp["w_h"], to_gpu(inp["w_h"]),
            False)


@pytest.mark.parametrize("dim,bf16", [(64, True), (128, False), (512, True)])
def test_select_k64_every_selector_width(d2, dim, bf16):
    w = synth.workload(0, B=2, K=64, V=5000, D=96, dim=dim, bf16_params=bf16, peak="decay")
    inp = synth.make_inputs(w)
    A64, B64, Ag, Bg, W64, Wg, wb = _tables(inp)
    logits, ver = to_gpu_bits(inp["logits_bits"]), to_gpu(inp["verified"])
    Hg = d2.context_gate(to_gpu(inp["h"]), Wg, to_gpu(inp["bias"]))
    Href, _, pre_abs = oracle.context_gate(inp["h"].reshape(-1, w.D), W64, inp["bias"], wb)
    assert_close_scaled(cpu(Hg).reshape(-1, dim), Href, 0.25 * pre_abs, what=f"gate dim {dim}")
    ridx, rval = oracle.topk16(inp["logits_bits"])
    H32 = cpu(Hg).astype(np.float64)
    Sref, Sabs, rst = oracle.pair_score(ridx, rval, inp["verified"], A64, B64, H32)
    for T, seed in ((0.0, 0), (0.7, 5)):
        print(f"select K=64 dim={dim} bf16={bf16} T={T}", flush=True)
        out = d2.select(logits, ver, Ag, Bg, Hg, T, seed)
        np.testing.assert_array_equal(cpu(out["cand_idx"]), ridx)
        assert_close_scaled(cpu(out["S"]), Sref, Sabs, what=f"S dim {dim}")
        np.testing.assert_array_equal(cpu(out["row_status"]), rst)
        stats = check_walk(Sref, ridx, cpu(out["tokens"]), cpu(out["slots"]), cpu(out["q"]), T, seed)
        print("walk stats", stats, flush=True)
        # the fused call equals the three separate calls bit for bit
        idx, val = d2.topk16(logits)
        S, st = d2.pair_score(idx, val, ver, Ag, Bg, Hg)
        tok, slots, q = d2.walk(S, idx, T, seed)
        for name, ref in (("S", S), ("tokens", tok), ("slots", slots), ("q", q)):
            a, b = cpu(out[name]), cpu(ref)
            np.testing.assert_array_equal(a.view(np.uint32) if a.dtype == np.float32 else a,
                                          b.view(np.uint32) if b.dtype == np.float32 else b, err_msg=name)


@pytest.mark.parametrize("dim,K,bf16", [(16, 7, True), (16, 17, False), (32, 16, True), (32, 3, False),
                                        (256, 16, True), (256, 17, True), (1024, 8, True), (1024, 9, False)])
def test_select_selector_widths_and_block_limit(d2, dim, K, bf16):
    """Each width with a draft block on either side of the walk's staging limit (the
    step distributions of K <= 16 positions are staged in LDS, longer blocks read them
    from memory): the oracle's candidates, scores within tolerance, the walk
    teacher-forced, and bit-identity with the three separate calls."""
    w = synth.workload(0, B=3, K=K, V=3000, D=64, dim=dim, bf16_params=bf16, peak="decay")
    inp = synth.make_inputs(w)
    A64, B64, Ag, Bg, W64, Wg, wb = _tables(inp)
    logits, ver = to_gpu_bits(inp["logits_bits"]), to_gpu(inp["verified"])
    Hg = d2.context_gate(to_gpu(inp["h"]), Wg, to_gpu(inp["bias"]))
    ridx, rval = oracle.topk16(inp["logits_bits"])
    Sref, Sabs, rst = oracle.pair_score(ridx, rval, inp["verified"], A64, B64, cpu(Hg).astype(np.float64))
    for T, seed in ((0.0, 0), (1.3, 8)):
        print(f"select dim={dim} K={K} bf16={bf16} T={T}", flush=True)
        out = d2.select(logits, ver, Ag, Bg, Hg, T, seed)
        np.testing.assert_array_equal(cpu(out["cand_idx"]), ridx)
        assert_close_scaled(cpu(out["S"]), Sref, Sabs, what=f"S dim {dim} K {K}")
        np.testing.assert_array_equal(cpu(out["row_status"]), rst)
        check_walk(Sref, ridx, cpu(out["tokens"]), cpu(out["slots"]), cpu(out["q"]), T, seed)
        idx, val = d2.topk16(logits)
        S, st = d2.pair_score(idx, val, ver, Ag, Bg, Hg)
        tok, slots, q = d2.walk(S, idx, T, seed)
        for name, ref in (("S", S), ("tokens", tok), ("slots", slots), ("q", q), ("row_status", st)):
            a, b = cpu(out[name]), cpu(ref)
            np.testing.assert_array_equal(a.view(np.uint32) if a.dtype == np.float32 else a,
                                          b.view(np.uint32) if b.dtype == np.float32 else b, err_msg=name)


def test_select_gated_k64(d2):
    import torch
    w = synth.workload(0, B=2, K=64, V=5000, D=200, dim=128, bf16_params=True, peak="decay")
    inp = synth.make_inputs(w)
    A64, B64, Ag, Bg, W64, Wg, _ = _tables(inp)
    logits, ver = to_gpu_bits(inp["logits_bits"]), to_gpu(inp["verified"])
    Hout = torch.empty((w.B, w.K, w.dim), dtype=torch.float32, device=logits.device)
    print("gated select K=64", flush=True)
    out = d2.select_gated(logits, ver, Ag, Bg, to_gpu(inp["h"]), Wg, to_gpu(inp["bias"]), "sigmoid", 0.9, 3,
                          H_out=Hout)
    Href, _, pre_abs = oracle.context_gate(inp["h"].reshape(-1, w.D), W64, inp["bias"], True)
    assert_close_scaled(cpu(Hout).reshape(-1, w.dim), Href, 0.25 * pre_abs, what="gated H K=64")
    ref = d2.select(logits, ver, Ag, Bg, Hout, 0.9, 3)
    for k in ref:
        a, b = cpu(out[k]), cpu(ref[k])
        np.testing.assert_array_equal(a.view(np.uint32) if a.dtype == np.float32 else a,
                                      b.view(np.uint32) if b.dtype == np.float32 else b, err_msg=k)


@pytest.mark.parametrize("V,ld", [(1 << 19, 1 << 19), (524285, 1 << 19)])
def test_topk16_largest_vocabulary(d2, V, ld):
    rng = np.random.default_rng(7)
    rows = 3
    logits = synth.f32_to_bf16_bits(rng.standard_normal((rows, ld), dtype=np.float32) * 3.0)
    logits[0, V - 1] = synth.f32_to_bf16_bits(np.array([40.0], dtype=np.float32))[0]   # best logit is the last one
    logits[1, :] = logits[1, 0]                                                          # a constant row
    print(f"topk16 V={V} ld={ld}", flush=True)
    g = to_gpu_bits(logits)[:, :V] if V != ld else to_gpu_bits(logits)
    idx, val, st = d2.topk16(g, row_status=True)
    ridx, rval = oracle.topk16(logits[:, :V])
    np.testing.assert_array_equal(cpu(idx), ridx)
    np.testing.assert_array_equal(cpu(val).astype(np.float64), rval)
    assert cpu(idx)[0, 0] == V - 1


@pytest.mark.parametrize("temperature", [0.0, 0.8])
def test_spec_accept_k64(d2, temperature):
    w = synth.workload(0, B=3, K=64, V=5000, D=96, dim=128, bf16_params=True, peak="decay")
    inp = synth.make_inputs(w)
    _, _, Ag, Bg, _, Wg, _ = _tables(inp)
    rng = np.random.default_rng(21)
    target = synth.f32_to_bf16_bits(rng.standard_normal((w.B, w.K + 1, w.V), dtype=np.float32) * 3.0)
    Hg = d2.context_gate(to_gpu(inp["h"]), Wg, to_gpu(inp["bias"]))
    out = d2.select(to_gpu_bits(inp["logits_bits"]), to_gpu(inp["verified"]), Ag, Bg, Hg, max(temperature, 0.5), 2)
    tokens, cand, q = cpu(out["tokens"]), cpu(out["cand_idx"]), cpu(out["q"])
    if temperature == 0.0:
        gmax = np.argmax(oracle.bf16_to_f64(target), axis=-1)
        for b, n in enumerate((0, 17, 64)):
            tokens[b, :n] = gmax[b, :n]
    else:
        # request 2's drafts carry almost all of the target's mass: every position is
        # accepted and the bonus token comes from row 64
        for t in range(w.K):
            target[2, t, tokens[2, t]] = synth.f32_to_bf16_bits(np.array([60.0], dtype=np.float32))[0]
    print(f"spec_accept K=64 T={temperature}", flush=True)
    o, n, st = d2.spec_accept(to_gpu_bits(target), to_gpu(tokens), to_gpu(cand), to_gpu(q), temperature, seed=13)
    stats = check_accept(target, tokens, cand, q, temperature, 13, cpu(o), cpu(n), cpu(st))
    if temperature == 0.0:
        assert cpu(n).tolist() == [0, 17, 64]
    else:
        assert cpu(n)[2] == 64
    print("verify stats", stats, flush=True)


@pytest.mark.parametrize("B", [8, 9, 17])
def test_select_and_verify_across_xcd_lanes(d2, B):
    """Batches at and just past whole lanes of 8 requests (the streams place each
    request's work-groups on one XCD, padding the grid to whole lanes): the select
    against the oracle and equal to the three separate calls, and the sampled, filtered
    and greedy verifies against the oracle."""
    w = synth.workload(0, B=B, K=3, V=3000, D=64, dim=64, bf16_params=True, peak="decay")
    inp = synth.make_inputs(w)
    A64, B64, Ag, Bg, W64, Wg, wb = _tables(inp)
    logits, ver = to_gpu_bits(inp["logits_bits"]), to_gpu(inp["verified"])
    Hg = d2.context_gate(to_gpu(inp["h"]), Wg, to_gpu(inp["bias"]))
    ridx, rval = oracle.topk16(inp["logits_bits"])
    Sref, Sabs, rst = oracle.pair_score(ridx, rval, inp["verified"], A64, B64, cpu(Hg).astype(np.float64))
    print(f"select B={B} (lanes of 8)", flush=True)
    out = d2.select(logits, ver, Ag, Bg, Hg, 1.0, 4)
    np.testing.assert_array_equal(cpu(out["cand_idx"]), ridx)
    assert_close_scaled(cpu(out["S"]), Sref, Sabs, what=f"S B {B}")
    np.testing.assert_array_equal(cpu(out["row_status"]), rst)
    check_walk(Sref, ridx, cpu(out["tokens"]), cpu(out["slots"]), cpu(out["q"]), 1.0, 4)
    idx, val = d2.topk16(logits)
    S, st = d2.pair_score(idx, val, ver, Ag, Bg, Hg)
    tok, slots, q = d2.walk(S, idx, 1.0, 4)
    for name, ref in (("S", S), ("tokens", tok), ("slots", slots), ("q", q)):
        a, b = cpu(out[name]), cpu(ref)
        np.testing.assert_array_equal(a.view(np.uint32) if a.dtype == np.float32 else a,
                                      b.view(np.uint32) if b.dtype == np.float32 else b, err_msg=name)
    rng = np.random.default_rng(40 + B)
    target = synth.f32_to_bf16_bits(rng.standard_normal((w.B, w.K + 1, w.V), dtype=np.float32) * 3.0)
    tokens, cand, qd = cpu(out["tokens"]), cpu(out["cand_idx"]), cpu(out["q"])
    for T, kw in ((1.0, {}), (1.0, {"top_k": 20, "top_p": 0.95}), (0.0, {})):
        print(f"verify B={B} T={T} {kw}", flush=True)
        if kw:
            o, n, vst = d2.spec_accept_filtered(to_gpu_bits(target), out["tokens"], out["cand_idx"], out["q"], T,
                                                seed=6, **kw)
        else:
            o, n, vst = d2.spec_accept(to_gpu_bits(target), out["tokens"], out["cand_idx"], out["q"], T, seed=6)
        check_accept(target, tokens, cand, qd, T, 6, cpu(o), cpu(n), cpu(vst), **kw)
