"""Parity of libdflash2 (HIP, gfx950) with the CPU oracle, through the C ABI.

Sizes: the tiny workload c0 and the full single-GPU workloads c1, c2, c4 in full; c3 with
the candidates and gate of all 960 rows and the scores and walk of 16 requests; ragged
vocabularies and degenerate rows for the edge cases.
"""

import numpy as np
import pytest

import oracle
from dflash_draft_selector_amd import synth
from parity_util import (REL, assert_close_scaled, check_accept, check_walk, cpu, to_gpu, to_gpu_bits)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def d2():
    import torch
    from dflash_draft_selector_amd import dflash2
    dflash2.load_library()
    torch.cuda.init()
    return dflash2


_INPUTS = {}


def inputs(i, **over):
    key = (i, tuple(sorted(over.items())))
    if key not in _INPUTS:
        _INPUTS[key] = synth.make_inputs(synth.workload(i, **over))
    return _INPUTS[key]


def tables(inp):
    if "emb_a_bits" in inp:
        return (oracle.bf16_to_f64(inp["emb_a_bits"]), oracle.bf16_to_f64(inp["emb_b_bits"]),
                to_gpu_bits(inp["emb_a_bits"]), to_gpu_bits(inp["emb_b_bits"]))
    return inp["emb_a"], inp["emb_b"], to_gpu(inp["emb_a"]), to_gpu(inp["emb_b"])


def gate_w(inp):
    if "w_h_bits" in inp:
        return oracle.bf16_to_f64(inp["w_h_bits"]), to_gpu_bits(inp["w_h_bits"]), True
    return inp["w_h"], to_gpu(inp["w_h"]), False


# ------------------------------------------------------------------ top-16 ----------


@pytest.mark.parametrize("wl", [0, 1, 2])
def test_topk16_exact(d2, wl):
    inp = inputs(wl)
    print(f"topk16 workload c{wl}", flush=True)
    idx, val, st = d2.topk16(to_gpu_bits(inp["logits_bits"]), row_status=True)
    ridx, rval = oracle.topk16(inp["logits_bits"])
    np.testing.assert_array_equal(cpu(idx), ridx)
    np.testing.assert_array_equal(cpu(val).astype(np.float64), rval)
    assert np.all(cpu(st) == 0)


def _bits_of(vals):
    return (np.asarray(vals, np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def test_topk16_edge_rows(d2):
    import torch
    rng = np.random.default_rng(31)
    for V in (16, 17, 23, 4096, 16384, 16392, 40003, 151936):
        rows = []
        rows.append(np.full(V, 0x4000, np.uint16))                                     # constant
        rows.append(_bits_of(np.arange(V, dtype=np.float32)))                           # increasing
        rows.append(_bits_of(-np.arange(V, dtype=np.float32)))                          # decreasing
        r = _bits_of(rng.choice([-1.0, -0.0, 0.0, 0.5], size=V).astype(np.float32))    # zeros and ties
        rows.append(r)
        r = synth.f32_to_bf16_bits(rng.standard_normal(V).astype(np.float32) * 3)
        r[rng.integers(0, V, max(1, V // 50))] = 0x7FC0                                 # NaNs
        rows.append(r)
        r = np.full(V, 0x7FC0, np.uint16)
        r[rng.integers(0, V, 5)] = synth.f32_to_bf16_bits(rng.standard_normal(5).astype(np.float32))
        rows.append(r)                                                                  # mostly NaN
        r = synth.f32_to_bf16_bits(-np.abs(rng.standard_normal(V).astype(np.float32)) - 1)
        rows.append(r)                                                                  # all negative
        r = synth.f32_to_bf16_bits(rng.standard_normal(V).astype(np.float32))
        r[rng.integers(0, V, 3)] = 0x7F80
        r[rng.integers(0, V, 3)] = 0xFF80
        rows.append(r)                                                                  # +-inf
        bits = np.stack(rows)
        ld = (V + 7) // 8 * 8 + 8 * int(rng.integers(0, 3))
        buf = np.zeros((bits.shape[0], ld), np.uint16)
        buf[:, :V] = bits
        g = to_gpu_bits(buf)[:, :V]
        print(f"topk16 edge rows V={V} ld={ld}", flush=True)
        idx, val, st = d2.topk16(g, row_status=True)
        ridx, rval = oracle.topk16(bits)
        np.testing.assert_array_equal(cpu(idx), ridx, err_msg=f"V={V}")
        np.testing.assert_array_equal(cpu(val).view(np.uint32) >> 16, _bits_of(rval.astype(np.float32)).astype(np.uint32))
        want_st = (~np.isfinite(rval)).any(axis=1).astype(np.int32)
        np.testing.assert_array_equal(cpu(st), want_st)
        torch.cuda.synchronize()


# ------------------------------------------------------------------ gate ------------


@pytest.mark.parametrize("wl", [0, 2, 3])
def test_context_gate(d2, wl):
    inp = inputs(wl)
    w = synth.workload(wl)
    W64, Wg, is_bf16 = gate_w(inp)
    h = inp["h"].reshape(-1, w.D)
    if wl == 3:
        h = h[:300]
    print(f"gate c{wl} rows={h.shape[0]}", flush=True)
    for act in ("sigmoid", "identity"):
        H = cpu(d2.context_gate(to_gpu(h), Wg, to_gpu(inp["bias"]), act=act))
        Href, pre, pre_abs = oracle.context_gate(h, W64, inp["bias"], is_bf16, act=act)
        scale = pre_abs * (0.25 if act == "sigmoid" else 1.0)
        assert_close_scaled(H, Href, scale, what=f"gate {act}")


def test_context_gate_ragged(d2):
    rng = np.random.default_rng(4)
    # From 256 rows a bf16 weight takes wide tiles (64 rows x 256 columns over parts of
    # the hidden dimension) when dim is a multiple of 256 and hidden of 128: two column
    # tiles with one-stage parts, one part (H written by the tiles), uneven parts of two
    # and three stages with a ragged last row group.
    for rows, hidden, dim in ((1, 8, 16), (17, 520, 64), (33, 1000, 128), (5, 4096, 1024), (300, 200, 128),
                              (257, 1032, 256), (300, 1024, 512), (300, 128, 256), (1000, 5120, 256),
                              (640, 384, 256)):
        h = rng.standard_normal((rows, hidden)).astype(np.float32)
        w = (rng.standard_normal((dim, hidden)) / np.sqrt(hidden)).astype(np.float32)
        wb = synth.f32_to_bf16_bits(w)
        b = rng.standard_normal(dim).astype(np.float32)
        print(f"gate ragged {rows}x{hidden}x{dim}", flush=True)
        H = cpu(d2.context_gate(to_gpu(h), to_gpu_bits(wb), to_gpu(b)))
        Href, _, pre_abs = oracle.context_gate(h, oracle.bf16_to_f64(wb), b, True)
        assert_close_scaled(H, Href, 0.25 * pre_abs, what="gate bf16 ragged")
        H = cpu(d2.context_gate(to_gpu(h), to_gpu(w), to_gpu(b)))
        Href, _, pre_abs = oracle.context_gate(h, w, b, False)
        assert_close_scaled(H, Href, 0.25 * pre_abs, what="gate f32 ragged")


def test_context_gate_bf16_h(d2):
    """h in bf16: within tolerance of the oracle, and bit-identical to the gate of the
    fp32 h that holds the same values (both weight dtypes)."""
    rng = np.random.default_rng(12)
    for rows, hidden, dim in ((1, 8, 16), (105, 5120, 256), (33, 1000, 128), (257, 1032, 64), (5, 4096, 1024),
                              (320, 1024, 256)):
        hb = synth.f32_to_bf16_bits(rng.standard_normal((rows, hidden)).astype(np.float32))
        h64 = oracle.bf16_to_f64(hb)
        w = (rng.standard_normal((dim, hidden)) / np.sqrt(hidden)).astype(np.float32)
        wb = synth.f32_to_bf16_bits(w)
        b = rng.standard_normal(dim).astype(np.float32)
        print(f"gate bf16 h {rows}x{hidden}x{dim}", flush=True)
        for Wg, W64, is_bf16 in ((to_gpu_bits(wb), oracle.bf16_to_f64(wb), True), (to_gpu(w), w, False)):
            H = cpu(d2.context_gate(to_gpu_bits(hb), Wg, to_gpu(b)))
            Href, _, pre_abs = oracle.context_gate(h64, W64, b, is_bf16)
            assert_close_scaled(H, Href, 0.25 * pre_abs, what=f"gate bf16 h (bf16 W: {is_bf16})")
            H32 = cpu(d2.context_gate(to_gpu(h64.astype(np.float32)), Wg, to_gpu(b)))
            np.testing.assert_array_equal(H.view(np.uint32), H32.view(np.uint32))


# ------------------------------------------------------------------ pair score ------


def _oracle_cands_and_H(inp, w):
    ridx, rval = oracle.topk16(inp["logits_bits"])
    W64, _, is_bf16 = gate_w(inp)
    H, _, _ = oracle.context_gate(inp["h"].reshape(-1, w.D), W64, inp["bias"], is_bf16)
    return ridx, rval, H.reshape(w.B, w.K, -1)


@pytest.mark.parametrize("wl", [0, 2])
def test_pair_score(d2, wl):
    inp = inputs(wl)
    w = synth.workload(wl)
    ridx, rval, H = _oracle_cands_and_H(inp, w)
    H32 = H.astype(np.float32)
    A64, B64, Ag, Bg = tables(inp)
    print(f"pair_score c{wl}", flush=True)
    S, st = d2.pair_score(to_gpu(ridx, None).int(), to_gpu(rval.astype(np.float32)), to_gpu(inp["verified"]), Ag, Bg,
                          to_gpu(H32))
    Sref, Sabs, rst = oracle.pair_score(ridx, rval, inp["verified"], A64, B64, H32)
    assert_close_scaled(cpu(S), Sref, Sabs, what="pair score")
    np.testing.assert_array_equal(cpu(st), rst)


def test_pair_score_bad_ids_are_clamped_and_flagged(d2):
    inp = inputs(0)
    w = synth.workload(0)
    ridx, rval, H = _oracle_cands_and_H(inp, w)
    ridx = ridx.copy()
    ridx[0, 2, 5] = w.V + 7
    ver = inp["verified"].copy()
    ver[0] = -3
    A64, B64, Ag, Bg = tables(inp)
    S, st = d2.pair_score(to_gpu(ridx, None).int(), to_gpu(rval.astype(np.float32)), to_gpu(ver), Ag, Bg,
                          to_gpu(H.astype(np.float32)))
    Sref, Sabs, rst = oracle.pair_score(ridx, rval, ver, A64, B64, H.astype(np.float32))
    np.testing.assert_array_equal(cpu(st), rst)
    assert rst[0, 0] == 2 and rst[0, 2] == 2 and rst[0, 3] == 2
    assert_close_scaled(cpu(S), Sref, Sabs, what="pair score clamped")


# ------------------------------------------------------------------ walk ------------


@pytest.mark.parametrize("temperature", [0.0, 1.0, 0.35])
def test_walk_on_oracle_scores(d2, temperature):
    rng = np.random.default_rng(9)
    B, K = 300, 7
    S = (rng.standard_normal((B, K, 16, 16)) * 2).astype(np.float32)
    S[:5] = np.round(S[:5])                       # exact ties in fp32
    S[5, 3, :, 4] = np.nan
    S[6, 2] = np.inf
    cand = rng.integers(0, 151936, (B, K, 16)).astype(np.int32)
    print(f"walk T={temperature}", flush=True)
    tok, slots, q = d2.walk(to_gpu(S), to_gpu(cand), temperature, seed=77)
    stats = check_walk(S.astype(np.float64), cand, cpu(tok), cpu(slots), cpu(q), temperature, 77)
    print("walk stats", stats)
    if temperature == 0.0:
        assert stats["band"] == 0                  # same fp32 scores -> same argmax


# ------------------------------------------------------------------ fused select ----


def _run_select(d2, inp, w, temperature, seed):
    Wg = gate_w(inp)[1]
    A64, B64, Ag, Bg = tables(inp)
    Hg = d2.context_gate(to_gpu(inp["h"].reshape(w.B, w.K, w.D)), Wg, to_gpu(inp["bias"]))
    out = d2.select(to_gpu_bits(inp["logits_bits"]), to_gpu(inp["verified"]), Ag, Bg, Hg, temperature, seed)
    return Hg, out


@pytest.mark.parametrize("wl", [0, 1, 2, 4])
def test_select_equals_three_calls(d2, wl):
    inp = inputs(wl)
    w = synth.workload(wl)
    T = w.temperature
    print(f"select vs three calls c{wl}", flush=True)
    Hg, out = _run_select(d2, inp, w, T, w.walk_seed)
    A64, B64, Ag, Bg = tables(inp)
    idx, val = d2.topk16(to_gpu_bits(inp["logits_bits"]))
    S, st = d2.pair_score(idx, val, to_gpu(inp["verified"]), Ag, Bg, Hg)
    tok, slots, q = d2.walk(S, idx, T, w.walk_seed)
    for name, ref in (("cand_idx", idx), ("cand_val", val), ("S", S), ("tokens", tok), ("slots", slots), ("q", q),
                      ("row_status", st)):
        np.testing.assert_array_equal(cpu(out[name]).view(np.uint32) if cpu(out[name]).dtype == np.float32 else cpu(out[name]),
                                      cpu(ref).view(np.uint32) if cpu(ref).dtype == np.float32 else cpu(ref), err_msg=name)


@pytest.mark.parametrize("wl", [0, 1, 2, 4])
def test_select_vs_oracle(d2, wl):
    inp = inputs(wl)
    w = synth.workload(wl)
    print(f"select vs oracle c{wl}", flush=True)
    Hg, out = _run_select(d2, inp, w, w.temperature, w.walk_seed)
    ridx, rval, H = _oracle_cands_and_H(inp, w)
    np.testing.assert_array_equal(cpu(out["cand_idx"]), ridx)
    np.testing.assert_array_equal(cpu(out["cand_val"]).astype(np.float64), rval)
    A64, B64, _, _ = tables(inp)
    Sref, Sabs, rst = oracle.pair_score(ridx, rval, inp["verified"], A64, B64, H)
    assert_close_scaled(cpu(out["S"]), Sref, Sabs, what="select S")
    np.testing.assert_array_equal(cpu(out["row_status"]), rst)
    stats = check_walk(Sref, ridx, cpu(out["tokens"]), cpu(out["slots"]), cpu(out["q"]), w.temperature, w.walk_seed)
    print(f"c{wl} walk stats", stats, flush=True)


@pytest.mark.parametrize("wl", [0, 1, 2, 4])
def test_select_gated(d2, wl):
    """The gated select's H_out follows the oracle gate, and every other output is
    bit-identical to dflash2_select called with that H."""
    import torch
    inp = inputs(wl)
    w = synth.workload(wl)
    if "w_h_bits" not in inp:
        pytest.skip("the gated select takes a bf16 gate weight")
    print(f"gated select c{wl}", flush=True)
    A64, B64, Ag, Bg = tables(inp)
    W64, Wg, _ = gate_w(inp)
    hg = to_gpu(inp["h"].reshape(w.B, w.K, w.D))
    logits, ver = to_gpu_bits(inp["logits_bits"]), to_gpu(inp["verified"])
    Hout = torch.empty((w.B, w.K, w.dim), dtype=torch.float32, device=hg.device)
    out = d2.select_gated(logits, ver, Ag, Bg, hg, Wg, to_gpu(inp["bias"]), "sigmoid", w.temperature, w.walk_seed,
                          H_out=Hout)
    Href, _, pre_abs = oracle.context_gate(inp["h"].reshape(-1, w.D), W64, inp["bias"], True)
    scale = 0.25 * pre_abs          # |d sigmoid / dx| <= 1/4
    assert_close_scaled(cpu(Hout).reshape(-1, w.dim), Href, scale, what="gated H")
    ref = d2.select(logits, ver, Ag, Bg, Hout, w.temperature, w.walk_seed)
    for k in ref:
        a, b = cpu(out[k]), cpu(ref[k])
        np.testing.assert_array_equal(a.view(np.uint32) if a.dtype == np.float32 else a,
                                      b.view(np.uint32) if b.dtype == np.float32 else b, err_msg=k)
    ridx, _ = oracle.topk16(inp["logits_bits"])
    np.testing.assert_array_equal(cpu(out["cand_idx"]), ridx)


def test_select_gated_ragged(d2):
    """Rows not a multiple of 16, a hidden size that is not a multiple of 32, dim 64, a
    bias, the identity activation and a sampled walk."""
    import torch
    w = synth.workload(0, B=3, K=5, V=5000, D=200, dim=64, bf16_params=True)
    inp = synth.make_inputs(w)
    rng = np.random.default_rng(11)
    bias = rng.normal(0.0, 0.5, size=w.dim).astype(np.float32)
    A64, B64, Ag, Bg = tables(inp)
    W64, Wg, _ = gate_w(inp)
    logits, ver = to_gpu_bits(inp["logits_bits"]), to_gpu(inp["verified"])
    for act, T in (("identity", 0.0), ("sigmoid", 0.7)):
        print(f"gated select ragged act={act} T={T}", flush=True)
        Hout = torch.empty((w.B, w.K, w.dim), dtype=torch.float32, device=logits.device)
        out = d2.select_gated(logits, ver, Ag, Bg, to_gpu(inp["h"]), Wg, to_gpu(bias), act, T, 9, H_out=Hout)
        Href, _, pre_abs = oracle.context_gate(inp["h"].reshape(-1, w.D), W64, bias, True, act=act)
        assert_close_scaled(cpu(Hout).reshape(-1, w.dim), Href, pre_abs * (0.25 if act == "sigmoid" else 1.0),
                            what=f"gated H {act}")
        ref = d2.select(logits, ver, Ag, Bg, Hout, T, 9)
        for k in ref:
            a, b = cpu(out[k]), cpu(ref[k])
            np.testing.assert_array_equal(a.view(np.uint32) if a.dtype == np.float32 else a,
                                          b.view(np.uint32) if b.dtype == np.float32 else b, err_msg=k)


def test_select_gated_300_rows(d2):
    """The gated select at 20 requests of 15 positions (300 rows, not a whole number of
    the gate's 16-row tiles' groups), hidden 1024, a bias, both activations, greedy and
    sampled: H_out within tolerance of the oracle's gate and every other output
    bit-identical to dflash2_select with that H; h in bf16 bit-identical to the fp32 h
    holding the same values."""
    import torch
    w = synth.workload(0, B=20, K=15, V=3000, D=1024, dim=256, bf16_params=True)
    inp = synth.make_inputs(w)
    rng = np.random.default_rng(21)
    bias = rng.normal(0.0, 0.5, size=w.dim).astype(np.float32)
    A64, B64, Ag, Bg = tables(inp)
    W64, Wg, _ = gate_w(inp)
    logits, ver = to_gpu_bits(inp["logits_bits"]), to_gpu(inp["verified"])
    hb = synth.f32_to_bf16_bits(inp["h"].reshape(-1, w.D))
    h64 = oracle.bf16_to_f64(hb)
    for act, T in (("sigmoid", 0.0), ("identity", 0.8)):
        print(f"gated select 300 rows act={act} T={T}", flush=True)
        Hout = torch.empty((w.B, w.K, w.dim), dtype=torch.float32, device=logits.device)
        out = d2.select_gated(logits, ver, Ag, Bg, to_gpu(h64.astype(np.float32).reshape(w.B, w.K, w.D)), Wg,
                              to_gpu(bias), act, T, 5, H_out=Hout)
        Href, _, pre_abs = oracle.context_gate(h64, W64, bias, True, act=act)
        assert_close_scaled(cpu(Hout).reshape(-1, w.dim), Href, pre_abs * (0.25 if act == "sigmoid" else 1.0),
                            what=f"gated H 300 rows {act}")
        ref = d2.select(logits, ver, Ag, Bg, Hout, T, 5)
        for k in ref:
            a, b = cpu(out[k]), cpu(ref[k])
            np.testing.assert_array_equal(a.view(np.uint32) if a.dtype == np.float32 else a,
                                          b.view(np.uint32) if b.dtype == np.float32 else b, err_msg=k)
        Hout_b = torch.empty_like(Hout)
        out_b = d2.select_gated(logits, ver, Ag, Bg, to_gpu_bits(hb.reshape(w.B, w.K, w.D)), Wg, to_gpu(bias), act, T,
                                5, H_out=Hout_b)
        np.testing.assert_array_equal(cpu(Hout_b).view(np.uint32), cpu(Hout).view(np.uint32))
        for k in out:
            a, b = cpu(out_b[k]), cpu(out[k])
            np.testing.assert_array_equal(a.view(np.uint32) if a.dtype == np.float32 else a,
                                          b.view(np.uint32) if b.dtype == np.float32 else b, err_msg=k)


def test_select_gated_bf16_h(d2):
    """The gated select at B 15, K 7 with h in bf16: every output, H_out included,
    bit-identical to the gated select on the fp32 h holding the same values; H_out
    within tolerance of the oracle's gate."""
    import torch
    w = synth.workload(2)
    inp = inputs(2)
    print("gated select bf16 h c2", flush=True)
    A64, B64, Ag, Bg = tables(inp)
    W64, Wg, _ = gate_w(inp)
    hb = synth.f32_to_bf16_bits(inp["h"])
    h64 = oracle.bf16_to_f64(hb)
    logits, ver = to_gpu_bits(inp["logits_bits"]), to_gpu(inp["verified"])
    for T in (0.0, 1.0):
        Hb = torch.empty((w.B, w.K, w.dim), dtype=torch.float32, device=logits.device)
        Hf = torch.empty_like(Hb)
        ob = d2.select_gated(logits, ver, Ag, Bg, to_gpu_bits(hb), Wg, to_gpu(inp["bias"]), "sigmoid", T, 3, H_out=Hb)
        of = d2.select_gated(logits, ver, Ag, Bg, to_gpu(h64.astype(np.float32)), Wg, to_gpu(inp["bias"]), "sigmoid",
                             T, 3, H_out=Hf)
        assert torch.equal(Hb, Hf)
        for k in ob:
            a, b = cpu(ob[k]), cpu(of[k])
            np.testing.assert_array_equal(a.view(np.uint32) if a.dtype == np.float32 else a,
                                          b.view(np.uint32) if b.dtype == np.float32 else b, err_msg=k)
        Href, _, pre_abs = oracle.context_gate(h64.reshape(-1, w.D), W64, inp["bias"], True)
        assert_close_scaled(cpu(Hb).reshape(-1, w.dim), Href, 0.25 * pre_abs, what="gated H bf16 h")


def test_select_gated_many_rows(d2):
    """The gated select at c3's 960 rows: H_out within tolerance on every row, and every
    output bit-identical to dflash2_select on that H."""
    import torch
    w = synth.workload(3)
    inp = inputs(3)
    print("gated select c3 (960 rows)", flush=True)
    A64, B64, Ag, Bg = tables(inp)
    W64, Wg, _ = gate_w(inp)
    logits, ver = to_gpu_bits(inp["logits_bits"]), to_gpu(inp["verified"])
    Hout = torch.empty((w.B, w.K, w.dim), dtype=torch.float32, device=logits.device)
    out = d2.select_gated(logits, ver, Ag, Bg, to_gpu(inp["h"]), Wg, to_gpu(inp["bias"]), "sigmoid", 0.0, 0,
                          H_out=Hout)
    Href, _, pre_abs = oracle.context_gate(inp["h"].reshape(-1, w.D), W64, inp["bias"], True)
    assert_close_scaled(cpu(Hout).reshape(-1, w.dim), Href, 0.25 * pre_abs, what="gated H c3")
    ref = d2.select(logits, ver, Ag, Bg, Hout, 0.0, 0)
    for k in ref:
        a, b = cpu(out[k]), cpu(ref[k])
        np.testing.assert_array_equal(a.view(np.uint32) if a.dtype == np.float32 else a,
                                      b.view(np.uint32) if b.dtype == np.float32 else b, err_msg=k)


def test_select_c3_all_rows(d2):
    """c3 (B 64, K 15, V 151936): the top-16 of all 960 rows bit-exact against the
    oracle's full sort; the scores and the walk (teacher-forced) of 16 requests spread
    over the batch; every request's tokens are its slots' candidates."""
    w = synth.workload(3)
    inp = inputs(3)
    print("select c3 (all 960 rows)", flush=True)
    Hg, out = _run_select(d2, inp, w, 0.0, 0)
    ridx, rval = oracle.topk16(inp["logits_bits"])
    np.testing.assert_array_equal(cpu(out["cand_idx"]), ridx)
    np.testing.assert_array_equal(cpu(out["cand_val"]).astype(np.float64), rval)
    reqs = list(range(0, w.B, 4))
    W64, _, _ = gate_w(inp)
    H, _, _ = oracle.context_gate(inp["h"][reqs].reshape(-1, w.D), W64, inp["bias"], True)
    A64, B64, _, _ = tables(inp)
    Sref, Sabs, rst = oracle.pair_score(ridx[reqs], rval[reqs], inp["verified"][reqs], A64, B64,
                                        H.reshape(len(reqs), w.K, -1))
    assert_close_scaled(cpu(out["S"])[reqs], Sref, Sabs, what="c3 S")
    np.testing.assert_array_equal(cpu(out["row_status"])[reqs], rst)
    check_walk(Sref, ridx[reqs], cpu(out["tokens"])[reqs], cpu(out["slots"])[reqs], cpu(out["q"])[reqs], 0.0, 0)
    tok, cand, slots = cpu(out["tokens"]), cpu(out["cand_idx"]), cpu(out["slots"])
    np.testing.assert_array_equal(tok, np.take_along_axis(cand, slots[..., None], axis=2)[..., 0])


def test_select_deterministic(d2):
    inp = inputs(2)
    w = synth.workload(2)
    _, a = _run_select(d2, inp, w, 1.0, 5)
    _, b = _run_select(d2, inp, w, 1.0, 5)
    for k in a:
        np.testing.assert_array_equal(cpu(a[k]), cpu(b[k]), err_msg=k)


def test_workspace_needs_no_init_and_serves_smaller_calls(d2):
    """Every call writes the workspace bytes it reads: a buffer full of garbage, shared by
    calls of two different sizes, gives the same results as fresh buffers."""
    import torch
    runs = []
    for wl in (0, 1):
        inp = inputs(wl)
        w = synth.workload(wl)
        runs.append((inp, w, _run_select(d2, inp, w, 1.0, 3)[1]))
    kinds = {}
    for key, buf in d2._ws_cache.items():
        kinds.setdefault(key[1], []).append(key)
    for kind, keys in kinds.items():
        big = torch.full((max(d2._ws_cache[k].numel() for k in keys),), 0xFF, dtype=torch.uint8,
                         device=d2._ws_cache[keys[0]].device)
        for k in keys:
            d2._ws_cache[k] = big
    print("select with one garbage-filled workspace per call kind", flush=True)
    for inp, w, ref in runs:
        _, again = _run_select(d2, inp, w, 1.0, 3)
        for k in ref:
            np.testing.assert_array_equal(cpu(again[k]), cpu(ref[k]), err_msg=f"V={w.V} {k}")
    d2._ws_cache.clear()


# ------------------------------------------------------------------ conv ------------


@pytest.mark.parametrize("wl", [0, 2, 3])
def test_conv2tap(d2, wl):
    inp = inputs(wl)
    print(f"conv c{wl}", flush=True)
    y = cpu(d2.conv2tap(to_gpu(inp["conv_x"]), to_gpu(inp["conv_prev"]), to_gpu(inp["conv_taps"])))
    yref, yabs = oracle.conv2tap(inp["conv_x"], inp["conv_prev"], inp["conv_taps"])
    assert_close_scaled(y, yref, yabs, what="conv")


def test_conv2tap_groups_and_odd_shapes(d2):
    rng = np.random.default_rng(3)
    for S_, B, K, D, g in ((1, 1, 1, 4, 1), (2, 3, 5, 12, 3), (1, 2, 9, 10, 1), (3, 1, 64, 64, 16), (1, 4, 7, 5120, 2)):
        x = rng.standard_normal((S_, B, K, D)).astype(np.float32)
        p = rng.standard_normal((S_, B, D)).astype(np.float32)
        k = rng.uniform(-1, 1, (S_, B, K, 2, D // g)).astype(np.float32)
        print(f"conv shape {(S_, B, K, D, g)}", flush=True)
        y = cpu(d2.conv2tap(to_gpu(x), to_gpu(p), to_gpu(k), group=g))
        yref, yabs = oracle.conv2tap(x, p, k, g)
        assert_close_scaled(y, yref, yabs, what=f"conv {(S_, B, K, D, g)}")


# ------------------------------------------------------------------ verify ----------


def _c4_draft(d2):
    inp = inputs(4)
    w = synth.workload(4)
    _, out = _run_select(d2, inp, w, w.temperature, w.walk_seed)
    return inp, w, out


@pytest.mark.parametrize("temperature", [1.0, 0.0, 0.6])
def test_spec_accept_c4(d2, temperature):
    inp, w, out = _c4_draft(d2)
    tb = inp["target_bits"]
    tokens, cand, q = cpu(out["tokens"]), cpu(out["cand_idx"]), cpu(out["q"])
    if temperature == 0.0:
        # make some drafts match the target argmax so prefixes of several lengths occur
        g = np.argmax(oracle.bf16_to_f64(tb), axis=-1)
        for b in range(w.B):
            n = b % (w.K + 1)
            tokens[b, :n] = g[b, :n]
    print(f"spec_accept c4 T={temperature}", flush=True)
    o, n, st = d2.spec_accept(to_gpu_bits(tb), to_gpu(tokens), to_gpu(cand), to_gpu(q), temperature, seed=11)
    stats = check_accept(tb, tokens, cand, q, temperature, 11, cpu(o), cpu(n), cpu(st))
    print("verify stats", stats)


def test_spec_accept_correlated_target(d2):
    # target = draft logits + N(0, 1): drafts are often accepted, so every branch
    # (accept, residual resample, bonus) is exercised against the oracle
    inp, w, out = _c4_draft(d2)
    rng = np.random.default_rng(8)
    draft = synth.bf16_bits_as_f32(inp["logits_bits"])
    # a target sharper than the draft: its mass sits on the draft's best candidates
    tgt = 4.0 * np.concatenate([draft, draft[:, -1:]], axis=1) + rng.standard_normal((w.B, w.K + 1, w.V)).astype(np.float32) * 0.3
    tb = synth.f32_to_bf16_bits(tgt)
    tokens, cand, q = cpu(out["tokens"]), cpu(out["cand_idx"]), cpu(out["q"])
    o, n, st = d2.spec_accept(to_gpu_bits(tb), to_gpu(tokens), to_gpu(cand), to_gpu(q), 1.0, seed=12)
    stats = check_accept(tb, tokens, cand, q, 1.0, 12, cpu(o), cpu(n), cpu(st))
    print("correlated verify stats", stats, "accepted", cpu(n).tolist())
    assert cpu(n).max() > 0


def test_spec_accept_fault_rows(d2):
    rng = np.random.default_rng(14)
    B, K, V = 6, 3, 5000
    tb = synth.f32_to_bf16_bits(rng.standard_normal((B, K + 1, V)).astype(np.float32))
    cand = np.stack([np.stack([rng.choice(V, 16, replace=False) for _ in range(K)]) for _ in range(B)]).astype(np.int32)
    q = np.full((B, K, 16), 1.0 / 16, np.float32)
    tokens = cand[:, :, 0].copy()
    tb[0, 1, 77] = 0x7FC0                 # NaN target -> bit 0
    q[1, 0, 3] = np.nan                   # NaN q -> bit 2
    q[2, 2] *= 0.5                        # wrong total -> bit 2
    tokens[3, 1] = V + 4                  # out-of-range draft -> bit 1
    q[4, 1, :] = 0.0                      # q(x) = 0 -> bit 2 (and wrong total)
    q[4, 1, 5] = 1.0
    tb[5, 0, 9] = 0x7F80                  # +inf target -> bit 0
    o, n, st = d2.spec_accept(to_gpu_bits(tb), to_gpu(tokens), to_gpu(cand), to_gpu(q), 1.0, seed=3)
    check_accept(tb, tokens, cand, q, 1.0, 3, cpu(o), cpu(n), cpu(st))
    assert cpu(st).tolist() == [1, 4, 4, 2, 4, 1]


@pytest.mark.parametrize("V", [16, 23, 77, 1003, 9729])
@pytest.mark.parametrize("temperature", [1.0, 0.3])
def test_spec_accept_sampled_small_and_ragged_vocab(d2, V, temperature):
    """Sampled verify where the vocabulary leaves sub-chunks empty (V = 16, 23), short,
    ragged (V % 8 != 0) or one vector past a whole sub-chunk (9729); the drafts are
    the target's own top candidates so accepts, residual draws and bonus draws occur."""
    rng = np.random.default_rng(V)
    B, K = 6, 4
    vals = rng.standard_normal((B, K + 1, V)).astype(np.float32) * 2.0
    tb = synth.f32_to_bf16_bits(vals)
    p = np.stack([[oracle.target_probs(tb[b, t], temperature) for t in range(K + 1)] for b in range(B)])
    cand = np.argsort(-p[:, :K], axis=-1, kind="stable")[..., :16].astype(np.int32)
    q = np.take_along_axis(p[:, :K], cand.astype(np.int64), axis=-1)
    q = (q / q.sum(-1, keepdims=True)).astype(np.float32)
    q = (0.5 * q + 0.5 * rng.dirichlet(np.ones(16), size=(B, K))).astype(np.float32)   # off the target's
    q /= q.sum(-1, keepdims=True)
    tokens = cand[:, :, 0].copy()
    ld = (V + 7) // 8 * 8                                # rows padded to the 16-byte stride rule
    buf = np.zeros((B, K + 1, ld), np.uint16)
    buf[..., :V] = tb
    print(f"sampled verify V={V} T={temperature}", flush=True)
    o, n, st = d2.spec_accept(to_gpu_bits(buf)[..., :V], to_gpu(tokens), to_gpu(cand), to_gpu(q.astype(np.float32)),
                              temperature, seed=V)
    stats = check_accept(tb, tokens, cand, q, temperature, V, cpu(o), cpu(n), cpu(st))
    print("verify stats", stats, "accepted", cpu(n).tolist(), flush=True)


@pytest.mark.parametrize("V", [5003, 40000])
def test_spec_accept_greedy_edge_rows(d2, V):
    """Greedy verify = argmax prefix match with NaN lowest, -0 == +0 and ties to the
    lowest id, on target rows built to hit every branch of the chunk argmax."""
    rng = np.random.default_rng(21)
    B, K = 8, 3
    vals = rng.standard_normal((B, K + 1, V)).astype(np.float32)
    tb = synth.f32_to_bf16_bits(vals)
    tb[0, 0, 11] = 0x7FC0                                # +NaN above every value: not the argmax
    tb[0, 1, :] = 0x7FC0                                 # all NaN: argmax = token 0
    tb[0, 1, 5::7] = 0xFFC1                              # with some -NaN
    tb[1, 0, :] = 0x8000                                 # all -0 ...
    tb[1, 0, 3000 % V] = 0x0000                          # ... one +0: ties with -0, lowest id wins
    tb[1, 1, :] = 0xFF80                                 # all -inf
    tb[2, 0, [17, 400, V - 1]] = 0x4400                  # tied maxima (value 512)
    tb[2, 1, V - 1] = 0x7F80                             # +inf in the ragged tail
    tb[3, 0, :] = 0xC000                                 # all -2 ...
    tb[3, 0, V // 2:] = 0x7FC0                           # ... and +NaN on the right half: fallback path
    tb[3, 1, :] = 0xFFC0                                 # all -NaN
    cand = np.stack([np.stack([rng.choice(V, 16, replace=False) for _ in range(K)]) for _ in range(B)]).astype(np.int32)
    q = np.full((B, K, 16), 1.0 / 16, np.float32)
    g = np.array([[int(oracle.bf16_argmax(tb[b, t])) for t in range(K + 1)] for b in range(B)])
    tokens = cand[:, :, 0].copy()
    for b in range(B):                                   # prefixes of several lengths
        n = b % (K + 1)
        tokens[b, :n] = g[b, :n]
    ld = (V + 7) // 8 * 8                                # rows padded to the 16-byte stride rule
    buf = np.zeros((B, K + 1, ld), np.uint16)
    buf[..., :V] = tb
    print(f"greedy verify edge rows V={V} ld={ld}", flush=True)
    o, n, st = d2.spec_accept(to_gpu_bits(buf)[..., :V], to_gpu(tokens), to_gpu(cand), to_gpu(q), 0.0, seed=1)
    check_accept(tb, tokens, cand, q, 0.0, 1, cpu(o), cpu(n), cpu(st))


def test_spec_accept_shared_target_matches_expanded(d2):
    inp, w, out = _c4_draft(d2)
    tb = inp["target_bits"][0]
    tokens, cand, q = out["tokens"], out["cand_idx"], out["q"]
    o1, n1, s1 = d2.spec_accept(to_gpu_bits(tb), tokens, cand, q, 1.0, seed=5, shared_target=True)
    full = np.broadcast_to(tb, (w.B,) + tb.shape)
    o2, n2, s2 = d2.spec_accept(to_gpu_bits(full), tokens, cand, q, 1.0, seed=5)
    np.testing.assert_array_equal(cpu(o1), cpu(o2))
    np.testing.assert_array_equal(cpu(n1), cpu(n2))
