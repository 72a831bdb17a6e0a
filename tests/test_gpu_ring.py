"""Draft-block attention over the per-request K/V ring (dflash2_ring_attention) through
the C ABI against the oracle (the window gathered into a dense key list, float64).

Tolerance, from the arithmetic: q k^T sums head_dim bf16 products in fp32 on the matrix
cores (32 per step, head_dim/32 steps), so a score is off by at most
(head_dim/32 + 33) 2^-24 max_k sum_d |q_d k_d| * scale (the scale in fp32 included);
a score error e moves the normalised output by at most 2e in units of
sum_k p_k |v_k|; p enters the p v product as two bf16 parts (2^-16); the p v sums run in
fp32 over the window's keys, chunk by chunk, and the splits.  Checked per element:
|out - ref| <= (2 (Dh/32 + 33) 2^-24 smax + 2^-15 + (nkeys/32 + 64) 2^-24) sum_k p_k |v_k|.
"""

import numpy as np
import pytest

import oracle
from dflash_draft_selector_amd import synth
from parity_util import cpu, to_gpu, to_gpu_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def d2():
    import torch
    from dflash_draft_selector_amd import dflash2
    dflash2.load_library()
    torch.cuda.init()
    return dflash2


def gpu_args(inp):
    """The inputs in the library's layouts: rings [B, ring, Hkv, Dh] as drawn become the
    tiled K and V rings (tests/test_ring_layout.py pins both re-layouts)."""
    import torch
    from dflash_draft_selector_amd import dflash2
    kr = dflash2.ring_k_tiles(inp["kr_bits"])
    vr = dflash2.ring_v_tiles(inp["vr_bits"])
    return (to_gpu_bits(inp["q_bits"]), to_gpu_bits(inp["kb_bits"]), to_gpu_bits(inp["vb_bits"]), to_gpu_bits(kr),
            to_gpu_bits(vr), torch.from_numpy(inp["ctx_len"]).cuda())


def run_and_check(d2, inp, window, what, scale=0.0):
    B, nq, hq, dh = inp["q_bits"].shape
    got = cpu(d2.ring_attention(*gpu_args(inp), window, scale))
    f = oracle.bf16_to_f64
    ref, pv_abs, smax = oracle.ring_attention(f(inp["q_bits"]), f(inp["kb_bits"]), f(inp["vb_bits"]),
                                              f(inp["kr_bits"]), f(inp["vr_bits"]), inp["ctx_len"], window,
                                              None if scale == 0.0 else scale)
    nkeys = np.minimum(np.maximum(inp["ctx_len"], 0), window - 1) + nq
    rel = 2 * (dh / 32 + 33) * 2.0**-24 * smax + 2.0**-15 + ((nkeys[:, None, None] / 32 + 64) * 2.0**-24)
    tol = rel[..., None] * pv_abs
    err = np.abs(got - ref)
    worst = np.max(err / np.maximum(tol, 1e-300))
    print(f"  {what}: worst error / bound = {worst:.3f}", flush=True)
    assert np.all(np.isfinite(got))
    assert np.all(err <= tol), f"{what}: {np.sum(err > tol)} elements over the bound (worst ratio {worst:.2f})"


@pytest.mark.parametrize("B,nq,hq,hkv,ring,window,ctx", [
    (3, 8, 8, 2, 2112, 2048, [0, 100, 5000]),          # block only; a partial window; a full window that wraps
    (3, 8, 8, 2, 2112, 2048, [1, 2049, 4229]),         # window starts off the 8-row grid, one wraps mid-group
    (2, 8, 12, 2, 2112, 2048, [2047, 2048]),            # 48 query rows (three row tiles); window just full
    (2, 1, 4, 4, 2112, 2048, [1, 3000]),               # one query row per K/V head
    (4, 8, 8, 8, 64, 33, [31, 32, 33, 77]),             # small ring: wraps, fewer steps than waves
    (2, 4, 8, 4, 64, 64, [63, 1000]),                   # window = ring
    (2, 8, 8, 2, 2112, 2048, [-5, 10]),                 # a negative length reads as 0
    (2, 4, 8, 2, 32, 1, [0, 13]),                       # window 1: the block's keys only
    (2, 8, 8, 2, 3968, 3906, [3905, 9000]),             # 123 context steps over 16 splits
    (2, 8, 8, 2, 20480, 20480, [20479, 30000]),         # 641 steps: 32 splits, several steps per wave
    (2, 8, 8, 2, 768, 700, [300, 650]),                 # 22 context steps: uneven shares per wave
    (3, 8, 8, 2, 2080, 2048, [2100, 4111, 5000]),       # ring of 65 tiles: the window wraps mid-ring
    (2, 8, 8, 2, 2112, 2048, [2**31 - 1, 2**31 - 77]),  # context lengths at the top of int32
])
def test_ring_attention_parity(d2, B, nq, hq, hkv, ring, window, ctx):
    print(f"ring attention B={B} nq={nq} hq={hq} hkv={hkv} ring={ring} window={window} ctx={ctx}", flush=True)
    inp = synth.ring_inputs(B, nq, hq, hkv, ring, ctx, seed=B * 7 + nq + hq + ring)
    run_and_check(d2, inp, window, "random")
    sharp = synth.ring_inputs(B, nq, hq, hkv, ring, ctx, seed=B * 7 + nq + hq + ring + 1, q_scale=4.0)
    run_and_check(d2, sharp, window, "sharp (q x 4)")


def test_ring_attention_never_reads_rows_outside_the_window(d2):
    # NaN in every ring row the window does not cover (stale, rejected or too old): the
    # output stays finite and equal to the clean run
    B, nq, hq, hkv, ring, window = 2, 8, 8, 2, 2112, 2048
    ctx = [3001, 501]                                     # windows starting off the 8-row grid
    inp = synth.ring_inputs(B, nq, hq, hkv, ring, ctx, seed=9)
    clean = cpu(d2.ring_attention(*gpu_args(inp), window))
    dirty = dict(inp)
    kr, vr = inp["kr_bits"].copy(), inp["vr_bits"].copy()
    for b in range(B):
        keep = set(oracle.ring_window_keys(ctx[b], window, ring))
        for row in range(ring):
            if row not in keep:
                kr[b, row] = 0x7FC0
                vr[b, row] = 0x7FC0
    dirty["kr_bits"], dirty["vr_bits"] = kr, vr
    got = cpu(d2.ring_attention(*gpu_args(dirty), window))
    assert np.all(np.isfinite(got))
    np.testing.assert_array_equal(got, clean)


def test_ring_attention_explicit_scale_and_garbage_workspace(d2):
    inp = synth.ring_inputs(2, 8, 8, 2, 2112, [1234, 4321], seed=21)
    run_and_check(d2, inp, 2048, "scale 0.05", scale=0.05)
    from dflash_draft_selector_amd import dflash2
    for buf in list(dflash2._ws_cache.values()):
        buf.fill_(0xA5)
    run_and_check(d2, inp, 2048, "scale 0.05, garbage workspace", scale=0.05)


def test_ring_attention_full_size(d2):
    # the benchmark's shape: 15 requests, [last token, mask x 7], 32 query heads over 8
    # K/V heads of 128, ring 2112, window 2048, context lengths past the window
    B, nq, hq, hkv = 15, 8, 32, 8
    ctx = list(np.random.default_rng(4).integers(2048, 8192, size=B))
    inp = synth.ring_inputs(B, nq, hq, hkv, 2112, ctx, seed=4)
    run_and_check(d2, inp, 2048, "full size")
