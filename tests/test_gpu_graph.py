"""One launch per proposer step: the gated select and the two-tap conv recorded into a
HIP graph by the library (dflash2_graph_begin / end / launch), replayed several times
with fresh inputs copied in between, each replay bit-identical to the same calls made
eagerly and matching the CPU oracle: candidates exactly, the gate, scores and conv
within the term-magnitude tolerance, and the walk teacher-forced within the tie band."""

import numpy as np
import pytest

from dflash_draft_selector_amd import synth
import oracle
from parity_util import assert_close_scaled, check_walk, cpu, to_gpu, to_gpu_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def d2():
    import torch
    from dflash_draft_selector_amd import dflash2
    dflash2.load_library()
    torch.cuda.init()
    return dflash2


@pytest.mark.parametrize("temperature", [0.0, 1.0])
def test_proposer_step_graph_replays_equal_eager(d2, temperature):
    import torch
    w = synth.workload(2, V=40000)                          # B 15, K 7, hidden 5120
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        inp = synth.make_inputs(w)
        logits, h, x = to_gpu_bits(inp["logits_bits"]), to_gpu(inp["h"]), to_gpu(inp["conv_x"])
        ver, A, B = to_gpu(inp["verified"]), to_gpu_bits(inp["emb_a_bits"]), to_gpu_bits(inp["emb_b_bits"])
        Wh, bias = to_gpu_bits(inp["w_h_bits"]), to_gpu(inp["bias"])
        xp, taps = to_gpu(inp["conv_prev"]), to_gpu(inp["conv_taps"])
        H = torch.empty((w.B, w.K, w.dim), dtype=torch.float32, device="cuda")
        y = torch.empty_like(x)
        out = d2.select_gated(logits, ver, A, B, h, Wh, bias, "sigmoid", temperature, 11, H_out=H)   # buffers exist
        d2.conv2tap(x, xp, taps, y=y)
        with d2.Graph() as g:
            d2.select_gated(logits, ver, A, B, h, Wh, bias, "sigmoid", temperature, 11, out=out, H_out=H)
            d2.conv2tap(x, xp, taps, y=y)
        for rep in range(3):
            fresh = synth.make_inputs(synth.workload(2, V=40000, seed=100 + rep))
            logits.copy_(to_gpu_bits(fresh["logits_bits"]))
            h.copy_(to_gpu(fresh["h"]))
            x.copy_(to_gpu(fresh["conv_x"]))
            g.launch()
            torch.cuda.synchronize()
            print(f"graph replay {rep} T={temperature}", flush=True)
            ref = d2.select_gated(logits, ver, A, B, h, Wh, bias, "sigmoid", temperature, 11,
                                  H_out=(Hr := torch.empty_like(H)))
            yr = d2.conv2tap(x, xp, taps)
            torch.cuda.synchronize()
            for k in ("cand_idx", "cand_val", "S", "tokens", "slots", "q", "row_status"):
                assert torch.equal(out[k], ref[k]), f"replay {rep}: {k} differs from the eager call"
            assert torch.equal(H, Hr) and torch.equal(y, yr)
            # the replay against the oracle on the inputs it ran on
            ridx, rval = oracle.topk16(fresh["logits_bits"])
            assert np.array_equal(cpu(out["cand_idx"]), ridx), f"replay {rep}: candidates differ from the oracle"
            assert np.array_equal(cpu(out["cand_val"]), rval.astype(np.float32))
            Href, _, pre_abs = oracle.context_gate(fresh["h"].reshape(-1, w.D), oracle.bf16_to_f64(inp["w_h_bits"]),
                                                   inp["bias"], True)
            assert_close_scaled(cpu(H).reshape(-1, w.dim), Href, 0.25 * pre_abs, what=f"replay {rep} gate")
            A64, B64 = oracle.bf16_to_f64(inp["emb_a_bits"]), oracle.bf16_to_f64(inp["emb_b_bits"])
            Sref, Sabs, _ = oracle.pair_score(ridx, rval, inp["verified"], A64, B64, cpu(H).astype(np.float64))
            assert_close_scaled(cpu(out["S"]), Sref, Sabs, what=f"replay {rep} scores")
            check_walk(Sref, ridx, cpu(out["tokens"]), cpu(out["slots"]), cpu(out["q"]), temperature, 11)
            yref, yabs = oracle.conv2tap(fresh["conv_x"], inp["conv_prev"], inp["conv_taps"])
            assert_close_scaled(cpu(y), yref, yabs, what=f"replay {rep} conv")
        g.close()
