"""dflash2_select_noalloc (the select on the library's own per-GPU scratch) against
dflash2_select (caller workspace): two calls in a row through the C ABI, the second on
a smaller request, every output bit-identical, greedy and sampled."""

import numpy as np
import pytest

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


def _inputs(d2, w):
    inp = synth.make_inputs(w)
    logits, ver = to_gpu_bits(inp["logits_bits"]), to_gpu(inp["verified"])
    if "emb_a_bits" in inp:
        A, B, Wh = to_gpu_bits(inp["emb_a_bits"]), to_gpu_bits(inp["emb_b_bits"]), to_gpu_bits(inp["w_h_bits"])
    else:
        A, B, Wh = to_gpu(inp["emb_a"]), to_gpu(inp["emb_b"]), to_gpu(inp["w_h"])
    H = d2.context_gate(to_gpu(inp["h"]), Wh, to_gpu(inp["bias"]))
    return logits, ver, A, B, H


def _same(a, b, what):
    for k in a:
        x, y = cpu(a[k]), cpu(b[k])
        np.testing.assert_array_equal(x.view(np.uint32) if x.dtype == np.float32 else x,
                                      y.view(np.uint32) if y.dtype == np.float32 else y, err_msg=f"{what}: {k}")


@pytest.mark.parametrize("temperature,seed", [(0.0, 0), (1.0, 4)])
def test_select_noalloc_equals_select_twice(d2, temperature, seed):
    import torch
    big = synth.workload(2)                                            # B 15, K 7, V 151936, bf16 tables
    small = synth.workload(0, B=3, K=5, V=40000, D=128, dim=64)        # fp32 tables, fewer rows, smaller V
    for w, what in ((big, "B15 K7 V151936"), (small, "B3 K5 V40000 fp32 dim 64")):
        print(f"select_noalloc {what} T={temperature}", flush=True)
        logits, ver, A, B, H = _inputs(d2, w)
        got = d2.select_noalloc(logits, ver, A, B, H, temperature, seed)
        ref = d2.select(logits, ver, A, B, H, temperature, seed)
        torch.cuda.synchronize()
        _same(got, ref, what)
