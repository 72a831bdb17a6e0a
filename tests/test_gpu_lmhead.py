"""LM head with the fused top-16 (dflash2_lmhead_topk16) through the C ABI against the
oracle (exact sum rounded once to bf16, then the top-16).

The kernel sums in fp32 on the matrix cores, so a logit within the accumulation error
of a bf16 rounding boundary may round the other way.  The bound used is the worst case
of that arithmetic: the D products summed 32 at a time per MFMA step (taken as 32
sequential fp32 roundings) and D/32 accumulator additions, |err| <= (D/32 + 32) 2^-24
sum_d |h_d W_vd|.  Checks per row:
  1. every returned value is a bf16 rounding of its id's exact logit within that bound;
  2. the list is sorted by (value desc, id asc) with distinct ids;
  3. nothing left out beats the 16th, even at the lowest rounding it could take;
  4. where no logit near the cut is within the bound of a rounding boundary, the list
     equals the oracle's exactly (ids and values).
"""

import numpy as np
import pytest

import oracle
from dflash_draft_selector_amd import synth
from parity_util import cpu, to_gpu_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def d2():
    import torch
    from dflash_draft_selector_amd import dflash2
    dflash2.load_library()
    torch.cuda.init()
    return dflash2


def _key(vals, ids):
    # (value desc, id asc) as one sortable float pair; -0 == +0
    return [(-float(v) + 0.0, int(i)) for v, i in zip(vals, ids)]


def check_rows(idx_g, val_g, h_bits, w_bits, rows_sel=None, vchunk=16384):
    """Checks 1-4 on rows ``rows_sel`` (all by default); returns (rows exactly equal to
    the oracle, rows compared exactly, rows with an ambiguous cut)."""
    h_bits = np.asarray(h_bits)
    R, D = h_bits.shape
    V = w_bits.shape[0]
    rows_sel = np.arange(R) if rows_sel is None else np.asarray(rows_sel)
    h = oracle.bf16_to_f64(h_bits[rows_sel])
    exact = np.empty((len(rows_sel), V))
    absdot = np.empty((len(rows_sel), V))
    for v0 in range(0, V, vchunk):
        wc = oracle.bf16_to_f64(w_bits[v0:v0 + vchunk])
        exact[:, v0:v0 + vchunk] = h @ wc.T
        absdot[:, v0:v0 + vchunk] = np.abs(h) @ np.abs(wc).T
    tol = (D / 32 + 32) * 2.0**-24 * absdot
    lo = oracle.round_to_bf16(exact - tol)
    hi = oracle.round_to_bf16(exact + tol)
    ref_bits = oracle.bf16_bits_of(oracle.round_to_bf16(exact))
    ridx, rval = oracle.topk16(ref_bits)
    n_equal = n_exact = n_amb = 0
    for k, r in enumerate(rows_sel):
        gi, gv = idx_g[r].astype(np.int64), val_g[r].astype(np.float64)
        assert len(set(gi.tolist())) == 16 and gi.min() >= 0 and gi.max() < V, f"row {r}: ids {gi}"
        bad = (gv < lo[k, gi]) | (gv > hi[k, gi])
        assert not np.any(bad), (f"row {r}: value outside its rounding band: ids {gi[bad]} got {gv[bad]} "
                                 f"exact {exact[k, gi[bad]]} tol {tol[k, gi[bad]]} band [{lo[k, gi[bad]]}, "
                                 f"{hi[k, gi[bad]]}]")
        keys = _key(gv, gi)
        assert keys == sorted(keys), f"row {r}: not sorted"
        last = keys[-1]
        out = np.ones(V, dtype=bool)
        out[gi] = False
        lo_keys = np.stack([-lo[k] + 0.0, np.arange(V)], axis=1)[out]
        beats = (lo_keys[:, 0] < last[0]) | ((lo_keys[:, 0] == last[0]) & (lo_keys[:, 1] < last[1]))
        assert not np.any(beats), f"row {r}: an omitted id beats the 16th at its lowest rounding"
        # the cut is unambiguous when every id whose band reaches the oracle's 16th has a
        # single rounding
        cut = rval[k, 15]
        near = hi[k] >= cut
        amb = np.any(lo[k, near] != hi[k, near])
        n_amb += int(amb)
        if not amb:
            n_exact += 1
            np.testing.assert_array_equal(gi, ridx[k], err_msg=f"row {r}")
            np.testing.assert_array_equal(gv, rval[k], err_msg=f"row {r}")
        n_equal += int(np.array_equal(gi, ridx[k]) and np.array_equal(gv, rval[k]))
    return n_equal, n_exact, n_amb


@pytest.mark.parametrize("rows,hidden,vocab,peaks", [
    (7, 256, 5003, True),        # one 16-row tile, ragged last column tile
    (20, 512, 4096, False),      # two row tiles, no planted peaks (dense ties)
    (40, 256, 2071, True),       # four row tiles
    (105, 512, 9000, True),      # eight row tiles (the B=15, K=7 row count)
    (130, 256, 3000, True),      # two row groups: 128 + 2
    (3, 256, 16, False),         # the smallest vocabulary: a permutation of all ids
    (5, 256, 270, False),        # a last tile with 14 columns (fewer than 16)
    # Vocabularies past one round of work-groups (256 compute units: one 512-thread
    # work-group each at 64+ rows, two at 16 rows or fewer) leave a last round under half
    # full, whose tiles are split along the hidden dimension and combined:
    (40, 2048, 70000, True),     # 274 tiles, 18 left over, split in 8 parts
    (100, 512, 70000, False),    # seven row tiles; the 18 left over split in 2 parts
    (5, 1024, 140000, True),     # 547 tiles, 35 left over past two per compute unit, 4 parts
    (140, 512, 70000, True),     # two row groups (128 + 12), each with its split last round
    (5, 768, 140000, True),      # three stages: the 35 left over split in 3 parts of one stage
    (40, 1280, 70000, False),    # five stages, 18 left over: 5 parts of one stage
    (40, 1280, 91000, True),     # 356 tiles, 100 left over: 2 parts of unequal length (2 + 3 stages)
    # One round of work-groups runs the tiles in turn, the W ring running on from one
    # tile into the next; with more than half a round left over nothing is split:
    (105, 512, 100000, True),    # 391 tiles: work-groups 0-134 run two whole tiles each
    (105, 256, 70000, False),    # one stage per tile, so every stage hands over to the next tile
    (7, 256, 200000, True),      # 782 tiles at two work-groups per compute unit: 270 run two
])
def test_lmhead_topk16_parity(d2, rows, hidden, vocab, peaks):
    inp = synth.lmhead_inputs(rows, hidden, vocab, seed=rows + hidden + vocab, peaks=peaks)
    print(f"lmhead rows={rows} hidden={hidden} vocab={vocab}", flush=True)
    idx, val, st = d2.lmhead_topk16(to_gpu_bits(inp["h_bits"]), to_gpu_bits(inp["w_bits"]), row_status=True)
    n_eq, n_ex, n_amb = check_rows(cpu(idx), cpu(val), inp["h_bits"], inp["w_bits"])
    print(f"  rows equal to the oracle {n_eq}/{rows}; exact-checked {n_ex}; ambiguous cut {n_amb}", flush=True)
    assert n_ex >= rows // 2
    assert not np.any(cpu(st))
    if peaks:
        hit = cpu(idx)[:, 0] == inp["peak_idx"]
        assert hit.mean() > 0.9


def test_lmhead_topk16_matches_topk16_of_its_own_rounding_on_exact_data(d2):
    # Small integers: every product and partial sum is exact in fp32, so the logits are
    # exact and the result must equal topk16 of the oracle's logits bit for bit, ties
    # (many, at these magnitudes) included.
    rng = np.random.default_rng(11)
    rows, hidden, vocab = 24, 512, 6000
    h = rng.integers(-3, 4, size=(rows, hidden)).astype(np.float32)
    w = rng.integers(-2, 3, size=(vocab, hidden)).astype(np.float32)
    hb, wb = synth.f32_to_bf16_bits(h), synth.f32_to_bf16_bits(w)
    idx, val = d2.lmhead_topk16(to_gpu_bits(hb), to_gpu_bits(wb))
    ridx, rval = oracle.lmhead_topk16(hb, wb)
    np.testing.assert_array_equal(cpu(idx), ridx)
    np.testing.assert_array_equal(cpu(val), rval)


def test_lmhead_topk16_nonfinite_and_garbage_workspace(d2):
    import torch
    rows, hidden, vocab = 4, 256, 1000
    inp = synth.lmhead_inputs(rows, hidden, vocab, seed=3, peaks=False)
    w = inp["w_bits"].copy()
    w[17, 5] = 0x7F80          # +inf in one weight: row logits of column 17 become +-inf or NaN
    hb = inp["h_bits"]
    idx, val, st = d2.lmhead_topk16(to_gpu_bits(hb), to_gpu_bits(w), row_status=True)
    h0 = oracle.bf16_to_f64(hb)[:, 5]
    for r in range(rows):
        if h0[r] > 0:          # +inf logit ranks first
            assert cpu(idx)[r, 0] == 17 and np.isposinf(cpu(val)[r, 0])
        else:                  # -inf: never above a finite logit
            assert 17 not in cpu(idx)[r].tolist()
    assert cpu(st).tolist() == [1 if x > 0 else 0 for x in h0]
    # a workspace full of garbage gives the same result as a fresh one
    from dflash_draft_selector_amd import dflash2
    for buf in list(dflash2._ws_cache.values()):
        buf.fill_(0xA5)
    idx2, val2 = d2.lmhead_topk16(to_gpu_bits(hb), to_gpu_bits(w))
    np.testing.assert_array_equal(cpu(idx2), cpu(idx))
    torch.cuda.synchronize()


def test_lmhead_topk16_full_size_sampled_rows(d2):
    # B=15, K=7 rows, hidden 5120, the Qwen vocabulary: the launch the benchmark times,
    # checked on eight rows
    rows, hidden, vocab = 105, 5120, synth.VOCAB_QWEN
    inp = synth.lmhead_inputs(rows, hidden, vocab, seed=2)
    print("lmhead full size: inputs drawn", flush=True)
    idx, val = d2.lmhead_topk16(to_gpu_bits(inp["h_bits"]), to_gpu_bits(inp["w_bits"]))
    sel = np.array([0, 1, 14, 52, 63, 64, 99, 104])
    n_eq, n_ex, n_amb = check_rows(cpu(idx), cpu(val), inp["h_bits"], inp["w_bits"], rows_sel=sel)
    print(f"  sampled rows equal to the oracle {n_eq}/8; exact-checked {n_ex}; ambiguous cut {n_amb}", flush=True)
    assert np.mean(cpu(idx)[:, 0] == inp["peak_idx"]) > 0.9


def pack_ref(w_bits):
    """The packed layout of include/dflash2.h (dflash2_lmhead_pack), written out with
    numpy: columns padded with zeros to whole 256-column tiles, then per tile and 32-dim
    step [nt][wave][g][i][8 dims] for column 256 T + 32 wave + 16 nt + i, dims
    32 k + 8 g .. + 7."""
    V, D = w_bits.shape
    T = (V + 255) // 256
    wp = np.zeros((T * 256, D), dtype=np.uint16)
    wp[:V] = w_bits
    t = wp.reshape(T, 8, 2, 16, D // 32, 4, 8)            # T, wave, nt, i, k, g, e
    return np.ascontiguousarray(t.transpose(0, 4, 2, 1, 5, 3, 6)).reshape(-1)


@pytest.mark.parametrize("vocab,hidden", [(300, 512), (4096, 256), (16, 768)])
def test_lmhead_pack_layout(d2, vocab, hidden):
    w = synth.lmhead_inputs(3, hidden, vocab, seed=vocab)["w_bits"]
    wp = d2.lmhead_pack(to_gpu_bits(w))
    np.testing.assert_array_equal(cpu(wp).view(np.uint16), pack_ref(w))


@pytest.mark.parametrize("rows,hidden,vocab", [
    (7, 256, 5003),              # one row tile, ragged last column tile
    (105, 512, 9000),            # eight row tiles
    (130, 256, 3000),            # two row groups
    (5, 256, 270),               # a last tile with 14 columns
    (40, 2048, 70000),           # split last round, 8 parts
    (40, 1280, 91000),           # split parts of unequal length
    (105, 256, 70000),           # tiles run in turn, one stage each
])
def test_lmhead_topk16_packed_is_bit_identical(d2, rows, hidden, vocab):
    inp = synth.lmhead_inputs(rows, hidden, vocab, seed=rows * 3 + vocab)
    print(f"lmhead packed rows={rows} hidden={hidden} vocab={vocab}", flush=True)
    h, w = to_gpu_bits(inp["h_bits"]), to_gpu_bits(inp["w_bits"])
    idx, val, st = d2.lmhead_topk16(h, w, row_status=True)
    pidx, pval, pst = d2.lmhead_topk16_packed(h, d2.lmhead_pack(w), vocab, row_status=True)
    np.testing.assert_array_equal(cpu(pidx), cpu(idx))
    np.testing.assert_array_equal(cpu(pval), cpu(val))
    np.testing.assert_array_equal(cpu(pst), cpu(st))
    if rows <= 40:
        n_eq, n_ex, n_amb = check_rows(cpu(pidx), cpu(pval), inp["h_bits"], inp["w_bits"])
        assert n_ex >= rows // 2


def test_lmhead_topk16_packed_full_size(d2):
    # the benchmark's launch on the packed weight: bit-identical to the row-major weight
    rows, hidden, vocab = 105, 5120, synth.VOCAB_QWEN
    inp = synth.lmhead_inputs(rows, hidden, vocab, seed=2)
    h, w = to_gpu_bits(inp["h_bits"]), to_gpu_bits(inp["w_bits"])
    idx, val = d2.lmhead_topk16(h, w)
    wp = d2.lmhead_pack(w)
    pidx, pval = d2.lmhead_topk16_packed(h, wp, vocab)
    np.testing.assert_array_equal(cpu(pidx), cpu(idx))
    np.testing.assert_array_equal(cpu(pval), cpu(val))
