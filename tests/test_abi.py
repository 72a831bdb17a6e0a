"""The C-ABI library loads, exports every symbol its header declares, and rejects bad
arguments on the host before touching the GPU (no compute calls here)."""

import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dflash2.h")


def _lib():
    from dflash_draft_selector_amd import dflash2
    if not os.path.exists(dflash2.LIB_PATH):
        from dflash_draft_selector_amd.build import build_library
        build_library()
    return dflash2, dflash2.load_library()


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dflash2_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_six_calls_and_the_fused_step():
    names = _declared()
    for n in ("dflash2_topk16", "dflash2_context_gate", "dflash2_pair_score", "dflash2_walk", "dflash2_conv2tap",
              "dflash2_spec_accept", "dflash2_select", "dflash2_spec_accept_filtered"):
        assert n in names


def test_every_declared_symbol_is_exported():
    d2, lib = _lib()
    out = subprocess.run(["nm", "-D", "--defined-only", d2.LIB_PATH], capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (dflash2_\w+)", out))
    missing = [n for n in _declared() if n not in exported]
    assert not missing, missing
    assert set(d2.EXPORTED) == set(_declared())
    assert lib.dflash2_abi_version() == 3


def test_header_compiles_as_c():
    res = subprocess.run(["gcc", "-fsyntax-only", "-x", "c", "-std=c99", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                          HEADER], capture_output=True, text=True)
    assert res.returncode == 0, res.stderr


def test_status_strings():
    d2, lib = _lib()
    assert d2.status_str(0) == "DFLASH2_OK"
    assert d2.status_str(5) == "DFLASH2_ERR_WORKSPACE"
    assert d2.status_str(99) == "DFLASH2_UNKNOWN_STATUS"


FAKE = ctypes.c_void_p(0x100000)          # 16-byte aligned, never dereferenced
MIS = ctypes.c_void_p(0x100002)
NULL = None


def test_host_validation_before_any_launch():
    d2, lib = _lib()
    ws = ctypes.c_void_p(0x200000)
    big = 1 << 30
    # topk16
    assert lib.dflash2_topk16(NULL, 4, 4096, 4096, FAKE, FAKE, NULL, ws, big, NULL) == 1
    assert lib.dflash2_topk16(FAKE, 4, 15, 16, FAKE, FAKE, NULL, ws, big, NULL) == 2
    assert lib.dflash2_topk16(FAKE, 4, 4096, 4000, FAKE, FAKE, NULL, ws, big, NULL) == 2
    assert lib.dflash2_topk16(FAKE, 4, (1 << 20) + 8, (1 << 20) + 8, FAKE, FAKE, NULL, ws, big, NULL) == 2
    assert lib.dflash2_topk16(FAKE, 4, 4100, 4100, FAKE, FAKE, NULL, ws, big, NULL) == 3
    assert lib.dflash2_topk16(MIS, 4, 4096, 4096, FAKE, FAKE, NULL, ws, big, NULL) == 3
    need = lib.dflash2_topk16_workspace(4, 4096)
    assert need > 0
    assert lib.dflash2_topk16(FAKE, 4, 4096, 4096, FAKE, FAKE, NULL, ws, need - 257, NULL) == 5
    assert lib.dflash2_topk16(FAKE, 4, 4096, 4096, FAKE, FAKE, NULL, NULL, big, NULL) == 5
    # context gate
    assert lib.dflash2_context_gate(FAKE, 0, FAKE, 7, NULL, 4, 512, 256, 0, FAKE, ws, big, NULL) == 4
    assert lib.dflash2_context_gate(FAKE, 2, FAKE, 1, NULL, 4, 512, 256, 0, FAKE, ws, big, NULL) == 4
    assert lib.dflash2_context_gate(FAKE, 1, FAKE, 1, NULL, 4, 512, 256, 9, FAKE, ws, big, NULL) == 4
    assert lib.dflash2_context_gate(FAKE, 0, FAKE, 1, NULL, 4, 500, 256, 0, FAKE, ws, big, NULL) == 2
    assert lib.dflash2_context_gate(FAKE, 1, FAKE, 1, NULL, 4, 512, 250, 0, FAKE, ws, big, NULL) == 2
    assert lib.dflash2_context_gate(FAKE, 0, MIS, 1, NULL, 4, 512, 256, 0, FAKE, ws, big, NULL) == 3
    assert lib.dflash2_context_gate(MIS, 1, FAKE, 0, NULL, 4, 512, 256, 0, FAKE, ws, big, NULL) == 3
    assert lib.dflash2_context_gate(NULL, 1, FAKE, 0, NULL, 4, 512, 256, 0, FAKE, ws, big, NULL) == 1
    # pair score
    assert lib.dflash2_pair_score(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 4096, 96, FAKE, 1, 7, FAKE, NULL, NULL) == 2
    assert lib.dflash2_pair_score(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 4096, 256, FAKE, 1, 65, FAKE, NULL, NULL) == 2
    assert lib.dflash2_pair_score(FAKE, FAKE, FAKE, FAKE, FAKE, 3, 4096, 256, FAKE, 1, 7, FAKE, NULL, NULL) == 4
    assert lib.dflash2_pair_score(FAKE, FAKE, NULL, FAKE, FAKE, 1, 4096, 256, FAKE, 1, 7, FAKE, NULL, NULL) == 1
    # walk
    assert lib.dflash2_walk(FAKE, FAKE, 1, 7, -1.0, 0, FAKE, FAKE, FAKE, NULL) == 6
    assert lib.dflash2_walk(FAKE, FAKE, 1, 7, float("nan"), 0, FAKE, FAKE, FAKE, NULL) == 6
    assert lib.dflash2_walk(FAKE, FAKE, 0, 7, 0.0, 0, FAKE, FAKE, FAKE, NULL) == 2
    # select
    assert lib.dflash2_select(FAKE, 4096, FAKE, FAKE, FAKE, 1, 4096, 256, FAKE, 1, 7, 0.0, 0, FAKE, FAKE, FAKE, FAKE,
                              FAKE, FAKE, NULL, ws, 16, NULL) == 5
    assert lib.dflash2_select(FAKE, 4096, FAKE, FAKE, FAKE, 1, 4096, 256, FAKE, 1, 0, 0.0, 0, FAKE, FAKE, FAKE, FAKE,
                              FAKE, FAKE, NULL, ws, big, NULL) == 2
    # gated select: the select checks, then the gate's
    sg = lambda w_dtype=1, hidden=512, act=0, h=FAKE, wsb=big, K=7, h_dtype=0: lib.dflash2_select_gated(
        FAKE, 4096, FAKE, FAKE, FAKE, 1, 4096, 256, h, h_dtype, FAKE, w_dtype, NULL, hidden, act, 1, K, 0.0, 0, NULL,
        FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, NULL, ws, wsb, NULL)
    assert sg(K=0) == 2
    assert sg(h=NULL) == 1
    assert sg(w_dtype=0) == 4
    assert sg(h_dtype=3) == 4
    assert sg(h_dtype=1, h=MIS) == 3
    assert sg(act=5) == 4
    assert sg(hidden=500) == 2
    assert sg(h=MIS) == 3
    assert lib.dflash2_select_gated_workspace(1, 7, 4096, 512, 256) > lib.dflash2_select_workspace(1, 7, 4096)
    assert sg(wsb=lib.dflash2_select_gated_workspace(1, 7, 4096, 512, 256) - 257) == 5
    # conv
    assert lib.dflash2_conv2tap(FAKE, FAKE, FAKE, 1, 1, 7, 512, 3, FAKE, NULL) == 2
    assert lib.dflash2_conv2tap(FAKE, NULL, FAKE, 1, 1, 7, 512, 1, FAKE, NULL) == 1
    # spec accept
    assert lib.dflash2_spec_accept(FAKE, 4096, 8 * 4096, FAKE, FAKE, NULL, 1, 7, 4096, 1.0, 0, FAKE, FAKE, NULL, ws,
                                   big, NULL) == 1
    assert lib.dflash2_spec_accept(FAKE, 4096, 100, FAKE, FAKE, FAKE, 2, 7, 4096, 1.0, 0, FAKE, FAKE, NULL, ws, big,
                                   NULL) == 2
    assert lib.dflash2_spec_accept(FAKE, 4096, 8 * 4096 + 4, FAKE, FAKE, FAKE, 2, 7, 4096, 1.0, 0, FAKE, FAKE, NULL, ws,
                                   big, NULL) == 3
    # filtered verify: the spec_accept checks, then top_k in [1, 32] and top_p in (0, 1]
    fv = lambda top_k=20, top_p=0.95, q=FAKE, T=1.0, wsb=big, K=7: lib.dflash2_spec_accept_filtered(
        FAKE, 4096, 8 * 4096, FAKE, FAKE, q, 2, K, 4096, T, top_k, top_p, 0, FAKE, FAKE, NULL, ws, wsb, NULL)
    assert fv(K=65) == 2
    assert fv(T=-1.0) == 6
    for bad_k, bad_p in ((0, 0.95), (33, 0.95), (-1, 0.95), (20, 0.0), (20, 1.5), (20, float("nan")), (20, -0.1)):
        assert fv(top_k=bad_k, top_p=bad_p) == 6, (bad_k, bad_p)
    assert fv(q=NULL) == 1
    assert fv(q=NULL, T=0.0, wsb=16) == 5               # q may be NULL when greedy; the workspace is still checked
    need = lib.dflash2_spec_accept_filtered_workspace(2, 7, 4096)
    assert need > lib.dflash2_spec_accept_workspace(2, 7, 4096)
    assert fv(wsb=need - 257) == 5


def test_binding_fails_loudly_without_library(tmp_path):
    from dflash_draft_selector_amd import dflash2
    with pytest.raises(dflash2.Dflash2Error):
        dflash2.load_library.__wrapped__(str(tmp_path / "missing.so")) if hasattr(dflash2.load_library, "__wrapped__") \
            else _load_missing(dflash2, tmp_path)


def _load_missing(dflash2, tmp_path):
    saved = dflash2._lib
    dflash2._lib = None
    try:
        dflash2.load_library(str(tmp_path / "missing.so"))
    finally:
        dflash2._lib = saved


def test_host_validation_lmhead_ring_and_graph():
    """The LM head, ring attention and graph entry points reject bad arguments before any
    launch (every call below returns on the host)."""
    d2, lib = _lib()
    ws = ctypes.c_void_p(0x200000)
    big = 1 << 31
    # LM head + top-16: hidden a multiple of 256, 16 <= vocab <= 2^19, 16-byte aligned h and W
    lm = lambda h=FAKE, w=FAKE, rows=105, hidden=5120, vocab=151936, idx=FAKE, wsb=big: lib.dflash2_lmhead_topk16(
        h, w, rows, hidden, vocab, idx, FAKE, NULL, ws, wsb, NULL)
    assert lm(h=NULL) == 1
    assert lm(idx=NULL) == 1
    for kw in ({"rows": 0}, {"hidden": 5000}, {"hidden": 128}, {"vocab": 15}, {"vocab": (1 << 19) + 1}):
        assert lm(**kw) == 2, kw
    assert lm(w=MIS) == 3
    need = lib.dflash2_lmhead_topk16_workspace(105, 151936)
    assert need >= 105 * 594 * 16 * 8
    assert lm(wsb=need - 257) == 5
    # the packed LM head: the same checks; the packed size covers whole 256-column tiles
    lmp = lambda h=FAKE, w=FAKE, rows=105, hidden=5120, vocab=151936, idx=FAKE, wsb=big: \
        lib.dflash2_lmhead_topk16_packed(h, w, rows, hidden, vocab, idx, FAKE, NULL, ws, wsb, NULL)
    assert lmp(w=NULL) == 1
    for kw in ({"rows": 0}, {"hidden": 5000}, {"vocab": 15}, {"vocab": (1 << 19) + 1}):
        assert lmp(**kw) == 2, kw
    assert lmp(h=MIS) == 3
    assert lmp(wsb=need - 257) == 5
    assert lib.dflash2_lmhead_packed_bytes(151936, 5120) == 594 * 256 * 5120 * 2
    assert lib.dflash2_lmhead_packed_bytes(151936, 5000) == 0 and lib.dflash2_lmhead_packed_bytes(15, 5120) == 0
    assert lib.dflash2_lmhead_pack(NULL, 151936, 5120, FAKE, NULL) == 1
    assert lib.dflash2_lmhead_pack(FAKE, 151936, 5000, FAKE, NULL) == 2
    assert lib.dflash2_lmhead_pack(FAKE, 151936, 5120, MIS, NULL) == 3
    # ring attention: head_dim 128, GQA rows <= 48, ring a multiple of 32, window <= ring,
    # scale >= 0 and finite
    ra = lambda q=FAKE, B=15, nq=8, hq=32, hkv=8, dh=128, ring=2112, window=2048, scale=0.0, wsb=big, ctx=FAKE: \
        lib.dflash2_ring_attention(q, FAKE, FAKE, FAKE, FAKE, ctx, B, nq, hq, hkv, dh, ring, window, scale, FAKE, ws,
                                   wsb, NULL)
    assert ra(ctx=NULL) == 1
    for kw in ({"dh": 64}, {"hq": 30}, {"hq": 56}, {"ring": 2100}, {"ring": 2056}, {"ring": 16, "window": 1},
               {"window": 2113}, {"window": 0}, {"B": 0}, {"ring": 4096, "window": 4097}):
        assert ra(**kw) == 2, kw
    assert ra(ring=1 << 20, window=1 << 20, scale=-1.0) == 6   # any window up to the ring passes the shape checks
    assert ra(scale=float("nan")) == 6
    assert ra(scale=float("inf")) == 6
    assert ra(q=MIS) == 3
    need = lib.dflash2_ring_attention_workspace(15, 8, 32, 8, 2048)
    assert need >= 15 * 8 * 32 * (128 + 2) * 4            # (max, sum, O) of every query row
    assert lib.dflash2_ring_attention_workspace(15, 8, 32, 8, 1 << 20) <= 15 * 8 * 32 * 32 * (128 + 2) * 4 + 4096
    assert ra(wsb=need - 257) == 5
    # graphs: the default stream cannot be captured; null handles are refused
    out = ctypes.c_void_p()
    assert lib.dflash2_graph_begin(NULL) == 1
    assert lib.dflash2_graph_end(NULL, ctypes.byref(out)) == 1
    assert lib.dflash2_graph_launch(NULL, NULL) == 1
    assert lib.dflash2_graph_destroy(NULL) == 1


def test_temperature_range_on_host():
    """A temperature is 0 or finite and at least FLT_MIN = 2^-126: below it 1/T overflows
    in fp32.  Subnormal temperatures are refused before any launch; FLT_MIN itself passes
    the check (the select then stops at its too-small workspace, status 5)."""
    d2, lib = _lib()
    ws = ctypes.c_void_p(0x200000)
    flt_min = 2.0 ** -126
    sel = lambda T: lib.dflash2_select(FAKE, 4096, FAKE, FAKE, FAKE, 1, 4096, 256, FAKE, 1, 7, T, 0, FAKE, FAKE, FAKE,
                                       FAKE, FAKE, FAKE, NULL, ws, 16, NULL)
    for T in (1e-39, 2.0 ** -127, 2.0 ** -149, -1e-39, float("inf"), float("-inf"), float("nan")):
        assert lib.dflash2_walk(FAKE, FAKE, 1, 7, T, 0, FAKE, FAKE, FAKE, NULL) == 6, T
        assert sel(T) == 6, T
        assert lib.dflash2_spec_accept(FAKE, 4096, 8 * 4096, FAKE, FAKE, FAKE, 1, 7, 4096, T, 0, FAKE, FAKE, NULL, ws,
                                       16, NULL) == 6, T
    for T in (0.0, flt_min, 1e-30, 1.0, 3.0e38):
        assert sel(T) == 5, T


def test_select_noalloc_refuses_requests_beyond_its_scratch():
    """The select without workspace checks its request against the 4 MiB scratch on the
    host: a request whose workspace would exceed it returns DFLASH2_ERR_WORKSPACE before
    any HIP call; the other argument checks are those of dflash2_select."""
    d2, lib = _lib()
    sel = lambda B, K, V=151936, T=0.0, S=FAKE: lib.dflash2_select_noalloc(
        FAKE, V, FAKE, FAKE, FAKE, 1, V, 256, FAKE, B, K, T, 0, FAKE, FAKE, S, FAKE, FAKE, FAKE, NULL, NULL)
    assert lib.dflash2_select_workspace(64, 64, 1 << 19) > 4 << 20
    assert sel(64, 64, 1 << 19) == 5
    assert sel(1, 0) == 2
    assert sel(15, 7, T=-1.0) == 6
    assert sel(15, 7, S=MIS) == 3
