"""Thin ctypes binding of libdflash2 (argument marshalling only).

Every function takes torch tensors that live on the GPU, checks dtypes, shapes and
contiguity, allocates the outputs, and calls the C-ABI entry point of the same name
on torch's current stream.  All arithmetic runs in the library's HIP kernels; there
is no CPU or PyTorch fallback: if libdflash2.so is missing or fails to load, every
call raises.
"""

from __future__ import annotations

import ctypes
import os
import threading

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdflash2.so")

NCAND = 16
F32, BF16 = 0, 1
GATE_SIGMOID, GATE_IDENTITY = 0, 1

_lib = None
_lock = threading.Lock()

_c_ptr = ctypes.c_void_p
_i64 = ctypes.c_int64
_u64 = ctypes.c_uint64
_f32 = ctypes.c_float
_size = ctypes.c_size_t
_int = ctypes.c_int

_SIGNATURES = {
    "dflash2_abi_version": ([], _int),
    "dflash2_status_str": ([_int], ctypes.c_char_p),
    "dflash2_topk16_workspace": ([_i64, _i64], _size),
    "dflash2_topk16": ([_c_ptr, _i64, _i64, _i64, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _size, _c_ptr], _int),
    "dflash2_lmhead_topk16_workspace": ([_i64, _i64], _size),
    "dflash2_lmhead_topk16": ([_c_ptr, _c_ptr, _i64, _i64, _i64, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _size, _c_ptr], _int),
    "dflash2_lmhead_packed_bytes": ([_i64, _i64], _size),
    "dflash2_lmhead_pack": ([_c_ptr, _i64, _i64, _c_ptr, _c_ptr], _int),
    "dflash2_lmhead_topk16_packed": ([_c_ptr, _c_ptr, _i64, _i64, _i64, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _size,
                                      _c_ptr], _int),
    "dflash2_graph_begin": ([_c_ptr], _int),
    "dflash2_graph_end": ([_c_ptr, ctypes.POINTER(ctypes.c_void_p)], _int),
    "dflash2_graph_launch": ([_c_ptr, _c_ptr], _int),
    "dflash2_graph_destroy": ([_c_ptr], _int),
    "dflash2_ring_attention_workspace": ([_i64, _i64, _i64, _i64, _i64], _size),
    "dflash2_ring_attention": ([_c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _i64, _i64, _i64, _i64, _i64, _i64,
                                _i64, _f32, _c_ptr, _c_ptr, _size, _c_ptr], _int),
    "dflash2_context_gate_workspace": ([_i64, _i64, _i64], _size),
    "dflash2_context_gate": ([_c_ptr, _int, _c_ptr, _int, _c_ptr, _i64, _i64, _i64, _int, _c_ptr, _c_ptr, _size, _c_ptr],
                             _int),
    "dflash2_pair_score": ([_c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _int, _i64, _i64, _c_ptr, _i64, _i64, _c_ptr,
                            _c_ptr, _c_ptr], _int),
    "dflash2_walk": ([_c_ptr, _c_ptr, _i64, _i64, _f32, _u64, _c_ptr, _c_ptr, _c_ptr, _c_ptr], _int),
    "dflash2_select_workspace": ([_i64, _i64, _i64], _size),
    "dflash2_select": ([_c_ptr, _i64, _c_ptr, _c_ptr, _c_ptr, _int, _i64, _i64, _c_ptr, _i64, _i64, _f32, _u64,
                        _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _size, _c_ptr], _int),
    "dflash2_select_noalloc": ([_c_ptr, _i64, _c_ptr, _c_ptr, _c_ptr, _int, _i64, _i64, _c_ptr, _i64, _i64, _f32,
                                _u64, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr], _int),
    "dflash2_select_gated_workspace": ([_i64, _i64, _i64, _i64, _i64], _size),
    "dflash2_select_gated": ([_c_ptr, _i64, _c_ptr, _c_ptr, _c_ptr, _int, _i64, _i64, _c_ptr, _int, _c_ptr, _int,
                              _c_ptr, _i64, _int, _i64, _i64, _f32, _u64, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr,
                              _c_ptr, _c_ptr, _c_ptr, _size, _c_ptr], _int),
    "dflash2_conv2tap": ([_c_ptr, _c_ptr, _c_ptr, _i64, _i64, _i64, _i64, _i64, _c_ptr, _c_ptr], _int),
    "dflash2_spec_accept_workspace": ([_i64, _i64, _i64], _size),
    "dflash2_spec_accept": ([_c_ptr, _i64, _i64, _c_ptr, _c_ptr, _c_ptr, _i64, _i64, _i64, _f32, _u64, _c_ptr,
                             _c_ptr, _c_ptr, _c_ptr, _size, _c_ptr], _int),
    "dflash2_spec_accept_filtered_workspace": ([_i64, _i64, _i64], _size),
    "dflash2_spec_accept_filtered": ([_c_ptr, _i64, _i64, _c_ptr, _c_ptr, _c_ptr, _i64, _i64, _i64, _f32,
                                      ctypes.c_int32, _f32, _u64, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _size, _c_ptr],
                                     _int),
}

EXPORTED = tuple(_SIGNATURES)


class Dflash2Error(RuntimeError):
    pass


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libdflash2.so (once) and declare every entry point's signature."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(path):
                raise Dflash2Error(f"{path} is not built: run __graft_entry__.build() (hipcc, gfx950) first")
            lib = ctypes.CDLL(path)
            for name, (args, res) in _SIGNATURES.items():
                fn = getattr(lib, name)
                fn.argtypes = args
                fn.restype = res
            _lib = lib
    return _lib


def status_str(code: int) -> str:
    return load_library().dflash2_status_str(code).decode()


def _check(code: int, what: str):
    if code != 0:
        raise Dflash2Error(f"{what}: {status_str(code)}")


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t, name, dtypes, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU device")
    if dtypes is not None and t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    return t


def _contig(t, name):
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


_BF16_LIKE = (torch.bfloat16, torch.int16, torch.uint16)

# Workspaces: one buffer per (device, call kind, shape, stream).  A call writes every
# workspace byte before it reads it, so no initialisation is needed; keeping one buffer
# per stream keeps calls that may overlap in time off each other's scratch.
_ws_cache: dict = {}


def workspace(kind: str, nbytes: int, device: torch.device, shape: tuple = ()) -> torch.Tensor:
    key = (device.index, kind, tuple(shape), _stream())
    buf = _ws_cache.get(key)
    if buf is None:
        buf = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
        _ws_cache[key] = buf
    return buf


def _rows_view(logits, name):
    """(rows, vocab, ld) of a [..., V] bf16 tensor whose last dim is contiguous and
    whose leading dims collapse to one row stride."""
    if logits.dim() < 2 or logits.stride(-1) != 1:
        raise ValueError(f"{name} must be [..., V] with a contiguous last dimension")
    V = logits.shape[-1]
    lead = logits.shape[:-1]
    ld = logits.stride(-2)
    # the leading dims must be uniformly strided by ld
    expect = ld
    for size, stride in zip(reversed(lead), reversed(logits.stride()[:-1])):
        if size > 1 and stride != expect:
            raise ValueError(f"{name}: leading dimensions must collapse to one row stride")
        expect *= size
    rows = 1
    for s in lead:
        rows *= s
    return rows, V, ld


# ---------------------------------------------------------------------------------------


def topk16(logits: torch.Tensor, row_status: bool = False):
    """Top-16 candidates of every [V]-row of bf16 `logits`: (idx int32 [..., 16], val f32 [..., 16])."""
    lib = load_library()
    _need(logits, "logits", _BF16_LIKE)
    rows, V, ld = _rows_view(logits, "logits")
    dev = logits.device
    idx = torch.empty(logits.shape[:-1] + (NCAND,), dtype=torch.int32, device=dev)
    val = torch.empty(logits.shape[:-1] + (NCAND,), dtype=torch.float32, device=dev)
    st = torch.empty(logits.shape[:-1], dtype=torch.int32, device=dev) if row_status else None
    nbytes = lib.dflash2_topk16_workspace(rows, V)
    ws = workspace("topk16", nbytes, dev, (rows, V))
    _check(lib.dflash2_topk16(_ptr(logits), rows, V, ld, _ptr(idx), _ptr(val), _ptr(st), _ptr(ws), ws.numel(),
                              _stream()), "dflash2_topk16")
    return (idx, val, st) if row_status else (idx, val)


def lmhead_topk16(h: torch.Tensor, w: torch.Tensor, row_status: bool = False):
    """Top-16 candidates of the bf16 logits h @ w.T without writing them: h bf16 [rows, D]
    (or [..., D]), w bf16 [V, D].  Returns (idx int32 [..., 16], val f32 [..., 16])."""
    lib = load_library()
    _contig(_need(h, "h", _BF16_LIKE), "h")
    _contig(_need(w, "w", _BF16_LIKE, h.device), "w")
    if h.dim() < 2 or w.dim() != 2 or w.shape[1] != h.shape[-1]:
        raise ValueError("lmhead_topk16: h [..., D] and w [V, D] must share D")
    D, V = h.shape[-1], w.shape[0]
    rows = h.numel() // D
    dev = h.device
    idx = torch.empty(h.shape[:-1] + (NCAND,), dtype=torch.int32, device=dev)
    val = torch.empty(h.shape[:-1] + (NCAND,), dtype=torch.float32, device=dev)
    st = torch.empty(h.shape[:-1], dtype=torch.int32, device=dev) if row_status else None
    nbytes = lib.dflash2_lmhead_topk16_workspace(rows, V)
    ws = workspace("lmhead_topk16", nbytes, dev, (rows, V))
    _check(lib.dflash2_lmhead_topk16(_ptr(h), _ptr(w), rows, D, V, _ptr(idx), _ptr(val), _ptr(st), _ptr(ws),
                                     ws.numel(), _stream()), "dflash2_lmhead_topk16")
    return (idx, val, st) if row_status else (idx, val)


def lmhead_pack(w: torch.Tensor) -> torch.Tensor:
    """The LM-head weight bf16 [V, D] in the packed layout lmhead_topk16_packed reads (a
    new bf16 tensor of dflash2_lmhead_packed_bytes, done once per weight)."""
    lib = load_library()
    _contig(_need(w, "w", _BF16_LIKE), "w")
    if w.dim() != 2:
        raise ValueError("lmhead_pack: w must be [V, D]")
    V, D = w.shape
    nbytes = lib.dflash2_lmhead_packed_bytes(V, D)
    if nbytes == 0:
        raise ValueError("lmhead_pack: unsupported shape")
    wp = torch.empty(nbytes // 2, dtype=w.dtype, device=w.device)
    _check(lib.dflash2_lmhead_pack(_ptr(w), V, D, _ptr(wp), _stream()), "dflash2_lmhead_pack")
    return wp


def lmhead_topk16_packed(h: torch.Tensor, w_packed: torch.Tensor, vocab: int, row_status: bool = False):
    """lmhead_topk16 on a weight packed by lmhead_pack (bit-identical results): h bf16
    [rows, D] (or [..., D]), w_packed from lmhead_pack of a [vocab, D] weight."""
    lib = load_library()
    _contig(_need(h, "h", _BF16_LIKE), "h")
    _contig(_need(w_packed, "w_packed", _BF16_LIKE, h.device), "w_packed")
    if h.dim() < 2:
        raise ValueError("lmhead_topk16_packed: h must be [..., D]")
    D, V = h.shape[-1], int(vocab)
    if w_packed.numel() * 2 != lib.dflash2_lmhead_packed_bytes(V, D):
        raise ValueError("lmhead_topk16_packed: w_packed does not hold a packed [vocab, D] weight")
    rows = h.numel() // D
    dev = h.device
    idx = torch.empty(h.shape[:-1] + (NCAND,), dtype=torch.int32, device=dev)
    val = torch.empty(h.shape[:-1] + (NCAND,), dtype=torch.float32, device=dev)
    st = torch.empty(h.shape[:-1], dtype=torch.int32, device=dev) if row_status else None
    nbytes = lib.dflash2_lmhead_topk16_workspace(rows, V)
    ws = workspace("lmhead_topk16", nbytes, dev, (rows, V))
    _check(lib.dflash2_lmhead_topk16_packed(_ptr(h), _ptr(w_packed), rows, D, V, _ptr(idx), _ptr(val), _ptr(st),
                                            _ptr(ws), ws.numel(), _stream()), "dflash2_lmhead_topk16_packed")
    return (idx, val, st) if row_status else (idx, val)


class Graph:
    """Records the library calls made on torch's current stream inside ``with`` into one
    HIP graph; ``launch()`` replays them with one launch on the same buffers.

    Make every recorded call once before recording, so that its workspace and outputs
    exist (pass ``out=`` / ``y=`` buffers); the current stream must not be the default
    stream.  Inputs are refreshed in place between launches."""

    def __init__(self):
        self._lib = load_library()
        self.handle = None

    def __enter__(self):
        s = _stream()
        if not s:
            raise Dflash2Error("Graph: record on a non-default stream (torch.cuda.stream(...))")
        _check(self._lib.dflash2_graph_begin(s), "dflash2_graph_begin")
        return self

    def __exit__(self, exc_type, exc, tb):
        h = ctypes.c_void_p()
        code = self._lib.dflash2_graph_end(_stream(), ctypes.byref(h))
        if exc_type is None:
            _check(code, "dflash2_graph_end")
            self.handle = h
        return False

    def launch(self):
        if self.handle is None:
            raise Dflash2Error("Graph: nothing recorded")
        _check(self._lib.dflash2_graph_launch(self.handle, _stream()), "dflash2_graph_launch")

    def close(self):
        if self.handle is not None:
            self._lib.dflash2_graph_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def ring_k_shape(B: int, hkv: int, ring: int, dh: int) -> tuple:
    """Shape of the K ring the library reads: tiles of 32 positions [B, Hkv, ring / 32,
    32 * Dh], each tile in the order the matrix cores read it (ring_k_tiles)."""
    if ring % 32:
        raise ValueError("ring_k_shape: ring must be a multiple of 32")
    return (B, hkv, ring // 32, 32 * dh)


def ring_k_tiles(k_rows):
    """A K ring held as rows [B, ring, Hkv, Dh] (Dh = 128) in the library's tiled layout:
    position p, dim d of tile p // 32 (pp = p % 32) at [(pp // 4) % 2][d // 32]
    [(d % 32) // 8][4 (pp // 8) + pp % 4][d % 8] within the tile's 32 * Dh elements (a
    copy; torch tensor or numpy array)."""
    B, ring, hkv, dh = k_rows.shape
    # source axes: b, tile, pp // 8, (pp // 4) % 2, pp % 4, head, d // 32, (d % 32) // 8, d % 8
    t = k_rows.reshape(B, ring // 32, 4, 2, 4, hkv, dh // 32, 4, 8)
    order = (0, 5, 1, 3, 6, 7, 2, 4, 8)
    if isinstance(t, torch.Tensor):
        return t.permute(*order).contiguous().reshape(B, hkv, ring // 32, 32 * dh)
    import numpy as np
    return np.ascontiguousarray(t.transpose(*order)).reshape(B, hkv, ring // 32, 32 * dh)


def ring_v_shape(B: int, hkv: int, ring: int, dh: int) -> tuple:
    """Shape of the V ring the library reads: tiles of 32 positions, transposed within the
    tile, [B, Hkv, ring / 32, Dh, 32] (position p, dim d at [p // 32, d, p % 32])."""
    if ring % 32:
        raise ValueError("ring_v_shape: ring must be a multiple of 32")
    return (B, hkv, ring // 32, dh, 32)


def ring_v_tiles(v_rows):
    """A V ring held as rows [B, ring, Hkv, Dh] in the library's tiled layout
    [B, Hkv, ring / 32, Dh, 32] (a copy; torch tensor or numpy array)."""
    B, ring, hkv, dh = v_rows.shape
    t = v_rows.reshape(B, ring // 32, 32, hkv, dh)
    if isinstance(t, torch.Tensor):
        return t.permute(0, 3, 1, 4, 2).contiguous()
    import numpy as np
    return np.ascontiguousarray(t.transpose(0, 3, 1, 4, 2))


def ring_attention(q, k_blk, v_blk, k_ring, v_ring, ctx_len, window: int = 2048, scale: float = 0.0):
    """Draft-block attention over each request's K/V ring: q bf16 [B, nq, Hq, Dh], k_blk /
    v_blk bf16 [B, nq, Hkv, Dh], k_ring bf16 [B, Hkv, ring / 32, 32 * Dh] (ring_k_shape /
    ring_k_tiles), v_ring bf16 [B, Hkv, ring / 32, Dh, 32] (ring_v_shape / ring_v_tiles),
    ctx_len int32 [B].  Returns float32 [B, nq, Hq, Dh]."""
    lib = load_library()
    for t, n in ((q, "q"), (k_blk, "k_blk"), (v_blk, "v_blk"), (k_ring, "k_ring"), (v_ring, "v_ring")):
        _contig(_need(t, n, _BF16_LIKE, q.device), n)
    _contig(_need(ctx_len, "ctx_len", (torch.int32,), q.device), "ctx_len")
    B, nq, hq, dh = q.shape
    hkv, ring = k_blk.shape[2], 32 * k_ring.shape[2]
    if k_blk.shape != (B, nq, hkv, dh) or v_blk.shape != k_blk.shape or k_ring.shape != ring_k_shape(B, hkv, ring, dh) \
            or v_ring.shape != ring_v_shape(B, hkv, ring, dh) or ctx_len.shape != (B,):
        raise ValueError("ring_attention: inconsistent shapes")
    out = torch.empty((B, nq, hq, dh), dtype=torch.float32, device=q.device)
    nbytes = lib.dflash2_ring_attention_workspace(B, nq, hq, hkv, window)
    ws = workspace("ring_attention", nbytes, q.device, (B, nq, hq, hkv, window))
    _check(lib.dflash2_ring_attention(_ptr(q), _ptr(k_blk), _ptr(v_blk), _ptr(k_ring), _ptr(v_ring), _ptr(ctx_len),
                                      B, nq, hq, hkv, dh, ring, window, scale, _ptr(out), _ptr(ws), ws.numel(),
                                      _stream()), "dflash2_ring_attention")
    return out


def context_gate(h: torch.Tensor, w_h: torch.Tensor, bias: torch.Tensor | None = None, act: str = "sigmoid",
                 out: torch.Tensor | None = None):
    """H = act(W_H h + b) for h [..., hidden] (fp32 or bf16) and W_H [dim, hidden] (fp32 or
    bf16).

    `out` may supply a contiguous fp32 tensor of shape [..., dim] to write H into."""
    lib = load_library()
    _contig(_need(h, "h", (torch.float32,) + _BF16_LIKE), "h")
    _contig(_need(w_h, "w_h", (torch.float32,) + _BF16_LIKE, h.device), "w_h")
    if bias is not None:
        _contig(_need(bias, "bias", (torch.float32,), h.device), "bias")
    dim, hidden = w_h.shape
    if h.shape[-1] != hidden:
        raise ValueError("h and w_h disagree on the hidden size")
    rows = h.numel() // hidden
    if out is None:
        H = torch.empty(h.shape[:-1] + (dim,), dtype=torch.float32, device=h.device)
    else:
        H = _contig(_need(out, "out", (torch.float32,), h.device), "out")
        if tuple(H.shape) != tuple(h.shape[:-1]) + (dim,):
            raise ValueError("out must have shape h.shape[:-1] + (dim,)")
    wdt = F32 if w_h.dtype == torch.float32 else BF16
    a = {"sigmoid": GATE_SIGMOID, "identity": GATE_IDENTITY}[act]
    nbytes = lib.dflash2_context_gate_workspace(rows, hidden, dim)
    ws = workspace("gate", nbytes, h.device, (rows, hidden, dim))
    hdt = F32 if h.dtype == torch.float32 else BF16
    _check(lib.dflash2_context_gate(_ptr(h), hdt, _ptr(w_h), wdt, _ptr(bias), rows, hidden, dim, a, _ptr(H), _ptr(ws),
                                    ws.numel(), _stream()), "dflash2_context_gate")
    return H


def _emb_dtype(emb_a, emb_b):
    if emb_a.dtype != emb_b.dtype:
        raise TypeError("emb_a and emb_b must share a dtype")
    return F32 if emb_a.dtype == torch.float32 else BF16


def pair_score(cand_idx, cand_val, verified, emb_a, emb_b, H):
    """S [B, K, 16, 16] and row_status [B, K] from candidates [B, K, 16] and gates H [B, K, dim]."""
    lib = load_library()
    dev = cand_idx.device
    _contig(_need(cand_idx, "cand_idx", (torch.int32,)), "cand_idx")
    _contig(_need(cand_val, "cand_val", (torch.float32,), dev), "cand_val")
    _contig(_need(verified, "verified", (torch.int32,), dev), "verified")
    _contig(_need(emb_a, "emb_a", (torch.float32,) + _BF16_LIKE, dev), "emb_a")
    _contig(_need(emb_b, "emb_b", (torch.float32,) + _BF16_LIKE, dev), "emb_b")
    _contig(_need(H, "H", (torch.float32,), dev), "H")
    B, K, _ = cand_idx.shape
    V, dim = emb_a.shape
    S = torch.empty((B, K, NCAND, NCAND), dtype=torch.float32, device=dev)
    st = torch.empty((B, K), dtype=torch.int32, device=dev)
    _check(lib.dflash2_pair_score(_ptr(cand_idx), _ptr(cand_val), _ptr(verified), _ptr(emb_a), _ptr(emb_b),
                                  _emb_dtype(emb_a, emb_b), V, dim, _ptr(H), B, K, _ptr(S), _ptr(st), _stream()),
           "dflash2_pair_score")
    return S, st


def walk(S, cand_idx, temperature: float = 0.0, seed: int = 0):
    """(tokens int32 [B, K], slots int32 [B, K], q f32 [B, K, 16]) of the greedy or sampled walk."""
    lib = load_library()
    dev = S.device
    _contig(_need(S, "S", (torch.float32,)), "S")
    _contig(_need(cand_idx, "cand_idx", (torch.int32,), dev), "cand_idx")
    B, K = S.shape[:2]
    tokens = torch.empty((B, K), dtype=torch.int32, device=dev)
    slots = torch.empty((B, K), dtype=torch.int32, device=dev)
    q = torch.empty((B, K, NCAND), dtype=torch.float32, device=dev)
    _check(lib.dflash2_walk(_ptr(S), _ptr(cand_idx), B, K, float(temperature), int(seed) & (2 ** 64 - 1), _ptr(tokens),
                            _ptr(slots), _ptr(q), _stream()), "dflash2_walk")
    return tokens, slots, q


def select(logits, verified, emb_a, emb_b, H, temperature: float = 0.0, seed: int = 0, out: dict | None = None):
    """Fused top-16 -> pair score -> walk in one launch.  logits [B, K, V] bf16.

    Returns a dict with cand_idx, cand_val, S, tokens, slots, q, row_status.  `out`
    may supply preallocated tensors of those names (reused, no allocation).
    """
    lib = load_library()
    dev = logits.device
    _need(logits, "logits", _BF16_LIKE)
    rows, V, ld = _rows_view(logits, "logits")
    B, K = logits.shape[0], logits.shape[1]
    _contig(_need(verified, "verified", (torch.int32,), dev), "verified")
    _contig(_need(emb_a, "emb_a", (torch.float32,) + _BF16_LIKE, dev), "emb_a")
    _contig(_need(emb_b, "emb_b", (torch.float32,) + _BF16_LIKE, dev), "emb_b")
    _contig(_need(H, "H", (torch.float32,), dev), "H")
    dim = emb_a.shape[1]
    if out is None:
        out = {
            "cand_idx": torch.empty((B, K, NCAND), dtype=torch.int32, device=dev),
            "cand_val": torch.empty((B, K, NCAND), dtype=torch.float32, device=dev),
            "S": torch.empty((B, K, NCAND, NCAND), dtype=torch.float32, device=dev),
            "tokens": torch.empty((B, K), dtype=torch.int32, device=dev),
            "slots": torch.empty((B, K), dtype=torch.int32, device=dev),
            "q": torch.empty((B, K, NCAND), dtype=torch.float32, device=dev),
            "row_status": torch.empty((B, K), dtype=torch.int32, device=dev),
        }
    nbytes = lib.dflash2_select_workspace(B, K, V)
    ws = workspace("select", nbytes, dev, (B, K, V))
    _check(lib.dflash2_select(_ptr(logits), ld, _ptr(verified), _ptr(emb_a), _ptr(emb_b), _emb_dtype(emb_a, emb_b), V,
                              dim, _ptr(H), B, K, float(temperature), int(seed) & (2 ** 64 - 1), _ptr(out["cand_idx"]),
                              _ptr(out["cand_val"]), _ptr(out["S"]), _ptr(out["tokens"]), _ptr(out["slots"]),
                              _ptr(out["q"]), _ptr(out["row_status"]), _ptr(ws), ws.numel(), _stream()),
           "dflash2_select")
    return out


def select_noalloc(logits, verified, emb_a, emb_b, H, temperature: float = 0.0, seed: int = 0,
                   out: dict | None = None):
    """select() through dflash2_select_noalloc: the library's own per-GPU scratch instead
    of a workspace (no device allocation by the library; with `out` given, none at all).
    Calls that overlap on one GPU race on that scratch."""
    lib = load_library()
    dev = logits.device
    _need(logits, "logits", _BF16_LIKE)
    rows, V, ld = _rows_view(logits, "logits")
    B, K = logits.shape[0], logits.shape[1]
    _contig(_need(verified, "verified", (torch.int32,), dev), "verified")
    _contig(_need(emb_a, "emb_a", (torch.float32,) + _BF16_LIKE, dev), "emb_a")
    _contig(_need(emb_b, "emb_b", (torch.float32,) + _BF16_LIKE, dev), "emb_b")
    _contig(_need(H, "H", (torch.float32,), dev), "H")
    dim = emb_a.shape[1]
    if out is None:
        out = {
            "cand_idx": torch.empty((B, K, NCAND), dtype=torch.int32, device=dev),
            "cand_val": torch.empty((B, K, NCAND), dtype=torch.float32, device=dev),
            "S": torch.empty((B, K, NCAND, NCAND), dtype=torch.float32, device=dev),
            "tokens": torch.empty((B, K), dtype=torch.int32, device=dev),
            "slots": torch.empty((B, K), dtype=torch.int32, device=dev),
            "q": torch.empty((B, K, NCAND), dtype=torch.float32, device=dev),
            "row_status": torch.empty((B, K), dtype=torch.int32, device=dev),
        }
    _check(lib.dflash2_select_noalloc(_ptr(logits), ld, _ptr(verified), _ptr(emb_a), _ptr(emb_b),
                                      _emb_dtype(emb_a, emb_b), V, dim, _ptr(H), B, K, float(temperature),
                                      int(seed) & (2 ** 64 - 1), _ptr(out["cand_idx"]), _ptr(out["cand_val"]),
                                      _ptr(out["S"]), _ptr(out["tokens"]), _ptr(out["slots"]), _ptr(out["q"]),
                                      _ptr(out["row_status"]), _stream()),
           "dflash2_select_noalloc")
    return out


def select_gated(logits, verified, emb_a, emb_b, h, w_h, bias=None, act: str = "sigmoid", temperature: float = 0.0,
                 seed: int = 0, out: dict | None = None, H_out: torch.Tensor | None = None):
    """Context gate + select in one call: h [B, K, hidden] fp32 or bf16, w_h [dim, hidden] bf16.

    Returns the dict of select(); H_out (fp32 [B, K, dim]) receives the gate values the
    scores used when given.
    """
    lib = load_library()
    dev = logits.device
    _need(logits, "logits", _BF16_LIKE)
    rows, V, ld = _rows_view(logits, "logits")
    B, K = logits.shape[0], logits.shape[1]
    _contig(_need(verified, "verified", (torch.int32,), dev), "verified")
    _contig(_need(emb_a, "emb_a", (torch.float32,) + _BF16_LIKE, dev), "emb_a")
    _contig(_need(emb_b, "emb_b", (torch.float32,) + _BF16_LIKE, dev), "emb_b")
    _contig(_need(h, "h", (torch.float32,) + _BF16_LIKE, dev), "h")
    _contig(_need(w_h, "w_h", _BF16_LIKE, dev), "w_h")
    if bias is not None:
        _contig(_need(bias, "bias", (torch.float32,), dev), "bias")
    dim = emb_a.shape[1]
    hidden = h.shape[-1]
    if tuple(h.shape) != (B, K, hidden) or tuple(w_h.shape) != (dim, hidden):
        raise ValueError("h must be [B, K, hidden] and w_h [dim, hidden] with dim = emb_a.shape[1]")
    if H_out is not None:
        _contig(_need(H_out, "H_out", (torch.float32,), dev), "H_out")
        if tuple(H_out.shape) != (B, K, dim):
            raise ValueError("H_out must be [B, K, dim]")
    if out is None:
        out = {
            "cand_idx": torch.empty((B, K, NCAND), dtype=torch.int32, device=dev),
            "cand_val": torch.empty((B, K, NCAND), dtype=torch.float32, device=dev),
            "S": torch.empty((B, K, NCAND, NCAND), dtype=torch.float32, device=dev),
            "tokens": torch.empty((B, K), dtype=torch.int32, device=dev),
            "slots": torch.empty((B, K), dtype=torch.int32, device=dev),
            "q": torch.empty((B, K, NCAND), dtype=torch.float32, device=dev),
            "row_status": torch.empty((B, K), dtype=torch.int32, device=dev),
        }
    a = {"sigmoid": GATE_SIGMOID, "identity": GATE_IDENTITY}[act]
    nbytes = lib.dflash2_select_gated_workspace(B, K, V, hidden, dim)
    ws = workspace("select_gated", nbytes, dev, (B, K, V, hidden, dim))
    _check(lib.dflash2_select_gated(_ptr(logits), ld, _ptr(verified), _ptr(emb_a), _ptr(emb_b),
                                    _emb_dtype(emb_a, emb_b), V, dim, _ptr(h), F32 if h.dtype == torch.float32 else BF16,
                                    _ptr(w_h), BF16, _ptr(bias), hidden, a, B, K, float(temperature), int(seed) & (2 ** 64 - 1), _ptr(H_out),
                                    _ptr(out["cand_idx"]), _ptr(out["cand_val"]), _ptr(out["S"]), _ptr(out["tokens"]),
                                    _ptr(out["slots"]), _ptr(out["q"]), _ptr(out["row_status"]), _ptr(ws), ws.numel(),
                                    _stream()), "dflash2_select_gated")
    return out


def conv2tap(x, x_prev, taps, group: int = 1, y=None):
    """Conv(x)_t = k_{t,0} x_t + k_{t,1} x_{t-1}; x [S, B, K, D], x_prev [S, B, D], taps [S, B, K, 2, D/group]."""
    lib = load_library()
    dev = x.device
    _contig(_need(x, "x", (torch.float32,)), "x")
    _contig(_need(x_prev, "x_prev", (torch.float32,), dev), "x_prev")
    _contig(_need(taps, "taps", (torch.float32,), dev), "taps")
    S_, B, K, D = x.shape
    if y is None:
        y = torch.empty_like(x)
    _check(lib.dflash2_conv2tap(_ptr(x), _ptr(x_prev), _ptr(taps), S_, B, K, D, int(group), _ptr(y), _stream()),
           "dflash2_conv2tap")
    return y


def spec_accept(target_logits, tokens, cand_idx, q, temperature: float, seed: int = 0, shared_target: bool = False):
    """Verify drafts [B, K] against target logits [B, K+1, V] (or [K+1, V] shared by every
    request when shared_target).  Returns (out_tokens [B, K+1], n_accepted [B], row_status [B])."""
    return _spec_accept(target_logits, tokens, cand_idx, q, temperature, seed, shared_target, None, None)


def spec_accept_filtered(target_logits, tokens, cand_idx, q, temperature: float, top_k: int, top_p: float,
                         seed: int = 0, shared_target: bool = False):
    """spec_accept against the target distribution after top-k (1..32) then top-p (0, 1]
    filtering; same layouts and outputs."""
    return _spec_accept(target_logits, tokens, cand_idx, q, temperature, seed, shared_target, top_k, top_p)


def _spec_accept(target_logits, tokens, cand_idx, q, temperature, seed, shared_target, top_k, top_p):
    lib = load_library()
    dev = tokens.device
    _need(target_logits, "target_logits", _BF16_LIKE, dev)
    _contig(_need(tokens, "tokens", (torch.int32,)), "tokens")
    _contig(_need(cand_idx, "cand_idx", (torch.int32,), dev), "cand_idx")
    if q is not None:
        _contig(_need(q, "q", (torch.float32,), dev), "q")
    B, K = tokens.shape
    if target_logits.stride(-1) != 1:
        raise ValueError("target_logits must have a contiguous last dimension")
    V = target_logits.shape[-1]
    ld = target_logits.stride(-2)
    if shared_target:
        if target_logits.dim() != 2 or target_logits.shape[0] != K + 1:
            raise ValueError("shared target_logits must be [K+1, V]")
        bstride = 0
    else:
        if target_logits.dim() != 3 or target_logits.shape[:2] != (B, K + 1):
            raise ValueError("target_logits must be [B, K+1, V]")
        bstride = target_logits.stride(0)
    out = torch.empty((B, K + 1), dtype=torch.int32, device=dev)
    nacc = torch.empty((B,), dtype=torch.int32, device=dev)
    st = torch.empty((B,), dtype=torch.int32, device=dev)
    seed = int(seed) & (2 ** 64 - 1)
    if top_k is None:
        nbytes = lib.dflash2_spec_accept_workspace(1 if shared_target else B, K, V)
        ws = workspace("spec_accept", nbytes, dev, (B if not shared_target else -1, K, V))
        _check(lib.dflash2_spec_accept(_ptr(target_logits), ld, bstride, _ptr(tokens), _ptr(cand_idx), _ptr(q), B, K,
                                       V, float(temperature), seed, _ptr(out), _ptr(nacc), _ptr(st), _ptr(ws),
                                       ws.numel(), _stream()), "dflash2_spec_accept")
    else:
        nbytes = lib.dflash2_spec_accept_filtered_workspace(1 if shared_target else B, K, V)
        ws = workspace("spec_accept_filtered", nbytes, dev, (B if not shared_target else -1, K, V))
        _check(lib.dflash2_spec_accept_filtered(_ptr(target_logits), ld, bstride, _ptr(tokens), _ptr(cand_idx),
                                                _ptr(q), B, K, V, float(temperature), int(top_k), float(top_p), seed,
                                                _ptr(out), _ptr(nacc), _ptr(st), _ptr(ws), ws.numel(), _stream()),
                                       "dflash2_spec_accept_filtered")
    return out, nacc, st
