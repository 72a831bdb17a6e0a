"""Seeded synthetic inputs for the DFlash 2 proposer hot path.

This module only draws random data with fixed seeds and a fixed draw order.  It
holds none of the method's arithmetic: it is shared by the tests (which hand the
same arrays to the CPU oracle and to the HIP library) and by the benchmark.

Workloads (sizes and distributions, seed = workload index):

  c0  tiny greedy     B=1  K=7  V=4096    D=512   fp32 tables and gate weight,
                      logits N(0, 3^2) rounded to bf16 (so exact bf16 ties occur)
  c1  single request  B=1  K=7  V=151936  D=5120  bf16 tables / gate weight,
                      one planted peak of +8 per position
  c2  batched greedy  B=15 K=7  V=151936  D=5120  peak +8-t at position t
  c3  throughput      B=64 K=15 V=151936  D=5120  peak +8-t, conv at 4 sites
  c4  sampled+verify  c2's draft side, T=1, target logits bf16 [B, K+1, V]
                      ~ N(0, 3^2), walk seed 4

Common to all: C=16 candidates, selector dim 256, A and B tables ~ N(0, 1/256),
h ~ N(0, 1), gate weight ~ N(0, 1/D) with zero bias, verified ids ~ U[0, V),
conv x and previous hidden ~ N(0, 1), conv taps ~ U(-1, 1), group size 1.

Draw order from ``numpy.random.default_rng(seed)`` (PCG64), all float32 draws:
logits, peak indices (if any), table A, table B, h, gate weight, verified ids,
conv x, conv previous hidden, conv taps, target logits (c4 only).  Planted peaks
are added in float32 before the bf16 rounding (round to nearest, ties to even).
"""

from __future__ import annotations

import dataclasses

import numpy as np

VOCAB_QWEN = 151936


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    B: int
    K: int
    V: int
    D: int
    dim: int = 256
    C: int = 16
    bf16_params: bool = True      # tables A, B and gate weight stored as bf16
    peak: str = "decay"           # "none" | "const" | "decay"
    sites: int = 1                # conv sites per position
    group: int = 1                # conv channel-group size
    temperature: float = 0.0      # walk / verify temperature (0 = greedy)
    walk_seed: int = 0
    target: bool = False          # also draw target logits [B, K+1, V]

    @property
    def rows(self) -> int:
        return self.B * self.K


WORKLOADS = {
    0: Workload("c0_tiny_greedy", 0, B=1, K=7, V=4096, D=512, bf16_params=False, peak="none"),
    1: Workload("c1_single_request_greedy", 1, B=1, K=7, V=VOCAB_QWEN, D=5120, peak="const"),
    2: Workload("c2_batched_greedy_b15_k7", 2, B=15, K=7, V=VOCAB_QWEN, D=5120, peak="decay"),
    3: Workload("c3_throughput_b64_k15", 3, B=64, K=15, V=VOCAB_QWEN, D=5120, peak="decay", sites=4),
    4: Workload("c4_sampled_verify_b15_k7", 4, B=15, K=7, V=VOCAB_QWEN, D=5120, peak="decay",
                temperature=1.0, walk_seed=4, target=True),
}


def workload(index: int, **overrides) -> Workload:
    """Return workload ``index``, optionally with fields replaced (e.g. a smaller V)."""
    return dataclasses.replace(WORKLOADS[index], **overrides)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round finite float32 data to bf16 (nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    u = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (u >> np.uint32(16)).astype(np.uint16)


def _normal(rng, shape, std):
    return rng.standard_normal(shape, dtype=np.float32) * np.float32(std)


def make_inputs(w: Workload) -> dict:
    """Draw every input of workload ``w``.

    Returns a dict of numpy arrays.  bf16 data is returned as uint16 bit patterns
    (``*_bits``); float32 data as float32.
    """
    rng = np.random.default_rng(w.seed)
    out: dict = {"workload": w}
    logits = _normal(rng, (w.B, w.K, w.V), 3.0)
    if w.peak != "none":
        pidx = rng.integers(0, w.V, size=(w.B, w.K))
        bump = np.full((w.B, w.K), 8.0, dtype=np.float32)
        if w.peak == "decay":
            bump = bump - np.arange(w.K, dtype=np.float32)[None, :]
        bi, ti = np.meshgrid(np.arange(w.B), np.arange(w.K), indexing="ij")
        logits[bi, ti, pidx] += bump
        out["peak_idx"] = pidx
    out["logits_bits"] = f32_to_bf16_bits(logits)
    del logits
    emb_a = _normal(rng, (w.V, w.dim), 1.0 / 16.0)
    emb_b = _normal(rng, (w.V, w.dim), 1.0 / 16.0)
    h = _normal(rng, (w.B, w.K, w.D), 1.0)
    w_h = _normal(rng, (w.dim, w.D), float(np.sqrt(1.0 / w.D)))
    if w.bf16_params:
        out["emb_a_bits"] = f32_to_bf16_bits(emb_a)
        out["emb_b_bits"] = f32_to_bf16_bits(emb_b)
        out["w_h_bits"] = f32_to_bf16_bits(w_h)
    else:
        out["emb_a"] = emb_a
        out["emb_b"] = emb_b
        out["w_h"] = w_h
    out["h"] = h
    out["bias"] = np.zeros(w.dim, dtype=np.float32)
    out["verified"] = rng.integers(0, w.V, size=w.B).astype(np.int32)
    out["conv_x"] = _normal(rng, (w.sites, w.B, w.K, w.D), 1.0)
    out["conv_prev"] = _normal(rng, (w.sites, w.B, w.D), 1.0)
    out["conv_taps"] = rng.uniform(-1.0, 1.0, size=(w.sites, w.B, w.K, 2, w.D // w.group)).astype(np.float32)
    if w.target:
        out["target_bits"] = f32_to_bf16_bits(_normal(rng, (w.B, w.K + 1, w.V), 3.0))
    return out


def make_target(w: Workload, seed: int) -> np.ndarray:
    """Target logits bf16 bits [B, K+1, V] ~ N(0, 3^2) from their own generator (the
    c4 recipe at any workload's shape)."""
    rng = np.random.default_rng(seed)
    return f32_to_bf16_bits(_normal(rng, (w.B, w.K + 1, w.V), 3.0))


def bf16_bits_as_f32(bits: np.ndarray) -> np.ndarray:
    """Reinterpret bf16 bit patterns as the float32 values they denote (exact widening)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def lmhead_inputs(rows: int, hidden: int, vocab: int, seed: int, peaks: bool = True) -> dict:
    """Inputs of the LM head with the fused top-16: draft hidden rows h ~ N(0, 1) and a
    weight W ~ N(0, 1/hidden), both rounded to bf16, drawn in that order from
    ``default_rng(seed)``.  With ``peaks`` every row r gets a planted peak: W row
    peak_r (uniform, drawn after W) is set to h_r * 8 / hidden, so its logit is about 8
    against N(0, 1) for the rest (the c1-c4 recipe of one strong candidate per slot).
    Returns uint16 bit patterns ``h_bits`` [rows, hidden] and ``w_bits`` [vocab, hidden]
    (and ``peak_idx``)."""
    rng = np.random.default_rng(seed)
    h = _normal(rng, (rows, hidden), 1.0)
    w = np.empty((vocab, hidden), dtype=np.uint16)
    step = 8192
    for v0 in range(0, vocab, step):
        w[v0:v0 + step] = f32_to_bf16_bits(_normal(rng, (min(step, vocab - v0), hidden), float(np.sqrt(1.0 / hidden))))
    out = {"h_bits": f32_to_bf16_bits(h), "w_bits": w}
    if peaks:
        pidx = rng.integers(0, vocab, size=rows)
        w[pidx] = f32_to_bf16_bits(h * np.float32(8.0 / hidden))
        out["peak_idx"] = pidx
    return out


def ring_inputs(B: int, nq: int, hq: int, hkv: int, ring: int, ctx_len, seed: int, dh: int = 128,
                q_scale: float = 1.0) -> dict:
    """Inputs of the draft-block ring attention: q (times q_scale), block K/V and ring K/V
    ~ N(0, 1) rounded to bf16, drawn in that order from ``default_rng(seed)``; ctx_len as
    given (an int per request).  Rows of the ring that the window does not cover hold
    the same kind of data (a ring is reused, so stale rows are ordinary numbers)."""
    rng = np.random.default_rng(seed)
    out = {"q_bits": f32_to_bf16_bits(_normal(rng, (B, nq, hq, dh), q_scale)),
           "kb_bits": f32_to_bf16_bits(_normal(rng, (B, nq, hkv, dh), 1.0)),
           "vb_bits": f32_to_bf16_bits(_normal(rng, (B, nq, hkv, dh), 1.0)),
           "kr_bits": f32_to_bf16_bits(_normal(rng, (B, ring, hkv, dh), 1.0)),
           "vr_bits": f32_to_bf16_bits(_normal(rng, (B, ring, hkv, dh), 1.0)),
           "ctx_len": np.asarray(ctx_len, dtype=np.int32)}
    return out
