"""The tiled K/V ring layouts of dflash2_ring_attention (include/dflash2.h): the binding's
re-layout helpers against the element formulas the header states, element by element,
and the K tile against the order in which a step's MFMA slices are read (lane
16 g + i of slice (t, s) takes dims 32 s + 8 g .. + 7 of tile position
8 (i / 4) + 4 t + i % 4).  CPU only."""

import numpy as np
import pytest
import torch

from dflash_draft_selector_amd import dflash2


def rows(B=2, ring=96, hkv=3, dh=128, seed=0):
    return np.random.default_rng(seed).integers(0, 65536, size=(B, ring, hkv, dh)).astype(np.uint16)


def test_k_tiles_follow_the_header_formula():
    a = rows()
    B, ring, hkv, dh = a.shape
    t = dflash2.ring_k_tiles(a)
    assert t.shape == dflash2.ring_k_shape(B, hkv, ring, dh) == (B, hkv, ring // 32, 32 * dh)
    for b in range(B):
        for p in range(ring):
            for h in range(hkv):
                pp = p % 32
                for d in range(dh):
                    off = ((((pp // 4) % 2) * 4 + d // 32) * 4 + (d % 32) // 8) * 128 + (4 * (pp // 8) + pp % 4) * 8 \
                        + d % 8
                    assert t[b, h, p // 32, off] == a[b, p, h, d]


def test_k_tile_slices_are_the_mfma_operand_order():
    a = rows(B=1, ring=64, hkv=2)
    t = dflash2.ring_k_tiles(a)
    for tile in range(2):
        for tt in range(2):
            for s in range(4):
                for lane in range(64):
                    g, i = lane // 16, lane % 16
                    key = 32 * tile + 8 * (i // 4) + 4 * tt + i % 4
                    seg = t[0, 1, tile, (4 * tt + s) * 512 + 8 * lane:(4 * tt + s) * 512 + 8 * lane + 8]
                    assert np.array_equal(seg, a[0, key, 1, 32 * s + 8 * g:32 * s + 8 * g + 8])


def test_v_tiles_follow_the_header_formula():
    a = rows(seed=1)
    B, ring, hkv, dh = a.shape
    t = dflash2.ring_v_tiles(a)
    assert t.shape == dflash2.ring_v_shape(B, hkv, ring, dh) == (B, hkv, ring // 32, dh, 32)
    for b in range(B):
        for p in range(ring):
            for h in range(hkv):
                assert np.array_equal(t[b, h, p // 32, :, p % 32], a[b, p, h, :])


def test_torch_and_numpy_agree_and_rings_must_be_whole_tiles():
    a = rows(seed=2)
    ta = torch.from_numpy(a.view(np.int16))
    assert np.array_equal(dflash2.ring_k_tiles(ta).numpy().view(np.uint16), dflash2.ring_k_tiles(a))
    assert np.array_equal(dflash2.ring_v_tiles(ta).numpy().view(np.uint16), dflash2.ring_v_tiles(a))
    for shape in (dflash2.ring_k_shape, dflash2.ring_v_shape):
        with pytest.raises(ValueError):
            shape(1, 1, 2100, 128)
