"""libdflash2: the DFlash 2 proposer hot path as HIP kernels for MI355X (gfx950).

The library itself is C-ABI (``include/dflash2.h``); ``dflash_draft_selector_amd.dflash2``
is a thin ctypes binding over it that takes torch tensors.  Importing this package
does not load the shared library; the first call does, and fails loudly if it has
not been built.
"""

__all__ = ["dflash2", "synth"]
