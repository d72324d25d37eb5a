"""MoDA joint sequence/depth attention forward on MI355X (gfx950).

The computation lives in libmoda_attn.so (hand-written HIP kernels behind the C
ABI declared in include/moda_attn.h); this package only marshals torch tensors.
"""
from ._lib import EXPORTS, ModaError, attn_fwd, lib  # noqa: F401

__all__ = ["attn_fwd", "lib", "ModaError", "EXPORTS"]
