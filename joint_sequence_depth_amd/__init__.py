"""MoDA joint sequence/depth attention forward (and decode step) on MI355X (gfx950).

The computation lives in libmoda_attn.so (hand-written HIP kernels behind the C
ABI declared in include/moda_attn.h); this package only marshals torch tensors.
"""
from ._lib import EXPORTS, ModaError, attn_decode, attn_fwd, decode_workspace_size, lib  # noqa: F401

__all__ = ["attn_fwd", "attn_decode", "decode_workspace_size", "lib", "ModaError", "EXPORTS"]
