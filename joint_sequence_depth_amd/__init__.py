"""MoDA joint sequence/depth attention on MI355X (gfx950): forward, backward,
decode step and depth-KV writer.

The computation lives in libmoda_attn.so (hand-written HIP kernels behind the C
ABI declared in include/moda_attn.h); this package only marshals torch tensors.
"""
from ._lib import (  # noqa: F401
    EXPORTS,
    ModaError,
    attn_bwd,
    attn_decode,
    attn_decode_noalloc,
    attn_fwd,
    bwd_workspace_size,
    decode_workspace_size,
    depth_kv_project,
    depth_kv_write,
    lib,
    topk_workspace_size,
)

__all__ = ["attn_fwd", "attn_bwd", "attn_decode", "attn_decode_noalloc", "depth_kv_write", "depth_kv_project", "bwd_workspace_size", "decode_workspace_size",
           "topk_workspace_size", "lib", "ModaError", "EXPORTS"]
