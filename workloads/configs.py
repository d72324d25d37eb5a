"""The five synthetic workloads of the MoDA joint sequence/depth attention forward.

Shapes follow the kernel notation of the MoDA deck (arXiv 2603.15619, slides
"One denominator allocates probability across both memories" and "Backup: grouped
indexing preserves the correct token map"): T tokens, H_q query heads sharing H_kv
key/value heads (G = H_q / H_kv), head dimension d, S depth slots per token.

Layouts (last dimension contiguous):
    q, out        [B, T, H_q, d]        varlen: [N, H_q, d]
    k, v          [B, T, H_kv, d]       varlen: [N, H_kv, d]
    k_depth, v_d  [B, T, S, H_kv, d]    varlen: [N, S, H_kv, d]
    lse           [B, H_q, T] float32   varlen: [H_q, N]
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

from . import gen

# tensor ids used by the generator
TID_Q, TID_K, TID_V, TID_KD, TID_VD = 1, 2, 3, 4, 5
TID_DO = 6  # upstream gradient of out (backward)
BATCH_TID_STRIDE = 16  # the i-th extra input batch uses tid + 16 * i


@dataclass(frozen=True)
class Workload:
    name: str
    desc: str
    dtype: str  # "f32" | "bf16"
    batch: int  # B (1 for varlen)
    seqlen: int  # T, or the packed total N for varlen
    n_heads_q: int
    n_heads_kv: int
    head_dim: int
    n_depth: int
    seed: int
    key_mult: float = 1.0  # multiplies k and k_depth (a power of two)
    causal: bool = True
    seqlens: Optional[tuple] = None  # varlen lengths, packed in this order
    depth_capacity: Optional[int] = None  # allocated slot axis (>= n_depth)

    @property
    def varlen(self) -> bool:
        return self.seqlens is not None

    @property
    def group(self) -> int:
        return self.n_heads_q // self.n_heads_kv

    @property
    def s_cap(self) -> int:
        return self.depth_capacity if self.depth_capacity is not None else self.n_depth

    @property
    def bf16(self) -> bool:
        return self.dtype == "bf16"

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.head_dim))

    @property
    def n_tokens(self) -> int:
        return self.batch * self.seqlen

    @property
    def lengths(self) -> tuple:
        return tuple(self.seqlens) if self.varlen else (self.seqlen,) * self.batch

    def cu_seqlens(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.lengths)]).astype(np.int32)

    # tensor shapes --------------------------------------------------------------
    def _lead(self):
        return (self.seqlen,) if self.varlen else (self.batch, self.seqlen)

    def shape_q(self):
        return self._lead() + (self.n_heads_q, self.head_dim)

    def shape_kv(self):
        return self._lead() + (self.n_heads_kv, self.head_dim)

    def shape_depth(self):
        return self._lead() + (self.s_cap, self.n_heads_kv, self.head_dim)

    def shape_lse(self):
        if self.varlen:
            return (self.n_heads_q, self.seqlen)
        return (self.batch, self.n_heads_q, self.seqlen)

    # algorithmic work (counted once per visible pair / per byte that must move) --
    def seq_flops(self) -> float:
        """QK^T and PV over causally visible pairs: 4 d H_q sum_L L(L+1)/2."""
        if self.causal:
            pairs = sum(L * (L + 1) // 2 for L in self.lengths)
        else:
            pairs = sum(L * L for L in self.lengths)
        return 4.0 * self.head_dim * self.n_heads_q * pairs

    def depth_flops(self) -> float:
        return 4.0 * self.n_tokens * self.n_heads_q * self.n_depth * self.head_dim

    def elem_bytes(self) -> int:
        return 2 if self.bf16 else 4

    def depth_bytes(self) -> float:
        """k_depth + v_depth, each (token, KV head, slot) row read once."""
        return 2.0 * self.n_tokens * self.n_depth * self.n_heads_kv * self.head_dim * self.elem_bytes()

    def other_bytes(self) -> float:
        """q, k, v read once, out written once, lse written once."""
        e = self.elem_bytes()
        n, d = self.n_tokens, self.head_dim
        return n * d * e * (2 * self.n_heads_q + 2 * self.n_heads_kv) + 4.0 * n * self.n_heads_q

    def total_bytes(self) -> float:
        return self.depth_bytes() + self.other_bytes()


def draw_packed_lengths(seed: int, n_seqs: int = 8, total: int = 65536, lo: int = 1024, hi: int = 16384):
    """Rejection draw of ``n_seqs`` lengths in [lo, hi] summing to ``total``.

    The first n_seqs-1 lengths are uniform on [lo, hi]; the last takes the remainder
    and the draw is repeated until it also lies in [lo, hi]; the accepted list is
    then shuffled with the same generator.
    """
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 99])))
    while True:
        head = rng.integers(lo, hi + 1, size=n_seqs - 1)
        last = total - int(head.sum())
        if lo <= last <= hi:
            lens = np.concatenate([head, [last]])
            rng.shuffle(lens)
            return tuple(int(x) for x in lens)


WORKLOADS = {
    "tiny_f32": Workload(
        "tiny_f32", "fp32 B=1 H=2 T=128 d=64 S=4", "f32", 1, 128, 2, 2, 64, 4, seed=0
    ),
    "small_bf16": Workload(
        "small_bf16", "bf16 B=2 H=8 T=1024 d=64 S=8, keys x0.5", "bf16", 2, 1024, 8, 8, 64, 8, seed=1, key_mult=0.5
    ),
    "mha_bf16": Workload(
        "mha_bf16", "bf16 B=4 H=16 T=4096 d=128 S=24", "bf16", 4, 4096, 16, 16, 128, 24, seed=2
    ),
    "gqa_bf16": Workload(
        "gqa_bf16", "bf16 GQA B=1 Hq=32 Hkv=8 T=8192 d=128 S=46", "bf16", 1, 8192, 32, 8, 128, 46, seed=3
    ),
    "packed_bf16": Workload(
        "packed_bf16",
        "bf16 varlen 8 seqs sum 65536 H=16 d=128 S=62",
        "bf16",
        1,
        65536,
        16,
        16,
        128,
        62,
        seed=4,
        seqlens=draw_packed_lengths(4),
    ),
}
ORDER = ["tiny_f32", "small_bf16", "mha_bf16", "gqa_bf16", "packed_bf16"]


def tids(batch_index: int = 0):
    o = BATCH_TID_STRIDE * batch_index
    return dict(q=TID_Q + o, k=TID_K + o, v=TID_V + o, kd=TID_KD + o, vd=TID_VD + o, do=TID_DO + o)


def make_host(w: Workload, batch_index: int = 0) -> dict:
    """All five inputs as float32 numpy arrays holding the stored values (small workloads)."""
    t = tids(batch_index)
    b = w.bf16
    out = dict(
        q=gen.tensor_np(w.seed, t["q"], w.shape_q(), 1.0, b),
        k=gen.tensor_np(w.seed, t["k"], w.shape_kv(), w.key_mult, b),
        v=gen.tensor_np(w.seed, t["v"], w.shape_kv(), 1.0, b),
    )
    if w.n_depth > 0:
        out["kd"] = gen.tensor_np(w.seed, t["kd"], w.shape_depth(), w.key_mult, b)
        out["vd"] = gen.tensor_np(w.seed, t["vd"], w.shape_depth(), 1.0, b)
    else:
        out["kd"] = out["vd"] = None
    return out


def make_device(w: Workload, device, batch_index: int = 0) -> dict:
    """All five inputs as torch tensors on ``device`` in the workload's dtype."""
    import torch

    dt = torch.bfloat16 if w.bf16 else torch.float32
    t = tids(batch_index)
    out = dict(
        q=gen.tensor_t(w.seed, t["q"], w.shape_q(), dt, device),
        k=gen.tensor_t(w.seed, t["k"], w.shape_kv(), dt, device, w.key_mult),
        v=gen.tensor_t(w.seed, t["v"], w.shape_kv(), dt, device),
    )
    if w.n_depth > 0:
        out["kd"] = gen.tensor_t(w.seed, t["kd"], w.shape_depth(), dt, device, w.key_mult)
        out["vd"] = gen.tensor_t(w.seed, t["vd"], w.shape_depth(), dt, device)
    else:
        out["kd"] = out["vd"] = None
    return out


def host_slice(w: Workload, name: str, index_arrays, batch_index: int = 0, bf16: bool = False) -> np.ndarray:
    """Regenerate selected elements of one input tensor on the host.

    ``index_arrays`` is a tuple of integer arrays (numpy fancy indexing over the
    tensor's shape); the result has their broadcast shape. The upstream gradient
    "do" is stored in the gradient dtype: ``bf16`` says whether it is bfloat16.
    """
    shape = {"q": w.shape_q(), "k": w.shape_kv(), "v": w.shape_kv(), "kd": w.shape_depth(), "vd": w.shape_depth(),
             "do": w.shape_q()}[name]
    mult = w.key_mult if name in ("k", "kd") else 1.0
    idx = np.ravel_multi_index(tuple(np.asarray(a, dtype=np.int64) for a in index_arrays), shape)
    rounded = bf16 if name == "do" else w.bf16
    return gen.values_np(w.seed, tids(batch_index)[name], idx, mult, rounded)


def make_dout_device(w: Workload, device, dtype, batch_index: int = 0):
    """Upstream gradient of out (shape of q) for the backward, N(0, 1), in ``dtype``
    (bfloat16 values are the float32 values rounded to nearest-even)."""
    return gen.tensor_t(w.seed, tids(batch_index)["do"], w.shape_q(), dtype, device)


def make_dout_host(w: Workload, bf16: bool, batch_index: int = 0) -> np.ndarray:
    return gen.tensor_np(w.seed, tids(batch_index)["do"], w.shape_q(), 1.0, bf16)


# ------------------------------------------------------------------------------ decode
#
# One decode step: one new token per sequence reads its sequence-cache prefix and
# its own depth slots (the decode-time caches of the MoDA paper's Table 1 as the
# deck quotes it on slide "Depth compute still accumulates quadratically in depth").
#
#   q                 [B, H_q, d]
#   k_cache, v_cache  [B, T_max, H_kv, d]   rows 0 .. cache_seqlens[b] - 1 are valid
#   k_depth, v_depth  [B, S_cap, H_kv, d]   the new token's depth slots
#   out [B, H_q, d]; lse [B, H_q] float32


def draw_cache_lengths(seed: int, batch: int, lo: int, hi: int) -> tuple:
    """``batch`` cache lengths uniform on [lo, hi]; the first is hi and the second lo
    (when batch allows), so every draw holds both extremes."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 77])))
    lens = [int(x) for x in rng.integers(lo, hi + 1, size=batch)]
    if batch >= 1:
        lens[0] = hi
    if batch >= 2:
        lens[1] = lo
    return tuple(lens)


@dataclass(frozen=True)
class DecodeWorkload:
    name: str
    desc: str
    dtype: str  # "f32" | "bf16"
    cache_lengths: tuple  # cache_seqlens, one per sequence (B = len)
    max_cache_len: int  # T_max (>= every length)
    n_heads_q: int
    n_heads_kv: int
    head_dim: int
    n_depth: int
    seed: int
    key_mult: float = 1.0
    depth_capacity: Optional[int] = None

    @property
    def batch(self) -> int:
        return len(self.cache_lengths)

    @property
    def group(self) -> int:
        return self.n_heads_q // self.n_heads_kv

    @property
    def s_cap(self) -> int:
        return self.depth_capacity if self.depth_capacity is not None else self.n_depth

    @property
    def bf16(self) -> bool:
        return self.dtype == "bf16"

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.head_dim))

    def elem_bytes(self) -> int:
        return 2 if self.bf16 else 4

    def shape_q(self):
        return (self.batch, self.n_heads_q, self.head_dim)

    def shape_cache(self):
        return (self.batch, self.max_cache_len, self.n_heads_kv, self.head_dim)

    def shape_depth(self):
        return (self.batch, self.s_cap, self.n_heads_kv, self.head_dim)

    # algorithmic bytes: each visible cache row and depth slot read once (K and V),
    # q read once, out and lse written once
    def cache_bytes(self) -> float:
        return 2.0 * sum(self.cache_lengths) * self.n_heads_kv * self.head_dim * self.elem_bytes()

    def depth_bytes(self) -> float:
        return 2.0 * self.batch * self.n_depth * self.n_heads_kv * self.head_dim * self.elem_bytes()

    def other_bytes(self, out_bytes: int = 2) -> float:
        n = self.batch * self.n_heads_q
        return n * self.head_dim * (self.elem_bytes() + out_bytes) + 4.0 * n

    def total_bytes(self, out_bytes: int = 2) -> float:
        return self.cache_bytes() + self.depth_bytes() + self.other_bytes(out_bytes)

    def flops(self) -> float:
        """QK and PV over every visible key: 4 d H_q (sum L + B n_depth)."""
        return 4.0 * self.head_dim * self.n_heads_q * (sum(self.cache_lengths) + self.batch * self.n_depth)


DECODE_WORKLOADS = {
    "decode_gqa_bf16": DecodeWorkload(
        "decode_gqa_bf16",
        "bf16 decode GQA B=16 Hq=32 Hkv=8 d=128 S=46, cache lengths 1024..8192",
        "bf16",
        draw_cache_lengths(5, 16, 1024, 8192),
        8192,
        32,
        8,
        128,
        46,
        seed=5,
    ),
    "decode_mha_bf16": DecodeWorkload(
        "decode_mha_bf16",
        "bf16 decode B=32 H=16 d=128 S=24, cache lengths 512..4096",
        "bf16",
        draw_cache_lengths(6, 32, 512, 4096),
        4096,
        16,
        16,
        128,
        24,
        seed=6,
    ),
}


def make_decode_host(w: DecodeWorkload) -> dict:
    """Every decode input as float32 numpy arrays of the stored values (small cases)."""
    b = w.bf16
    out = dict(
        q=gen.tensor_np(w.seed, TID_Q, w.shape_q(), 1.0, b),
        k=gen.tensor_np(w.seed, TID_K, w.shape_cache(), w.key_mult, b),
        v=gen.tensor_np(w.seed, TID_V, w.shape_cache(), 1.0, b),
        kd=gen.tensor_np(w.seed, TID_KD, w.shape_depth(), w.key_mult, b) if w.s_cap > 0 else None,
        vd=gen.tensor_np(w.seed, TID_VD, w.shape_depth(), 1.0, b) if w.s_cap > 0 else None,
        seqlens=np.asarray(w.cache_lengths, dtype=np.int32),
    )
    return out


def make_decode_device(w: DecodeWorkload, device) -> dict:
    import torch

    dt = torch.bfloat16 if w.bf16 else torch.float32
    out = dict(
        q=gen.tensor_t(w.seed, TID_Q, w.shape_q(), dt, device),
        k=gen.tensor_t(w.seed, TID_K, w.shape_cache(), dt, device, w.key_mult),
        v=gen.tensor_t(w.seed, TID_V, w.shape_cache(), dt, device),
        kd=gen.tensor_t(w.seed, TID_KD, w.shape_depth(), dt, device, w.key_mult) if w.s_cap > 0 else None,
        vd=gen.tensor_t(w.seed, TID_VD, w.shape_depth(), dt, device) if w.s_cap > 0 else None,
        seqlens=torch.tensor(w.cache_lengths, dtype=torch.int32, device=device),
    )
    return out


def decode_host_slice(w: DecodeWorkload, name: str, index_arrays) -> np.ndarray:
    """Regenerate selected elements of one decode input on the host."""
    shape = {"q": w.shape_q(), "k": w.shape_cache(), "v": w.shape_cache(), "kd": w.shape_depth(),
             "vd": w.shape_depth()}[name]
    tid = {"q": TID_Q, "k": TID_K, "v": TID_V, "kd": TID_KD, "vd": TID_VD}[name]
    mult = w.key_mult if name in ("k", "kd") else 1.0
    idx = np.ravel_multi_index(tuple(np.asarray(a, dtype=np.int64) for a in index_arrays), shape)
    return gen.values_np(w.seed, tid, idx, mult, w.bf16)
