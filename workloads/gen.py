"""Seeded synthetic tensors, bit-identical on the host (numpy) and on the device (torch).

This module holds none of the attention arithmetic. It turns a triple
(seed, tensor id, flat element index) into one value, so that any slice of any
tensor can be regenerated on its own: the CPU checker recomputes exactly the
elements it needs while the device side fills whole tensors in place.

Definition of element ``e`` of tensor ``tid`` under ``seed``:

    mix(x)   = Mueller's 32-bit integer hash: three xor-shift-16 steps with two
               multiplications by 0x45d9f3b in between, all modulo 2**32
    key      = mix(mix(seed) ^ (tid * 0x9E3779B1 mod 2**32))
    h        = mix(lo32(e) ^ mix(hi32(e) ^ key))
    value    = QTAB[h >> 16] * mult                      (float32)

``QTAB`` holds the 65536 standard-normal quantiles at (i + 0.5) / 65536, rounded to
float32, so ``value`` follows a 16-bit quantile grid of N(0, mult**2) (variance
0.99998 mult**2, tails cut at 4.32 sigma). ``mult`` must be a power of two, which
keeps ``QTAB[i] * mult`` exact. bfloat16 tensors take that float32 value rounded
to nearest-even. Every step is an integer operation, a table lookup, an exact
power-of-two product or one IEEE rounding, so numpy and torch (CPU or GPU) give
the same bits. All integer products stay below 2**63, so no signed overflow
occurs in torch's int64 arithmetic.
"""
from __future__ import annotations

import math

import numpy as np

M32 = 0xFFFFFFFF
_MUL = 0x45D9F3B
_GOLD = 0x9E3779B1


def _quantile_table() -> np.ndarray:
    from scipy.special import ndtri

    i = np.arange(65536, dtype=np.float64)
    return ndtri((i + 0.5) / 65536.0).astype(np.float32)


QTAB = _quantile_table()


def _mix_py(x: int) -> int:
    x &= M32
    x = ((x ^ (x >> 16)) * _MUL) & M32
    x = ((x ^ (x >> 16)) * _MUL) & M32
    return x ^ (x >> 16)


def tensor_key(seed: int, tid: int) -> int:
    return _mix_py(_mix_py(seed) ^ ((tid * _GOLD) & M32))


def _check_mult(mult: float) -> None:
    m, _ = math.frexp(mult)
    if mult <= 0 or m != 0.5:
        raise ValueError(f"mult must be a positive power of two, got {mult}")


# ----------------------------------------------------------------------------- numpy


def _mix_np(x: np.ndarray) -> np.ndarray:
    x = ((x ^ (x >> 16)) * _MUL) & M32
    x = ((x ^ (x >> 16)) * _MUL) & M32
    return x ^ (x >> 16)


def values_np(seed: int, tid: int, flat_index, mult: float = 1.0, bf16: bool = False) -> np.ndarray:
    """float32 values of the given flat element indices (any integer array shape).

    With ``bf16`` the float32 result already carries the bfloat16-rounded value,
    which is exact in float32.
    """
    _check_mult(mult)
    e = np.asarray(flat_index, dtype=np.int64)
    if e.size and e.min() < 0:
        raise ValueError("negative element index")
    key = np.int64(tensor_key(seed, tid))
    lo = e & M32
    hi = e >> 32
    h = _mix_np(lo ^ _mix_np(hi ^ key))
    val = QTAB[(h >> 16).astype(np.intp)] * np.float32(mult)
    if bf16:
        val = round_bf16_np(val)
    return val


def round_bf16_np(x: np.ndarray) -> np.ndarray:
    """float32 -> nearest-even bfloat16, returned as float32 (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def tensor_np(seed: int, tid: int, shape, mult: float = 1.0, bf16: bool = False) -> np.ndarray:
    n = int(np.prod(shape, dtype=np.int64))
    return values_np(seed, tid, np.arange(n, dtype=np.int64), mult, bf16).reshape(shape)


# ----------------------------------------------------------------------------- torch


def _mix_t(x):
    x = ((x ^ (x >> 16)) * _MUL) & M32
    x = ((x ^ (x >> 16)) * _MUL) & M32
    return x ^ (x >> 16)


_QTAB_CACHE: dict = {}


def _qtab_t(device):
    import torch

    key = str(device)
    if key not in _QTAB_CACHE:
        _QTAB_CACHE[key] = torch.from_numpy(QTAB.copy()).to(device)
    return _QTAB_CACHE[key]


def fill_(out, seed: int, tid: int, mult: float = 1.0, chunk: int = 1 << 28):
    """Fill a contiguous torch tensor (float32 or bfloat16, any device) in place."""
    import torch

    _check_mult(mult)
    if not out.is_contiguous():
        raise ValueError("fill_ needs a contiguous tensor")
    if out.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError(f"unsupported dtype {out.dtype}")
    flat = out.view(-1)
    n = flat.numel()
    dev = out.device
    tab = _qtab_t(dev)
    key = tensor_key(seed, tid)
    for s in range(0, n, chunk):
        c = min(chunk, n - s)
        e = torch.arange(s, s + c, dtype=torch.int64, device=dev)
        h = _mix_t((e & M32) ^ _mix_t((e >> 32) ^ key))
        val = tab[h >> 16]
        if mult != 1.0:
            val = val * mult
        flat[s : s + c].copy_(val)  # float32 -> bfloat16 copy rounds to nearest-even
        del e, h, val
    return out


def tensor_t(seed: int, tid: int, shape, dtype, device, mult: float = 1.0):
    import torch

    out = torch.empty(tuple(shape), dtype=dtype, device=device)
    return fill_(out, seed, tid, mult)
