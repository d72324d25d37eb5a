"""The C ABI library on the host: it loads, exports every declared symbol, and its
host-side checks reject bad arguments before any device work (no GPU needed: no
call here reaches a launch)."""
import ctypes
import math
import os
import re

import pytest

from joint_sequence_depth_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moda_attn.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moda_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = _lib.lib()
    names = declared_functions()
    assert set(names) == set(_lib.EXPORTS)
    for n in names:
        assert hasattr(L, n), n
    assert L.moda_abi_version() == 7


def test_status_codes_match_header():
    text = open(HEADER).read()
    codes = {m.group(1): int(m.group(2)) for m in re.finditer(r"#define (MODA_(?:OK|ERR_\w+))\s+(\d+)", text)}
    assert {v: k for k, v in codes.items()} == _lib.STATUS_NAMES


# Fake, 16-byte aligned addresses: every case below must fail validation, which
# runs before any HIP call. Skipped where a GPU is present, so that a wrong
# expectation can never turn into a launch on fake pointers.
P = 0x10000
A = dict(q=P, k=P, v=P, kd=P, vd=P, out=P, lse=P, dtype=1, odt=1, B=1, T=16, Hq=4, Hkv=2, d=64, Scap=4, S=4, causal=1,
         scale=0.125)


@pytest.fixture(autouse=True)
def _no_gpu_here():
    try:
        import torch

        if torch.cuda.is_available():
            pytest.skip("host-only validation tests run where no GPU can be reached")
    except ImportError:
        pass


def call(**kw):
    a = dict(A)
    a.update(kw)
    L = _lib.lib()
    return L.moda_attn_fwd(a["q"], a["k"], a["v"], a["kd"], a["vd"], a["out"], a["lse"], a["dtype"], a["odt"], a["B"], a["T"],
                           a["Hq"], a["Hkv"], a["d"], a["Scap"], a["S"], a["causal"], a["scale"], None)


def callv(cu=P, n_seqs=2, N=16, max_len=8, **kw):
    a = dict(A)
    a.update(kw)
    L = _lib.lib()
    return L.moda_attn_fwd_varlen(a["q"], a["k"], a["v"], a["kd"], a["vd"], a["out"], a["lse"], a["dtype"], a["odt"], cu,
                                  n_seqs, N, max_len, a["Hq"], a["Hkv"], a["d"], a["Scap"], a["S"], a["causal"],
                                  a["scale"], None)


def err():
    return _lib.lib().moda_last_error().decode()


@pytest.mark.parametrize(
    "kw,code",
    [
        (dict(q=None), 1),
        (dict(out=None), 1),
        (dict(kd=None), 1),
        (dict(dtype=2), 3),
        (dict(dtype=-1), 3),
        (dict(odt=5), 3),
        (dict(dtype=0, odt=1), 3),
        (dict(Hq=3, Hkv=2), 2),
        (dict(Hkv=0), 2),
        (dict(d=96), 5),
        (dict(d=256), 5),
        (dict(S=5, Scap=4), 2),
        (dict(S=-1), 2),
        (dict(B=-1), 2),
        (dict(T=-5), 2),
        (dict(q=P + 8), 4),
        (dict(vd=P + 2), 4),
        (dict(lse=P + 2), 4),
        (dict(scale=0.0), 7),
        (dict(scale=-1.0), 7),
        (dict(scale=math.inf), 7),
        (dict(scale=math.nan), 7),
        (dict(causal=2), 7),
    ],
)
def test_validation_rejects(kw, code):
    assert call(**kw) == code
    assert err()


def test_depth_pointers_optional_without_slots():
    # n_depth == 0 with NULL depth pointers passes the depth checks; make it fail
    # later on purpose (bad head_dim) to stay host-only.
    assert call(kd=None, vd=None, S=0, Scap=0, d=96) == 5


def test_empty_problems_are_ok_without_launch():
    assert call(B=0) == 0
    assert call(T=0, q=None) == 0
    assert callv(n_seqs=0) == 0
    assert callv(N=0) == 0
    assert err() == ""


@pytest.mark.parametrize(
    "kw,code",
    [
        (dict(cu=None), 1),
        (dict(cu=P + 2), 4),
        (dict(max_len=17), 2),
        (dict(n_seqs=-1), 2),
        (dict(N=-3), 2),
        (dict(d=32), 5),
    ],
)
def test_varlen_validation_rejects(kw, code):
    assert callv(**kw) == code
    assert err()


def callp(phase, **kw):
    a = dict(A)
    a.update(kw)
    L = _lib.lib()
    return L.moda_attn_fwd_phases(a["q"], a["k"], a["v"], a["kd"], a["vd"], a["out"], a["lse"], a["dtype"],
                                  a["odt"], a["B"], a["T"], a["Hq"], a["Hkv"], a["d"], a["Scap"], a["S"], a["causal"],
                                  a["scale"], phase, None)


def callvp(phase, cu=P, n_seqs=2, N=16, max_len=8, **kw):
    a = dict(A)
    a.update(kw)
    L = _lib.lib()
    return L.moda_attn_fwd_varlen_phases(a["q"], a["k"], a["v"], a["kd"], a["vd"], a["out"], a["lse"], a["dtype"],
                                         a["odt"], cu, n_seqs, N, max_len, a["Hq"], a["Hkv"], a["d"], a["Scap"],
                                         a["S"], a["causal"], a["scale"], phase, None)


@pytest.mark.parametrize("phase", [0, 4, -1, 7])
def test_phases_reject_unknown_mask(phase):
    assert callp(phase) == 7 and "phase_mask" in err()
    assert callvp(phase) == 7 and "phase_mask" in err()


def test_depth_phase_needs_slots():
    assert callp(2, S=0, kd=None, vd=None) == 7 and "n_depth" in err()
    assert callvp(2, S=0, kd=None, vd=None) == 7 and "n_depth" in err()


def test_phases_check_like_the_fused_call():
    # the same argument checks run first (bad head_dim), and empty problems stay no-ops
    for phase in (1, 2, 3):
        assert callp(phase, d=96) == 5
        assert callvp(phase, d=96) == 5
        assert callp(phase, B=0) == 0
        assert callvp(phase, n_seqs=0) == 0


def test_packed_call_needs_max_seqlen(monkeypatch):
    # the binding never copies cu_seqlens back to the host: max_seqlen is required
    import torch

    class Dev:  # a stand-in with the attributes the binding checks before the library call
        def __init__(self, shape, dtype=torch.bfloat16):
            self.shape, self.dtype = torch.Size(shape), dtype
            self.device = torch.device("cuda", 0)

        def dim(self):
            return len(self.shape)

        def is_contiguous(self):
            return True

        def numel(self):
            n = 1
            for x in self.shape:
                n *= x
            return n

        def element_size(self):
            return 2

        def data_ptr(self):
            return P

    q, k = Dev((16, 4, 64)), Dev((16, 2, 64))
    out, lse = Dev((16, 4, 64)), Dev((4, 16), torch.float32)
    cu = Dev((3,), torch.int32)
    monkeypatch.setattr(torch.cuda, "current_stream", lambda *a: type("S", (), {"cuda_stream": 0})())
    with pytest.raises(ValueError, match="max_seqlen"):
        _lib.attn_fwd(q, k, k, out=out, lse=lse, cu_seqlens=cu)


def callt(topk=2, recent=1, ws=P, ws_bytes=1 << 30, **kw):
    a = dict(A)
    a.update(kw)
    L = _lib.lib()
    return L.moda_attn_fwd_topk(a["q"], a["k"], a["v"], a["kd"], a["vd"], a["out"], a["lse"], a["dtype"], a["odt"],
                                a["B"], a["T"], a["Hq"], a["Hkv"], a["d"], a["Scap"], a["S"], topk, recent,
                                a["causal"], a["scale"], ws, ws_bytes, None)


def callvt(topk=2, recent=1, ws=P, ws_bytes=1 << 30, cu=P, n_seqs=2, N=16, max_len=8, **kw):
    a = dict(A)
    a.update(kw)
    L = _lib.lib()
    return L.moda_attn_fwd_varlen_topk(a["q"], a["k"], a["v"], a["kd"], a["vd"], a["out"], a["lse"], a["dtype"],
                                       a["odt"], cu, n_seqs, N, max_len, a["Hq"], a["Hkv"], a["d"], a["Scap"], a["S"],
                                       topk, recent, a["causal"], a["scale"], ws, ws_bytes, None)


@pytest.mark.parametrize(
    "kw,code",
    [
        (dict(topk=-1), 7),
        (dict(recent=-2), 7),
        (dict(S=65, Scap=65), 5),
        (dict(ws=None), 1),
        (dict(ws=P + 8), 4),
        (dict(ws_bytes=16 * 4 * 8 - 1), 2),
        (dict(d=96), 5),
        (dict(q=None), 1),
    ],
)
def test_topk_validation_rejects(kw, code):
    assert callt(**kw) == code and err()
    assert callvt(**kw) == code and err()


def test_topk_workspace_size():
    L = _lib.lib()
    assert L.moda_attn_fwd_topk_workspace_size(16, 4) == 16 * 4 * 8
    assert L.moda_attn_fwd_topk_workspace_size(-1, 4) == -1
    assert L.moda_attn_fwd_topk_workspace_size(16, 0) == -1
    assert callt(B=0) == 0 and callvt(n_seqs=0) == 0


def test_python_binding_fails_loudly_without_library(monkeypatch):
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "LIB_PATH", "/nonexistent/libmoda_attn.so")
    with pytest.raises(RuntimeError, match="missing"):
        _lib.lib()


def test_ctypes_signatures():
    L = _lib.lib()
    assert len(L.moda_attn_fwd.argtypes) == 19
    assert len(L.moda_attn_fwd_varlen.argtypes) == 21
    assert len(L.moda_attn_fwd_phases.argtypes) == 20
    assert len(L.moda_attn_fwd_varlen_phases.argtypes) == 22
    assert len(L.moda_attn_fwd_topk.argtypes) == 23
    assert len(L.moda_attn_fwd_varlen_topk.argtypes) == 25
    assert len(L.moda_attn_fwd_topk_workspace_size.argtypes) == 2
    assert len(L.moda_attn_decode.argtypes) == 21
    assert len(L.moda_attn_decode_noalloc.argtypes) == 19
    assert len(L.moda_attn_decode_workspace_size.argtypes) == 5
    assert L.moda_attn_decode_workspace_size.restype is ctypes.c_int64
    assert len(L.moda_attn_bwd.argtypes) == 27
    assert len(L.moda_attn_bwd_varlen.argtypes) == 29
    assert len(L.moda_attn_bwd_workspace_size.argtypes) == 4
    assert len(L.moda_depth_kv_write.argtypes) == 11
    assert len(L.moda_depth_kv_project.argtypes) == 12
    assert L.moda_last_error.restype is ctypes.c_char_p


def calld(seqlens=P, Tmax=32, ws=P, ws_bytes=1 << 30, **kw):
    a = dict(A)
    a.update(kw)
    L = _lib.lib()
    return L.moda_attn_decode(a["q"], a["k"], a["v"], a["kd"], a["vd"], a["out"], a["lse"], a["dtype"], a["odt"],
                              seqlens, a["B"], Tmax, a["Hq"], a["Hkv"], a["d"], a["Scap"], a["S"], a["scale"], ws,
                              ws_bytes, None)


@pytest.mark.parametrize(
    "kw,code",
    [
        (dict(seqlens=None), 1),
        (dict(seqlens=P + 2), 4),
        (dict(ws=None), 1),
        (dict(ws=P + 8), 4),
        (dict(ws_bytes=16), 2),
        (dict(Tmax=0), 2),
        (dict(Tmax=-4), 2),
        (dict(B=-1), 2),
        (dict(q=None), 1),
        (dict(kd=None), 1),
        (dict(Hq=6, Hkv=4), 2),
        (dict(d=32), 5),
        (dict(dtype=0, odt=1), 3),
        (dict(scale=0.0), 7),
        (dict(S=5, Scap=4), 2),
    ],
)
def test_decode_validation_rejects(kw, code):
    assert calld(**kw) == code
    assert err()


def test_decode_noalloc_rejects_steps_beyond_its_scratch():
    # B = 256, Hq = Hkv = 64, d = 128: two chunks of 132 floats per (sequence, head)
    # need 17.3 MB > MODA_DECODE_SCRATCH_BYTES; rejected on the host, before any
    # HIP call (without a GPU a HIP call would report MODA_ERR_HIP instead)
    L = _lib.lib()
    B, Hq, Hkv, d, T = 256, 64, 64, 128, 16
    assert L.moda_attn_decode_workspace_size(B, Hq, Hkv, d, T) > _lib.DECODE_SCRATCH_BYTES
    rc = L.moda_attn_decode_noalloc(P, P, P, None, None, P, None, 1, 1, P, B, T, Hq, Hkv, d, 0, 0, 0.088, None)
    assert rc == 2 and "scratch" in err()
    # the same argument checks as moda_attn_decode run first
    assert L.moda_attn_decode_noalloc(None, P, P, None, None, P, None, 1, 1, P, 1, T, 2, 2, 64, 0, 0, 0.1, None) == 1
    assert L.moda_attn_decode_noalloc(P, P, P, None, None, P, None, 1, 1, P, 1, T, 2, 2, 96, 0, 0, 0.1, None) == 5
    assert L.moda_attn_decode_noalloc(P, P, P, None, None, P, None, 1, 1, P, 0, T, 2, 2, 64, 0, 0, 0.1, None) == 0


def test_decode_empty_batch_is_ok_without_launch():
    assert calld(B=0, ws=None, seqlens=None) == 0
    assert err() == ""


def test_decode_workspace_size():
    L = _lib.lib()
    assert L.moda_attn_decode_workspace_size(1, 4, 2, 96, 16) == -1
    assert L.moda_attn_decode_workspace_size(1, 3, 2, 64, 16) == -1
    assert L.moda_attn_decode_workspace_size(1, 4, 2, 64, 0) == -1
    assert L.moda_attn_decode_workspace_size(0, 4, 2, 64, 16) == 0
    for B, Hq, Hkv, d, T in [(1, 4, 2, 64, 16), (16, 32, 8, 128, 8192), (3, 8, 8, 128, 100000)]:
        n = L.moda_attn_decode_workspace_size(B, Hq, Hkv, d, T)
        # one fp32 record (d accumulators, max, sum, 2 pad) per (row, head, chunk),
        # with at least one sequence chunk and the depth chunk
        rec = (d + 4) * 4
        assert n > 0 and n % (B * Hq * rec) == 0
        assert n // (B * Hq * rec) >= 2
    # a workspace one byte short is refused
    need = L.moda_attn_decode_workspace_size(1, 4, 2, 64, 32)
    assert calld(ws_bytes=need - 1) == 2
    assert "workspace" in err()


BIG_WS = 1 << 40
WS = 0x100000  # 256-byte aligned fake address


def callb(ws=WS, ws_bytes=BIG_WS, dout=P, lse=P, dq=P, dk=P, dv=P, dkd=P, dvd=P, gdt=1, **kw):
    a = dict(A)
    a.update(kw)
    L = _lib.lib()
    return L.moda_attn_bwd(a["q"], a["k"], a["v"], a["kd"], a["vd"], a["out"], dout, lse, dq, dk, dv, dkd, dvd,
                           a["dtype"], gdt, a["B"], a["T"], a["Hq"], a["Hkv"], a["d"], a["Scap"], a["S"], a["causal"],
                           a["scale"], ws, ws_bytes, None)


def callbv(cu=P, n_seqs=2, N=16, max_len=8, ws=WS, ws_bytes=BIG_WS, **kw):
    a = dict(A)
    a.update(kw)
    L = _lib.lib()
    return L.moda_attn_bwd_varlen(a["q"], a["k"], a["v"], a["kd"], a["vd"], a["out"], P, P, P, P, P, P, P,
                                  a["dtype"], 1, cu, n_seqs, N, max_len, a["Hq"], a["Hkv"], a["d"], a["Scap"], a["S"],
                                  a["causal"], a["scale"], ws, ws_bytes, None)


@pytest.mark.parametrize(
    "kw,code",
    [
        (dict(dout=None), 1),
        (dict(lse=None), 1),
        (dict(dq=None), 1),
        (dict(dk=None), 1),
        (dict(dvd=None), 1),
        (dict(out=None), 1),
        (dict(ws=None), 1),
        (dict(ws=WS + 16), 4),
        (dict(ws_bytes=100), 2),
        (dict(dv=P + 8), 4),
        (dict(dkd=P + 4), 4),
        (dict(lse=P + 2), 4),
        (dict(gdt=5), 3),
        (dict(dtype=0, gdt=1), 3),
        (dict(Hq=34, Hkv=2), 5),
        (dict(Hq=3, Hkv=2), 2),
        (dict(d=96), 5),
        (dict(S=5, Scap=4), 2),
        (dict(scale=0.0), 7),
        (dict(causal=3), 7),
        (dict(B=-1), 2),
    ],
)
def test_bwd_validation_rejects(kw, code):
    assert callb(**kw) == code
    assert err()


def test_bwd_depth_grads_optional_without_slots():
    # n_depth == 0 accepts NULL depth gradients; fail later on purpose (bad head_dim)
    assert callb(kd=None, vd=None, dkd=None, dvd=None, S=0, Scap=0, d=96) == 5


def test_bwd_empty_problems_are_ok_without_launch():
    assert callb(B=0) == 0
    assert callb(T=0, q=None) == 0
    assert callbv(n_seqs=0) == 0
    assert err() == ""


@pytest.mark.parametrize("kw,code", [(dict(cu=None), 1), (dict(cu=P + 2), 4), (dict(max_len=17), 2),
                                     (dict(n_seqs=-1), 2), (dict(d=32), 5)])
def test_bwd_varlen_validation_rejects(kw, code):
    assert callbv(**kw) == code
    assert err()


def test_bwd_workspace_size():
    L = _lib.lib()
    assert L.moda_attn_bwd_workspace_size(16, 4, 96, 2) == -1
    assert L.moda_attn_bwd_workspace_size(-1, 4, 64, 2) == -1
    assert L.moda_attn_bwd_workspace_size(0, 4, 64, 2) == 0
    # fp32 delta [Hq, N], then the depth share of dq [N, Hq, d] when there are slots
    assert L.moda_attn_bwd_workspace_size(64, 4, 64, 0) == 1024
    assert L.moda_attn_bwd_workspace_size(64, 4, 64, 3) == 1024 + 64 * 4 * 64 * 4
    need = L.moda_attn_bwd_workspace_size(16, 4, 64, 4)
    assert callb(ws_bytes=need - 1) == 2 and "workspace" in err()


def callw(ks=P, vs=P, kd=P, vd=P, dtype=1, N=16, Hkv=2, d=64, Scap=4, slot=1):
    return _lib.lib().moda_depth_kv_write(ks, vs, kd, vd, dtype, N, Hkv, d, Scap, slot, None)


@pytest.mark.parametrize(
    "kw,code",
    [
        (dict(ks=None), 1),
        (dict(vd=None), 1),
        (dict(dtype=7), 3),
        (dict(slot=4), 2),
        (dict(slot=-1), 2),
        (dict(Scap=0, slot=0), 2),
        (dict(Hkv=0), 2),
        (dict(N=-1), 2),
        (dict(Hkv=1, d=4), 2),  # 8-byte rows
        (dict(kd=P + 8), 4),
    ],
)
def test_writer_validation_rejects(kw, code):
    assert callw(**kw) == code
    assert err()


def test_writer_empty_is_ok():
    assert callw(N=0, ks=None) == 0
    assert err() == ""


def callp_(x=P, w=P, kd=P, vd=P, dtype=1, n=16, dm=128, hkv=2, d=64, scap=3, slot=1):
    return _lib.lib().moda_depth_kv_project(x, w, kd, vd, dtype, n, dm, hkv, d, scap, slot, None)


@pytest.mark.parametrize(
    "kw,code",
    [
        (dict(x=None), 1),
        (dict(w=None), 1),
        (dict(dtype=3), 3),
        (dict(d=96), 5),
        (dict(dm=100), 5),
        (dict(dm=0), 5),
        (dict(slot=3), 2),
        (dict(slot=-1), 2),
        (dict(hkv=0), 2),
        (dict(n=-1), 2),
        (dict(kd=P + 4), 4),
    ],
)
def test_projection_validation_rejects(kw, code):
    assert callp_(**kw) == code and err()


def test_projection_empty_is_ok():
    assert callp_(n=0, x=None) == 0


# Sizes whose products would overflow int64 (or reach 2^56 elements) are refused
# before any size is computed from them; the size queries answer -1. Every call
# stays host-only (rejected by validation).
HUGE = 1 << 62


def test_oversized_problems_are_refused():
    assert call(B=(1 << 31) - 1, T=1 << 40) == 2 and "too large" in err()
    assert call(B=1, T=HUGE, S=0, kd=None, vd=None) == 2 and "too large" in err()
    assert call(B=1 << 20, T=1 << 20, Scap=1 << 30, S=1) == 2 and "too large" in err()
    assert callv(n_seqs=(1 << 31) - 1, N=1 << 40, max_len=(1 << 31) - 1) == 2 and "too large" in err()
    assert callv(n_seqs=(1 << 31) - 1, N=(1 << 31) - 1, max_len=(1 << 31) - 1, Hq=1 << 20, Hkv=1) == 2
    assert calld(B=(1 << 31) - 1, Tmax=(1 << 31) - 1, Hq=1 << 20, Hkv=1 << 20) == 2 and "too large" in err()
    assert callb(B=1, T=HUGE) == 2 and "too large" in err()
    assert callbv(n_seqs=(1 << 31) - 1, N=1 << 40, max_len=(1 << 31) - 1) == 2 and "too large" in err()
    assert callw(N=HUGE) == 2 and "too large" in err()
    assert callp_(n=HUGE) == 2 and "too large" in err()


def test_size_queries_refuse_overflowing_sizes():
    L = _lib.lib()
    assert L.moda_attn_bwd_workspace_size(HUGE, 64, 128, 64) == -1
    assert L.moda_attn_bwd_workspace_size(1 << 40, 1 << 30, 128, 0) == -1
    assert L.moda_attn_fwd_topk_workspace_size(HUGE, 1 << 30) == -1
    assert L.moda_attn_decode_workspace_size(HUGE, 64, 8, 128, 1 << 30) == -1
    assert L.moda_attn_decode_workspace_size((1 << 31) - 1, 1 << 30, 1 << 30, 128, (1 << 31) - 1) == -1
    # large but representable sizes still answer
    assert L.moda_attn_bwd_workspace_size(1 << 30, 64, 128, 8) > 0


def test_poisoned_lds_build_is_instrumented():
    # the debug build's kernels carry the NaN fill pattern (0x7fc07fc0) as an
    # immediate and the normal build's do not: the GPU comparison of the two
    # builds compares instrumented kernels against plain ones
    from joint_sequence_depth_amd import build

    pattern = (0x7FC07FC0).to_bytes(4, "little")
    for path in (build.LIB_PATH, build.POISON_LIB_PATH):
        if not os.path.exists(path):
            pytest.skip("the library is not built")
    assert open(build.LIB_PATH, "rb").read().count(pattern) == 0
    assert open(build.POISON_LIB_PATH, "rb").read().count(pattern) >= 20
