"""The FFN input's KV projection into one depth slot (moda_depth_kv_project) on
the HIP path vs the fp64 oracle (oracle.depth_kv_projection), on an MI355X.

MoDA deck, slide "Reuse attention KV; add a projection for FFN inputs": slot s
of every token receives x W_k^T and x W_v^T; every other slot is untouched.

Bounds: bf16 inputs (fp32 accumulation, one rounding to bf16 per output) take
the forward's rule, 2e-2 x RMS of the reference slot plus half a bf16 ulp; fp32
inputs take the worst-case bound of an fp32 dot product of length K,
K u sum_k |x_k| |w_k| with u = 2^-24 (the output is O(1) only for scaled
weights, so a fixed 1e-5 would not be a property of the arithmetic).
"""
import sys

import numpy as np
import pytest

import oracle
from parity_util import check_out
from workloads import gen

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

TID_X, TID_W, TID_KD, TID_VD = 60, 61, 62, 63
W_MULT = 2.0**-5  # weights N(0, 2^-10): outputs of unit scale at D_model = 1024


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _inputs(N, D, Hkv, d, S_cap, seed, bf16):
    dt = torch.bfloat16 if bf16 else torch.float32
    dev = dict(x=gen.tensor_t(seed, TID_X, (N, D), dt, "cuda"),
               w=gen.tensor_t(seed, TID_W, (2 * Hkv * d, D), dt, "cuda", W_MULT),
               kd=gen.tensor_t(seed, TID_KD, (N, S_cap, Hkv, d), dt, "cuda"),
               vd=gen.tensor_t(seed, TID_VD, (N, S_cap, Hkv, d), dt, "cuda"))
    host = dict(x=gen.tensor_np(seed, TID_X, (N, D), 1.0, bf16),
                w=gen.tensor_np(seed, TID_W, (2 * Hkv * d, D), W_MULT, bf16),
                kd=gen.tensor_np(seed, TID_KD, (N, S_cap, Hkv, d), 1.0, bf16),
                vd=gen.tensor_np(seed, TID_VD, (N, S_cap, Hkv, d), 1.0, bf16))
    return dev, host


class _W:  # the fields check_out reads
    def __init__(self, bf16, name):
        self.bf16, self.name = bf16, name


def _compare(got, ref, x, w, bf16, tag):
    if bf16:
        return check_out(_W(True, tag), got, ref, tag, out_bf16=True)
    K = x.shape[1]
    mag = np.abs(x.astype(np.float64)) @ np.abs(w.astype(np.float64)).T  # [N, 2 Hkv d]
    tol = K * 2.0**-24 * mag.reshape(got.shape) + 1e-30
    ratio = float(np.max(np.abs(got - ref) / tol))
    assert ratio <= 1.0, f"{tag}: worst error/bound {ratio:.3f}"
    return float(np.max(np.abs(got - ref))), ratio


@pytest.mark.parametrize("bf16", [True, False])
@pytest.mark.parametrize("N,D,Hkv,d,S_cap,slot", [
    (1, 64, 1, 64, 1, 0), (5, 256, 2, 128, 3, 2), (127, 128, 1, 64, 4, 1), (128, 1024, 8, 64, 2, 0),
    (300, 2048, 4, 128, 3, 1), (1000, 512, 16, 128, 2, 1),
])
def test_projection_matches_oracle(bf16, N, D, Hkv, d, S_cap, slot):
    from joint_sequence_depth_amd import depth_kv_project

    tag = f"projection N={N} D={D} Hkv={Hkv} d={d} slot={slot}/{S_cap} bf16={bf16}"
    _say(tag)
    dev, h = _inputs(N, D, Hkv, d, S_cap, seed=N + D + slot, bf16=bf16)
    before_k, before_v = dev["kd"].clone(), dev["vd"].clone()
    depth_kv_project(dev["x"], dev["w"], dev["kd"], dev["vd"], slot)
    torch.cuda.synchronize()
    rk, rv = oracle.depth_kv_projection(h["x"], h["w"], h["kd"], h["vd"], slot, Hkv, d)
    gk = dev["kd"].float().cpu().numpy().astype(np.float64)
    gv = dev["vd"].float().cpu().numpy().astype(np.float64)
    hd = Hkv * d
    for name, got, ref, wpart in (("k", gk, rk, h["w"][:hd]), ("v", gv, rv, h["w"][hd:])):
        err, ratio = _compare(got[:, slot], ref[:, slot], h["x"], wpart, bf16, f"{tag} {name}")
        _say(f"  {name}: max err {err:.3e}, error/bound {ratio:.3f}")
    others = [i for i in range(S_cap) if i != slot]
    assert torch.equal(dev["kd"][:, others], before_k[:, others])
    assert torch.equal(dev["vd"][:, others], before_v[:, others])


def test_projection_full_size_sampled_tokens():
    """The benchmark's shapes (16384 tokens, D_model 2048, 16 KV heads of 128):
    256 sampled tokens against the oracle, RMS over those tokens' whole slot rows."""
    from joint_sequence_depth_amd import depth_kv_project

    N, D, Hkv, d, S_cap, slot = 16384, 2048, 16, 128, 24, 23
    x = gen.tensor_t(7, TID_X, (N, D), torch.bfloat16, "cuda")
    w = gen.tensor_t(7, TID_W, (2 * Hkv * d, D), torch.bfloat16, "cuda", W_MULT)
    kd = torch.zeros((N, S_cap, Hkv, d), dtype=torch.bfloat16, device="cuda")
    vd = torch.zeros_like(kd)
    depth_kv_project(x, w, kd, vd, slot)
    torch.cuda.synchronize()
    rng = np.random.default_rng(3)
    toks = np.unique(np.concatenate([[0, 127, 128, N - 1], rng.integers(0, N, size=252)]))
    xs = gen.values_np(7, TID_X, (toks[:, None] * D + np.arange(D)[None, :]), 1.0, True)
    wh = gen.tensor_np(7, TID_W, (2 * Hkv * d, D), W_MULT, True)
    rk, rv = oracle.depth_kv_projection(xs, wh, np.zeros((len(toks), 1, Hkv, d)), np.zeros((len(toks), 1, Hkv, d)),
                                        0, Hkv, d)
    tt = torch.from_numpy(toks).cuda()
    gk = kd[tt, slot].float().cpu().numpy().astype(np.float64)
    gv = vd[tt, slot].float().cpu().numpy().astype(np.float64)
    for name, got, ref in (("k", gk, rk[:, 0]), ("v", gv, rv[:, 0])):
        err, ratio = check_out(_W(True, "projection full size"), got, ref, f"projection full size {name}")
        _say(f"full size {name}: {len(toks)} tokens, max err {err:.3e}, error/bound {ratio:.3f}")
    assert float(kd[:, :slot].abs().max()) == 0.0  # the other slots stay untouched
