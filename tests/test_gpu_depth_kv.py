"""Depth-KV writer and bounded slot buffers on the HIP path.

The writer is a copy, checked bit for bit (and that nothing else is written).
The bounded buffer is checked through the forward against the oracle: a ring of
S_cap slots after more than S_cap writes, read whole, must equal the joint
attention over the most recent S_cap entries; a window of slots read through
``slot_offset`` must equal the oracle on that slice of the slot axis.
"""
import numpy as np
import pytest

import oracle
from parity_util import check_out, to_np, workload
from workloads import configs, gen

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("lead,Hkv,d,S_cap,slot", [((2, 33), 2, 64, 5, 3), ((70,), 8, 128, 3, 0), ((1, 1), 1, 64, 1, 0),
                                                   ((3, 100), 4, 128, 62, 61)])
def test_writer_copies_one_slot(dtype, lead, Hkv, d, S_cap, slot):
    from joint_sequence_depth_amd import depth_kv_write

    shape = lead + (Hkv, d)
    ks = gen.tensor_t(5, 1, shape, dtype, "cuda")
    vs = gen.tensor_t(5, 2, shape, dtype, "cuda")
    kd = torch.full(lead + (S_cap, Hkv, d), 7.0, dtype=dtype, device="cuda")
    vd = torch.full(lead + (S_cap, Hkv, d), -3.0, dtype=dtype, device="cuda")
    depth_kv_write(ks, vs, kd, vd, slot)
    torch.cuda.synchronize()
    sl = (slice(None),) * len(lead)
    assert torch.equal(kd[sl + (slot,)], ks) and torch.equal(vd[sl + (slot,)], vs)
    others = [i for i in range(S_cap) if i != slot]
    if others:
        assert torch.all(kd[sl + (others,)] == 7.0) and torch.all(vd[sl + (others,)] == -3.0)


def _entries(w, n_entries):
    """n_entries seeded [B,T,Hkv,d] key/value pairs (host float32 values and device tensors)."""
    dt = torch.bfloat16 if w.bf16 else torch.float32
    shape = (w.batch, w.seqlen, w.n_heads_kv, w.head_dim)
    host, dev = [], []
    for e in range(n_entries):
        host.append((gen.tensor_np(w.seed, 40 + 2 * e, shape, 1.0, w.bf16), gen.tensor_np(w.seed, 41 + 2 * e, shape, 1.0,
                                                                                          w.bf16)))
        dev.append((gen.tensor_t(w.seed, 40 + 2 * e, shape, dt, "cuda"), gen.tensor_t(w.seed, 41 + 2 * e, shape, dt, "cuda")))
    return host, dev


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("S_cap,n_written", [(4, 7), (3, 3), (5, 12), (1, 4)])
def test_ring_buffer_is_a_sliding_window(dtype, S_cap, n_written):
    from joint_sequence_depth_amd import attn_fwd, depth_kv_write

    w = workload(dtype=dtype, head_dim=64, seqlen=150, batch=2, n_heads_q=4, n_heads_kv=2, n_depth=S_cap,
                 seed=60 + S_cap)
    dt = torch.bfloat16 if w.bf16 else torch.float32
    x = configs.make_device(w, "cuda")
    host_e, dev_e = _entries(w, n_written)
    kd = torch.zeros((w.batch, w.seqlen, S_cap, w.n_heads_kv, w.head_dim), dtype=dt, device="cuda")
    vd = torch.zeros_like(kd)
    for e in range(n_written):  # entry e goes to slot e mod S_cap
        depth_kv_write(dev_e[e][0], dev_e[e][1], kd, vd, e % S_cap)
    n_valid = min(n_written, S_cap)
    out, lse = attn_fwd(x["q"], x["k"], x["v"], kd, vd, n_depth=n_valid)
    torch.cuda.synchronize()
    # oracle: the most recent n_valid entries, in the order they were written
    recent = host_e[n_written - n_valid:]
    kd_h = np.stack([e[0] for e in recent], axis=2)
    vd_h = np.stack([e[1] for e in recent], axis=2)
    h = configs.make_host(w)
    ref_o, ref_l = oracle.joint_attention(h["q"], h["k"], h["v"], kd_h, vd_h, n_valid, True, w.scale)
    check_out(w, to_np(out), ref_o, "ring buffer")
    assert np.max(np.abs(to_np(lse) - ref_l)) <= (1e-3 if w.bf16 else 1e-5)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("offset,n", [(2, 3), (0, 6), (5, 1), (6, 0)])
def test_slot_window(dtype, offset, n):
    from joint_sequence_depth_amd import attn_fwd

    w = workload(dtype=dtype, head_dim=128, seqlen=130, batch=1, n_heads_q=2, n_heads_kv=1, n_depth=6,
                 depth_capacity=6, seed=70 + offset)
    x = configs.make_device(w, "cuda")
    out, lse = attn_fwd(x["q"], x["k"], x["v"], x["kd"], x["vd"], n_depth=n, slot_offset=offset)
    torch.cuda.synchronize()
    h = configs.make_host(w)
    kd = np.ascontiguousarray(h["kd"][:, :, offset:offset + n])
    vd = np.ascontiguousarray(h["vd"][:, :, offset:offset + n])
    ref_o, ref_l = oracle.joint_attention(h["q"], h["k"], h["v"], kd, vd, n, True, w.scale)
    check_out(w, to_np(out), ref_o, "slot window")
    assert np.max(np.abs(to_np(lse) - ref_l)) <= (1e-3 if w.bf16 else 1e-5)
