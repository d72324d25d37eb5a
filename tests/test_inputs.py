"""The seeded input generator: numpy and torch give identical bits, slices
regenerate on their own, and the workload table matches its description."""
import numpy as np
import torch

from workloads import configs, gen


def test_numpy_torch_bit_identical():
    for bf16, dt, mult in [(True, torch.bfloat16, 0.5), (False, torch.float32, 1.0), (True, torch.bfloat16, 1.0)]:
        a = gen.tensor_np(7, 3, (333, 65), mult, bf16)
        b = gen.tensor_t(7, 3, (333, 65), dt, "cpu", mult).float().numpy()
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_chunked_fill_matches():
    out = torch.empty(10007, dtype=torch.bfloat16)
    gen.fill_(out, 2, 9, 1.0, chunk=1000)
    ref = gen.tensor_np(2, 9, (10007,), 1.0, True)
    assert np.array_equal(out.float().numpy().view(np.uint32), ref.view(np.uint32))


def test_indices_beyond_2_pow_32():
    e = np.array([0, 1, 2**32 - 1, 2**32, 2**32 + 1, 3 * 2**32 + 7], dtype=np.int64)
    a = gen.values_np(4, 4, e)
    t = torch.from_numpy(e)
    key = gen.tensor_key(4, 4)
    h = gen._mix_t((t & gen.M32) ^ gen._mix_t((t >> 32) ^ key))
    b = torch.from_numpy(gen.QTAB)[h >> 16].numpy()
    assert np.array_equal(a, b)
    assert len(set(a.tolist())) == len(a)


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(100000) * np.exp(rng.uniform(-20, 20, 100000))).astype(np.float32)
    a = gen.round_bf16_np(x)
    b = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_distribution_and_independence():
    x = gen.tensor_np(1, 1, (1 << 18,)).astype(np.float64)
    assert abs(x.mean()) < 0.01 and abs(x.var() - 1.0) < 0.01
    assert abs(np.corrcoef(x[:-1], x[1:])[0, 1]) < 0.01
    y = gen.tensor_np(1, 2, (1 << 18,)).astype(np.float64)
    assert abs(np.corrcoef(x, y)[0, 1]) < 0.01
    z = gen.tensor_np(2, 1, (1 << 18,)).astype(np.float64)
    assert abs(np.corrcoef(x, z)[0, 1]) < 0.01
    # fourth moment of a normal is 3
    assert abs((x**4).mean() - 3.0) < 0.1


def test_host_slice_matches_full_tensor():
    w = configs.WORKLOADS["small_bf16"]
    full = configs.make_host(w)
    idx = (np.array([0, 1, 1]), np.array([5, 1023, 0]), np.array([2, 7, 0]), np.array([1, 7, 0]), np.array([0, 63, 9]))
    got = configs.host_slice(w, "kd", idx)
    assert np.array_equal(got, full["kd"][idx])
    qi = idx[:2] + (np.array([7, 0, 3]), np.array([1, 2, 63]))
    got = configs.host_slice(w, "q", qi)
    assert np.array_equal(got, full["q"][qi])


def test_workload_table():
    w = configs.WORKLOADS
    assert w["tiny_f32"].dtype == "f32" and w["tiny_f32"].shape_depth() == (1, 128, 4, 2, 64)
    assert w["small_bf16"].key_mult == 0.5 and w["small_bf16"].n_depth == 8
    assert w["mha_bf16"].shape_depth() == (4, 4096, 24, 16, 128)
    g = w["gqa_bf16"]
    assert g.group == 4 and g.n_depth == 46 and g.seqlen == 8192
    p = w["packed_bf16"]
    assert p.varlen and sum(p.seqlens) == 65536 and len(p.seqlens) == 8
    assert all(1024 <= L <= 16384 for L in p.seqlens)
    assert p.shape_depth() == (65536, 62, 16, 128)
    assert configs.draw_packed_lengths(4) == p.seqlens
