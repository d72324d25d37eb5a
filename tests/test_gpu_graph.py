"""Graph capture: each entry point captured in a HIP graph, replayed several
times with eager work and synchronisations in between, must reproduce the eager
call's results bit for bit on every replay (no memsets inside the library's
launches, workspace contents on entry irrelevant)."""
import pytest

from parity_util import workload
from workloads import configs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _replays_match(fn, outs, n_replays=3):
    """fn() writes into the tensors of `outs`. Eager reference, then capture and
    replays with unrelated eager work in between."""
    fn()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    junk = torch.randn(1 << 20, device="cuda")
    for i in range(n_replays):
        for t in outs:
            t.fill_(float("nan"))  # stale results must not survive a replay
        junk.mul_(1.0001)  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(outs, ref):
            assert torch.equal(a, b), f"replay {i} differs from the eager call"


def test_graph_forward_backward():
    from joint_sequence_depth_amd import attn_bwd, attn_fwd, bwd_workspace_size

    w = workload(dtype="bf16", head_dim=128, seqlen=300, batch=2, n_heads_q=8, n_heads_kv=2, n_depth=5, seed=2024)
    x = configs.make_device(w, "cuda")
    out = torch.empty(w.shape_q(), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(w.shape_lse(), dtype=torch.float32, device="cuda")
    _replays_match(lambda: attn_fwd(x["q"], x["k"], x["v"], x["kd"], x["vd"], n_depth=w.n_depth, out=out, lse=lse),
                   [out, lse])
    dout = configs.make_dout_device(w, "cuda", torch.bfloat16)
    grads = (torch.empty_like(x["q"]), torch.empty_like(x["k"]), torch.empty_like(x["v"]), torch.zeros_like(x["kd"]),
             torch.zeros_like(x["vd"]))
    ws = torch.empty(bwd_workspace_size(w.n_tokens, w.n_heads_q, w.head_dim, w.n_depth), dtype=torch.uint8,
                     device="cuda")
    _replays_match(lambda: attn_bwd(x["q"], x["k"], x["v"], x["kd"], x["vd"], out, dout, lse, n_depth=w.n_depth,
                                    grads=grads, workspace=ws), list(grads[:3]) + [grads[3][:, :, :5], grads[4][:, :, :5]])


def test_graph_decode_and_writer():
    from joint_sequence_depth_amd import attn_decode, decode_workspace_size, depth_kv_write

    dw = configs.DecodeWorkload("g", "", "bf16", (700, 1, 333), 700, 8, 2, 128, 7, seed=77)
    x = configs.make_decode_device(dw, "cuda")
    out = torch.empty(dw.shape_q(), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((dw.batch, dw.n_heads_q), dtype=torch.float32, device="cuda")
    ws = torch.empty(decode_workspace_size(dw.batch, 8, 2, 128, 700), dtype=torch.uint8, device="cuda")
    _replays_match(lambda: attn_decode(x["q"], x["k"], x["v"], x["seqlens"], x["kd"], x["vd"], n_depth=dw.n_depth,
                                       out=out, lse=lse, workspace=ws), [out, lse])
    kd = torch.zeros((3, 50, 4, 2, 64), dtype=torch.bfloat16, device="cuda")
    vd = torch.zeros_like(kd)
    ks = torch.randn((3, 50, 2, 64), device="cuda").to(torch.bfloat16)
    vs = torch.randn((3, 50, 2, 64), device="cuda").to(torch.bfloat16)
    _replays_match(lambda: depth_kv_write(ks, vs, kd, vd, 2), [kd[:, :, 2], vd[:, :, 2]])
