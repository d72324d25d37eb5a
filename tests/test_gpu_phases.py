"""The two parts of the forward, one at a time, through moda_attn_fwd_phases /
moda_attn_fwd_varlen_phases, on an MI355X.

MoDA deck, slide "Shared online-softmax states preserve the joint operator": the
sequence blocks and the depth blocks update one running softmax state, so each
part alone is a softmax of its own and the operator is their log-sum-exp merge
(oracle pin p4 checks that identity on the CPU). Here:
  * phase 1 (sequence keys only) against oracle.sequence_only,
  * phase 2 (depth slots only) against oracle.depth_only,
  * the merge of the two GPU results against the joint oracle, and
  * phase 3 through the phases entry point bit-identical to moda_attn_fwd,
on shapes that reach every tile schedule of the bf16 kernel (split and shared
tiles, one, two and four heads per workgroup, both head dims), packed sequences
with an empty one, and the fp32 path.
"""
import sys

import numpy as np
import pytest

import oracle
from parity_util import check_lse, check_out, to_np, workload
from workloads import configs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


CASES = {
    "split_d64": dict(dtype="bf16", head_dim=64, seqlen=300, batch=1, n_heads_q=2, n_heads_kv=2, n_depth=5,
                      kernel="<64, 1, 2, {}, false, true>"),
    "split_d128_g2": dict(dtype="bf16", head_dim=128, seqlen=257, batch=2, n_heads_q=4, n_heads_kv=2, n_depth=7,
                          kernel="<128, 2, 2, {}, false, true>"),
    "shared2_d64_g4": dict(dtype="bf16", head_dim=64, seqlen=1024, batch=1, n_heads_q=32, n_heads_kv=8, n_depth=5,
                           kernel="<64, 4, 2, {}, false, false>"),
    "shared2_d128_g4": dict(dtype="bf16", head_dim=128, seqlen=2048, batch=1, n_heads_q=16, n_heads_kv=4,
                            n_depth=9, kernel="<128, 4, 2, {}, false, false>"),
    "shared4_d128_g1": dict(dtype="bf16", head_dim=128, seqlen=1024, batch=1, n_heads_q=64, n_heads_kv=64,
                            n_depth=3, kernel="<128, 1, 4, {}, false, false>"),
    "packed_d128": dict(dtype="bf16", head_dim=128, seqlens=(5, 1, 130, 64, 0, 257), n_heads_q=4, n_heads_kv=4,
                        n_depth=6, kernel=None),
    "fp32_d64": dict(dtype="f32", head_dim=64, seqlen=129, batch=2, n_heads_q=4, n_heads_kv=2, n_depth=4,
                     kernel=None),
}


def _case(name):
    kw = {k: v for k, v in CASES[name].items() if k != "kernel"}
    return workload(name=name, seed=60 + list(CASES).index(name), **kw)


def _run(w, x, phase, out_f32):
    from joint_sequence_depth_amd import attn_fwd

    cu = torch.from_numpy(w.cu_seqlens()).cuda() if w.varlen else None
    out, lse = attn_fwd(x["q"], x["k"], x["v"], x["kd"], x["vd"], n_depth=w.n_depth, causal=w.causal, scale=w.scale,
                        cu_seqlens=cu, max_seqlen=max(w.lengths) if w.varlen else None,
                        out_dtype=torch.float32 if out_f32 else None, phase=phase)
    torch.cuda.synchronize()
    return out, lse


def _lse_rows(w, lse):
    """lse [B,Hq,T] or [Hq,N] -> [N, Hq] (token-major, like out)."""
    if w.varlen:
        return lse.T
    return lse.transpose(0, 2, 1).reshape(-1, w.n_heads_q)


@pytest.mark.parametrize("name", list(CASES))
def test_phases_merge_to_the_operator(name):
    import bench

    w = _case(name)
    _say(f"phases {name}: {w}")
    kern = CASES[name]["kernel"]
    if kern is not None:
        for phase, mode in ((1, 0), (2, 2), (3, 1)):
            assert bench.kernel_name(w, phase=phase).endswith(kern.format(mode)), bench.kernel_name(w, phase=phase)
    x = configs.make_device(w, "cuda")
    h = configs.make_host(w)
    cu = w.cu_seqlens() if w.varlen else None
    ref_j, ref_jl = oracle.joint_attention(h["q"], h["k"], h["v"], h["kd"], h["vd"], w.n_depth, w.causal, w.scale,
                                           cu_seqlens=cu)
    ref_s, ref_sl = oracle.sequence_only(h["q"], h["k"], h["v"], w.causal, w.scale, cu_seqlens=cu)
    ref_d, ref_dl = oracle.depth_only(h["q"], h["k"], h["v"], h["kd"], h["vd"], w.n_depth, w.scale, cu_seqlens=cu)
    for out_f32 in ([False, True] if w.bf16 else [False]):
        got = {}
        for phase, ref, ref_l in ((1, ref_s, ref_sl), (2, ref_d, ref_dl), (3, ref_j, ref_jl)):
            o, l = _run(w, x, phase, out_f32)
            tag = f"{name} phase {phase} out_f32={out_f32}"
            r = check_out(w, to_np(o), ref, tag, out_bf16=w.bf16 and not out_f32)
            check_lse(w, to_np(l), ref_l, tag)
            _say(f"  {tag}: max err {r[0]:.3e}, error/bound {r[1]:.3f}")
            got[phase] = (o, l)
        # phase 3 through the phases entry point is the fused call itself
        o3, l3 = _run(w, x, 3, out_f32)
        from joint_sequence_depth_amd import attn_fwd

        cu_t = torch.from_numpy(cu).cuda() if w.varlen else None
        of, lf = attn_fwd(x["q"], x["k"], x["v"], x["kd"], x["vd"], n_depth=w.n_depth, causal=w.causal,
                          scale=w.scale, cu_seqlens=cu_t, max_seqlen=max(w.lengths) if w.varlen else None,
                          out_dtype=torch.float32 if out_f32 else None)
        torch.cuda.synchronize()
        assert torch.equal(o3, of) and torch.equal(l3, lf)
        if w.bf16 and not out_f32:
            continue  # the merge is checked on unrounded (fp32) partial outputs
        # log-sum-exp merge of the two parts (fp64 on the host) = the operator
        o_s, o_d = to_np(got[1][0]), to_np(got[2][0])
        l_s, l_d = _lse_rows(w, to_np(got[1][1])), _lse_rows(w, to_np(got[2][1]))
        lm = np.logaddexp(l_s, l_d)
        shape = (-1, w.n_heads_q, 1)
        merged = (np.exp(l_s - lm).reshape(shape) * o_s.reshape(-1, w.n_heads_q, w.head_dim)
                  + np.exp(l_d - lm).reshape(shape) * o_d.reshape(-1, w.n_heads_q, w.head_dim)).reshape(o_s.shape)
        tag = f"{name} merge of phases 1+2 out_f32={out_f32}"
        r = check_out(w, merged, ref_j, tag, out_bf16=False)
        _say(f"  {tag}: max err {r[0]:.3e}, error/bound {r[1]:.3f}")
        assert np.max(np.abs(lm - _lse_rows(w, ref_jl))) <= (1e-3 if w.bf16 else 1e-5)
