"""Host logic of bench.py (CPU only): the one-GPU contract, the kernel names it
reports (checked against the names rocprofv3 recorded on the GPU in the committed
traces), and the profile summaries written from rocprofv3 output (synthetic
fixtures in a temporary directory; the committed profiles are never touched)."""
import json
import os

import pytest

import bench
from workloads import configs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().err


@pytest.mark.parametrize("name", ["packed_bf16", "mha_bf16", "gqa_bf16"])
def test_kernel_names_match_the_traced_launches(name):
    # the traces list the kernels the library really launched (names from the GPU):
    # the fused instance and the two one-part instances bench.py reports must be there
    path = os.path.join(ROOT, "profiles", f"moda_fwd_{name}_kernel_trace.txt")
    if not os.path.exists(path):
        pytest.skip("no committed trace")
    traced = [line for line in open(path) if line.startswith("| `")]
    w = configs.WORKLOADS[name]
    for phase in (3, 1, 2):
        assert any(bench.kernel_name(w, phase=phase) in line for line in traced), (name, phase)


def test_bounded_reads_name_the_selecting_instance():
    w = configs.WORKLOADS["packed_bf16"]

    class A:
        depth_topk, depth_recent = 16, 0

    assert bench._selects(w, A)
    assert bench.kernel_name(w, select=True).endswith("<128, 1, 4, 3, false, false>")
    A.depth_topk = 62  # every slot stays: the operator itself
    assert not bench._selects(w, A)
    A.depth_topk, A.depth_recent = 10, 60  # 10 >= 62 - 60
    assert not bench._selects(w, A)
    A.depth_topk = None
    assert not bench._selects(w, A)


def _write_csv(path, header, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w") as f:
        f.write(",".join(header) + "\n")
        for r in rows:
            f.write(",".join(str(x) for x in r) + "\n")


def test_trace_summary_from_rocprof_output(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    os.makedirs(tmp_path / "profiles")
    w = configs.WORKLOADS["mha_bf16"]
    k = bench.kernel_name(w)
    _write_csv(str(tmp_path / "tr" / "run_kernel_stats.csv"), ["Name", "Calls", "AverageNs", "MinNs", "MaxNs", "Percentage"],
               [[f'"void moda::(anonymous namespace)::{k}(moda::Params)"', 100, 800000.0, 790000.0, 900000.0, 70.0],
                ['"void at::native::other_kernel"', 10, 1000.0, 900.0, 1100.0, 1.0]])
    line = {"metric": "m", "value": 350.0, "unit": "TFLOP/s", "steps": 100, "ms_per_step": 0.808,
            "kernel_source_sha": "abc", "roofline": {"bound": "hbm", "achieved": 4300.0, "unit": "GB/s", "frac": 0.5375}}
    log = tmp_path / "tr.log"
    log.write_text("# something\n" + json.dumps(line) + "\n")
    bench.write_trace_summary(w, str(tmp_path / "tr"), str(log), "rocprofv3 ... -- python3 R/bench.py")
    text = (tmp_path / "profiles" / "moda_fwd_mha_bf16_kernel_trace.txt").read_text()
    assert k in text and "800.00" in text
    assert "808.00 us per step; trace average 800.00 us (+1.0 %)" in text
    assert "frac 0.537" in text


def test_traffic_from_counter_output(tmp_path, monkeypatch):
    # scale factors from the 1 GiB copy, per-launch bytes and ratios against the
    # algorithmic bytes
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_sha", lambda sources=None: "fixture")
    os.makedirs(tmp_path / "profiles")
    w = configs.WORKLOADS["mha_bf16"]
    k = bench.kernel_name(w)
    hdr = ["Kernel_Name", "Counter_Name", "Counter_Value"]
    alg_rd = w.total_bytes() - w.n_tokens * w.n_heads_q * (w.head_dim * w.elem_bytes() + 4)
    alg_wr = w.total_bytes() - alg_rd
    # the kernel reads 1.05x and writes exactly its algorithmic bytes; FETCH_SIZE
    # counts half the bytes (as the copy shows), WRITE_SIZE all of them
    _write_csv(str(tmp_path / "f" / "run_counter_collection.csv"), hdr,
               [[f'"{k}"', "FETCH_SIZE", 1.05 * alg_rd / 2 / 1024]] * 2)
    _write_csv(str(tmp_path / "w" / "run_counter_collection.csv"), hdr, [[f'"{k}"', "WRITE_SIZE", alg_wr / 1024]] * 2)
    _write_csv(str(tmp_path / "cf" / "run_counter_collection.csv"), hdr, [["copyBuffer", "FETCH_SIZE", 524288.0]])
    _write_csv(str(tmp_path / "cw" / "run_counter_collection.csv"), hdr, [["copyBuffer", "WRITE_SIZE", 1048576.0]])
    bench.write_traffic(w, str(tmp_path / "f"), str(tmp_path / "w"), str(tmp_path / "cf"), str(tmp_path / "cw"),
                        ["cmd"])
    rec = json.load(open(tmp_path / "profiles" / "traffic_mha_bf16.json"))
    assert rec["scale_fetch"] == pytest.approx(2.0) and rec["scale_write"] == pytest.approx(1.0)
    assert rec["read_bytes"] / rec["algorithmic_read_bytes"] == pytest.approx(1.05)
    assert rec["write_bytes"] == pytest.approx(alg_wr)
    assert rec["kernel_source_sha"] == "fixture"
    text = (tmp_path / "profiles" / "moda_fwd_mha_bf16_hbm_counters.txt").read_text()
    assert "| read |" in text and "1.050 |" in text
