"""Benchmark of the MoDA joint sequence/depth attention forward on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--gpus 1]

One step = one launch of the fused forward (sequence + depth, all rows, all heads)
over one batch of seeded synthetic inputs already resident in HBM. The default
workload is packed_bf16 (8 packed sequences, 65536 tokens, 16 heads, d = 128, 62
depth slots), the largest configuration that fits one GPU. Consecutive steps
cycle through enough independent input batches that the 256 MB Infinity Cache
cannot hold them, so every step streams its operands from HBM. The timed steps
are replayed as a HIP graph (one graph launch per pass over the batches) so that
host launch overhead does not enter the per-step time.

Prints one JSON line. ``value`` = (sequence + depth FLOPs) per step / step time.
``roofline`` rates the fused kernel against the bound that limits it at this
workload (HBM bytes or bf16 MFMA FLOPs, whichever takes longer at peak).
``parts`` times the sequence part alone (TFLOP/s, fraction of bf16 MFMA peak)
and the depth part alone (depth-KV GB/s, fraction of HBM peak) with the same
kernel code, next to the rates this GPU attains on a plain streaming read and a
register-only MFMA loop. ``cpu_baseline`` times the fp64 oracle on a bounded
sample on the host.
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
for _p in (ROOT, os.path.join(ROOT, "tests")):
    if _p not in sys.path:
        sys.path.insert(0, _p)

METRIC = "fused seq+depth attention fwd TFLOP/s; % MFMA peak and depth-KV HBM GB/s"
PEAK_HBM_GBS = 8000.0  # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3  # MI355X fp32 vector
CACHE_DEFEAT_BYTES = 768 << 20  # > 256 MB Infinity Cache + 8 x 4 MB L2
KERNEL_SOURCES = ["moda_fwd_bf16.hip", "moda_fwd_f32.hip", "moda_attn.hip", "moda_internal.h", "moda_rowops.h",
                  "moda_lds_load.h"]  # the forward path
DECODE_SOURCES = ["moda_decode.hip", "moda_attn.hip", "moda_internal.h", "moda_rowops.h"]
BWD_SOURCES = ["moda_bwd.hip", "moda_attn.hip", "moda_internal.h", "moda_rowops.h"]
WRITER_SOURCES = ["moda_depth_kv.hip", "moda_attn.hip", "moda_internal.h"]
PROJECT_SOURCES = ["moda_depth_kv_project.hip", "moda_attn.hip", "moda_internal.h", "moda_lds_load.h"]
WRITER_METRIC = "depth-KV writer HBM GB/s (one layer's K/V rows into one slot of the depth cache)"
BWD_METRIC = "fused seq+depth attention bwd TFLOP/s (dq, dk, dv, dk_depth, dv_depth)"
DECODE_METRIC = "MoDA decode step (joint seq+depth softmax, one token per sequence) HBM GB/s"


def kernel_source_sha(sources=None) -> str:
    h = hashlib.sha256()
    for f in sources or KERNEL_SOURCES:
        with open(os.path.join(ROOT, "joint_sequence_depth_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def kernel_name(w, phase: int = 3, select: bool = False) -> str:
    """The kernel instance the library launches for this workload (mirrors the
    host dispatch: heads per workgroup, waves per workgroup, depth schedule,
    shared or split tiles); ``phase`` 1 or 2 names the sequence-only or
    depth-only launch, ``select`` the bounded depth reads (bf16: selection in
    the depth pass)."""
    if _is_decode(w):
        G = w.group
        gd = next(g for g in (8, 4, 2, 1) if G % g == 0)
        return f"moda_decode_partial_kernel<{w.head_dim}, {gd}, {str(w.bf16).lower()}>"
    if not w.bf16:
        return f"moda_fwd_f32_kernel<{w.head_dim}>"
    G = w.group
    gb = 4 if G % 4 == 0 else 2 if G % 2 == 0 else 1
    n_hg = G // gb
    n_pairs = len(w.lengths) * w.n_heads_kv
    max_len = max(w.lengths)
    waves, split = 0, False
    for nw in (4, 2):
        tok = 32 * nw // gb
        if n_pairs * n_hg * ((max_len + tok - 1) // tok) >= 512:
            waves = nw
            break
    if waves == 0:
        waves, split = 2, True
    mode = 2 if phase == 2 else 0 if (w.n_depth == 0 or phase == 1) else 3 if select else 1
    return f"moda_fwd_bf16_kernel<{w.head_dim}, {gb}, {waves}, {mode}, false, {str(split).lower()}>"


def _is_decode(w) -> bool:
    from workloads import configs

    return isinstance(w, configs.DecodeWorkload)


def _sources(w):
    return DECODE_SOURCES if _is_decode(w) else KERNEL_SOURCES


def _summary_prefix(w) -> str:
    return "moda_decode" if _is_decode(w) else "moda_fwd"


def roofline(w, sec_per_launch: float) -> dict:
    flops = w.seq_flops() + w.depth_flops()
    nbytes = w.total_bytes()
    peak_f = PEAK_BF16_TFLOPS if w.bf16 else PEAK_F32_TFLOPS
    t_mfma = flops / (peak_f * 1e12)
    t_hbm = nbytes / (PEAK_HBM_GBS * 1e9)
    if t_hbm >= t_mfma:
        achieved = nbytes / sec_per_launch / 1e9
        return {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": achieved / PEAK_HBM_GBS, "traffic": traffic_from_profile(w, nbytes)}
    achieved = flops / sec_per_launch / 1e12
    return {"bound": "mfma", "achieved": achieved, "peak": peak_f, "unit": "TFLOP/s", "frac": achieved / peak_f,
            "traffic": traffic_from_profile(w, nbytes)}


def traffic_from_profile(w, algorithmic_bytes):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was
    taken on the current kernel sources (else None)."""
    path = os.path.join(ROOT, "profiles", f"traffic_{w.name}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_sha") != kernel_source_sha(_sources(w)):
        return None
    return rec.get("hbm_bytes_per_launch")


# ------------------------------------------------------------------ profile summaries


def _read_csv(path):
    import csv

    with open(path) as f:
        return list(csv.DictReader(f))


def _counter_kib(run_dir, counter, name_part):
    """Mean per-dispatch value of `counter` over the dispatches whose kernel name
    contains `name_part` (rocprofv3 --pmc csv output)."""
    vals = [float(r["Counter_Value"]) for r in _read_csv(os.path.join(run_dir, "run_counter_collection.csv"))
            if r["Counter_Name"] == counter and name_part in r["Kernel_Name"]]
    if not vals:
        raise SystemExit(f"no {counter} rows for '{name_part}' in {run_dir}")
    return sum(vals) / len(vals), len(vals)


def write_traffic(w, fetch_dir, write_dir, copy_fetch_dir, copy_write_dir, cmds) -> None:
    """profiles/traffic_<workload>.json and a text summary from four rocprofv3 --pmc
    runs: FETCH_SIZE and WRITE_SIZE on the workload and on the 1 GiB copy."""
    kname = kernel_name(w)  # the full instance: the bench also launches the one-part instances
    copy_name = "copyBuffer"
    f_k, n_fk = _counter_kib(fetch_dir, "FETCH_SIZE", kname)
    w_k, n_wk = _counter_kib(write_dir, "WRITE_SIZE", kname)
    f_c, _ = _counter_kib(copy_fetch_dir, "FETCH_SIZE", copy_name)
    w_c, _ = _counter_kib(copy_write_dir, "WRITE_SIZE", copy_name)
    copy_bytes = float(1 << 30)
    scale_f = copy_bytes / (f_c * 1024.0)
    scale_w = copy_bytes / (w_c * 1024.0)
    rd = f_k * 1024.0 * scale_f
    wr = w_k * 1024.0 * scale_w
    if _is_decode(w):  # the partial kernel: reads q, the visible cache rows and the depth slots once
        alg_rd = w.cache_bytes() + w.depth_bytes() + w.batch * w.n_heads_q * w.head_dim * w.elem_bytes()
        alg_wr = 0.0  # its writes are the chunk states in the workspace, not part of the operator's output
    else:
        alg_rd = w.total_bytes() - w.n_tokens * w.n_heads_q * (w.head_dim * w.elem_bytes() + 4)
        alg_wr = w.total_bytes() - alg_rd
    sha = kernel_source_sha(_sources(w))
    rec = {"workload": w.name, "kernel": kernel_name(w), "kernel_source_sha": sha,
           "hbm_bytes_per_launch": rd + wr, "read_bytes": rd, "write_bytes": wr,
           "algorithmic_read_bytes": alg_rd, "algorithmic_write_bytes": alg_wr,
           "fetch_size_kib": f_k, "write_size_kib": w_k, "dispatches": [n_fk, n_wk],
           "copy_fetch_size_kib": f_c, "copy_write_size_kib": w_c, "scale_fetch": scale_f, "scale_write": scale_w}
    with open(os.path.join(ROOT, "profiles", f"traffic_{w.name}.json"), "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    lines = [f"# HBM traffic of {kernel_name(w)} on {w.name} ({w.desc})", "",
             "Commands (on the GPU host, from the repository root; R = repository root):"]
    lines += [f"    {c}" for c in cmds]
    lines += ["",
              "Calibration: a plain 1 GiB device-to-device copy (bench.py --copy-calibration) reads",
              f"FETCH_SIZE = {f_c:.1f} KiB and WRITE_SIZE = {w_c:.1f} KiB per copy; scale factors",
              f"{scale_f:.4f} (reads) and {scale_w:.4f} (writes) turn counter KiB into bytes.", "",
              "| per launch | counter (KiB) | scaled bytes | algorithmic bytes | ratio |", "|---|---|---|---|---|",
              f"| read | {f_k:.1f} | {rd / 1e6:.2f} MB | {alg_rd / 1e6:.2f} MB | {rd / alg_rd:.3f} |",
              f"| write | {w_k:.1f} | {wr / 1e6:.2f} MB | {alg_wr / 1e6:.2f} MB | "
              f"{(wr / alg_wr if alg_wr else float('nan')):.3f} |",
              f"| total | | {(rd + wr) / 1e6:.2f} MB | {(alg_rd + alg_wr) / 1e6:.2f} MB | "
              f"{(rd + wr) / (alg_rd + alg_wr):.3f} |",
              "", f"Means over {n_fk} and {n_wk} dispatches; kernel sources sha {sha}."]
    if _is_decode(w):
        lines.append("Algorithmic reads: q, the visible cache K/V rows and the depth K/V slots once; the kernel's "
                     "writes are the per-chunk fp32 states that the merge kernel reads.")
    else:
        lines.append("Algorithmic reads: q, k, v and the depth K/V rows once; writes: out and lse once.")
    with open(os.path.join(ROOT, "profiles", f"{_summary_prefix(w)}_{w.name}_hbm_counters.txt"), "w") as f:
        f.write("\n".join(lines) + "\n")


def _selects(w, args) -> bool:
    """Whether a bounded-read run launches the bf16 selecting instance (some slots
    dropped: 0 < topk < n_depth - recent)."""
    if args.depth_topk is None or not w.bf16:
        return False
    recent = min(args.depth_recent, w.n_depth)
    return 0 < args.depth_topk < w.n_depth - recent


def write_trace_summary(w, trace_dir, log_path, cmd, backward=False, writer=False, project=False,
                        depth_topk=None) -> None:
    """Text summary of a rocprofv3 --kernel-trace --stats run of bench.py."""
    stats = _read_csv(os.path.join(trace_dir, "run_kernel_stats.csv"))
    bench_line = None
    with open(log_path) as f:
        for line in f:
            if line.startswith("{") and '"metric"' in line:
                bench_line = json.loads(line)
    if backward:  # a backward step is three kernels
        parts = ["moda_bwd_prep_kernel", "moda_bwd_dq", "moda_bwd_dkv"]
        kname = "backward (prep + dq + dk/dv kernels)"
    elif writer:
        parts = ["moda_depth_kv_write_kernel"]
        kname = parts[0]
    elif project:
        parts = ["moda_depth_kv_project_bf16_kernel" if w.bf16 else "moda_depth_kv_project_f32_kernel"]
        kname = parts[0]
    elif _is_decode(w):  # a decode step is the partial kernel and the merge kernel
        parts = [kernel_name(w), "moda_decode_merge_kernel"]
        kname = kernel_name(w)
    else:
        parts = [kernel_name(w, select=depth_topk is not None and w.bf16)]
        kname = parts[0]
    rows = [next((r for r in stats if part in r["Name"]), None) for part in parts]
    if any(r is None for r in rows) or bench_line is None:
        raise SystemExit(f"kernels {parts} or the bench line missing in {trace_dir}")
    bench_us = bench_line["ms_per_step"] * 1e3
    step_us = sum(float(r["AverageNs"]) / 1e3 for r in rows)
    lines = [f"# rocprofv3 kernel trace: {kname} on {w.name} ({w.desc})", "",
             "Command (on the GPU host; R = repository root):", f"    {cmd}", "",
             "| kernel | calls | avg (us) | min (us) | max (us) | share of GPU time |", "|---|---|---|---|---|---|"]
    shown = [r for r in stats if "moda" in r["Name"]]  # the library's kernels, then the largest others
    shown += [r for r in stats if "moda" not in r["Name"]][: max(0, 6 - len(shown))]
    for r in shown:
        name = r["Name"]
        short = name if len(name) < 90 else name[:87] + "..."
        lines.append(f"| `{short}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | {float(r['MinNs']) / 1e3:.2f} "
                     f"| {float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.2f} % |")
    lines += ["", f"bench.py (same run, HIP events over {bench_line['steps']} graph-replayed steps): "
                  f"{bench_us:.2f} us per step; trace average {step_us:.2f} us "
                  + (f"(sum over {len(parts)} kernels) " if len(parts) > 1 else "")
                  + f"({100 * (bench_us / step_us - 1):+.1f} %).",
              f"value {bench_line['value']} {bench_line['unit']}; roofline {bench_line['roofline']['bound']} "
              f"{bench_line['roofline']['achieved']:.1f} {bench_line['roofline']['unit']} "
              f"(frac {bench_line['roofline']['frac']:.3f}); kernel sources sha {bench_line['kernel_source_sha']}."]
    parts = bench_line.get("parts") or {}
    for part in ("sequence_only", "depth_only"):
        if part in parts:
            row = next((r for r in stats if parts[part]["kernel"] in r["Name"]), None)
            trace = f"; trace average {float(row['AverageNs']) / 1e3:.2f} us" if row else ""
            rate = (f"{parts[part]['tflops']} TFLOP/s = {parts[part]['mfma_frac_of_peak']:.3f} of bf16 MFMA peak"
                    if part == "sequence_only" else
                    f"{parts[part]['depth_kv_gbs']} GB/s of depth K/V = {parts[part]['hbm_frac_of_peak']:.3f} of HBM peak")
            lines.append(f"{part.replace('_', ' ')} ({parts[part]['kernel']}): bench {parts[part]['ms'] * 1e3:.2f} us"
                         f"{trace}; {rate}.")
    prefix = ("moda_bwd" if backward else "moda_depth_kv" if writer else "moda_depth_kv_project" if project
              else _summary_prefix(w))
    tag = f"_top{depth_topk}" if depth_topk is not None else ""
    with open(os.path.join(ROOT, "profiles", f"{prefix}_{w.name}{tag}_kernel_trace.txt"), "w") as f:
        f.write("\n".join(lines) + "\n")


def cpu_baseline(w, budget_s: float) -> dict:
    """The fp64 oracle as it stands, on (segment, KV-head group) units of the same
    workload, as many as fit in about ``budget_s`` seconds."""
    import numpy as np

    import oracle
    from workloads import configs

    try:
        from threadpoolctl import threadpool_info

        cores = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:  # threadpoolctl missing: report the affinity set
        cores = len(os.sched_getaffinity(0))
    G, d = w.group, w.head_dim
    units = [(s, hk) for s in range(len(w.lengths)) for hk in range(w.n_heads_kv)]
    rng = np.random.default_rng(0)
    rng.shuffle(units)
    prepared = []
    t_start = time.perf_counter()
    for s, hk in units:  # regenerate the unit's operands (not timed)
        L = w.lengths[s]
        lead = _lead_index(w, s, L)
        hq = np.arange(hk * G, (hk + 1) * G)
        c = np.arange(d)
        q = configs.host_slice(w, "q", _ix(lead, hq, c))
        k = configs.host_slice(w, "k", _ix(lead, np.array([hk]), c))
        v = configs.host_slice(w, "v", _ix(lead, np.array([hk]), c))
        if w.n_depth > 0:
            i = np.arange(w.n_depth)
            kd = configs.host_slice(w, "kd", _ix(lead, i, np.array([hk]), c))[None]
            vd = configs.host_slice(w, "vd", _ix(lead, i, np.array([hk]), c))[None]
        else:
            kd = vd = None
        pairs = L * (L + 1) / 2 if w.causal else L * L
        unit_flops = 4.0 * d * G * pairs + 4.0 * L * G * w.n_depth * d
        prepared.append((q[None], k[None], v[None], kd, vd, unit_flops))
        if time.perf_counter() - t_start > budget_s or len(prepared) * q.nbytes * (2 + w.n_depth) > (4 << 30):
            break
    flops = 0.0
    calls = 0
    compute_s = 0.0
    while compute_s < budget_s:  # cycle over the prepared units until the budget is spent
        q, k, v, kd, vd, unit_flops = prepared[calls % len(prepared)]
        t0 = time.perf_counter()
        oracle.joint_attention(q, k, v, kd, vd, w.n_depth, w.causal, w.scale)
        compute_s += time.perf_counter() - t0
        flops += unit_flops
        calls += 1
    done = len(prepared)
    return {"value": flops / compute_s / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{calls} oracle calls over {done} of the {len(units)} (sequence, KV-head group) units of "
                      f"{w.name} ({flops / 1e9:.2f} GFLOP in {compute_s:.1f} s; operands regenerated on the host, "
                      "generation not timed)"}


def cpu_baseline_decode(w, budget_s: float) -> dict:
    """The fp64 oracle's decode on whole sequences of the workload (operands
    regenerated on the host, not timed), cycled until about ``budget_s`` seconds."""
    import numpy as np

    import oracle
    from workloads import configs

    cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info

        cores = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [cores])
    except Exception:
        pass
    d, S, Hkv = w.head_dim, w.n_depth, w.n_heads_kv
    c = np.arange(d)
    prepared = []
    t_start = time.perf_counter()
    for b in range(w.batch):
        L = w.cache_lengths[b]
        q = configs.decode_host_slice(w, "q", np.ix_([b], np.arange(w.n_heads_q), c))
        kidx = np.ix_([b], np.arange(L), np.arange(Hkv), c)
        k = configs.decode_host_slice(w, "k", kidx)
        v = configs.decode_host_slice(w, "v", kidx)
        if S > 0:
            didx = np.ix_([b], np.arange(S), np.arange(Hkv), c)
            kd, vd = configs.decode_host_slice(w, "kd", didx), configs.decode_host_slice(w, "vd", didx)
        else:
            kd = vd = None
        nbytes = 2.0 * (L + S) * Hkv * d * w.elem_bytes() + w.n_heads_q * d * (w.elem_bytes() + 2) + 4 * w.n_heads_q
        prepared.append((q, k, v, kd, vd, np.array([L]), nbytes))
        if time.perf_counter() - t_start > budget_s:
            break
    done, nbytes_total, compute_s, calls = 0, 0.0, 0.0, 0
    while compute_s < budget_s:
        q, k, v, kd, vd, lens, nbytes = prepared[calls % len(prepared)]
        t0 = time.perf_counter()
        oracle.decode(q, k, v, lens, kd, vd, S, w.scale)
        compute_s += time.perf_counter() - t0
        nbytes_total += nbytes
        calls += 1
    done = len(prepared)
    return {"value": nbytes_total / compute_s / 1e9, "unit": "GB/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{calls} oracle decode calls over {done} of the {w.batch} sequences of {w.name} "
                      f"({nbytes_total / 1e9:.2f} GB of operand bytes in {compute_s:.1f} s; operands regenerated "
                      "on the host, generation not timed)"}


def bench_decode(args, w, dev) -> int:
    """One step = one decode call (partial + merge kernels) for every sequence of
    the workload, inputs resident in HBM, cycling through enough input batches to
    defeat the Infinity Cache, replayed as a HIP graph."""
    import torch

    from joint_sequence_depth_amd import attn_decode, decode_workspace_size
    from workloads import configs

    batch_bytes = w.total_bytes()
    n_batches = max(1, min(32, math.ceil(CACHE_DEFEAT_BYTES / batch_bytes)))
    print(f"# workload {w.name}: {w.desc}; {n_batches} input batch(es) of {batch_bytes / 1e6:.1f} MB", file=sys.stderr,
          flush=True)
    inputs = []
    for i in range(n_batches):
        wi = dataclasses.replace(w, seed=w.seed + 1000 * i)
        inputs.append(configs.make_decode_device(wi, dev))
    odt = torch.bfloat16 if w.bf16 else torch.float32
    outs = [torch.empty(w.shape_q(), dtype=odt, device=dev) for _ in range(n_batches)]
    lses = [torch.empty((w.batch, w.n_heads_q), dtype=torch.float32, device=dev) for _ in range(n_batches)]
    ws = torch.empty(decode_workspace_size(w.batch, w.n_heads_q, w.n_heads_kv, w.head_dim, w.max_cache_len),
                     dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    def step(i):
        x = inputs[i % n_batches]
        attn_decode(x["q"], x["k"], x["v"], x["seqlens"], x["kd"], x["vd"], n_depth=w.n_depth, scale=w.scale,
                    out=outs[i % n_batches], lse=lses[i % n_batches], workspace=ws)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(n_batches):
        step(i)
    torch.cuda.synchronize()
    rough = (time.perf_counter() - t0) / n_batches
    steps = args.steps or max(n_batches, int(1.0 / max(rough, 1e-6)))
    steps = max(n_batches, (steps // n_batches) * n_batches)

    stream = torch.cuda.current_stream(dev)
    use_graph = not args.no_graph
    graph = None
    if use_graph:
        side = torch.cuda.Stream(dev)
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            step(0)
        stream.wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(n_batches):
                step(i)
        torch.cuda.synchronize()
        for _ in range(2):
            graph.replay()
        torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    if use_graph:
        for _ in range(steps // n_batches):
            graph.replay()
    else:
        for i in range(steps):
            step(i)
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    sec = ms / 1e3

    # the last replayed batch's results must equal an eager call (bitwise)
    last = (steps - 1) % n_batches
    ref_out, ref_lse = torch.empty_like(outs[0]), torch.empty_like(lses[0])
    x = inputs[last]
    attn_decode(x["q"], x["k"], x["v"], x["seqlens"], x["kd"], x["vd"], n_depth=w.n_depth, scale=w.scale,
                out=ref_out, lse=ref_lse, workspace=ws)
    torch.cuda.synchronize()
    replay_ok = bool(torch.equal(ref_out, outs[last]) and torch.equal(ref_lse, lses[last]))
    if not replay_ok:
        print("error: timed replays differ from an eager call", file=sys.stderr)

    nbytes = w.total_bytes(out_bytes=w.elem_bytes())
    gbs = nbytes / sec / 1e9
    rec = {
        "metric": DECODE_METRIC,
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.bf16 else "f32",
        "data": "synthetic (seeded counter-based N(0,1) quantile grid)",
        "config": {
            "workload": w.name,
            "batch": w.batch,
            "cache_lengths": list(w.cache_lengths),
            "max_cache_len": w.max_cache_len,
            "n_heads_q": w.n_heads_q,
            "n_heads_kv": w.n_heads_kv,
            "head_dim": w.head_dim,
            "n_depth": w.n_depth,
            "input_batches": n_batches,
            "graph": use_graph,
        },
        "parts": {
            "tflops": round(w.flops() / sec / 1e12, 3),
            "cache_kv_gbs": round(w.cache_bytes() / sec / 1e9, 1),
            "depth_kv_gbs": round(w.depth_bytes() / sec / 1e9, 1),
        },
        "kernel": kernel_name(w),
        "kernel_source_sha": kernel_source_sha(DECODE_SOURCES),
        "replay_matches_eager": replay_ok,
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": gbs / PEAK_HBM_GBS,
                     "traffic": traffic_from_profile(w, nbytes)},
        "cpu_baseline": None,
    }
    del inputs, outs, lses, graph, ws
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline_decode(w, args.cpu_budget)
    print(json.dumps(rec), flush=True)
    return 0 if replay_ok else 1


def bwd_bytes(w) -> float:
    """Algorithmic HBM bytes of one backward step: q, k, v, out, dout, lse and the
    depth slots read once; dq, dk, dv and the depth-slot gradients written once."""
    e, n, d = w.elem_bytes(), w.n_tokens, w.head_dim
    rows = n * d * e * (w.n_heads_q * 4 + w.n_heads_kv * 4)  # q, out, dout, dq; k, v, dk, dv
    return 2.0 * w.depth_bytes() + rows + 4.0 * n * w.n_heads_q


def bench_backward(args, w, dev) -> int:
    """One step = one backward call (prep/depth, dq and dk/dv kernels) over the
    whole workload, with q, k, v, the depth slots, out, dout and lse resident in
    HBM (out and lse from the library's forward), replayed as a HIP graph."""
    import torch

    from joint_sequence_depth_amd import attn_bwd, attn_fwd, bwd_workspace_size
    from workloads import configs

    gdt = torch.bfloat16 if w.bf16 else torch.float32
    per_batch = 2 * w.total_bytes() + 2 * w.n_tokens * w.n_heads_q * w.head_dim * w.elem_bytes()
    n_batches = max(1, min(8, math.ceil(CACHE_DEFEAT_BYTES / per_batch)))
    print(f"# backward of {w.name}: {w.desc}; {n_batches} input batch(es)", file=sys.stderr, flush=True)
    cu = torch.from_numpy(w.cu_seqlens()).to(dev) if w.varlen else None
    max_len = max(w.lengths)
    sets = []
    for i in range(n_batches):
        x = configs.make_device(w, dev, i)
        out, lse = attn_fwd(x["q"], x["k"], x["v"], x["kd"], x["vd"], n_depth=w.n_depth, causal=w.causal,
                            scale=w.scale, cu_seqlens=cu, max_seqlen=max_len, out_dtype=gdt)
        dout = configs.make_dout_device(w, dev, gdt, i)
        grads = (torch.empty_like(x["q"]), torch.empty_like(x["k"]), torch.empty_like(x["v"]),
                 None if x["kd"] is None else torch.zeros_like(x["kd"]),
                 None if x["vd"] is None else torch.zeros_like(x["vd"]))
        sets.append((x, out, dout, lse, grads))
    ws = torch.empty(max(256, bwd_workspace_size(w.n_tokens, w.n_heads_q, w.head_dim, w.n_depth)), dtype=torch.uint8,
                     device=dev)
    torch.cuda.synchronize()

    def step(i, grads=None):
        x, out, dout, lse, g = sets[i % n_batches]
        return attn_bwd(x["q"], x["k"], x["v"], x["kd"], x["vd"], out, dout, lse, n_depth=w.n_depth, causal=w.causal,
                        scale=w.scale, cu_seqlens=cu, max_seqlen=max_len, grads=grads or g, workspace=ws)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(n_batches):
        step(i)
    torch.cuda.synchronize()
    rough = (time.perf_counter() - t0) / n_batches
    steps = args.steps or max(n_batches, int(2.0 / max(rough, 1e-6)))
    steps = max(n_batches, (steps // n_batches) * n_batches)
    stream = torch.cuda.current_stream(dev)
    use_graph = not args.no_graph
    graph = None
    if use_graph:
        side = torch.cuda.Stream(dev)
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            step(0)
        stream.wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(n_batches):
                step(i)
        torch.cuda.synchronize()
        for _ in range(2):
            graph.replay()
        torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    if use_graph:
        for _ in range(steps // n_batches):
            graph.replay()
    else:
        for i in range(steps):
            step(i)
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    sec = ms / 1e3

    # the last replayed batch's gradients must equal an eager call's (bitwise)
    last = (steps - 1) % n_batches
    g_ref = tuple(None if t is None else torch.zeros_like(t) for t in sets[last][4])
    step(last, grads=g_ref)
    torch.cuda.synchronize()
    replay_ok = all(a is None or torch.equal(a, b) for a, b in zip(sets[last][4], g_ref))
    if not replay_ok:
        print("error: timed replays differ from an eager call", file=sys.stderr)

    # algorithmic work: dP, dS-weighted dQ and dK, and P-weighted dV over the same
    # visible pairs and slots as the forward: twice the forward's products
    flops = 2.0 * (w.seq_flops() + w.depth_flops())
    tflops = flops / sec / 1e12
    peak = PEAK_BF16_TFLOPS if w.bf16 else PEAK_F32_TFLOPS
    nbytes = bwd_bytes(w)
    if nbytes / (PEAK_HBM_GBS * 1e9) >= flops / (peak * 1e12):  # the bound that takes longer at peak
        gbs = nbytes / sec / 1e9
        roof = {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": gbs / PEAK_HBM_GBS,
                "traffic": None}
    else:
        roof = {"bound": "mfma" if w.bf16 else "alu", "achieved": tflops, "peak": peak, "unit": "TFLOP/s",
                "frac": tflops / peak, "traffic": None}
    rec = {
        "metric": BWD_METRIC,
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.bf16 else "f32",
        "data": "synthetic (seeded counter-based N(0,1) quantile grid)",
        "config": {"workload": w.name, "pass": "backward", "batch": w.batch, "seq_len": w.seqlen,
                   "seqlens": list(w.seqlens) if w.varlen else None, "n_heads_q": w.n_heads_q,
                   "n_heads_kv": w.n_heads_kv, "head_dim": w.head_dim, "n_depth": w.n_depth, "causal": w.causal,
                   "input_batches": n_batches, "graph": use_graph},
        "kernel": "moda_bwd_prep_kernel + moda_bwd_dq_kernel + moda_bwd_dkv8_kernel" if w.bf16 else
                  "moda_bwd_prep_kernel + moda_bwd_dq_f32_kernel + moda_bwd_dkv_f32_kernel",
        "kernel_source_sha": kernel_source_sha(BWD_SOURCES),
        "replay_matches_eager": replay_ok,
        "parts": {"all_bytes_gbs": round(nbytes / sec / 1e9, 1), "mfma_frac_of_peak": round(tflops / peak, 4)},
        "roofline": roof,
        "cpu_baseline": None,
    }
    del sets, graph, ws
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline_backward(w, args.cpu_budget)
    print(json.dumps(rec), flush=True)
    return 0 if replay_ok else 1


def cpu_baseline_backward(w, budget_s: float) -> dict:
    """The fp64 oracle's backward on (segment, KV head) units of the workload."""
    import numpy as np

    import oracle
    from parity_util import unit_operands

    cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info

        cores = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [cores])
    except Exception:
        pass
    units = [(s, hk) for s in range(len(w.lengths)) for hk in range(w.n_heads_kv)]
    np.random.default_rng(0).shuffle(units)
    flops = compute_s = 0.0
    calls = 0
    for s, hk in units:
        ops = unit_operands(w, s, hk, w.bf16)
        L = w.lengths[s]
        pairs = L * (L + 1) / 2 if w.causal else L * L
        unit_flops = 2.0 * (4.0 * w.head_dim * w.group * pairs + 4.0 * L * w.group * w.n_depth * w.head_dim)
        t0 = time.perf_counter()
        oracle.joint_attention_backward(*ops[:5], w.n_depth, ops[5], w.causal, w.scale)
        compute_s += time.perf_counter() - t0
        flops += unit_flops
        calls += 1
        if compute_s > budget_s:
            break
    return {"value": flops / compute_s / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{calls} of the {len(units)} (sequence, KV head) units of {w.name}, backward "
                      f"({flops / 1e9:.2f} GFLOP in {compute_s:.1f} s; operands regenerated on the host, not timed)"}


def bench_writer(args, w, dev) -> int:
    """One step = one depth-KV write: every token's K and V rows of the workload
    into one slot of its depth cache (slots cycling over S_cap, as a layer stack or
    a bounded ring buffer writes them)."""
    import torch

    from joint_sequence_depth_amd import depth_kv_write
    from workloads import configs

    dt = torch.bfloat16 if w.bf16 else torch.float32
    x = configs.make_device(w, dev)
    S_cap = max(1, w.s_cap)
    kd = torch.zeros(w.shape_depth()[:-3] + (S_cap, w.n_heads_kv, w.head_dim), dtype=dt, device=dev)
    vd = torch.zeros_like(kd)
    torch.cuda.synchronize()

    def step(i):
        depth_kv_write(x["k"], x["v"], kd, vd, i % S_cap)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    steps = args.steps or 200
    steps = max(S_cap, steps // S_cap * S_cap)
    stream = torch.cuda.current_stream(dev)
    graph = None
    if not args.no_graph:
        side = torch.cuda.Stream(dev)
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            step(0)
        stream.wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(S_cap):
                step(i)
        torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    if graph is not None:
        for _ in range(steps // S_cap):
            graph.replay()
    else:
        for i in range(steps):
            step(i)
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    ok = bool(torch.equal(kd[..., S_cap - 1, :, :], x["k"]) and torch.equal(vd[..., 0, :, :], x["v"]))
    nbytes = 4.0 * w.n_tokens * w.n_heads_kv * w.head_dim * w.elem_bytes()
    gbs = nbytes / (ms / 1e3) / 1e9
    rec = {
        "metric": WRITER_METRIC, "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16" if w.bf16 else "f32",
        "data": "synthetic (seeded counter-based N(0,1) quantile grid)",
        "config": {"workload": w.name, "pass": "depth-kv writer", "tokens": w.n_tokens, "n_heads_kv": w.n_heads_kv,
                   "head_dim": w.head_dim, "depth_capacity": S_cap, "graph": graph is not None},
        "kernel": "moda_depth_kv_write_kernel", "kernel_source_sha": kernel_source_sha(WRITER_SOURCES),
        "copies_match": ok,
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": gbs / PEAK_HBM_GBS,
                     "traffic": None},
        "cpu_baseline": None,
    }
    print(json.dumps(rec), flush=True)
    return 0 if ok else 1


PROJECT_METRIC = "FFN-input KV projection into a depth slot, bf16 MFMA TFLOP/s"


def bench_project(args, w, dev) -> int:
    """One step = the FFN input's KV projection of every token of the workload
    into one slot of its depth cache: x [N, D_model = H_q d] times [W_k; W_v]
    [2 H_kv d, D_model], the rows stored straight into slot s of [N, S_cap, H_kv, d]
    (slots cycling over S_cap). Bound: bf16 MFMA."""
    import torch

    from joint_sequence_depth_amd import depth_kv_project
    from workloads import gen

    dt = torch.bfloat16 if w.bf16 else torch.float32
    N, D, Hkv, d = w.n_tokens, w.n_heads_q * w.head_dim, w.n_heads_kv, w.head_dim
    S_cap = max(1, w.s_cap)
    x = gen.tensor_t(w.seed, 60, (N, D), dt, dev)
    wkv = gen.tensor_t(w.seed, 61, (2 * Hkv * d, D), dt, dev, 2.0**-5)
    kd = torch.zeros((N, S_cap, Hkv, d), dtype=dt, device=dev)
    vd = torch.zeros_like(kd)
    torch.cuda.synchronize()

    def step(i):
        depth_kv_project(x, wkv, kd, vd, i % S_cap)

    class _A:  # time_steps' view of the arguments: S_cap steps per graph pass
        steps, warmup, no_graph = args.steps, args.warmup, args.no_graph

    ms, steps, use_graph = time_steps(step, S_cap, _A, dev, torch.cuda.current_stream(dev))
    flops = 2.0 * N * D * 2 * Hkv * d
    tf = flops / (ms / 1e3) / 1e12
    peak = PEAK_BF16_TFLOPS if w.bf16 else PEAK_F32_TFLOPS
    rec = {
        "metric": PROJECT_METRIC, "value": round(tf, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16" if w.bf16 else "f32",
        "data": "synthetic (seeded counter-based N(0,1) quantile grid; weights x 2^-5)",
        "config": {"workload": w.name, "pass": "FFN-input KV projection", "tokens": N, "d_model": D,
                   "n_heads_kv": Hkv, "head_dim": d, "depth_capacity": S_cap, "graph": use_graph},
        "kernel": "moda_depth_kv_project_bf16_kernel" if w.bf16 else "moda_depth_kv_project_f32_kernel",
        "kernel_source_sha": kernel_source_sha(PROJECT_SOURCES),
        "roofline": {"bound": "mfma", "achieved": tf, "peak": peak, "unit": "TFLOP/s", "frac": tf / peak,
                     "traffic": None},
        "cpu_baseline": None,
    }
    print(json.dumps(rec), flush=True)
    return 0


def _lead_index(w, s, L):
    import numpy as np

    if w.varlen:
        return (np.arange(int(w.cu_seqlens()[s]), int(w.cu_seqlens()[s]) + L),)
    return (np.array([s]), np.arange(L))


def _ix(lead, *rest):
    """Open-mesh index tuple over the leading token index and the remaining axes."""
    import numpy as np

    if len(lead) == 2:  # (b, t): drop the batch axis afterwards
        idx = np.ix_(lead[0], lead[1], *rest)
        return tuple(a[0] for a in idx)
    return np.ix_(lead[0], *rest)


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None, help="timed steps (default: about 2 s of GPU time)")
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="packed_bf16")
    ap.add_argument("--backward", action="store_true", help="time the backward pass of the workload instead")
    ap.add_argument("--writer", action="store_true", help="time the depth-KV writer on the workload's shapes instead")
    ap.add_argument("--project", action="store_true",
                    help="time the FFN-input KV projection into a depth slot on the workload's shapes instead")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle time for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="launch every step from the host")
    ap.add_argument("--no-parts", action="store_true", help="skip the sequence-only and depth-only timings")
    ap.add_argument("--depth-topk", type=int, default=None,
                    help="time the bounded depth reads: each row keeps this many top-logit slots")
    ap.add_argument("--depth-recent", type=int, default=0, help="... plus this many most recent slots")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 1 GiB device copy (for scaling HBM counters)")
    ap.add_argument("--summarize-trace", nargs=2, metavar=("TRACE_DIR", "LOG"),
                    help="write the profiles/ summary of a rocprofv3 --kernel-trace --stats run (no GPU)")
    ap.add_argument("--write-traffic", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR", "COPY_WRITE_DIR"),
                    help="write profiles/traffic_<workload>.json from four rocprofv3 --pmc runs (no GPU)")
    ap.add_argument("--profile-cmd", action="append", default=[], help="command text recorded in a summary")
    args = ap.parse_args(argv)

    if args.summarize_trace or args.write_traffic:
        from workloads import configs

        w = configs.WORKLOADS.get(args.workload) or configs.DECODE_WORKLOADS[args.workload]
        if args.summarize_trace:
            write_trace_summary(w, args.summarize_trace[0], args.summarize_trace[1], " ".join(args.profile_cmd),
                                backward=args.backward, writer=args.writer, project=args.project,
                                depth_topk=args.depth_topk)
        if args.write_traffic:
            write_traffic(w, *args.write_traffic, args.profile_cmd)
        return 0

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the multi-GPU sharding of this path is a design note, not built.", file=sys.stderr)
        return 2

    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    dev = torch.device("cuda:0")

    if args.copy_calibration:
        n = 1 << 30
        a = torch.empty(n, dtype=torch.uint8, device=dev)
        a.fill_(1)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n, "launches": 3}))
        return 0

    from joint_sequence_depth_amd import attn_fwd, lib
    from workloads import configs

    lib()  # fail loudly before any work if the HIP library is missing
    if args.workload in configs.DECODE_WORKLOADS:
        return bench_decode(args, configs.DECODE_WORKLOADS[args.workload], dev)
    w = configs.WORKLOADS[args.workload]
    if args.backward:
        return bench_backward(args, w, dev)
    if args.writer:
        return bench_writer(args, w, dev)
    if args.project:
        return bench_project(args, w, dev)
    peaks = attained_peaks(dev)
    print(f"# attained peaks: {peaks}", file=sys.stderr, flush=True)
    batch_bytes = w.total_bytes()
    n_batches = max(1, min(32, math.ceil(CACHE_DEFEAT_BYTES / batch_bytes)))
    print(f"# workload {w.name}: {w.desc}; {n_batches} input batch(es) of {batch_bytes / 1e6:.1f} MB", file=sys.stderr,
          flush=True)
    inputs = [configs.make_device(w, dev, i) for i in range(n_batches)]
    cu = torch.from_numpy(w.cu_seqlens()).to(dev) if w.varlen else None
    max_len = max(w.lengths)
    odt = torch.bfloat16 if w.bf16 else torch.float32
    outs = [torch.empty(w.shape_q(), dtype=odt, device=dev) for _ in range(n_batches)]
    lses = [torch.empty(w.shape_lse(), dtype=torch.float32, device=dev) for _ in range(n_batches)]
    torch.cuda.synchronize()
    print("# inputs generated", file=sys.stderr, flush=True)
    stream = torch.cuda.current_stream(dev)

    sel = {}
    if args.depth_topk is not None:  # bounded depth reads: slot masks in a preallocated workspace
        from joint_sequence_depth_amd import topk_workspace_size

        sel = dict(depth_topk=args.depth_topk, depth_recent=args.depth_recent,
                   workspace=torch.empty(topk_workspace_size(w.n_tokens, w.n_heads_q), dtype=torch.uint8, device=dev))

    def make_step(phase):
        def step(i):
            x = inputs[i % n_batches]
            attn_fwd(x["q"], x["k"], x["v"], x["kd"], x["vd"], n_depth=w.n_depth, causal=w.causal, scale=w.scale,
                     cu_seqlens=cu, max_seqlen=max_len, out=outs[i % n_batches], lse=lses[i % n_batches],
                     phase=phase, **sel)
        return step

    step = make_step(3)
    ms, steps, use_graph = time_steps(step, n_batches, args, dev, stream)
    sec = ms / 1e3

    # replayed results must equal an eager call on the same inputs (bitwise)
    ref_out = torch.empty_like(outs[0])
    ref_lse = torch.empty_like(lses[0])
    x0 = inputs[0]
    attn_fwd(x0["q"], x0["k"], x0["v"], x0["kd"], x0["vd"], n_depth=w.n_depth, causal=w.causal, scale=w.scale,
             cu_seqlens=cu, max_seqlen=max_len, out=ref_out, lse=ref_lse, **sel)
    torch.cuda.synchronize()
    replay_ok = bool(torch.equal(ref_out, outs[0]) and torch.equal(ref_lse, lses[0]))
    if not replay_ok:
        print("error: timed replays differ from an eager call", file=sys.stderr)

    # the two parts alone, from the same kernel code (the other part compiled out)
    part_ms = {}
    if w.bf16 and w.n_depth > 0 and not args.no_parts and not sel:
        for phase in (1, 2):
            part_ms[phase], _, _ = time_steps(make_step(phase), n_batches, args, dev, stream)
            print(f"# phase {phase}: {part_ms[phase]:.4f} ms per launch", file=sys.stderr, flush=True)

    flops = w.seq_flops() + w.depth_flops()
    tflops = flops / sec / 1e12
    peak_f = PEAK_BF16_TFLOPS if w.bf16 else PEAK_F32_TFLOPS
    if sel:
        # bounded reads: every slot key is scored, only the kept slots' values are weighted
        kept = min(w.n_depth, args.depth_topk + args.depth_recent)
        flops = w.seq_flops() + 2.0 * w.n_tokens * w.n_heads_q * w.head_dim * (w.n_depth + kept)
        tflops = flops / sec / 1e12
    parts = {
        "fused": {
            "ms": round(ms, 5),
            "seq_tflops": round(w.seq_flops() / sec / 1e12, 3),
            "mfma_frac_of_peak": round(tflops / peak_f, 4),
            "depth_kv_gbs": round(w.depth_bytes() / sec / 1e9, 1),
            "all_bytes_gbs": round(w.total_bytes() / sec / 1e9, 1),
            "hbm_frac_of_peak": round(w.total_bytes() / sec / 1e9 / PEAK_HBM_GBS, 4),
        },
        "attained_peaks": peaks,
    }
    if part_ms:
        s1, s2 = part_ms[1] / 1e3, part_ms[2] / 1e3
        seq_tf = w.seq_flops() / s1 / 1e12
        dep_gbs = w.depth_bytes() / s2 / 1e9
        dep_all = (w.depth_bytes() + depth_phase_other_bytes(w)) / s2 / 1e9
        parts["sequence_only"] = {
            "ms": round(part_ms[1], 5), "kernel": kernel_name(w, phase=1), "tflops": round(seq_tf, 2),
            "mfma_frac_of_peak": round(seq_tf / PEAK_BF16_TFLOPS, 4),
            "mfma_frac_of_attained": round(seq_tf / peaks["mfma_bf16_tflops"], 4),
        }
        parts["depth_only"] = {
            "ms": round(part_ms[2], 5), "kernel": kernel_name(w, phase=2), "depth_kv_gbs": round(dep_gbs, 1),
            "hbm_frac_of_peak": round(dep_gbs / PEAK_HBM_GBS, 4),
            "hbm_frac_of_attained": round(dep_gbs / peaks["hbm_stream_read_gbs"], 4),
            "all_bytes_gbs": round(dep_all, 1),
        }
        # depth bytes over the time the fused launch spends beyond the sequence part alone
        extra = sec - s1
        parts["depth_kv_gbs_beside_sequence"] = round(w.depth_bytes() / extra / 1e9, 1) if extra > 0 else None
    if sel:
        kept = min(w.n_depth, args.depth_topk + args.depth_recent)
        alg = w.n_tokens * w.n_heads_kv * w.head_dim * w.elem_bytes() * (w.n_depth + kept) + w.other_bytes()
        alg += 16.0 * w.n_tokens * w.n_heads_q  # slot masks written and read
        parts["bounded_depth_reads"] = {
            "depth_topk": args.depth_topk, "depth_recent": args.depth_recent, "kept_slots": kept,
            "algorithmic_bytes": alg, "gbs": round(alg / sec / 1e9, 1),
            "hbm_frac_of_peak": round(alg / sec / 1e9 / PEAK_HBM_GBS, 4),
            "note": "keys of every slot are read to rank them, values of the kept slots only (bf16: selected "
                    "inside the depth pass; grouped heads read the union of their kept slots)",
        }
    rec = {
        "metric": METRIC,
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.bf16 else "f32",
        "data": "synthetic (seeded counter-based N(0,1) quantile grid)",
        "config": {
            "workload": w.name,
            "batch": w.batch,
            "seq_len": w.seqlen,
            "seqlens": list(w.seqlens) if w.varlen else None,
            "n_heads_q": w.n_heads_q,
            "n_heads_kv": w.n_heads_kv,
            "head_dim": w.head_dim,
            "n_depth": w.n_depth,
            "causal": w.causal,
            "input_batches": n_batches,
            "graph": use_graph,
            "depth_topk": args.depth_topk,
            "depth_recent": args.depth_recent if sel else None,
        },
        "parts": parts,
        "kernel": kernel_name(w, select=_selects(w, args)),
        "kernel_source_sha": kernel_source_sha(),
        "replay_matches_eager": replay_ok,
        "roofline": roofline(w, sec) if not sel else {
            "bound": "hbm", "achieved": parts["bounded_depth_reads"]["gbs"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": parts["bounded_depth_reads"]["hbm_frac_of_peak"], "traffic": None},
        "cpu_baseline": None,
    }
    del inputs, outs, lses
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(w, args.cpu_budget)
    print(json.dumps(rec), flush=True)
    return 0 if replay_ok else 1


def depth_phase_other_bytes(w) -> float:
    """Bytes the depth-only launch moves besides the depth slots: q read, out and
    lse written once."""
    e = w.elem_bytes()
    return w.n_tokens * w.n_heads_q * (2 * w.head_dim * e + 4.0)


def time_steps(step, n_batches, args, dev, stream):
    """Warm-up, then whole passes over the input batches replayed as one HIP graph
    per pass (or launched from the host with --no-graph), timed with events on the
    stream the kernels run on. Returns (ms per step, steps, graph used)."""
    import torch

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # rough per-step time to size the timed region
    t0 = time.perf_counter()
    for i in range(n_batches):
        step(i)
    torch.cuda.synchronize()
    rough = (time.perf_counter() - t0) / n_batches
    steps = args.steps or max(n_batches, int(2.0 / max(rough, 1e-6)))
    steps = max(n_batches, (steps // n_batches) * n_batches)  # whole passes over the batches
    use_graph = not args.no_graph
    graph = None
    if use_graph:
        side = torch.cuda.Stream(dev)
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            step(0)  # one eager call on the capture stream before capture
        stream.wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(n_batches):
                step(i)
        torch.cuda.synchronize()
        for _ in range(2):
            graph.replay()
        torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    if use_graph:
        for _ in range(steps // n_batches):
            graph.replay()
    else:
        for i in range(steps):
            step(i)
    end.record(stream)
    torch.cuda.synchronize()
    del graph
    return start.elapsed_time(end) / steps, steps, use_graph


def attained_peaks(dev) -> dict:
    """The rates this GPU reaches on a plain 16-byte streaming read of 4 GiB and on
    a register-only bf16 MFMA loop (libmoda_peaks.so), each the best of 5 timed
    launches after one warm-up."""
    import ctypes

    import torch

    from joint_sequence_depth_amd import build as _b

    L = ctypes.CDLL(_b.PEAKS_PATH)
    L.moda_peak_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int32,
                                        ctypes.c_void_p]
    L.moda_peak_mfma_bf16.argtypes = [ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p]
    L.moda_peak_mfma_flops_per_launch.argtypes = [ctypes.c_int32, ctypes.c_int32]
    L.moda_peak_mfma_flops_per_launch.restype = ctypes.c_double
    stream = torch.cuda.current_stream(dev)
    nbytes, wg_read = 4 << 30, 4096
    buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    buf.fill_(7)
    sink = torch.empty(8192, dtype=torch.float32, device=dev)
    iters, wg_mfma = 2048, 2048

    def best(fn):
        fn()
        ts = []
        for _ in range(5):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b) / 1e3)
        return min(ts)

    def read():
        rc = L.moda_peak_stream_read(buf.data_ptr(), nbytes, sink.data_ptr(), wg_read, stream.cuda_stream)
        assert rc == 0, rc

    def mfma():
        rc = L.moda_peak_mfma_bf16(iters, sink.data_ptr(), wg_mfma, stream.cuda_stream)
        assert rc == 0, rc

    t_read = best(read)
    t_mfma = best(mfma)
    del buf, sink
    torch.cuda.empty_cache()
    return {"hbm_stream_read_gbs": round(nbytes / t_read / 1e9, 1),
            "mfma_bf16_tflops": round(L.moda_peak_mfma_flops_per_launch(iters, wg_mfma) / t_mfma / 1e12, 1)}


if __name__ == "__main__":
    sys.exit(main())
