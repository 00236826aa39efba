"""Benchmark of the MI355X exact attention forward (one JSON line on stdout).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c2] [--dtype bf16]

A step is one full forward call (attn_fwd: the fused kernel, plus the combine
kernel when the key range is split) over one batch of synthetic inputs that is
already resident in HBM. The default workload is the non-causal MHA forward
q/k/v [1, 20480, 56, 128] in bf16 (video joint-attention shape).

Reported:
  value       whole-job TFLOP/s (GB/s when the workload is HBM-bound: decode, short-query
              cached prediction) over the K timed steps
  roofline    achieved / peak of the dominant kernel: algorithmic FLOPs (or bytes) per
              launch / its mean duration from HIP events on the launch stream;
              traffic = HBM bytes per launch from FETCH_SIZE / WRITE_SIZE counters
              (profiles/traffic_*.txt), null when the kernel sources changed since
  cpu_baseline the fp64 CPU oracle timed on a bounded sample of rows of the same
              workload, scaled to the same unit
  check       GPU vs oracle on those sampled rows
  decode      (after a prefill workload) the decode workload c5b timed in the same run:
              GB/s over its own timed calls, kernel_ms from HIP events, HBM fraction

Algorithmic work: 2*D + 2*Dv FLOPs per visible (query row, key, head) triple (2*D for
QK^T, 2*Dv for PV); masked, padded and skipped pairs count nothing. Decode bytes: every valid
K and V element once, plus q, O and LSE.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

REPO = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, REPO)

METRIC = "attn fwd TFLOP/s & % MI355X bf16 MFMA peak; decode GB/s & % HBM peak"
PEAK_MFMA_TFLOPS = 2500.0   # MI355X dense bf16 / fp16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
DECODE = ("c5b",)

DESCRIPTION = {
    "c1": "non-causal MHA [1,257,8,128]",
    "c2": "non-causal MHA [1,20480,56,128] (video joint attention)",
    "c3": "varlen causal GQA 32/8 D128 + rel_bias E256, 8 seqs len U[512,8192]",
    "c3r": "c3 with the bias produced in the kernel from r [T,32,16] . rel_proj [16,256]",
    "c4a": "self-attention [256,10000,6,64]",
    "c4b": "feature attention [100,100000,4,16]",
    "c4c": "cross attention q[1,1000,6,64] k/v[1,1e6,6,64], split-KV heuristic",
    "c5a": "8:1 pack-GQA D256 q[4,1024,8,256] k/v[4,2048,1,256] seqused_k U[600,2048]",
    "c5b": "D256 decode q[32,1,8,256] k/v[32,131072,1,256] causal, split-KV + combine",
    "n1a": "cached prediction fp16 MQA 8:1 D64, q[1,16,8,64] k/v[1,300000,1,64], split-KV",
    "n1b": "cached prediction fp16 MQA 8:1 D64, q[1,64,8,64] k/v[1,300000,1,64], split-KV",
    "n1c": "cached prediction fp16 MQA 8:1 D64, q[1,256,8,64] k/v[1,300000,1,64], split-KV",
    "n2a": "non-causal MHA bf16 [2,8192,32,48] (head dim 48: class-64 tiles, 48-column arithmetic)",
    "n2b": "non-causal MHA bf16 [2,8192,32,72] (head dim 72: class-128 tiles, 96-column arithmetic)",
    "n2c": "non-causal MHA bf16 [2,8192,32,128] (head dim 128, for comparison)",
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def lengths(spec, x):
    if spec.varlen:
        ql = np.diff(x["cu_seqlens_q"].astype(np.int64))
        kl = np.diff(x["cu_seqlens_k"].astype(np.int64))
    else:
        ql = np.full(spec.B, spec.Sq, dtype=np.int64)
        kl = np.full(spec.B, spec.Sk, dtype=np.int64)
    if "seqused_k" in x:
        kl = x["seqused_k"].astype(np.int64)
    return ql, kl


def visible_keys(causal, ql, kl):
    """Visible keys of each query row of one sequence (bottom-right causal alignment)."""
    if not causal:
        return np.full(ql, kl, dtype=np.int64)
    return np.clip(np.arange(ql, dtype=np.int64) + (kl - ql) + 1, 0, kl)


def algorithmic_flops(spec, x):
    ql, kl = lengths(spec, x)
    pairs = sum(int(visible_keys(spec.causal, int(a), int(b)).sum()) for a, b in zip(ql, kl))
    return pairs * spec.Hq * (2 * spec.D + 2 * spec.Dv)


def algorithmic_bytes(spec, x):
    ql, kl = lengths(spec, x)
    kv = int(kl.sum()) * spec.Hkv * (spec.D + spec.Dv) * 2
    rows = int(ql.sum()) * spec.Hq
    return kv + rows * (spec.D * 2 + spec.Dv * 2 + 4)


def hbm_bound(spec, x):
    return algorithmic_flops(spec, x) < algorithmic_bytes(spec, x) * (PEAK_MFMA_TFLOPS * 1e12) / (PEAK_HBM_GBS * 1e9)


def kernel_source_hash():
    h = hashlib.sha256()
    csrc = os.path.join(REPO, "exact_attention_forward_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".hpp", ".h", ".cpp")):
            with open(os.path.join(csrc, f), "rb") as fh:
                h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def read_traffic(workload, dtype):
    """HBM bytes per launch from committed counter data, if taken on the current kernel sources."""
    path = os.path.join(REPO, "profiles", f"traffic_{workload}_{dtype}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if "=" in line and not line.startswith("#"):
                a, b = line.split("=", 1)
                kv[a.strip()] = b.strip()
    if kv.get("kernel_source_hash") != kernel_source_hash():
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


COPY_BYTES = 1 << 30  # bytes read and written by each calibration copy


def counter_means(run_dir, counter):
    """Per-dispatch values of one counter from a rocprofv3 --pmc run: (attention fwd, copies)."""
    import csv
    import glob
    files = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if len(files) != 1:
        raise SystemExit(f"expected one counter_collection.csv under {run_dir}, found {files}")
    fwd, other = [], []
    with open(files[0]) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            v = float(r["Counter_Value"]) * 1024.0  # the counter is in KiB
            (fwd if "attn_fwd_kernel" in r["Kernel_Name"] else other).append(
                (v, r["Kernel_Name"]))
    # the calibration copies are the three elementwise launches that move the most bytes
    copies = sorted(v for v, name in other if "elementwise" in name)[-3:]
    if not fwd or len(copies) != 3:
        raise SystemExit(f"{run_dir}: {len(fwd)} forward dispatches, {len(copies)} copies")
    return [v for v, _ in fwd], copies


def write_traffic(args, fetch_dir, write_dir):
    """profiles/traffic_<workload>_<dtype>.txt from a FETCH_SIZE run and a WRITE_SIZE run.

    Each counter is scaled by the ratio of the bytes a plain 1 GiB copy moves to what
    the same counter reads for it, so the figure is HBM-side bytes per forward launch.
    """
    from workloads import configs
    spec = configs.workload(args.workload, args.dtype)
    f_fwd, f_copy = counter_means(fetch_dir, "FETCH_SIZE")
    w_fwd, w_copy = counter_means(write_dir, "WRITE_SIZE")
    f_scale = COPY_BYTES / float(np.mean(f_copy))
    w_scale = COPY_BYTES / float(np.mean(w_copy))
    fetch = float(np.mean(f_fwd)) * f_scale
    write = float(np.mean(w_fwd)) * w_scale
    path = os.path.join(REPO, "profiles", f"traffic_{args.workload}_{spec.dtype}.txt")
    cmd = (f"python3 -u bench.py --no-cpu --decode-steps 0 --steps 3 --warmup 1 --workload {args.workload} "
           f"--dtype {spec.dtype} --copy-calibration")
    with open(path, "w") as f:
        f.write(f"# HBM traffic of attn_fwd_kernel per launch, {args.workload} "
                f"({DESCRIPTION[args.workload]}), {spec.dtype}\n")
        f.write(f"# counters: rocprofv3 --pmc FETCH_SIZE -- {cmd}\n")
        f.write(f"#           rocprofv3 --pmc WRITE_SIZE -- {cmd}\n")
        f.write("# scale = bytes of a plain 1 GiB elementwise copy / what the counter reads for it\n")
        f.write(f"fetch_dispatches = {len(f_fwd)}\n")
        f.write(f"fetch_raw_bytes_per_launch = {np.mean(f_fwd):.0f}\n")
        f.write(f"fetch_scale = {f_scale:.4f}\n")
        f.write(f"write_raw_bytes_per_launch = {np.mean(w_fwd):.0f}\n")
        f.write(f"write_scale = {w_scale:.4f}\n")
        f.write(f"fetch_bytes_per_launch = {fetch:.0f}\n")
        f.write(f"write_bytes_per_launch = {write:.0f}\n")
        f.write(f"hbm_bytes_per_launch = {fetch + write:.0f}\n")
        f.write(f"kernel_source_hash = {kernel_source_hash()}\n")
    print(open(path).read())


# SQ counter passes (one rocprofv3 --pmc run each: at most 8 SQ and 2 GRBM counters a pass)
COUNTER_PASSES = (
    "SQ_INSTS_VALU SQ_INSTS_MFMA SQ_INSTS_LDS SQ_INSTS_VALU_TRANS_F32 SQ_INSTS_SALU SQ_INSTS_VMEM "
    "SQ_WAVES GRBM_GUI_ACTIVE",
    "SQ_VALU_MFMA_BUSY_CYCLES SQ_ACTIVE_INST_VALU SQ_LDS_IDX_ACTIVE SQ_WAIT_INST_LDS SQ_WAVE_CYCLES "
    "SQ_WAIT_INST_ANY SQ_ACTIVE_INST_LDS SQ_BUSY_CYCLES GRBM_GUI_ACTIVE",
    "SQ_VALU_MFMA_COEXEC_CYCLES SQ_ACTIVE_INST_VALU2 SQ_WAIT_ANY SQ_ACTIVE_INST_ANY SQ_ACTIVE_INST_MISC "
    "SQ_ACTIVE_INST_SCA SQ_ACTIVE_INST_VALU GRBM_GUI_ACTIVE",
)


def _csv_rows(run_dir, suffix):
    import csv
    import glob
    files = glob.glob(os.path.join(run_dir, "**", "*" + suffix), recursive=True)
    if len(files) != 1:
        raise SystemExit(f"expected one *{suffix} under {run_dir}, found {files}")
    with open(files[0]) as f:
        return list(csv.DictReader(f))


def _simd_count(run_dir):
    for r in _csv_rows(run_dir, "agent_info.csv"):
        if r.get("Agent_Type") == "GPU":
            return int(r["Simd_Count"])
    return 1024


def pass_counters(run_dir):
    """Counter means over the forward-kernel dispatches of one --pmc run (the first, cold
    dispatch left out), plus each dispatch's duration."""
    per = {}
    for r in _csv_rows(run_dir, "counter_collection.csv"):
        if "attn_fwd_kernel" not in r["Kernel_Name"]:
            continue
        d = per.setdefault(int(r["Dispatch_Id"]), {"_ns": int(r["End_Timestamp"]) - int(r["Start_Timestamp"])})
        d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    ids = sorted(per)[1:] or sorted(per)
    if not ids:
        raise SystemExit(f"{run_dir}: no forward-kernel dispatch")
    names = {n for i in ids for n in per[i]}
    return {n: float(np.mean([per[i].get(n, 0.0) for i in ids])) for n in names}, len(ids)


def kernel_stats(trace_dir):
    rows = _csv_rows(trace_dir, "kernel_stats.csv")
    return [(r["Name"], int(r["Calls"]), float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
             float(r["MaxNs"]) / 1e3) for r in rows]


def timed_forward_us(trace_dir, steps):
    """Durations of the last `steps` forward-kernel dispatches (the timed calls) in us."""
    rows = _csv_rows(trace_dir, "kernel_trace.csv")
    fwd = sorted((int(r["Dispatch_Id"]), (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
                 for r in rows if "attn_fwd_kernel" in r["Kernel_Name"])
    return [d for _, d in fwd[-steps:]]


def write_summary(args):
    """profiles/attn_fwd_d<class>_<dtype>_<workload>.md from a kernel-trace run and the SQ
    counter passes of COUNTER_PASSES (no GPU run)."""
    from workloads import configs
    spec = configs.workload(args.workload, args.dtype)
    x = configs.make_inputs(spec)
    flops = algorithmic_flops(spec, x)
    nbytes = algorithmic_bytes(spec, x)
    trace_dir, pmc_dirs = args.summarize[0], args.summarize[1:]
    dclass = next(c for c in (16, 64, 128, 256) if max(spec.D, spec.Dv) <= c)
    name = f"attn_fwd_d{dclass}_{spec.dtype}_{args.workload}"
    wl = f"--workload {args.workload} --dtype {spec.dtype}"
    lines = [f"# {name}: {DESCRIPTION[args.workload]}", ""]
    lines += ["Commands, from the repository root with TMPDIR=/tmp (rocprofv3 writes CSV under -d):", "", "```"]
    lines.append(f"rocprofv3 --kernel-trace --stats --output-format csv -d {trace_dir} -o run -- "
                 f"python3 -u bench.py --no-cpu --decode-steps 0 --steps {args.steps} --warmup 3 {wl}")
    for i, d in enumerate(pmc_dirs):
        lines.append(f"rocprofv3 --pmc {COUNTER_PASSES[i]} --output-format csv -d {d} -o run -- "
                     f"python3 -u bench.py --no-cpu --decode-steps 0 --steps 3 --warmup 1 --warmup-seconds 0 {wl}")
    lines.append(f"python3 bench.py {wl} --steps {args.steps} --summarize {trace_dir} {' '.join(pmc_dirs)}")
    lines += ["```", ""]
    lines += ["Kernel statistics over every dispatch of the trace run (the first call, warm-up and "
              "timed calls):", "", "| kernel | calls | average us | min us | max us |", "|---|---|---|---|---|"]
    for n, c, a, mn, mx in kernel_stats(trace_dir):
        lines.append(f"| `{n[:110]}` | {c} | {a:.1f} | {mn:.1f} | {mx:.1f} |")
    t = timed_forward_us(trace_dir, args.steps)
    fwd_us = float(np.mean(t))
    lines += ["", f"The {len(t)} timed forward dispatches: mean {fwd_us:.1f} us (min {min(t):.1f}, max {max(t):.1f}).",
              f"Algorithmic work per call: {flops:.4g} FLOP (2*D + 2*Dv per visible (row, key, head)), "
              f"{nbytes:.4g} bytes (K and V of every valid key once, plus q, O, LSE).",
              f"Forward kernel alone: {flops / (fwd_us * 1e-6) / 1e12:.1f} TFLOP/s = "
              f"{flops / (fwd_us * 1e-6) / 1e12 / PEAK_MFMA_TFLOPS:.3f} of {PEAK_MFMA_TFLOPS:.0f} TFLOP/s; "
              f"{nbytes / (fwd_us * 1e-6) / 1e9:.0f} GB/s = {nbytes / (fwd_us * 1e-6) / 1e9 / PEAK_HBM_GBS:.3f} "
              f"of {PEAK_HBM_GBS:.0f} GB/s."]
    if pmc_dirs:
        simd = _simd_count(pmc_dirs[0])
        merged, derived = {}, {}
        for d in pmc_dirs:
            c, n = pass_counters(d)
            gui = c["GRBM_GUI_ACTIVE"] / 8.0  # summed over the 8 XCDs, which run in lockstep
            if "SQ_VALU_MFMA_COEXEC_CYCLES" in c:
                derived["coexec"] = c["SQ_VALU_MFMA_COEXEC_CYCLES"] / (gui * simd)
            if "SQ_VALU_MFMA_BUSY_CYCLES" in c:
                derived["mfma_busy"] = c["SQ_VALU_MFMA_BUSY_CYCLES"] / (gui * simd)
                derived["lds_wait"] = c["SQ_WAIT_INST_LDS"] / c["SQ_WAVE_CYCLES"]
                derived["any_wait"] = c["SQ_WAIT_INST_ANY"] / c["SQ_WAVE_CYCLES"]
                derived["clock"] = gui / c["_ns"]
                # SQ_ACTIVE_INST_VALU counts 4-cycle units (summed over waves, which cannot issue
                # VALU on one SIMD in the same cycle): the share of SIMD cycles issuing VALU
                derived["valu_active"] = 4.0 * c["SQ_ACTIVE_INST_VALU"] / (gui * simd)
            for kname, val in c.items():
                if kname != "_ns" and kname != "GRBM_GUI_ACTIVE":
                    merged[kname] = val
            merged.setdefault("GRBM_GUI_ACTIVE (per XCD)", gui)
        if "SQ_INSTS_MFMA" in merged and merged["SQ_INSTS_MFMA"] > 0:
            derived["valu_per_mfma"] = (merged["SQ_INSTS_VALU"] - merged["SQ_INSTS_MFMA"]) / merged["SQ_INSTS_MFMA"]
        elif "SQ_INSTS_VALU" in merged:
            derived["valu_per_mfma"] = float("inf")
        lines += ["", f"SQ counters per forward dispatch (mean over the dispatches after the first; {simd} SIMDs):",
                  "", "| counter | value |", "|---|---|"]
        for kname in sorted(merged):
            lines.append(f"| {kname} | {merged[kname]:.4g} |")
        lines += ["", "Derived:", ""]
        if "mfma_busy" in derived:
            lines.append(f"- MFMA busy: {derived['mfma_busy']:.3f} = SQ_VALU_MFMA_BUSY_CYCLES / "
                         f"(GRBM_GUI_ACTIVE / 8 x {simd} SIMDs)")
            lines.append(f"- LDS-wait share: {derived['lds_wait']:.3f} = SQ_WAIT_INST_LDS / SQ_WAVE_CYCLES "
                         f"(any wait: {derived['any_wait']:.3f} = SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES)")
            lines.append(f"- VALU active: {derived['valu_active']:.3f} = 4 x SQ_ACTIVE_INST_VALU / "
                         f"(GRBM_GUI_ACTIVE / 8 x {simd} SIMDs) (MFMA issue included)")
            lines.append(f"- shader clock while counting: {derived['clock']:.2f} GHz = GRBM_GUI_ACTIVE / 8 / "
                         f"dispatch duration")
        if "coexec" in derived and "mfma_busy" in derived:
            idle = 1.0 - (derived["mfma_busy"] + derived["valu_active"] - derived["coexec"])
            lines.append(f"- MFMA and VALU both busy: {derived['coexec']:.3f} = SQ_VALU_MFMA_COEXEC_CYCLES / "
                         f"(GRBM_GUI_ACTIVE / 8 x {simd} SIMDs); neither: {idle:.3f} "
                         f"(1 - MFMA busy - VALU active + both)")
        if "valu_per_mfma" in derived:
            lines.append(f"- VALU per MFMA: {derived['valu_per_mfma']:.2f} = (SQ_INSTS_VALU - SQ_INSTS_MFMA) / "
                         f"SQ_INSTS_MFMA")
        if "SQ_INSTS_VALU_TRANS_F32" in merged and merged.get("SQ_INSTS_VALU"):
            lines.append(f"- transcendental share of VALU: "
                         f"{merged['SQ_INSTS_VALU_TRANS_F32'] / merged['SQ_INSTS_VALU']:.3f}")
    tr = read_traffic(args.workload, spec.dtype)
    lines += ["", (f"HBM traffic per forward launch (FETCH_SIZE + WRITE_SIZE, calibrated): {tr:.4g} bytes "
                   f"(profiles/traffic_{args.workload}_{spec.dtype}.txt)") if tr is not None else
              "HBM traffic: not taken on these kernel sources."]
    lines += ["", f"Kernel sources hash {kernel_source_hash()}.", ""]
    path = os.path.join(REPO, "profiles", name + ".md")
    with open(path, "w") as f:
        f.write("\n".join(lines))
    print("\n".join(lines))


def graph_timing(fa, q, k, v, kw, steps, eager_ms_step, kernel_ms):
    """Microseconds per call: eager (the timed loop above), one call captured in a HIP
    graph and replayed back to back, and the kernels alone (events)."""
    import torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fa.attn_fwd(q, k, v, **kw)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fa.attn_fwd(q, k, v, **kw)
    torch.cuda.synchronize()
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        g.replay()
    torch.cuda.synchronize()
    graph_us = (time.perf_counter() - t0) * 1e6 / steps
    # the floor of either way of launching: a one-element fill kernel, launched directly
    # and as a captured one-kernel graph, back to back
    tiny = torch.zeros(1, device="cuda")
    n = max(steps, 200)

    def per_call_us(fn):
        for _ in range(10):
            fn()
        torch.cuda.synchronize()
        t = time.perf_counter()
        for _ in range(n):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t) * 1e6 / n

    eager_fill_us = per_call_us(lambda: tiny.fill_(1.0))
    g2 = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        tiny.fill_(0.0)
    torch.cuda.synchronize()
    with torch.cuda.graph(g2):
        tiny.fill_(1.0)
    torch.cuda.synchronize()
    graph_fill_us = per_call_us(g2.replay)
    return {"eager_us_per_call": eager_ms_step * 1e3, "graph_us_per_call": graph_us,
            "kernel_us_per_call": kernel_ms * 1e3, "fill_kernel_eager_us_per_call": eager_fill_us,
            "fill_kernel_graph_us_per_call": graph_fill_us}


def sample_rows(spec, x, n, seed=12345):
    """Deterministic sample of (b, h, i) rows spread over batches, heads and positions."""
    from workloads import gen
    ql, _ = lengths(spec, x)
    rng = gen.make_rng(seed)
    bs = np.nonzero(ql > 0)[0]
    b = rng.choice(bs, size=n)
    h = rng.integers(0, spec.Hq, size=n)
    i = (rng.random(n) * ql[b]).astype(np.int64)
    return np.stack([b, h, i], axis=1).astype(np.int32)


def cpu_baseline(spec, x, out, lse, target_s, threads):
    """Time the oracle on a bounded row sample; also compare those rows with the GPU result."""
    from oracle import oracle as oracle_mod
    from workloads import gen
    ql, kl = lengths(spec, x)
    kw = dict(dtype=spec.dtype, B=spec.B, Sq=spec.Sq, Sk=spec.Sk, Hq=spec.Hq, Hkv=spec.Hkv,
              D=spec.D, Dv=spec.Dv, scale=spec.scale, causal=spec.causal,
              cu_seqlens_q=x.get("cu_seqlens_q"), cu_seqlens_k=x.get("cu_seqlens_k"),
              seqused_k=x.get("seqused_k"), rel_bias=x.get("rel_bias"), threads=threads)
    if "rel_r" in x:  # fused producer: the oracle gets the bias r . rel_proj makes
        kw["rel_bias"] = oracle_mod.rel_bias_from_proj(x["rel_r"], x["rel_proj"], spec.dtype)
    cu = x.get("cu_seqlens_q")

    def row_flops(rows):
        tot = 0
        for b, _, i in rows:
            vk = visible_keys(spec.causal, int(ql[b]), int(kl[b]))
            tot += int(vk[i])
        return tot * (2 * spec.D + 2 * spec.Dv)

    n = max(threads, 8)
    rows = sample_rows(spec, x, n)
    t0 = time.perf_counter()
    oracle_mod.attn_rows(x["q"], x["k"], x["v"], rows=rows, **kw)
    dt = time.perf_counter() - t0
    n = int(min(200000, max(n, n * target_s / max(dt, 1e-3))))
    rows = sample_rows(spec, x, n, seed=777)
    t0 = time.perf_counter()
    o_ref, l_ref = oracle_mod.attn_rows(x["q"], x["k"], x["v"], rows=rows, **kw)
    dt = time.perf_counter() - t0
    flops = row_flops(rows)
    # compare the sampled rows with the GPU output
    b, h, i = (rows[:, c].astype(np.int64) for c in range(3))
    import torch
    if cu is not None:
        t = cu.astype(np.int64)[b] + i
        og = out.view(torch.int16)[torch.from_numpy(t).cuda(), torch.from_numpy(h).cuda()]
        lg = lse.cpu().numpy()[h, t]
    else:
        og = out.view(torch.int16)[torch.from_numpy(b).cuda(), torch.from_numpy(i).cuda(),
                                   torch.from_numpy(h).cuda()]
        lg = lse.cpu().numpy()[b, h, i]
    og = gen.bits_to_f32(og.cpu().numpy().view(np.uint16), spec.dtype).astype(np.float64)
    fin = np.isfinite(l_ref)
    check = {"rows": int(n),
             "o_max_abs_err": float(np.abs(og - o_ref).max()) if n else 0.0,
             "lse_max_abs_err": float(np.abs(lg[fin] - l_ref[fin]).max()) if fin.any() else 0.0}
    sample = (f"{n} (batch, head, query) rows drawn uniformly from the workload, each over all "
              f"of its visible keys ({flops / n:.3g} FLOP per row on average)")
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": sample, "seconds": round(dt, 3), "sample_flop": flops}, check


class Run:
    """One workload's inputs resident in HBM, its preallocated outputs, and its timings."""


def time_workload(workload, dtype, steps, warmup, warmup_seconds, copy_calibration=False, num_splits=None):
    """Generate the workload's synthetic inputs, copy them to the GPU, warm up, then time
    exactly `steps` calls (wall clock around all of them, HIP events around each one on
    the launch stream). `num_splits`, when given, replaces the workload's split request."""
    import torch

    import exact_attention_forward_amd as fa
    from workloads import configs

    r = Run()
    spec = configs.workload(workload, dtype)
    if num_splits is not None:
        spec.num_splits = num_splits
    log(f"generating {workload} ({DESCRIPTION[workload]}) {spec.dtype}")
    x = configs.make_inputs(spec)
    tdt = {"bf16": torch.bfloat16, "fp16": torch.float16}[spec.dtype]

    def dev16(a):
        return torch.from_numpy(a.view(np.int16)).cuda().view(tdt)

    q, k, v = dev16(x["q"]), dev16(x["k"]), dev16(x["v"])
    kw = dict(causal=spec.causal, scale=spec.scale, num_splits=spec.num_splits,
              pack_gqa=spec.pack_gqa)
    varlen = spec.varlen
    if varlen:
        kw.update(cu_seqlens_q=torch.from_numpy(x["cu_seqlens_q"]).cuda(),
                  cu_seqlens_k=torch.from_numpy(x["cu_seqlens_k"]).cuda(),
                  max_seqlen_q=x["max_seqlen_q"], max_seqlen_k=x["max_seqlen_k"])
    if "seqused_k" in x:
        kw["seqused_k"] = torch.from_numpy(x["seqused_k"]).cuda()
    if "rel_bias" in x:
        kw["rel_bias"] = dev16(x["rel_bias"])
    if "rel_r" in x:
        kw["rel_r"] = dev16(x["rel_r"])
        kw["rel_proj"] = dev16(x["rel_proj"])
    # preallocate everything: the timed calls allocate nothing
    out, lse = fa.attn_fwd(q, k, v, **kw)
    ns = fa.num_splits(spec.B, spec.Sq, spec.Sk, spec.Hq, spec.Hkv, spec.D, spec.Dv,
                       causal=spec.causal, is_varlen=varlen, max_seqlen_q=x.get("max_seqlen_q", 0),
                       max_seqlen_k=x.get("max_seqlen_k", 0), pack_gqa=spec.pack_gqa,
                       requested=spec.num_splits)
    ws = None
    if ns > 1:
        ws = torch.empty(fa.workspace_size(spec.B, spec.Sq, spec.Hq, spec.Dv, is_varlen=varlen,
                                           splits=ns), dtype=torch.uint8, device="cuda")
    kw.update(out=out, lse=lse, workspace=ws)
    torch.cuda.synchronize()

    if copy_calibration:
        src = torch.empty(1 << 29, dtype=torch.float16, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst
        log("copy calibration: 3 x elementwise copy of 1 GiB")

    t_w = time.perf_counter()
    n_warm = 0
    while n_warm < warmup or time.perf_counter() - t_w < warmup_seconds:
        fa.attn_fwd(q, k, v, **kw)
        n_warm += 1
        if n_warm % 16 == 0:
            torch.cuda.synchronize()  # keep the host from running ahead of the clock
    torch.cuda.synchronize()
    log(f"warm-up: {n_warm} untimed steps in {time.perf_counter() - t_w:.2f} s")
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e0, e1 in ev:
        e0.record(stream)
        fa.attn_fwd(q, k, v, **kw)
        e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_call_ms = [e0.elapsed_time(e1) for e0, e1 in ev]
    r.spec, r.x, r.q, r.k, r.v, r.kw, r.out, r.lse = spec, x, q, k, v, kw, out, lse
    r.varlen, r.ns, r.n_warm = varlen, ns, n_warm
    r.ms_step = wall * 1e3 / steps
    r.mean_call_ms = float(np.mean(per_call_ms))
    return r


def decode_summary(r):
    """The decode sub-object: HBM-bound split-KV forward + combine."""
    nbytes = algorithmic_bytes(r.spec, r.x)
    achieved = nbytes / (r.mean_call_ms * 1e-3) / 1e9
    return {"workload": f"c5b: {DESCRIPTION['c5b']}", "value": nbytes / (r.ms_step * 1e-3) / 1e9,
            "unit": "GB/s", "ms_per_step": r.ms_step, "kernel_ms": r.mean_call_ms,
            "achieved": achieved, "peak": PEAK_HBM_GBS, "frac": achieved / PEAK_HBM_GBS,
            "algorithmic_bytes": nbytes, "num_splits": r.ns, "kernels_per_launch": 2 if r.ns > 1 else 1,
            "dtype": r.spec.dtype}


def _parse_smi_power(text):
    """Socket power (W) and per-XCD GFX clocks (MHz) from one `amd-smi metric -p -c` sample."""
    import re
    power, clocks, gfx = None, [], False
    for line in text.splitlines():
        m = re.match(r"\s*SOCKET_POWER:\s*([0-9.]+)\s*W", line)
        if m:
            power = float(m.group(1))
            continue
        if re.match(r"\s*GFX_\d+:\s*$", line):
            gfx = True
            continue
        if re.match(r"\s*[A-Z][A-Z0-9_]*:\s*$", line):
            gfx = False  # another clock domain (memory, video, ...)
            continue
        m = re.match(r"\s*CLK:\s*([0-9.]+)\s*MHz", line)
        if gfx and m:
            clocks.append(float(m.group(1)))
    return power, clocks


def power_run(fa, q, k, v, kw, seconds, path, workload, dtype):
    """Keep calling the forward for `seconds` while a child process takes `amd-smi metric -p -c`
    samples (socket power and GFX clocks); write the samples and their means to `path`."""
    import shutil
    import subprocess
    import torch
    if shutil.which("amd-smi") is None:
        raise SystemExit("bench.py --power needs amd-smi on PATH")
    cmd = ["amd-smi", "metric", "-p", "-c", "-g", "0"]
    torch.cuda.synchronize()
    time.sleep(3.0)  # the readings are averages over about a second: let the load fade first
    idle = subprocess.run(cmd, capture_output=True, text=True, timeout=60).stdout
    samples = []
    t0 = time.perf_counter()
    child, t_last = None, t0
    calls = 0
    while time.perf_counter() - t0 < seconds:
        now = time.perf_counter()
        # one sample a second (the readings refresh about that often), from the second second on
        if child is None and now - t0 > 1.0 and now - t_last >= 1.0:
            child, t_last = subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                                             text=True), now
        elif child is not None and child.poll() is not None:
            samples.append(_parse_smi_power(child.stdout.read()))
            child = None
        fa.attn_fwd(q, k, v, **kw)
        calls += 1
        if calls % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    if child is not None:
        child.wait()
    p_idle, c_idle = _parse_smi_power(idle)
    good = [(p, c) for p, c in samples if p is not None and c]
    with open(path, "w") as f:
        f.write(f"# socket power and GFX clocks while {workload} ({DESCRIPTION[workload]}, {dtype}) runs back to back\n")
        f.write(f"# command: python3 bench.py --no-cpu --decode-steps 0 --workload {workload} --dtype {dtype} "
                f"--power {os.path.relpath(path, REPO)}\n")
        f.write("# sampler: amd-smi metric -p -c -g 0 in a child process, one sample a second from the "
                "second second of load on; idle = 3 s after the timed steps, before this load\n")
        f.write(f"idle_socket_power_w = {p_idle}\n")
        for i, (p, c) in enumerate(good):
            f.write(f"sample_{i} = socket_power_w {p:.0f}, gfx_clock_mhz mean {np.mean(c):.0f} "
                    f"min {min(c):.0f} max {max(c):.0f} over {len(c)} XCDs\n")
        if good:
            f.write(f"mean_socket_power_w = {np.mean([p for p, _ in good]):.0f}\n")
            f.write(f"mean_gfx_clock_mhz = {np.mean([np.mean(c) for _, c in good]):.0f}\n")
        f.write(f"calls = {calls}\n")
    log(open(path).read())


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--warmup-seconds", type=float, default=1.0,
                    help="keep warming up (untimed steps) until this much time has passed as well: "
                         "the GPU needs some hundred milliseconds of load to reach its steady clocks, "
                         "longer than a few steps of a sub-millisecond call")
    ap.add_argument("--workload", default="c2", choices=sorted(DESCRIPTION))
    ap.add_argument("--dtype", default=None, choices=["bf16", "fp16"])
    ap.add_argument("--num-splits", type=int, default=None,
                    help="replace the workload's split request (0 = the heuristic); traffic is then null")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target wall time of the oracle sample")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle leg (profiling runs)")
    ap.add_argument("--decode-steps", type=int, default=100,
                    help="timed calls of the decode workload (c5b) reported in the line's 'decode' "
                         "object after a prefill workload; 0 skips it (profiling runs)")
    ap.add_argument("--graph", action="store_true",
                    help="also time the call captured in a HIP graph and replayed (host "
                         "dispatch overhead: eager vs graph microseconds per call)")
    ap.add_argument("--power", metavar="FILE",
                    help="after the timed steps, keep calling the forward for --power-seconds while "
                         "amd-smi samples socket power and GFX clocks; write them to FILE")
    ap.add_argument("--power-seconds", type=float, default=8.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB elementwise copy (counter calibration)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="no GPU run: turn the counter CSVs of two rocprofv3 --pmc runs of "
                         "bench.py --copy-calibration (FETCH_SIZE, then WRITE_SIZE) into "
                         "profiles/traffic_<workload>_<dtype>.txt")
    ap.add_argument("--summarize", nargs="+", metavar="DIR",
                    help="no GPU run: write profiles/attn_fwd_d<class>_<dtype>_<workload>.md from a "
                         "rocprofv3 --kernel-trace --stats run (first DIR) and --pmc runs of the "
                         "counter passes in order (further DIRs); --steps = the trace run's timed calls")
    args = ap.parse_args()
    if args.summarize:
        write_summary(args)
        return
    if args.traffic_from:
        write_traffic(args, *args.traffic_from)
        return
    if args.gpus != 1:
        print(f"bench.py: measures one GPU only (asked for {args.gpus}); the path would "
              "shard over (batch, KV head) with no exchange, or over the key range with one "
              "LSE combine step", file=sys.stderr)
        sys.exit(2)

    import torch

    import exact_attention_forward_amd as fa

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    fa.load()
    r = time_workload(args.workload, args.dtype, args.steps, args.warmup, args.warmup_seconds,
                      args.copy_calibration, args.num_splits)
    spec, x, q, k, v, kw, out, lse = r.spec, r.x, r.q, r.k, r.v, r.kw, r.out, r.lse
    varlen, ns, n_warm, ms_step, mean_call_ms = r.varlen, r.ns, r.n_warm, r.ms_step, r.mean_call_ms

    flops = algorithmic_flops(spec, x)
    # the bound follows the arithmetic intensity: below the machine balance (MFMA peak /
    # HBM peak, about 312 FLOP per byte) the algorithmic bytes cannot arrive faster than HBM
    # delivers them (decode, the short-query cached prediction), above it the MFMAs bound
    decode = args.workload in DECODE or hbm_bound(spec, x)
    if decode:
        nbytes = algorithmic_bytes(spec, x)
        value = nbytes / (ms_step * 1e-3) / 1e9
        unit = "GB/s"
        achieved = nbytes / (mean_call_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": achieved / PEAK_HBM_GBS}
    else:
        value = flops / (ms_step * 1e-3) / 1e12
        unit = "TFLOP/s"
        achieved = flops / (mean_call_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": PEAK_MFMA_TFLOPS, "unit": "TFLOP/s",
                "frac": achieved / PEAK_MFMA_TFLOPS}
    # the counters behind the traffic figure were taken at the workload's own split request
    roof["traffic"] = read_traffic(args.workload, spec.dtype) if args.num_splits is None else None
    roof["kernel_ms"] = mean_call_ms
    roof["kernels_per_launch"] = 2 if ns > 1 else 1
    log(f"{args.workload}: {ms_step:.4f} ms/step wall, {mean_call_ms:.4f} ms/call events, "
        f"{flops:.4g} FLOP, splits={ns}")

    result = {
        "metric": METRIC, "value": value, "unit": unit, "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "warmup_steps_run": n_warm, "ms_per_step": ms_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": spec.dtype, "data": "synthetic",
        "config": {"workload": f"{args.workload}: {DESCRIPTION[args.workload]}", "B": spec.B,
                   "Sq": spec.Sq, "Sk": spec.Sk, "Hq": spec.Hq, "Hkv": spec.Hkv, "D": spec.D,
                   "causal": spec.causal, "varlen": varlen, "rel_extent": spec.rel_extent,
                   "num_splits": ns, "algorithmic_flop": flops, "seed": spec.seed,
                   "parallelism": "single GPU"},
        "roofline": roof,
    }
    if args.power:
        power_run(fa, q, k, v, kw, args.power_seconds, os.path.abspath(args.power), args.workload, spec.dtype)
    if args.graph:
        result["dispatch"] = graph_timing(fa, q, k, v, kw, args.steps, ms_step, mean_call_ms)
        log(f"dispatch: {result['dispatch']}")
    if not args.no_cpu:
        threads = min(16, os.cpu_count() or 1)
        cb, check = cpu_baseline(spec, x, out, lse, args.cpu_seconds, threads)
        if decode:
            # the sample's share of the algorithmic bytes, by its share of the visible pairs
            cb["value"] = nbytes * (cb["sample_flop"] / flops) / cb["seconds"] / 1e9
            cb["unit"] = "GB/s"
        result["cpu_baseline"] = cb
        result["check"] = check
    if args.workload not in DECODE and args.decode_steps > 0:
        # the metric's decode half, measured in the same run on its own inputs
        del r, q, k, v, kw, out, lse, x
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        rd = time_workload(DECODE[0], None, args.decode_steps, args.warmup, args.warmup_seconds)
        result["decode"] = decode_summary(rd)
        log(f"decode {DECODE[0]}: {rd.ms_step:.4f} ms/step wall, {rd.mean_call_ms:.4f} ms/call events, "
            f"{result['decode']['frac']:.3f} of HBM peak")
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
