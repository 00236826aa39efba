"""Benchmark of the MI355X exact attention forward (one JSON line on stdout).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c2] [--dtype bf16]

A step is one full forward call (attn_fwd: the fused kernel, plus the combine
kernel when the key range is split) over one batch of synthetic inputs that is
already resident in HBM. The default workload is the non-causal MHA forward
q/k/v [1, 20480, 56, 128] in bf16 (video joint-attention shape).

Reported:
  value       whole-job TFLOP/s (GB/s for the decode workload) over the K timed steps
  roofline    achieved / peak of the dominant kernel: algorithmic FLOPs (or bytes) per
              launch / its mean duration from HIP events on the launch stream;
              traffic = HBM bytes per launch from FETCH_SIZE / WRITE_SIZE counters
              (profiles/traffic_*.txt), null when the kernel sources changed since
  cpu_baseline the fp64 CPU oracle timed on a bounded sample of rows of the same
              workload, scaled to the same unit
  check       GPU vs oracle on those sampled rows

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
    cmd = (f"python -u bench.py --no-cpu --steps 3 --warmup 1 --workload {args.workload} "
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
    return {"eager_us_per_call": eager_ms_step * 1e3, "graph_us_per_call": graph_us,
            "kernel_us_per_call": kernel_ms * 1e3}


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
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target wall time of the oracle sample")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle leg (profiling runs)")
    ap.add_argument("--graph", action="store_true",
                    help="also time the call captured in a HIP graph and replayed (host "
                         "dispatch overhead: eager vs graph microseconds per call)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB elementwise copy (counter calibration)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="no GPU run: turn the counter CSVs of two rocprofv3 --pmc runs of "
                         "bench.py --copy-calibration (FETCH_SIZE, then WRITE_SIZE) into "
                         "profiles/traffic_<workload>_<dtype>.txt")
    args = ap.parse_args()
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
    from workloads import configs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    fa.load()
    spec = configs.workload(args.workload, args.dtype)
    log(f"generating {args.workload} ({DESCRIPTION[args.workload]}) {spec.dtype}")
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

    if args.copy_calibration:
        src = torch.empty(1 << 29, dtype=torch.float16, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        log("copy calibration: 3 x elementwise copy of 1 GiB")

    t_w = time.perf_counter()
    n_warm = 0
    while n_warm < args.warmup or time.perf_counter() - t_w < args.warmup_seconds:
        fa.attn_fwd(q, k, v, **kw)
        n_warm += 1
        if n_warm % 16 == 0:
            torch.cuda.synchronize()  # keep the host from running ahead of the clock
    torch.cuda.synchronize()
    log(f"warm-up: {n_warm} untimed steps in {time.perf_counter() - t_w:.2f} s")
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e0, e1 in ev:
        e0.record(stream)
        fa.attn_fwd(q, k, v, **kw)
        e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_call_ms = [e0.elapsed_time(e1) for e0, e1 in ev]
    ms_step = wall * 1e3 / args.steps
    mean_call_ms = float(np.mean(per_call_ms))

    flops = algorithmic_flops(spec, x)
    decode = args.workload in DECODE
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
    roof["traffic"] = read_traffic(args.workload, spec.dtype)
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
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
