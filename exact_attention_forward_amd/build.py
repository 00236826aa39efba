"""Build libmi355attn.so (gfx950) in-tree with hipcc.

Every .hip / .cpp under csrc/ is compiled to an object in parallel, then
linked into exact_attention_forward_amd/libmi355attn.so.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmi355attn.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# -packed-fp32-ops: no v_pk_{add,mul,fma}_f32 are generated; some of their forms
#   have given wrong results on gfx950 now and then, with no error
# max-ilp scheduling: LDS operands are read well ahead of the MFMAs that use them
#   (the default strategy trades that latency hiding for registers the kernels do
#   not need at their occupancy)
COMMON = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-mllvm", "-amdgpu-sched-strategy=max-ilp",
          "-I" + os.path.join(os.path.dirname(HERE), "include")]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


# per-kernel register, spill, occupancy and LDS figures the compiler reports, kept beside
# the objects (tests/test_kernel_resources.py reads them)
RESOURCES = os.path.join(BUILD, "kernel_resources.txt")


def _resources(stderr: str) -> list[str]:
    """'<kernel> <key>: <value>' lines from the compiler's kernel-resource-usage remarks."""
    out, name = [], None
    for line in stderr.splitlines():
        if "[-Rpass-analysis=kernel-resource-usage]" not in line or "remark:" not in line:
            continue
        body = line.split("remark:", 1)[1].replace("[-Rpass-analysis=kernel-resource-usage]", "").strip()
        if body.startswith("Function Name:"):
            name = body.split(":", 1)[1].strip()
        elif name and ":" in body:
            out.append(f"{name} {body}")
    return out


def _compile(src: str) -> tuple[str, list[str]]:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    extra = ["-Rpass-analysis=kernel-resource-usage"] if src.endswith(".hip") else []
    cmd = [HIPCC] + COMMON + extra + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj, _resources(r.stderr)


def build(jobs: int = 8, verbose: bool = False) -> str:
    """Compile every source (always) and link the shared library. Returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        done = list(ex.map(_compile, srcs))
    objs = [o for o, _ in done]
    with open(RESOURCES, "w") as f:
        for _, lines in done:
            for line in lines:
                f.write(line + "\n")
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(jobs=int(sys.argv[1]) if len(sys.argv) > 1 else 8, verbose=True)
