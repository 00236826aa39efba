"""Compiler-reported resources of the forward kernels the benchmark workloads run.

The build keeps the compiler's kernel-resource-usage figures in
exact_attention_forward_amd/_build/kernel_resources.txt. The instances checked here must
spill no scalar registers and keep two waves per SIMD where the tile geometry relies on it:
a scalar spill lands in a vector lane and costs a VALU instruction at each use. One such
regression (masked-tile visibility compares formed ahead of the tile-kind branch, with the
masks kept in spilled scalar pairs) made the head-dim-16 fp16 forward 27% slower.
"""
import os
import re

import pytest

RES = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "exact_attention_forward_amd", "_build", "kernel_resources.txt")


def _kernel(D, bf16, causal=False, varlen=False, bias=False, split=False, dsplit=False, W=None):
    b = lambda x: "Lb1E" if x else "Lb0E"  # noqa: E731
    return (f"_ZN9mi355attn15attn_fwd_kernelILi{D}E{b(bf16)}{b(causal)}{b(varlen)}{b(bias)}{b(split)}"
            f"{b(dsplit)}Li{W or D}EEEvNS_9FwdParamsE")


def _load():
    if not os.path.exists(RES):
        pytest.skip("no resource report: build the library with exact_attention_forward_amd.build")
    res = {}
    for line in open(RES):
        m = re.match(r"(\S+) (.+?): (\S+)", line.strip())
        if m:
            res.setdefault(m.group(1), {})[m.group(2)] = m.group(3)
    return res


# (kernel, waves per SIMD it is built for): the dense bf16 D128 prefill, fp16 D64 and D16
# (tabular), bf16 D256 pack-GQA prefill, and the varlen causal GQA + bias prefill
CASES = [
    (_kernel(128, True), 2),
    (_kernel(64, False), 2),
    (_kernel(16, False), 2),
    (_kernel(256, True), 1),
    (_kernel(128, True, causal=True, varlen=True), 2),
]


@pytest.mark.parametrize("name,waves", CASES, ids=[c[0][30:80] for c in CASES])
def test_benchmarked_instances_spill_no_scalars(name, waves):
    res = _load()
    assert name in res, f"{name} missing from the resource report"
    r = res[name]
    assert int(r["SGPRs Spill"]) == 0, f"{name}: {r['SGPRs Spill']} scalar registers spilled"
    assert int(r["Occupancy [waves/SIMD]"]) >= waves, f"{name}: occupancy {r['Occupancy [waves/SIMD]']}"


def test_report_covers_every_forward_instance():
    res = _load()
    fwd = [n for n in res if n.startswith("_ZN9mi355attn15attn_fwd_kernel")]
    # classes 16, 64, 128: 32 instances each (dtype x causal x varlen x bias x split); class
    # 256 also has the decode form with the O columns split over the waves (64); the three
    # narrowed sets (96, 48, 192 columns) 32 each
    assert len(fwd) == 3 * 32 + 64 + 3 * 32, len(fwd)


def test_combine_kernels_spill_nothing():
    """Both split-KV merges (a work-group per row, a wave per row), every class and dtype."""
    res = _load()
    names = [n for n in res if re.search(r"attn_combine(_rows)?_kernel", n)]
    assert len(names) == 2 * 4 * 2, names  # two kernels x classes 16/64/128/256 x bf16/fp16
    for n in names:
        assert int(res[n]["SGPRs Spill"]) == 0, n
        assert int(res[n]["VGPRs Spill"]) == 0, n
