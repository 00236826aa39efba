"""attn_fwd_rel_proj: the relative bias produced inside the kernel from r and rel_proj.

Checked against the oracle run with the bias that r . rel_proj makes (summed in
fp64, stored in the dtype), and against attn_fwd fed that materialised bias.
"""
import numpy as np
import pytest
import torch

import exact_attention_forward_amd as fa
from tests.gpu_common import Case, dev16, full_check, host_f64, say
from workloads import gen

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    fa.load()


def case(seed, *, dtype, qls, kls, Hq, Hkv, D, Dv, d_rel, E, causal, num_splits=1):
    rng = gen.make_rng(seed)
    cu_q, cu_k = gen.cu_seqlens(qls), gen.cu_seqlens(kls)
    Tq, Tk = int(cu_q[-1]), int(cu_k[-1])
    q = gen.normal_bits(rng, (Tq, Hq, D), dtype)
    k = gen.normal_bits(rng, (Tk, Hkv, D), dtype)
    v = gen.normal_bits(rng, (Tk, Hkv, Dv), dtype)
    r = gen.normal_bits(rng, (Tq, Hq, d_rel), dtype)
    pj = gen.normal_bits(rng, (d_rel, E), dtype, 0.5 / np.sqrt(d_rel))
    return Case(dtype=dtype, B=len(qls), Sq=Tq, Sk=Tk, Hq=Hq, Hkv=Hkv, D=D, Dv=Dv, causal=causal,
                q=q, k=k, v=v, cu_q=cu_q, cu_k=cu_k, max_q=max(1, max(qls)), max_k=max(1, max(kls)),
                num_splits=num_splits, rel_r=r, rel_proj=pj,
                name=f"rel_proj {dtype} D{D} Dv{Dv} d_rel{d_rel} E{E} causal={causal}")


@pytest.mark.parametrize("dtype,D,Dv,d_rel,E,causal,splits", [
    ("bf16", 128, 128, 16, 256, True, 1),
    ("fp16", 128, 128, 8, 128, True, 1),
    ("bf16", 64, 64, 40, 384, True, 3),
    ("bf16", 72, 48, 64, 128, False, 1),
    ("fp16", 16, 16, 24, 256, True, 0),
    ("bf16", 256, 256, 16, 128, True, 1),
    ("bf16", 128, 128, 16, 512, True, 1),
    ("fp16", 256, 200, 32, 384, False, 1),
])
def test_fused_bias_matches_oracle_and_materialised(dtype, D, Dv, d_rel, E, causal, splits):
    c = case(8100 + D + d_rel + E, dtype=dtype, qls=[300, 0, 130, 517], kls=[300, 40, 200, 517],
             Hq=8, Hkv=2, D=D, Dv=Dv, d_rel=d_rel, E=E, causal=causal, num_splits=splits)
    out_f, lse_f = c.run_gpu()
    full_check(c, out_lse=(out_f, lse_f))
    # the same call with the materialised bias: equal up to the rounding of ties
    rr, pp = c.rel_r, c.rel_proj
    c.rel_r = None
    out_m, lse_m = c.run_gpu()
    c.rel_r = rr
    d_o = np.abs(host_f64(out_f, dtype) - host_f64(out_m, dtype)).max()
    fin = torch.isfinite(lse_m)
    d_l = (lse_f[fin] - lse_m[fin]).abs().max().item() if fin.any() else 0.0
    say(f"  fused vs materialised: O max diff {d_o:.3e}, LSE max diff {d_l:.3e}")
    assert d_o <= 5e-3 and d_l <= 1e-3
