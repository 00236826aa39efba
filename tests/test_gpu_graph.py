"""attn_fwd captured in a HIP graph (through torch.cuda.CUDAGraph) and replayed.

The call is stream-ordered, launches only kernels (no memset, no allocation, no
host synchronisation) when out / lse / workspace are passed in, so a capture
holds the forward kernel (and the combine kernel for a split key range). Each
replay is compared bit for bit with the eager call, with eager work and
synchronisations between the replays.
"""
import numpy as np
import pytest
import torch

import exact_attention_forward_amd as fa
from tests.gpu_common import dev16, full_check, Case, say
from workloads import gen

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    fa.load()


def _inputs(dtype, B, Sq, Sk, Hq, Hkv, D, seed):
    rng = gen.make_rng(seed)
    q = gen.normal_bits(rng, (B, Sq, Hq, D), dtype)
    k = gen.normal_bits(rng, (B, Sk, Hkv, D), dtype)
    v = gen.normal_bits(rng, (B, Sk, Hkv, D), dtype)
    return q, k, v


@pytest.mark.parametrize("shape", [
    # dtype, B, Sq, Sk, Hq, Hkv, D, causal, num_splits
    ("bf16", 1, 257, 257, 8, 8, 128, False, 1),
    ("fp16", 1, 16, 20000, 8, 1, 64, False, 0),    # short query, split key range + combine
    ("bf16", 2, 1, 9000, 8, 1, 256, True, 0),      # decode
])
def test_graph_replays_match_eager(shape):
    dtype, B, Sq, Sk, Hq, Hkv, D, causal, ns_req = shape
    qb, kb, vb = _inputs(dtype, B, Sq, Sk, Hq, Hkv, D, seed=4242 + D)
    q, k, v = dev16(qb, dtype), dev16(kb, dtype), dev16(vb, dtype)
    scale = float(np.float32(1.0 / np.sqrt(D)))
    ns = fa.num_splits(B, Sq, Sk, Hq, Hkv, D, D, causal=causal, requested=ns_req)
    ws_bytes = fa.workspace_size(B, Sq, Hq, D, splits=ns)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(q)
    lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device="cuda")
    kw = dict(causal=causal, scale=scale, num_splits=ns, out=out, lse=lse, workspace=ws)
    say(f"  graph case {shape}: splits={ns} workspace={ws_bytes} B")

    fa.attn_fwd(q, k, v, **kw)
    torch.cuda.synchronize()
    o_ref, l_ref = out.clone(), lse.clone()

    # warm-up on a side stream, as capture requires, then capture one call
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

    for rep in range(4):
        out.fill_(float("nan"))
        lse.fill_(0.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), o_ref.view(torch.int16)), f"replay {rep}: O differs"
        assert torch.equal(lse, l_ref), f"replay {rep}: LSE differs"
        # eager work on the same buffers between replays
        fa.attn_fwd(q, k, v, **kw)
        torch.cuda.synchronize()

    # and the eager result itself is right (small enough for the full oracle)
    if B * Sq * Hq * Sk <= 20_000_000:
        c = Case(dtype=dtype, B=B, Sq=Sq, Sk=Sk, Hq=Hq, Hkv=Hkv, D=D, scale=scale, causal=causal,
                 q=qb, k=kb, v=vb, num_splits=ns, name=f"graph {shape}")
        full_check(c, out_lse=(o_ref, l_ref))
