"""Results do not depend on what else runs on the GPU.

Each case runs alone, then again while a large forward call on a second stream (default
priority) competes for the compute units, so its work-groups land on other CUs, in another
order and next to other work-groups; the two results must be bitwise equal. A kernel that
read LDS or workspace data another work-group (or an earlier call) left behind, or that
depended on the order work-groups run in, would differ.
"""
import numpy as np
import pytest
import torch

import exact_attention_forward_amd as fa
from tests.gpu_common import dev16, dev_i32, random_case, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    fa.load()


CASES = [
    dict(name="varlen causal bias", seed=961, dtype="bf16", B=0, Sq=0, Sk=0, Hq=8, Hkv=2, D=128, causal=True,
         lens=([300, 77, 1000, 5], [300, 77, 1000, 5]), E=128, splits=1),
    dict(name="dense split", seed=962, dtype="fp16", B=2, Sq=90, Sk=3000, Hq=4, Hkv=1, D=64, causal=False,
         splits=6),
    dict(name="dense D128 pipelined", seed=963, dtype="bf16", B=1, Sq=700, Sk=900, Hq=4, Hkv=4, D=128,
         causal=False, splits=1),
    dict(name="decode D256", seed=964, dtype="bf16", B=4, Sq=1, Sk=5000, Hq=8, Hkv=1, D=256, causal=True,
         splits=0),
]


def _kw(c, ns):
    kw = dict(causal=c.causal, scale=c.scale, num_splits=ns)
    if c.varlen:
        kw.update(cu_seqlens_q=dev_i32(c.cu_q), cu_seqlens_k=dev_i32(c.cu_k), max_seqlen_q=int(c.max_q),
                  max_seqlen_k=int(c.max_k))
    if c.bias is not None:
        kw["rel_bias"] = dev16(c.bias, c.dtype)
    return kw


@pytest.mark.parametrize("cfg", CASES, ids=[c["name"] for c in CASES])
def test_bitwise_under_contention(cfg):
    c = random_case(cfg["seed"], dtype=cfg["dtype"], B=cfg["B"], Sq=cfg["Sq"], Sk=cfg["Sk"], Hq=cfg["Hq"],
                    Hkv=cfg["Hkv"], D=cfg["D"], causal=cfg["causal"], varlen_lens=cfg.get("lens"),
                    E=cfg.get("E", 0), name="race " + cfg["name"])
    q, k, v = dev16(c.q, c.dtype), dev16(c.k, c.dtype), dev16(c.v, c.dtype)
    ns = fa.num_splits(c.B, c.Sq, c.Sk, c.Hq, c.Hkv, c.D, c.Dv, causal=c.causal, is_varlen=c.varlen,
                       max_seqlen_q=int(c.max_q or 0), max_seqlen_k=int(c.max_k or 0), requested=cfg["splits"])
    out1, lse1 = fa.attn_fwd(q, k, v, **_kw(c, ns))
    torch.cuda.synchronize()
    # background: a dense non-causal forward of a few milliseconds on its own stream
    g = torch.Generator(device="cpu").manual_seed(965)
    bq = torch.randn(1, 8192, 16, 128, generator=g).to(torch.bfloat16).cuda()
    bk = torch.randn(1, 8192, 16, 128, generator=g).to(torch.bfloat16).cuda()
    bv = torch.randn(1, 8192, 16, 128, generator=g).to(torch.bfloat16).cuda()
    bout = torch.empty_like(bq)
    side = torch.cuda.Stream()
    main = torch.cuda.current_stream()
    side.wait_stream(main)
    for rep in range(3):
        out2 = torch.full_like(out1, 5.0)
        lse2 = torch.full_like(lse1, 5.0)
        kw = dict(_kw(c, ns), out=out2, lse=lse2)
        say(f"  GPU {c.name}: repeat {rep} beside a [1,8192,16,128] forward on a second stream")
        with torch.cuda.stream(side):
            fa.attn_fwd(bq, bk, bv, out=bout)
        fa.attn_fwd(q, k, v, **kw)
        torch.cuda.synchronize()
        assert torch.equal(out2.view(torch.int16), out1.view(torch.int16)), f"{c.name}: O differs (repeat {rep})"
        assert torch.equal(lse2.view(torch.int32), lse1.view(torch.int32)), f"{c.name}: LSE differs (repeat {rep})"
    assert np.isfinite(bout.float().cpu().numpy()).all()
