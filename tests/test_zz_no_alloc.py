"""attn_fwd_noalloc (the entry point that allocates nothing) against attn_fwd.

Two calls in a row through the C ABI, the second on a smaller input with a different
split count and partial layout, each compared bitwise with attn_fwd given its own
workspace and the same split count (the same kernels over the same partials), and
within the tolerance of the oracle. Then a call that needs no split, a decode call
with the heuristic's split count, and a call whose partials exceed the library's
array, which must be refused before anything is written.
"""
import numpy as np
import pytest
import torch

import exact_attention_forward_amd as fa
from tests.gpu_common import check_lse, check_o, dev16, dev_i32, host_f64, random_case, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    fa.load()


def _kw(c, ns):
    kw = dict(causal=c.causal, scale=c.scale, pack_gqa=c.pack_gqa, num_splits=ns)
    if c.varlen:
        kw.update(cu_seqlens_q=dev_i32(c.cu_q), cu_seqlens_k=dev_i32(c.cu_k), max_seqlen_q=int(c.max_q),
                  max_seqlen_k=int(c.max_k))
    if c.seqused is not None:
        kw["seqused_k"] = dev_i32(c.seqused)
    if c.bias is not None:
        kw["rel_bias"] = dev16(c.bias, c.dtype)
    return kw


def _splits(c, requested):
    return fa.num_splits(c.B, c.Sq, c.Sk, c.Hq, c.Hkv, c.D, c.Dv, causal=c.causal, is_varlen=c.varlen,
                         max_seqlen_q=int(c.max_q or 0), max_seqlen_k=int(c.max_k or 0), pack_gqa=c.pack_gqa,
                         requested=requested)


def _out_shapes(c):
    if c.varlen:
        return (c.Sq, c.Hq, c.Dv), (c.Hq, c.Sq)
    return (c.B, c.Sq, c.Hq, c.Dv), (c.B, c.Hq, c.Sq)


def _compare(c, requested, *, expect_split):
    """attn_fwd_noalloc vs attn_fwd (bitwise) and vs the oracle; returns the split count."""
    ns = _splits(c, requested)
    assert (ns > 1) == expect_split, (c.name, ns)
    n_ws = fa.workspace_size(c.B, c.Sq, c.Hq, c.Dv, is_varlen=c.varlen, splits=ns)
    assert n_ws <= fa.SCRATCH_BYTES, (c.name, n_ws)
    q, k, v = dev16(c.q, c.dtype), dev16(c.k, c.dtype), dev16(c.v, c.dtype)
    kw = _kw(c, ns)
    o_shape, l_shape = _out_shapes(c)
    tdt = torch.bfloat16 if c.dtype == "bf16" else torch.float16
    out_n = torch.full(o_shape, 7.0, dtype=tdt, device="cuda")
    lse_n = torch.full(l_shape, 7.0, dtype=torch.float32, device="cuda")
    say(f"  GPU {c.name}: attn_fwd_noalloc, {ns} splits, {n_ws} bytes of partials")
    fa.attn_fwd_noalloc(q, k, v, out=out_n, lse=lse_n, **kw)
    torch.cuda.synchronize()
    ws = torch.empty(max(n_ws, 16), dtype=torch.uint8, device="cuda")
    say(f"  GPU {c.name}: attn_fwd with its own workspace")
    out_w, lse_w = fa.attn_fwd(q, k, v, workspace=ws if ns > 1 else None, **kw)
    torch.cuda.synchronize()
    assert torch.equal(out_n.view(torch.int16), out_w.view(torch.int16)), f"{c.name}: O differs from attn_fwd"
    assert torch.equal(lse_n.view(torch.int32), lse_w.view(torch.int32)), f"{c.name}: LSE differs from attn_fwd"
    O_ref, L_ref = c.oracle_full()
    check_o(host_f64(out_n, c.dtype), O_ref, c.dtype, c.name)
    check_lse(lse_n.cpu().numpy().astype(np.float64), L_ref, c.name)
    return ns, n_ws


def test_two_calls_in_a_row():
    # first call: dense, causal with q_len < k_len, 6 splits (most of the array's 16 MiB is not
    # needed; what matters is that the second call's partials sit at other offsets)
    big = random_case(951, dtype="bf16", B=2, Sq=200, Sk=3000, Hq=8, Hkv=2, D=128, causal=True,
                      name="noalloc call 1 dense")
    ns1, n1 = _compare(big, 6, expect_split=True)
    # second call, smaller: varlen fp16, D = 64, 3 splits, an empty key range
    small = random_case(952, dtype="fp16", B=0, Sq=0, Sk=0, Hq=4, Hkv=1, D=64, causal=False,
                        varlen_lens=([33, 70, 1], [500, 0, 260]), name="noalloc call 2 varlen")
    ns2, n2 = _compare(small, 3, expect_split=True)
    assert n2 < n1 and ns2 < ns1


def test_no_split_and_decode():
    # one split: the array is not touched, the call is attn_fwd's unsplit path
    c = random_case(953, dtype="bf16", B=1, Sq=300, Sk=260, Hq=4, Hkv=4, D=128, Dv=96,
                    name="noalloc no split")
    _compare(c, 1, expect_split=False)
    # decode: the heuristic splits the key range
    c = random_case(954, dtype="bf16", B=4, Sq=1, Sk=4096, Hq=8, Hkv=1, D=128, causal=True,
                    name="noalloc decode")
    _compare(c, 0, expect_split=True)


def test_refuses_oversized_partials():
    # 256 rows x 16 heads x (128 + 1) floats per split: 8 splits need more than 16 MiB
    B, Sq, Sk, H, D = 1, 256, 1024, 16, 128
    assert fa.workspace_size(B, Sq, H, D, splits=8) > fa.SCRATCH_BYTES
    g = torch.Generator(device="cpu").manual_seed(955)
    q = torch.randn(B, Sq, H, D, generator=g).to(torch.bfloat16).cuda()
    k = torch.randn(B, Sk, H, D, generator=g).to(torch.bfloat16).cuda()
    v = torch.randn(B, Sk, H, D, generator=g).to(torch.bfloat16).cuda()
    out = torch.full((B, Sq, H, D), 3.0, dtype=torch.bfloat16, device="cuda")
    lse = torch.full((B, H, Sq), 3.0, dtype=torch.float32, device="cuda")
    say("  GPU noalloc oversized: 8 splits of 256 x 16 rows, expect ATTN_ERR_SCRATCH")
    with pytest.raises(fa.AttnError) as e:
        fa.attn_fwd_noalloc(q, k, v, out=out, lse=lse, num_splits=8)
    assert e.value.status == fa.CODE["ATTN_ERR_SCRATCH"]
    torch.cuda.synchronize()
    assert bool((out == 3.0).all().item()) and bool((lse == 3.0).all().item()), "refused call wrote output"
    # seven splits fit; the result then matches attn_fwd bitwise
    fa.attn_fwd_noalloc(q, k, v, out=out, lse=lse, num_splits=7)
    ws = torch.empty(fa.workspace_size(B, Sq, H, D, splits=7), dtype=torch.uint8, device="cuda")
    out_w, lse_w = fa.attn_fwd(q, k, v, num_splits=7, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out_w.view(torch.int16))
    assert torch.equal(lse.view(torch.int32), lse_w.view(torch.int32))
