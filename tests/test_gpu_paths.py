"""Accepted paths of the boundary that the main parity tests do not reach, against the oracle.

- attn_combine called on its own (the split-KV merge outside the forward call that the
  returned LSE allows: TabPFN issue #1235, closing comment) on the partials attn_fwd left
  in a caller-owned workspace: dense and varlen LSE layouts, Dv below its head-dim class,
  rows whose splits are all empty, few rows with many splits (a work-group per row) and many
  rows with few splits (a wave per row); bitwise equal to attn_fwd's own merge and within
  the tolerance of the oracle.
- scale = 0 and a negative scale (every tile then takes the masked softmax pass).
- lse = NULL, with and without splits.
- guard bands: out, lse and the workspace sit inside larger buffers filled with a
  sentinel; nothing outside them may change (dense, varlen + bias, split, decode, Dv
  below its class).
"""
import math

import numpy as np
import pytest
import torch

import exact_attention_forward_amd as fa
from tests.gpu_common import LSE_TOL, Case, check_lse, check_o, dev16, dev_i32, full_check, host_f64, random_case, say
from workloads import gen

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    fa.load()


def _kw(c):
    kw = dict(causal=c.causal, scale=c.scale, pack_gqa=c.pack_gqa)
    if c.varlen:
        kw.update(cu_seqlens_q=dev_i32(c.cu_q), cu_seqlens_k=dev_i32(c.cu_k), max_seqlen_q=int(c.max_q),
                  max_seqlen_k=int(c.max_k))
    if c.seqused is not None:
        kw["seqused_k"] = dev_i32(c.seqused)
    if c.bias is not None:
        kw["rel_bias"] = dev16(c.bias, c.dtype)
    return kw


def _tensors(c):
    return dev16(c.q, c.dtype), dev16(c.k, c.dtype), dev16(c.v, c.dtype)


def _splits(c, requested):
    return fa.num_splits(c.B, c.Sq, c.Sk, c.Hq, c.Hkv, c.D, c.Dv, causal=c.causal, is_varlen=c.varlen,
                         max_seqlen_q=int(c.max_q or 0), max_seqlen_k=int(c.max_k or 0), pack_gqa=c.pack_gqa,
                         requested=requested)


COMBINE_CASES = [
    # dense, causal with q_len > k_len: the first 43 rows of each sequence see no key, so
    # all their splits are empty (LSE -inf, O 0); Dv = 96 below its class (128)
    dict(name="dense Dv96", seed=901, dtype="bf16", B=2, Sq=300, Sk=257, Hq=4, Hkv=2, D=128, Dv=96,
         causal=True, splits=3),
    # varlen with an empty key range and an empty query range; fp16, D = Dv = 64
    dict(name="varlen fp16", seed=902, dtype="fp16", B=0, Sq=0, Sk=0, Hq=8, Hkv=2, D=64, Dv=64,
         causal=False, splits=4, lens=([40, 0, 130, 7], [300, 5, 0, 900])),
    # decode-like: one query row, D = 256, many splits
    dict(name="decode D256", seed=903, dtype="bf16", B=3, Sq=1, Sk=2000, Hq=8, Hkv=1, D=256, Dv=256,
         causal=True, splits=9, full_rows=True),
    # at least 8192 (row, head) items and at most 64 splits: the wave-per-row merge
    dict(name="many rows dense Dv96", seed=904, dtype="bf16", B=2, Sq=1100, Sk=1000, Hq=4, Hkv=2, D=128,
         Dv=96, causal=True, splits=2),
    dict(name="many rows varlen fp16", seed=905, dtype="fp16", B=0, Sq=0, Sk=0, Hq=2, Hkv=1, D=64, Dv=64,
         causal=False, splits=3, lens=([3000, 0, 2500, 7], [300, 5, 0, 900])),
    # pack-GQA D256 with seqused_k: every row of batch 0 is empty
    dict(name="many rows D256 seqused", seed=906, dtype="bf16", B=2, Sq=600, Sk=1200, Hq=8, Hkv=1, D=256,
         Dv=256, causal=False, splits=5, seqused=[0, 1100], pack_gqa=1),
    dict(name="many rows D16 64 splits", seed=907, dtype="fp16", B=1, Sq=2100, Sk=8192, Hq=4, Hkv=4, D=16,
         Dv=16, causal=True, splits=64, full_rows=True),
    # 2048..8191 items with at most two rounds of partial reads per lane (splits * class <= 4096):
    # also the wave-per-row merge (the short-query split calls)
    dict(name="short query 48 splits", seed=908, dtype="fp16", B=1, Sq=300, Sk=6000, Hq=8, Hkv=1, D=64,
         Dv=64, causal=False, splits=48, full_rows=True, pack_gqa=1),
]


@pytest.mark.parametrize("cfg", COMBINE_CASES, ids=[c["name"] for c in COMBINE_CASES])
def test_standalone_combine(cfg):
    c = random_case(cfg["seed"], dtype=cfg["dtype"], B=cfg["B"], Sq=cfg["Sq"], Sk=cfg["Sk"], Hq=cfg["Hq"],
                    Hkv=cfg["Hkv"], D=cfg["D"], Dv=cfg["Dv"], causal=cfg["causal"], varlen_lens=cfg.get("lens"),
                    seqused=cfg.get("seqused"), pack_gqa=cfg.get("pack_gqa", -1), name="combine " + cfg["name"])
    q, k, v = _tensors(c)
    ns = _splits(c, cfg["splits"])
    assert ns == cfg["splits"], ns
    ws = torch.empty(fa.workspace_size(c.B, c.Sq, c.Hq, c.Dv, is_varlen=c.varlen, splits=ns),
                     dtype=torch.uint8, device="cuda")
    say(f"  GPU {c.name}: attn_fwd with {ns} splits, then attn_combine on its workspace")
    out1, lse1 = fa.attn_fwd(q, k, v, num_splits=ns, workspace=ws, **_kw(c))
    torch.cuda.synchronize()
    o_p, l_p = fa.split_partials(ws, ns, B=c.B, Sq=c.Sq, Hq=c.Hq, Dv=c.Dv, is_varlen=c.varlen)
    out2 = torch.full_like(out1, 7.0)
    lse2 = torch.full_like(lse1, 7.0)
    fa.attn_combine(o_p, l_p, out=out2, lse=lse2, B=c.B, Sq=c.Sq, is_varlen=c.varlen)
    out3 = torch.full_like(out1, 7.0)
    fa.attn_combine(o_p, l_p, out=out3, lse=None, B=c.B, Sq=c.Sq, is_varlen=c.varlen)
    torch.cuda.synchronize()
    # the same partials through the same merge: bitwise what attn_fwd returned
    assert torch.equal(out2.view(torch.int16), out1.view(torch.int16))
    assert torch.equal(out3.view(torch.int16), out1.view(torch.int16))
    assert torch.equal(lse2.view(torch.int32), lse1.view(torch.int32))
    O_ref, L_ref = c.oracle_full()
    check_o(host_f64(out2, c.dtype), O_ref, c.dtype, c.name)
    check_lse(lse2.cpu().numpy().astype(np.float64), L_ref, c.name)
    if not cfg.get("full_rows"):
        assert np.isneginf(L_ref).any(), "the case should hold rows with no visible key"


# A varlen batch whose query side, or key side, is empty in every sequence: max_seqlen is then
# 0 on that side. No query rows: nothing is launched or written. No keys: every row is empty
# (O = 0, LSE = -inf).
@pytest.mark.parametrize("qls,kls,splits", [([0], [112], 1), ([0, 0, 0], [5, 0, 300], 0),
                                             ([40, 0, 7], [0, 0, 0], 1), ([40, 0, 7], [0, 0, 0], 3)])
def test_varlen_side_entirely_empty(qls, kls, splits):
    c = random_case(930 + len(qls), dtype="fp16", B=len(qls), Sq=0, Sk=0, Hq=8, Hkv=2, D=136, Dv=32,
                    causal=True, varlen_lens=(qls, kls), num_splits=splits,
                    name=f"varlen q {qls} k {kls} ns{splits}")
    say(f"  GPU {c.name}")
    full_check(c)


# The largest K / V tile the validation accepts: a 64-key tile of Hkv heads spans 2^30 bytes at
# head dim 128 (Hkv = 2^16) and just under it at 120 (Hkv = 69905, narrowed columns past D), so the
# buffer ranges, the per-lane load offsets and the past-the-range offset of the padding columns
# run at their limit. Q, K and V are zero but for a few heads drawn from the generator: those are
# checked against the oracle, and every other head must give O = 0 and LSE = ln(Sk) (equal
# scores over zero values).
@pytest.mark.parametrize("D", [128, 120])
def test_largest_kv_tile(D):
    dtype, B, Sq, Sk = "bf16", 1, 2, 200
    Hkv = (1 << 30) // (64 * D * 2)
    heads = [0, 1, Hkv // 2, Hkv - 2, Hkv - 1]
    say(f"  GPU largest K/V tile: D={D} Hkv={Hkv} Sk={Sk}, {64 * Hkv * D * 2} bytes per 64-key tile")
    tdt = torch.bfloat16
    q = torch.zeros((B, Sq, Hkv, D), dtype=tdt, device="cuda")
    k = torch.zeros((B, Sk, Hkv, D), dtype=tdt, device="cuda")
    v = torch.zeros((B, Sk, Hkv, D), dtype=tdt, device="cuda")
    cases = []
    for j, h in enumerate(heads):
        qh = gen.stream_normal_bits(970 + j, 1, (B, Sq, 1, D), dtype)
        kh = gen.stream_normal_bits(970 + j, 2, (B, Sk, 1, D), dtype)
        vh = gen.stream_normal_bits(970 + j, 3, (B, Sk, 1, D), dtype)
        q[:, :, h:h + 1] = dev16(qh, dtype)
        k[:, :, h:h + 1] = dev16(kh, dtype)
        v[:, :, h:h + 1] = dev16(vh, dtype)
        cases.append(Case(dtype=dtype, B=B, Sq=Sq, Sk=Sk, Hq=1, Hkv=1, D=D, q=qh, k=kh, v=vh,
                          name=f"largest tile D{D} head {h}"))
    out, lse = fa.attn_fwd(q, k, v)
    torch.cuda.synchronize()
    for h, c in zip(heads, cases):
        O_ref, L_ref = c.oracle_full()
        check_o(host_f64(out[:, :, h:h + 1], dtype), O_ref, dtype, c.name)
        check_lse(lse[:, h:h + 1].cpu().numpy().astype(np.float64), L_ref, c.name)
    rest = torch.ones(Hkv, dtype=torch.bool, device="cuda")
    rest[heads] = False
    assert int(torch.count_nonzero(out[:, :, rest])) == 0, "heads with zero inputs must give O = 0"
    err = float((lse[:, rest].double() - math.log(Sk)).abs().max())
    assert err <= LSE_TOL, f"heads with zero inputs: LSE off ln(Sk) by {err:.3e}"
    del q, k, v, out, lse
    torch.cuda.empty_cache()


# Outputs of more than 2^31 elements (rows_q * Hq * Dv): the Q loads and O stores index past any
# 32-bit range. Q is zero but for rows at both ends drawn from the generator; the call is
# non-causal, so each checked row is the oracle's row of a small case with the same K and V.
def test_outputs_beyond_2_31_elements():
    dtype, B, Sq, Sk, H, D = "bf16", 1, 163840, 96, 128, 128
    assert B * Sq * H * D > 1 << 31
    rows = [0, 1, Sq // 2, Sq - 2, Sq - 1]
    say(f"  GPU outputs beyond 2^31 elements: [{B},{Sq},{H},{D}] ({B * Sq * H * D} elements)")
    kh = gen.stream_normal_bits(980, 2, (B, Sk, H, D), dtype)
    vh = gen.stream_normal_bits(980, 3, (B, Sk, H, D), dtype)
    qh = gen.stream_normal_bits(980, 1, (B, len(rows), H, D), dtype)
    q = torch.zeros((B, Sq, H, D), dtype=torch.bfloat16, device="cuda")
    for j, i in enumerate(rows):
        q[:, i:i + 1] = dev16(qh[:, j:j + 1], dtype)
    out, lse = fa.attn_fwd(q, dev16(kh, dtype), dev16(vh, dtype))
    torch.cuda.synchronize()
    c = Case(dtype=dtype, B=B, Sq=len(rows), Sk=Sk, Hq=H, Hkv=H, D=D, q=qh, k=kh, v=vh,
             name="rows of a [1,163840,128,128] call")
    O_ref, L_ref = c.oracle_full()
    check_o(host_f64(out[:, rows], dtype), O_ref, dtype, c.name)
    check_lse(lse[:, :, rows].cpu().numpy().astype(np.float64), L_ref, c.name)
    # a zero query row weighs every key equally: O is the mean of V, LSE = ln(Sk)
    zero = host_f64(out[:, Sq - 3:Sq - 2], dtype)[0, 0]
    mean_v = gen.bits_to_f32(vh, dtype).astype(np.float64)[0].mean(axis=0)
    check_o(zero[None, None], mean_v[None, None], dtype, "zero query row near the end")
    err = float((lse[:, :, Sq - 3].double() - math.log(Sk)).abs().max())
    assert err <= LSE_TOL, f"zero query row: LSE off ln(Sk) by {err:.3e}"
    del q, out, lse
    torch.cuda.empty_cache()


@pytest.mark.parametrize("scale", [0.0, -0.125, -1.5])
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_nonpositive_scale(scale, dtype):
    for causal, splits in ((False, 1), (True, 3)):
        c = random_case(910 + int(causal), dtype=dtype, B=2, Sq=150, Sk=330, Hq=4, Hkv=2, D=64,
                        causal=causal, num_splits=splits, name=f"scale {scale} {dtype} c{int(causal)} ns{splits}")
        c.scale = float(np.float32(scale))
        full_check(c)
    # D = 128 (eight-wave work-groups without the causal mask)
    c = random_case(912, dtype=dtype, B=1, Sq=300, Sk=200, Hq=2, Hkv=2, D=128, name=f"scale {scale} D128")
    c.scale = float(np.float32(scale))
    full_check(c)


@pytest.mark.parametrize("splits", [1, 3])
@pytest.mark.parametrize("D", [64, 128])
def test_lse_null(splits, D):
    c = random_case(920 + D, dtype="bf16", B=2, Sq=100, Sk=700, Hq=4, Hkv=1, D=D, causal=True,
                    num_splits=splits, name=f"lse NULL D{D} ns{splits}")
    out, lse = c.run_gpu(return_lse=False)
    assert lse is None
    O_ref, _ = c.oracle_full()
    check_o(host_f64(out, c.dtype), O_ref, c.dtype, c.name)


GUARD = 4096  # bytes of sentinel on each side


def _guarded(n_bytes, fill):
    """A byte buffer with n_bytes in the middle (16-byte aligned) and GUARD sentinel bytes around."""
    buf = torch.full((n_bytes + 2 * GUARD,), fill, dtype=torch.uint8, device="cuda")
    return buf, buf[GUARD:GUARD + n_bytes]


def _intact(buf, n_bytes, fill):
    head = buf[:GUARD]
    tail = buf[GUARD + n_bytes:]
    return bool((head == fill).all().item()) and bool((tail == fill).all().item())


GUARD_CASES = [
    dict(name="dense D128", seed=930, dtype="bf16", B=2, Sq=260, Sk=333, Hq=4, Hkv=4, D=128, causal=False, splits=1),
    dict(name="varlen bias", seed=931, dtype="bf16", B=0, Sq=0, Sk=0, Hq=8, Hkv=2, D=128, causal=True, splits=1,
         lens=([77, 300, 5], [77, 300, 5]), E=128),
    dict(name="split D64", seed=932, dtype="fp16", B=2, Sq=70, Sk=1500, Hq=4, Hkv=1, D=64, causal=True, splits=5),
    dict(name="decode D256", seed=933, dtype="bf16", B=4, Sq=1, Sk=3000, Hq=8, Hkv=1, D=256, causal=True, splits=0),
    dict(name="Dv below class", seed=934, dtype="bf16", B=1, Sq=129, Sk=200, Hq=2, Hkv=2, D=128, Dv=72,
         causal=False, splits=3),
    # the wave-per-row merge (>= 8192 items, <= 64 splits), 10198 items: the last work-group
    # holds two items, so two of its waves have no row
    dict(name="many rows merge", seed=935, dtype="fp16", B=0, Sq=0, Sk=0, Hq=2, Hkv=1, D=128, Dv=104,
         causal=False, splits=3, lens=([4097, 0, 1002], [600, 77, 0])),
]


@pytest.mark.parametrize("cfg", GUARD_CASES, ids=[c["name"] for c in GUARD_CASES])
def test_guard_bands(cfg):
    Dv = cfg.get("Dv", cfg["D"])
    c = random_case(cfg["seed"], dtype=cfg["dtype"], B=cfg["B"], Sq=cfg["Sq"], Sk=cfg["Sk"], Hq=cfg["Hq"],
                    Hkv=cfg["Hkv"], D=cfg["D"], Dv=Dv, causal=cfg["causal"], varlen_lens=cfg.get("lens"),
                    E=cfg.get("E", 0), name="guard " + cfg["name"])
    q, k, v = _tensors(c)
    ns = _splits(c, cfg["splits"])
    rows_q = c.Sq if c.varlen else c.B * c.Sq
    out_shape = (c.Sq, c.Hq, Dv) if c.varlen else (c.B, c.Sq, c.Hq, Dv)
    lse_shape = (c.Hq, c.Sq) if c.varlen else (c.B, c.Hq, c.Sq)
    n_out = rows_q * c.Hq * Dv * 2
    n_lse = rows_q * c.Hq * 4
    n_ws = fa.workspace_size(c.B, c.Sq, c.Hq, Dv, is_varlen=c.varlen, splits=ns)
    ob, out_b = _guarded(n_out, 0xA5)
    lb, lse_b = _guarded(n_lse, 0x5A)
    wb, ws_b = _guarded(max(n_ws, 16), 0xC3)
    out = out_b.view(torch.bfloat16 if c.dtype == "bf16" else torch.float16).view(out_shape)
    lse = lse_b.view(torch.float32).view(lse_shape)
    say(f"  GPU {c.name}: {ns} splits, guarded out / lse / workspace ({n_out}, {n_lse}, {n_ws} bytes)")
    fa.attn_fwd(q, k, v, num_splits=ns, out=out, lse=lse, workspace=ws_b if ns > 1 else None, **_kw(c))
    torch.cuda.synchronize()
    assert _intact(ob, n_out, 0xA5), f"{c.name}: a write outside out"
    assert _intact(lb, n_lse, 0x5A), f"{c.name}: a write outside lse"
    assert _intact(wb, max(n_ws, 16), 0xC3), f"{c.name}: a write outside the workspace"
    if ns <= 1:
        assert bool((ws_b == 0xC3).all().item()), f"{c.name}: the unused workspace was written"
    full_check(c, out_lse=(out, lse))
