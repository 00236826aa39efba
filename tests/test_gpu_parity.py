"""GPU path vs the fp64 oracle, element by element, at sizes the oracle finishes quickly.

Covers every head dim and dtype, causal / non-causal with q_len <, =, > k_len,
ragged tiles, GQA with and without packing, varlen with empty sequences,
rel_bias bands, seqused_k with NaN padding, split-KV with several split counts,
decode, empty rows and empty problems. Masks, offsets and the band are checked
bit-exactly with probe inputs.
"""
import numpy as np
import pytest
import torch

import exact_attention_forward_amd as fa
from tests.gpu_common import (Case, check_lse, check_o, dev16, dev_i32, full_check, host_f64,
                              random_case, say)
from workloads import gen

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    fa.load()


@pytest.mark.parametrize("D", [16, 64, 128, 256])
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("causal", [False, True])
def test_dense_gqa_ragged(D, dtype, causal):
    # q_len > k_len with causal gives fully masked leading rows; tails are ragged
    for (Sq, Sk, Hq, Hkv) in [(300, 257, 4, 2), (129, 333, 2, 2)]:
        c = random_case(100 + D + Sq, dtype=dtype, B=2, Sq=Sq, Sk=Sk, Hq=Hq, Hkv=Hkv, D=D,
                        causal=causal, name=f"dense D{D} {dtype} c{int(causal)} {Sq}x{Sk}")
        full_check(c)


@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("splits", [2, 7, 0])
def test_split_kv(D, splits):
    c = random_case(200 + D, dtype="bf16", B=2, Sq=70, Sk=1500, Hq=4, Hkv=1, D=D, causal=True,
                    num_splits=splits, name=f"split D{D} ns={splits}")
    full_check(c)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("E", [128, 256])
@pytest.mark.parametrize("causal", [True, False])
def test_varlen_rel_bias(dtype, E, causal):
    qls = [1, 77, 300, 0, 513, 129, 5]
    kls = [1, 77, 300, 0, 513, 129, 5] if causal else [3, 200, 64, 9, 513, 0, 700]
    c = random_case(300 + E, dtype=dtype, B=0, Sq=0, Sk=0, Hq=8, Hkv=2, D=128, causal=causal,
                    varlen_lens=(qls, kls), E=E, name=f"varlen bias E{E} {dtype} c{int(causal)}")
    full_check(c)
    full_check(c, num_splits=3)


def test_varlen_d64_fp16_no_bias():
    qls = [33, 0, 1, 260]
    kls = [40, 7, 1, 255]
    c = random_case(350, dtype="fp16", B=0, Sq=0, Sk=0, Hq=6, Hkv=6, D=64, causal=True,
                    varlen_lens=(qls, kls), name="varlen D64 fp16")
    full_check(c)


@pytest.mark.parametrize("pack", [1, 0])
def test_seqused_nan_padding(pack):
    c = random_case(400, dtype="bf16", B=4, Sq=200, Sk=700, Hq=8, Hkv=1, D=256,
                    seqused=[700, 1, 0, 333], nan_pad=True, pack_gqa=pack,
                    name=f"seqused NaN pad pack={pack}")
    full_check(c)
    c.causal = True
    full_check(c)


@pytest.mark.parametrize("splits", [1, 0, 5])
def test_decode(splits):
    c = random_case(500, dtype="bf16", B=3, Sq=1, Sk=3000, Hq=8, Hkv=1, D=256, causal=True,
                    num_splits=splits, name=f"decode ns={splits}")
    full_check(c)


def test_pack_gqa_bitwise_and_determinism():
    c = random_case(600, dtype="bf16", B=2, Sq=150, Sk=310, Hq=8, Hkv=2, D=128, causal=True,
                    name="pack vs unpacked")
    o1, l1 = c.run_gpu(pack_gqa=1)
    o2, l2 = c.run_gpu(pack_gqa=0)
    o3, l3 = c.run_gpu(pack_gqa=1)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)), "pack-GQA changed O"
    assert torch.equal(l1, l2), "pack-GQA changed LSE"
    assert torch.equal(o1.view(torch.int16), o3.view(torch.int16)) and torch.equal(l1, l3), \
        "two identical calls differ"


def test_gqa_equals_repeated_kv():
    c = random_case(650, dtype="fp16", B=1, Sq=100, Sk=130, Hq=6, Hkv=2, D=64, causal=False,
                    name="gqa")
    o1, l1 = c.run_gpu(pack_gqa=0)
    G = 3
    c2 = Case(dtype="fp16", B=1, Sq=100, Sk=130, Hq=6, Hkv=6, D=64, q=c.q,
              k=np.repeat(c.k, G, axis=2), v=np.repeat(c.v, G, axis=2), name="repeated kv")
    o2, l2 = c2.run_gpu()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)


def test_empty_keys_and_problems():
    # Sk = 0: every row empty -> O = 0, LSE = -inf
    c = random_case(700, dtype="bf16", B=2, Sq=5, Sk=0, Hq=2, Hkv=1, D=64, name="Sk=0")
    out, lse = c.run_gpu()
    assert torch.all(out.float() == 0) and torch.all(torch.isneginf(lse))
    # B = 0 and Sq = 0: nothing launched, OK status
    q = torch.zeros((0, 4, 2, 64), dtype=torch.bfloat16, device="cuda")
    out, lse = fa.attn_fwd(q, q, q)
    assert out.shape == (0, 4, 2, 64)
    q = torch.zeros((2, 0, 2, 64), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((2, 4, 2, 64), dtype=torch.bfloat16, device="cuda")
    out, lse = fa.attn_fwd(q, k, k)
    assert out.shape == (2, 0, 2, 64)


def test_large_magnitude_scores():
    # scores up to ~1e2 exercise the running-max subtraction
    c = random_case(750, dtype="bf16", B=1, Sq=130, Sk=260, Hq=2, Hkv=2, D=128, q_std=30.0,
                    causal=True, name="large scores")
    full_check(c)


def test_grid_beyond_65535_batches():
    # batch * heads * tiles far above 65535 (a 1-D grid has no such limit)
    B, S = 70000, 16
    c = random_case(800, dtype="fp16", B=B, Sq=S, Sk=S, Hq=1, Hkv=1, D=64, causal=False,
                    name="70000 batches")
    out, lse = c.run_gpu()
    rows = np.array([[b, 0, i] for b in (0, 1, 12345, 65535, 65536, B - 1) for i in range(S)],
                    dtype=np.int32)
    o_ref, l_ref = c.oracle_rows(rows)
    o = host_f64(out, "fp16")
    lv = lse.cpu().numpy()
    check_o(o[rows[:, 0], rows[:, 2], 0], o_ref, "fp16", "grid")
    check_lse(lv[rows[:, 0], 0, rows[:, 2]], l_ref, "grid")


def test_varlen_beyond_65535_sequences():
    # 70000 varlen sequences of 0..3 query and key rows (empty ones among them), causal,
    # pack-GQA 2:1 with a bias band: the per-sequence offsets, the chunk-wise XCD deal and the
    # 1-D grid at a sequence count far above 65535, against the full oracle
    rng = gen.make_rng(810)
    B = 70000
    qls = [int(x) for x in rng.integers(0, 4, B)]
    kls = [int(x) for x in rng.integers(0, 4, B)]
    c = random_case(811, dtype="fp16", B=B, Sq=0, Sk=0, Hq=2, Hkv=1, D=64, causal=True,
                    varlen_lens=(qls, kls), E=128, name="70000 varlen sequences")
    say(f"  GPU {c.name}: total_q {sum(qls)}, total_k {sum(kls)}")
    full_check(c)


# ---------------------------------------------------------------- bit-exact probes

def _probe_visibility(dtype, B, Sq, Sk, Hq, Hkv, causal, cu=None, seqused=None, pack=-1, ns=1):
    """q = k = 0 and one-hot V windows: the nonzero pattern of O is the visibility mask."""
    Dv = 128
    one = gen.to_bits(np.float32(1.0), dtype).item()
    if cu is not None:
        cu_q, cu_k = cu
        Tq, Tk = int(cu_q[-1]), int(cu_k[-1])
        qshape, kshape = (Tq, Hq, Dv), (Tk, Hkv, Dv)
        max_q, max_k = int(np.diff(cu_q).max()), int(np.diff(cu_k).max())
        klens = np.diff(cu_k)
    else:
        cu_q = cu_k = max_q = max_k = None
        qshape, kshape = (B, Sq, Hq, Dv), (B, Sk, Hkv, Dv)
        klens = np.full(B, Sk)
    q = np.zeros(qshape, dtype=np.uint16)
    k = np.zeros(kshape, dtype=np.uint16)
    kmax = int(klens.max())
    for off in range(0, max(kmax, 1), Dv):
        v = np.zeros(kshape, dtype=np.uint16)
        for b in range(len(klens)):
            for j in range(off, min(off + Dv, int(klens[b]))):
                if cu is not None:
                    v[cu_k[b] + j, :, j - off] = one
                else:
                    v[b, j, :, j - off] = one
        c = Case(dtype=dtype, B=B if cu is None else len(cu_q) - 1, Sq=qshape[-3] if cu is None else Tq,
                 Sk=kshape[-3] if cu is None else Tk, Hq=Hq, Hkv=Hkv, D=Dv, causal=causal, q=q, k=k,
                 v=v, cu_q=cu_q, cu_k=cu_k, max_q=max_q, max_k=max_k, seqused=seqused,
                 num_splits=ns, pack_gqa=pack, name=f"visibility probe off={off}")
        out, lse = c.run_gpu()
        O_ref, _ = c.oracle_full()
        got = host_f64(out, dtype) != 0.0
        want = O_ref != 0.0
        assert np.array_equal(got, want), f"mask pattern differs at window {off}"


@pytest.mark.parametrize("causal", [False, True])
def test_mask_probe_dense(causal):
    for Sq, Sk in [(257, 257), (100, 300), (300, 100), (1, 129)]:
        _probe_visibility("bf16", 2, Sq, Sk, 4, 2, causal)


def test_mask_probe_varlen_seqused_pack_split():
    cu_q = gen.cu_seqlens([3, 130, 0, 257, 64])
    cu_k = gen.cu_seqlens([5, 129, 7, 257, 1])
    _probe_visibility("fp16", 0, 0, 0, 8, 2, True, cu=(cu_q, cu_k), pack=1)
    _probe_visibility("bf16", 0, 0, 0, 8, 2, True, cu=(cu_q, cu_k), pack=0, ns=3)
    _probe_visibility("bf16", 3, 40, 300, 8, 1, True, seqused=np.array([300, 17, 0], np.int32), pack=1)


def _dominant_keys(o, n_keys):
    """Per row: the key holding more than half of the weight, else -1."""
    w = o[..., :n_keys]
    idx = np.argmax(w, axis=-1)
    top = np.take_along_axis(w, idx[..., None], axis=-1)[..., 0]
    return np.where(top > 0.5, idx, -1)


@pytest.mark.parametrize("causal", [True, False])
def test_band_probe_varlen(causal):
    """A single +30 bias entry at index d: the selected key must be exactly j = i + delta - d."""
    dtype, E, Hq, Hkv, D = "bf16", 128, 2, 1, 128
    lens_q = [5, 140, 1, 77]
    lens_k = [5, 140, 1, 77] if causal else [9, 100, 128, 77]
    cu_q, cu_k = gen.cu_seqlens(lens_q), gen.cu_seqlens(lens_k)
    Tq, Tk = int(cu_q[-1]), int(cu_k[-1])
    one = gen.to_bits(np.float32(1.0), dtype).item()
    thirty = gen.to_bits(np.float32(30.0), dtype).item()
    q = np.zeros((Tq, Hq, D), dtype=np.uint16)
    k = np.zeros((Tk, Hkv, D), dtype=np.uint16)
    v = np.zeros((Tk, Hkv, D), dtype=np.uint16)
    for b in range(len(lens_k)):
        for j in range(min(lens_k[b], D)):
            v[cu_k[b] + j, :, j] = one
    for d in [0, 1, 2, 63, 64, 127]:
        rb = np.zeros((Tq, Hq, E), dtype=np.uint16)
        rb[:, :, d] = thirty
        c = Case(dtype=dtype, B=len(lens_q), Sq=Tq, Sk=Tk, Hq=Hq, Hkv=Hkv, D=D, causal=causal,
                 q=q, k=k, v=v, cu_q=cu_q, cu_k=cu_k, max_q=max(lens_q), max_k=max(lens_k),
                 bias=rb, scale=1.0, name=f"band probe d={d}")
        out, _ = c.run_gpu()
        O_ref, _ = c.oracle_full()
        got = _dominant_keys(host_f64(out, dtype), D)
        want = _dominant_keys(O_ref, D)
        assert np.array_equal(got, want), f"band selection differs for d={d}"
        say(f"  d={d}: {int((want >= 0).sum())} rows with a selected key, all identical")


def test_short_rows_bf16_accuracy():
    """Rows whose weight sits on 1-4 keys: the worst case for rounding P to bf16."""
    lens = [1, 2, 3, 4] * 60
    c = random_case(900, dtype="bf16", B=0, Sq=0, Sk=0, Hq=8, Hkv=2, D=128, causal=True,
                    varlen_lens=(lens, lens), E=128, name="short rows bf16")
    full_check(c)
    c2 = random_case(901, dtype="bf16", B=0, Sq=0, Sk=0, Hq=4, Hkv=4, D=64, causal=True,
                     varlen_lens=(lens, lens), q_std=4.0, name="short rows bf16 peaked")
    full_check(c2)


@pytest.mark.parametrize("D,causal", [(128, False), (128, True), (256, False), (64, False)],
                         ids=["d128", "d128-causal", "d256", "d64"])
def test_long_rows_few_effective_keys_bf16(D, causal):
    """bf16, 2500 keys per row. (1) Peaked scores (q std 3): most weight on a few keys in
    every tile. (2) A near-tie of three keys late in the row (keys 2100..2102 scaled up),
    arriving after the remainder bookkeeping has paused, so it must resume: in the rows those
    keys dominate (>= 90% of the weight), O rounded to bfloat16 must match the correctly
    rounded oracle in all but a few elements (without the remainder about a quarter differ,
    by a simulation of the same arithmetic)."""
    c = random_case(920 + D + causal, dtype="bf16", B=1, Sq=160, Sk=2500, Hq=8, Hkv=2, D=D,
                    causal=causal, q_std=3.0, name=f"peaked long rows D={D}")
    full_check(c)
    c = random_case(930 + D + causal, dtype="bf16", B=1, Sq=160, Sk=2500, Hq=8, Hkv=2, D=D,
                    causal=causal, name=f"late near-tie D={D}")
    kf = gen.bits_to_f32(c.k, "bf16").astype(np.float64)
    kf[:, 2100] *= 8.0
    kf[:, 2101] = 0.97 * kf[:, 2100]
    kf[:, 2102] = 0.94 * kf[:, 2100]
    c.k = gen.to_bits(kf.astype(np.float32), "bf16")
    out, lse = c.run_gpu()
    O_ref, L_ref = c.oracle_full()
    o = host_f64(out, "bf16")
    check_o(o, O_ref, "bf16", c.name)
    # weight of the three keys per (row, head), from the inputs and the oracle's LSE
    qf = gen.bits_to_f32(c.q, "bf16").astype(np.float64)[0]          # [Sq, Hq, D]
    kt = gen.bits_to_f32(c.k, "bf16").astype(np.float64)[0, 2100:2103]  # [3, Hkv, D]
    G = c.Hq // c.Hkv
    s = np.einsum("ihd,jhd->ihj", qf, np.repeat(kt, G, axis=1)) * c.scale
    w = np.exp(s - L_ref[0].T[:, :, None]).sum(-1)                    # [Sq, Hq]
    dom = w >= 0.9
    assert dom.sum() >= 50, f"only {dom.sum()} dominated rows"
    want = gen.to_bits(O_ref[0].astype(np.float32), "bf16")
    got = out.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)[0]
    frac = float((got[dom] != want[dom]).mean())
    say(f"  {int(dom.sum())} dominated rows: {frac:.4f} of their O elements differ from the rounded oracle")
    assert frac <= 0.03, f"{c.name}: {frac:.3f} of the dominated rows' elements differ from the rounded oracle"
