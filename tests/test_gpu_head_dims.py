"""The head-dim family: D and Dv any multiples of 8 up to 256, Dv may differ from D.

Each pair runs on the kernel of the next class size (16, 64, 128, 256) with the
columns past D / Dv zero; every case is checked against the full oracle at
sizes that span several row and key tiles and end in ragged ones.
"""
import pytest
import torch

import exact_attention_forward_amd as fa
from tests.gpu_common import full_check, random_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    fa.load()


PAIRS = [(8, 8), (24, 24), (32, 32), (48, 48), (72, 72), (96, 96), (120, 120), (136, 136),
         (160, 160), (200, 200), (248, 248), (128, 64), (64, 128), (192, 128), (72, 128),
         (40, 24), (256, 8), (8, 256), (256, 128), (128, 256)]


@pytest.mark.parametrize("D,Dv", PAIRS)
def test_dense_gqa_ragged(D, Dv):
    dtype = "bf16" if (D + Dv) % 16 == 0 else "fp16"
    causal = (D // 8) % 2 == 1
    c = random_case(7000 + D * 3 + Dv, dtype=dtype, B=2, Sq=133, Sk=270, Hq=4, Hkv=2, D=D, Dv=Dv,
                    causal=causal, name=f"D{D} Dv{Dv} {dtype} causal={causal}")
    full_check(c)


@pytest.mark.parametrize("D,Dv", [(72, 72), (48, 96), (200, 136), (24, 24)])
def test_varlen_split_seqused_pack(D, Dv):
    qls, kls = [37, 0, 150, 5], [300, 17, 180, 64]
    c = random_case(7500 + D + Dv, dtype="bf16", B=4, Sq=0, Sk=0, Hq=8, Hkv=2, D=D, Dv=Dv,
                    causal=True, varlen_lens=(qls, kls), num_splits=3,
                    name=f"varlen D{D} Dv{Dv} split 3")
    full_check(c)
    c = random_case(7600 + D + Dv, dtype="fp16", B=3, Sq=40, Sk=500, Hq=8, Hkv=1, D=D, Dv=Dv,
                    seqused=[500, 123, 7], nan_pad=True, num_splits=0, pack_gqa=1,
                    name=f"seqused NaN pad D{D} Dv{Dv} pack")
    full_check(c)


@pytest.mark.parametrize("D", [72, 48])
def test_rel_bias_band(D):
    qls, kls = [200, 70], [260, 70]
    c = random_case(7700 + D, dtype="bf16", B=2, Sq=0, Sk=0, Hq=4, Hkv=2, D=D, causal=True,
                    varlen_lens=(qls, kls), E=128, name=f"rel_bias D{D}")
    full_check(c)


@pytest.mark.parametrize("D,Dv", [(256, 256), (200, 136), (136, 256), (256, 8)])
@pytest.mark.parametrize("Sq,G", [(1, 8), (4, 8), (3, 2), (1, 1)])
def test_decode_rows_share_waves(D, Dv, Sq, G):
    """Class 256 with at most 32 rows per tile: every wave takes the same rows and a
    quarter of the V columns. Causal, padded keys, several splits."""
    c = random_case(7800 + D + Dv + 10 * Sq + G, dtype="bf16", B=3, Sq=Sq, Sk=2100, Hq=2 * G, Hkv=2,
                    D=D, Dv=Dv, causal=True, seqused=[2100, 1333, 40], nan_pad=True, num_splits=0,
                    name=f"decode D{D} Dv{Dv} Sq{Sq} G{G}")
    full_check(c)


@pytest.mark.parametrize("D,Dv,causal,splits", [(72, 72, False, 1), (96, 80, True, 1), (48, 48, False, 1),
                                                 (40, 48, True, 3), (88, 64, False, 4), (160, 160, False, 1),
                                                 (136, 192, True, 2), (192, 128, False, 1)])
def test_narrowed_equals_zero_padded_full_width(D, Dv, causal, splits):
    """Head dims that run the narrowed instances (max(D, Dv) <= 96 on class 128, <= 48 on
    class 64, <= 192 on class 256) give bitwise the result of the full-width kernel of their
    class on the same inputs padded with zero columns: the steps the narrowed kernel leaves out
    add exact zeros."""
    import numpy as np
    dclass = 64 if max(D, Dv) <= 64 else 128 if max(D, Dv) <= 128 else 256
    g = torch.Generator(device="cpu").manual_seed(7900 + D + Dv)
    B, Sq, Sk, Hq, Hkv = 2, 150, 333, 4, 2
    q = torch.randn(B, Sq, Hq, D, generator=g).to(torch.bfloat16)
    k = torch.randn(B, Sk, Hkv, D, generator=g).to(torch.bfloat16)
    v = torch.randn(B, Sk, Hkv, Dv, generator=g).to(torch.bfloat16)

    def pad(t, width):
        z = torch.zeros(*t.shape[:-1], width, dtype=t.dtype)
        z[..., :t.shape[-1]] = t
        return z

    scale = float(np.float32(1.0 / np.sqrt(D)))
    kw = dict(causal=causal, scale=scale, num_splits=splits)
    out_n, lse_n = fa.attn_fwd(q.cuda(), k.cuda(), v.cuda(), **kw)
    out_f, lse_f = fa.attn_fwd(pad(q, dclass).cuda(), pad(k, dclass).cuda(), pad(v, dclass).cuda(), **kw)
    torch.cuda.synchronize()
    assert torch.equal(out_n.view(torch.int16), out_f[..., :Dv].contiguous().view(torch.int16))
    assert torch.equal(lse_n.view(torch.int32), lse_f.view(torch.int32))
    assert not out_f[..., Dv:].any()
