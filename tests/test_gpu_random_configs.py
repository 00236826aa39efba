"""Seeded random configurations against the full oracle.

Each case draws a combination of the features the library supports (dtype, head
dims D / Dv in the 8..256 family, GQA ratio and pack-GQA on / off / auto, causal,
dense or varlen with empty and ragged sequences, padded seqused_k with NaN
padding, a rel_bias band, split count) at sizes that span a few tiles, runs it
through the C ABI and compares O and LSE with the fp64 oracle on every row.
The draw is fixed by the case number, so a failure names a reproducible case.
"""
import numpy as np
import pytest
import torch

import exact_attention_forward_amd as fa
from tests.gpu_common import full_check, random_case, say
from workloads import gen

pytestmark = pytest.mark.gpu

N_CASES = 296


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    fa.load()


def draw(case_no):
    rng = gen.make_rng(90_000 + case_no)
    pick = lambda xs: xs[int(rng.integers(len(xs)))]
    dtype = pick(["bf16", "fp16"])
    D = int(pick([8, 16, 24, 48, 64, 72, 96, 128, 136, 192, 256]))
    Dv = D if rng.random() < 0.6 else int(pick([8, 32, 64, 104, 128, 256]))
    Hkv = int(pick([1, 2, 3]))
    G = int(pick([1, 2, 4, 8]))
    causal = bool(rng.random() < 0.5)
    kw = dict(dtype=dtype, Hq=Hkv * G, Hkv=Hkv, D=D, Dv=Dv, causal=causal,
              pack_gqa=int(pick([-1, 0, 1])), num_splits=int(pick([1, 1, 0, 3])))
    mode = pick(["dense", "varlen", "seqused"])
    if mode == "varlen":
        B = int(rng.integers(1, 5))
        qls = [int(x) for x in rng.integers(0, 300, B)]
        kls = [int(x) for x in rng.integers(0, 400, B)]
        if rng.random() < 0.5:
            kls = qls  # self-attention lengths
        kw.update(B=B, Sq=0, Sk=0, varlen_lens=(qls, kls))
        if rng.random() < 0.4:
            kw["E"] = 128
    elif mode == "seqused":
        B = int(rng.integers(1, 4))
        Sk = int(rng.integers(1, 500))
        kw.update(B=B, Sq=int(rng.integers(1, 200)), Sk=Sk, nan_pad=True,
                  seqused=[int(x) for x in rng.integers(0, Sk + 1, B)])
    else:
        kw.update(B=int(rng.integers(1, 3)), Sq=int(rng.integers(1, 260)), Sk=int(rng.integers(1, 520)))
        if rng.random() < 0.3:
            kw["E"] = 256
    return kw


@pytest.mark.parametrize("case_no", range(N_CASES))
def test_random_config(case_no):
    kw = draw(case_no)
    say(f"  case {case_no}: {kw if 'varlen_lens' not in kw else {**kw, 'varlen_lens': '...'}}")
    c = random_case(91_000 + case_no, name=f"random case {case_no}", **kw)
    full_check(c)


N_PEAKED = 100


@pytest.mark.parametrize("case_no", range(N_PEAKED))
def test_random_config_peaked_bf16(case_no):
    """The same draws in bf16 with peaked rows (q std 2, 3, 4): few keys hold a row's weight,
    where the rounding of P to bf16 matters most and the remainder correction must engage."""
    kw = dict(draw(case_no), dtype="bf16")
    q_std = (2.0, 3.0, 4.0)[case_no % 3]
    say(f"  peaked case {case_no} (q std {q_std})")
    c = random_case(95_000 + case_no, name=f"peaked case {case_no}", q_std=q_std, **kw)
    full_check(c)
