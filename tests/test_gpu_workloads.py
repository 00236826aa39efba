"""The workloads at full size on the GPU, checked against the oracle on sampled rows
(config 1 in full). Inputs come from workloads.configs (seeded, synthetic)."""
import numpy as np
import pytest
import torch

import exact_attention_forward_amd as fa
from tests.gpu_common import Case, NAN16, full_check, sample_rows, sampled_check, say
from workloads import configs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    fa.load()


def make_case(name, dtype=None, nan_pad=False):
    spec = configs.workload(name, dtype)
    x = configs.make_inputs(spec)
    su = x.get("seqused_k")
    if nan_pad and su is not None:
        for b in range(spec.B):
            x["k"][b, su[b]:] = NAN16[spec.dtype]
            x["v"][b, su[b]:] = NAN16[spec.dtype]
    return Case(dtype=spec.dtype, B=spec.B, Sq=spec.Sq, Sk=spec.Sk, Hq=spec.Hq, Hkv=spec.Hkv,
                D=spec.D, scale=spec.scale, causal=spec.causal, q=x["q"], k=x["k"], v=x["v"],
                cu_q=x.get("cu_seqlens_q"), cu_k=x.get("cu_seqlens_k"),
                max_q=x.get("max_seqlen_q"), max_k=x.get("max_seqlen_k"), seqused=su,
                bias=x.get("rel_bias"), num_splits=spec.num_splits, pack_gqa=spec.pack_gqa,
                name=f"{name} {spec.dtype}", rel_r=x.get("rel_r"), rel_proj=x.get("rel_proj"))


def test_c1_full():
    full_check(make_case("c1"))


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_c2_sampled(dtype):
    c = make_case("c2", dtype)
    sampled_check(c, rows=sample_rows(c, max_pairs=8, per_seq_rows=24, tile=256))


def test_c3_sampled():
    c = make_case("c3")
    say(f"  c3 lengths {np.diff(c.cu_q).tolist()}")
    sampled_check(c, rows=sample_rows(c, max_pairs=10, per_seq_rows=40, tile=64))


def test_c3r_fused_bias_sampled():
    c = make_case("c3r")
    sampled_check(c, rows=sample_rows(c, max_pairs=10, per_seq_rows=40, tile=64))


def test_c4a_sampled():
    c = make_case("c4a")
    sampled_check(c, rows=sample_rows(c, max_pairs=8, per_seq_rows=20))


def test_c4b_sampled():
    c = make_case("c4b")
    sampled_check(c, rows=sample_rows(c, max_pairs=6, per_seq_rows=16))


def test_c4c_sampled():
    c = make_case("c4c")
    say(f"  c4c splits {fa.num_splits(1, 1000, 1000000, 6, 6, 64, 64, requested=0)}")
    sampled_check(c, rows=sample_rows(c, max_pairs=4, per_seq_rows=10))


def test_c5a_nan_padded():
    c = make_case("c5a", nan_pad=True)
    say(f"  c5a seqused_k {c.seqused.tolist()}")
    sampled_check(c, rows=sample_rows(c, max_pairs=12, per_seq_rows=40))


def test_c5b_decode():
    c = make_case("c5b")
    rows = np.array([[b, h, 0] for b in range(0, 32, 3) for h in range(8)], dtype=np.int32)
    sampled_check(c, rows=rows)


@pytest.mark.parametrize("name", ["n1a", "n1b", "n1c"])
def test_n1_cached_prediction(name):
    c = make_case(name)
    say(f"  {name} splits {fa.num_splits(1, c.Sq, c.Sk, 8, 1, 64, 64, requested=0)}")
    # every query row of every head: the rows are few, the keys many
    rows = np.array([[0, h, i] for h in range(8) for i in range(0, c.Sq, max(1, c.Sq // 16))],
                    dtype=np.int32)
    sampled_check(c, rows=rows)


@pytest.mark.parametrize("name", ["n2a", "n2b"])
def test_n2_head_dims_below_class(name):
    # head dim 48 on the class-64 kernel, 72 on the class-128 kernel, at the timed size
    c = make_case(name)
    sampled_check(c, rows=sample_rows(c, max_pairs=6, per_seq_rows=24, tile=256))
