"""The attention-forward workloads, as shapes + seeds, and their synthetic inputs.

Each workload stands in for a kind of call the pages describe (video-diffusion
joint attention, a causal GQA decoder with a relative bias, tabular in-context
learning in fp16, a D=256 8:1 GQA encoder with padded K/V, and D=256 decode).
No model, weight or dataset is involved: every input is a seeded draw from
``workloads.gen``.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence

import numpy as np

from . import gen


@dataclasses.dataclass
class Spec:
    name: str
    dtype: str
    B: int
    Sq: int              # dense: per-batch query length; varlen: filled with total_q
    Sk: int              # dense: per-batch key length (padded length when seqused_k); varlen: total_k
    Hq: int
    Hkv: int
    D: int
    Dv: int
    causal: bool
    scale: float         # float32 value used by both sides
    seed: int
    # varlen: either explicit lengths or a [lo, hi] range drawn from the seed (q and k share them)
    varlen: bool = False
    lengths: Optional[Sequence[int]] = None
    len_range: Optional[Sequence[int]] = None
    # padded K/V: seqused_k drawn uniform in [lo, hi] (or explicit)
    seqused_range: Optional[Sequence[int]] = None
    seqused: Optional[Sequence[int]] = None
    rel_extent: int = 0  # E; 0 = no relative bias
    bias_std: float = 0.5
    d_rel: int = 0       # > 0: the bias comes as r [rows_q, Hq, d_rel] and rel_proj [d_rel, E]
    num_splits: int = 1  # <= 0: heuristic
    pack_gqa: int = -1   # -1 auto, 0 off, 1 on
    q_std: float = 1.0
    k_std: float = 1.0
    v_std: float = 1.0

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv


def f32(x: float) -> float:
    return float(np.float32(x))


def make_inputs(spec: Spec) -> dict:
    """Draw the inputs of ``spec`` (uint16 bit patterns for 16-bit tensors, int32 metadata).

    Integer metadata comes from stream 0 (lengths, then seqused_k); q, k, v and
    rel_bias from streams 1-4 (see workloads.gen).
    """
    rng = gen.make_rng(spec.seed, gen.STREAM_META)
    out: dict = {}
    if spec.varlen:
        if spec.lengths is not None:
            lens = np.asarray(spec.lengths, dtype=np.int32)
        else:
            lo, hi = spec.len_range
            lens = gen.uniform_ints(rng, lo, hi, spec.B)
        cu = gen.cu_seqlens(lens)
        out["cu_seqlens_q"] = cu
        out["cu_seqlens_k"] = cu.copy()
        out["max_seqlen_q"] = int(lens.max()) if len(lens) else 0
        out["max_seqlen_k"] = int(lens.max()) if len(lens) else 0
        Tq = int(cu[-1])
        Tk = int(cu[-1])
        spec.Sq = Tq
        spec.Sk = Tk
        qshape = (Tq, spec.Hq, spec.D)
        kshape = (Tk, spec.Hkv, spec.D)
        vshape = (Tk, spec.Hkv, spec.Dv)
        nrows_q = Tq
    else:
        qshape = (spec.B, spec.Sq, spec.Hq, spec.D)
        kshape = (spec.B, spec.Sk, spec.Hkv, spec.D)
        vshape = (spec.B, spec.Sk, spec.Hkv, spec.Dv)
        nrows_q = spec.B * spec.Sq
    if spec.seqused is not None:
        out["seqused_k"] = np.asarray(spec.seqused, dtype=np.int32)
    elif spec.seqused_range is not None:
        lo, hi = spec.seqused_range
        out["seqused_k"] = gen.uniform_ints(rng, lo, hi, spec.B)
    out["q"] = gen.stream_normal_bits(spec.seed, gen.STREAM_Q, qshape, spec.dtype, spec.q_std)
    out["k"] = gen.stream_normal_bits(spec.seed, gen.STREAM_K, kshape, spec.dtype, spec.k_std)
    out["v"] = gen.stream_normal_bits(spec.seed, gen.STREAM_V, vshape, spec.dtype, spec.v_std)
    if spec.rel_extent and spec.d_rel:
        # r ~ N(0, 1), rel_proj ~ N(0, bias_std^2 / d_rel): the product has std bias_std
        out["rel_r"] = gen.stream_normal_bits(spec.seed, gen.STREAM_REL_R, (nrows_q, spec.Hq, spec.d_rel),
                                              spec.dtype, 1.0)
        out["rel_proj"] = gen.stream_normal_bits(spec.seed, gen.STREAM_REL_PROJ,
                                                 (spec.d_rel, spec.rel_extent), spec.dtype,
                                                 spec.bias_std / math.sqrt(spec.d_rel))
    elif spec.rel_extent:
        out["rel_bias"] = gen.stream_normal_bits(spec.seed, gen.STREAM_BIAS,
                                                 (nrows_q, spec.Hq, spec.rel_extent),
                                                 spec.dtype, spec.bias_std)
    return out


def workload(name: str, dtype: Optional[str] = None) -> Spec:
    """The named full-size workloads.

    c1   non-causal MHA bf16 [1,257,8,128]                   (small; full oracle)
    c2   non-causal MHA bf16 [1,20480,56,128] (also fp16)     (video joint attention)
    c3   varlen causal GQA 32/8 D128, rel_bias E=256, bf16    (8 seqs, len U[512,8192])
    c4a  fp16 self-attention [256,10000,6,64]
    c4b  fp16 feature attention [100,100000,4,16]
    c4c  fp16 cross attention q[1,1000,6,64] k/v[1,1e6,6,64], split-KV heuristic
    c5a  bf16 D256 8:1 pack-GQA, q[4,1024,8,256], k/v[4,2048,1,256], seqused_k U[600,2048]
    c3r  c3 with the bias produced in the kernel from r [T,32,16] and rel_proj [16,256]
    c5b  bf16 D256 decode q[32,1,8,256], k/v[32,131072,1,256], causal, split-KV + combine
    n1a/b/c  fp16 cached prediction: q[1,R,8,64] against k/v[1,300000,1,64] (MQA 8:1),
             R = 16 / 64 / 256 query rows, non-causal, split-KV heuristic
    n2a/b/c  bf16 non-causal MHA [2,8192,32,D] with D = 48 / 72 / 128 (the D48/D72/D128 family)
    """
    s128 = f32(1.0 / math.sqrt(128.0))
    if name == "c1":
        return Spec(name, dtype or gen.BF16, 1, 257, 257, 8, 8, 128, 128, False, s128, 1)
    if name == "c2":
        return Spec(name, dtype or gen.BF16, 1, 20480, 20480, 56, 56, 128, 128, False, s128, 2)
    if name == "c3":
        return Spec(name, dtype or gen.BF16, 8, 0, 0, 32, 8, 128, 128, True, s128, 3,
                    varlen=True, len_range=(512, 8192), rel_extent=256, bias_std=0.5)
    if name == "c3r":
        return Spec(name, dtype or gen.BF16, 8, 0, 0, 32, 8, 128, 128, True, s128, 3,
                    varlen=True, len_range=(512, 8192), rel_extent=256, bias_std=0.5, d_rel=16)
    if name == "c4a":
        return Spec(name, dtype or gen.FP16, 256, 10000, 10000, 6, 6, 64, 64, False, f32(1 / 8), 41)
    if name == "c4b":
        return Spec(name, dtype or gen.FP16, 100, 100000, 100000, 4, 4, 16, 16, False, f32(1 / 4), 42)
    if name == "c4c":
        return Spec(name, dtype or gen.FP16, 1, 1000, 1000000, 6, 6, 64, 64, False, f32(1 / 8), 43,
                    num_splits=0)
    if name == "c5a":
        return Spec(name, dtype or gen.BF16, 4, 1024, 2048, 8, 1, 256, 256, False, f32(1 / 16), 51,
                    seqused_range=(600, 2048), pack_gqa=1)
    if name == "c5b":
        return Spec(name, dtype or gen.BF16, 32, 1, 131072, 8, 1, 256, 256, True, f32(1 / 16), 52,
                    num_splits=0, pack_gqa=1)
    if name in N2_DIMS:
        D = N2_DIMS[name]
        return Spec(name, dtype or gen.BF16, 2, 8192, 8192, 32, 32, D, D, False, f32(1.0 / math.sqrt(D)),
                    N2_SEEDS[name])
    if name in N1_ROWS:
        return Spec(name, dtype or gen.FP16, 1, N1_ROWS[name], 300000, 8, 1, 64, 64, False, f32(1 / 8),
                    N1_SEEDS[name], num_splits=0)
    raise KeyError(name)


# head dims of the D48 / D72 / D128 family on one prefill shape, and seeds
N2_DIMS = {"n2a": 48, "n2b": 72, "n2c": 128}
N2_SEEDS = {"n2a": 71, "n2b": 72, "n2c": 73}

# short-query cached prediction: query rows per call and seeds
N1_ROWS = {"n1a": 16, "n1b": 64, "n1c": 256}
N1_SEEDS = {"n1a": 61, "n1b": 62, "n1c": 63}

WORKLOADS = ("c1", "c2", "c3", "c3r", "c4a", "c4b", "c4c", "c5a", "c5b", "n1a", "n1b", "n1c", "n2a", "n2b",
             "n2c")

