"""Helpers shared by the GPU parity tests: device transfer, the comparison bar, row sampling.

The bar (float outputs): every O element satisfies
    |O_gpu - O_ref| <= max(5e-3, 1 ulp of O_ref in the output dtype)
which equals the literal 5e-3 for every fp16 output and for every bf16 output
with |O| < 1 (where half a bf16 ulp is at most 2^-9); it only widens where a
bf16 output of magnitude >= 1 cannot hold 5e-3 after rounding at all. LSE:
|LSE_gpu - LSE_ref| <= 1e-3, and -inf exactly where the oracle has -inf.
"""
from __future__ import annotations

import math
import os
import sys

import numpy as np
import torch

import exact_attention_forward_amd as fa
from oracle import oracle as oracle_mod
from workloads import gen

O_TOL = 5e-3
LSE_TOL = 1e-3
TORCH_DT = {"bf16": torch.bfloat16, "fp16": torch.float16}
NAN16 = {"bf16": 0x7FC0, "fp16": 0x7E00}


def say(*a):
    """Progress line, flushed before each GPU step."""
    print(*a, flush=True)
    sys.stdout.flush()


def dev16(bits: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.to("cuda").view(TORCH_DT[dtype])


def dev_i32(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(np.asarray(a, dtype=np.int32))).to("cuda")


def host_f64(t: torch.Tensor, dtype: str) -> np.ndarray:
    bits = t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return gen.bits_to_f32(bits, dtype).astype(np.float64)


def ulp(x: np.ndarray, dtype: str) -> np.ndarray:
    """Spacing of the 16-bit format at |x| (normal range; subnormal spacing below it)."""
    ax = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    if dtype == "bf16":
        return np.exp2(np.maximum(e, -126) - 7)
    return np.exp2(np.maximum(e, -14) - 10)


def check_o(o_gpu, o_ref, dtype, what=""):
    o_gpu = np.asarray(o_gpu, dtype=np.float64)
    o_ref = np.asarray(o_ref, dtype=np.float64)
    assert o_gpu.shape == o_ref.shape, (what, o_gpu.shape, o_ref.shape)
    assert np.all(np.isfinite(o_gpu)), f"{what}: non-finite O from the GPU"
    err = np.abs(o_gpu - o_ref)
    allowed = np.maximum(O_TOL, ulp(o_ref, dtype))
    n_ulp_clause = int(np.count_nonzero(err > O_TOL))
    bad = err > allowed
    mx = float(err.max()) if err.size else 0.0
    say(f"  {what}: O max abs err {mx:.3e}, mean {float(err.mean()) if err.size else 0:.2e}, "
        f"elements over 5e-3 (allowed by the ulp clause) {n_ulp_clause}")
    assert not bad.any(), (f"{what}: {int(bad.sum())} O elements over the bar; max err {mx:.3e} "
                           f"at ref {o_ref[np.unravel_index(np.argmax(err - allowed), err.shape)]:.4f}")
    return mx


def check_lse(l_gpu, l_ref, what=""):
    l_gpu = np.asarray(l_gpu, dtype=np.float64)
    l_ref = np.asarray(l_ref, dtype=np.float64)
    assert l_gpu.shape == l_ref.shape, (what, l_gpu.shape, l_ref.shape)
    ninf = np.isneginf(l_ref)
    assert np.array_equal(np.isneginf(l_gpu), ninf), f"{what}: -inf LSE positions differ"
    fin = ~ninf
    assert np.all(np.isfinite(l_gpu[fin])), f"{what}: non-finite LSE"
    mx = float(np.abs(l_gpu[fin] - l_ref[fin]).max()) if fin.any() else 0.0
    say(f"  {what}: LSE max abs err {mx:.3e}")
    assert mx <= LSE_TOL, f"{what}: LSE err {mx:.3e} > {LSE_TOL}"
    return mx


class Case:
    """One attention call: host inputs (16-bit patterns) plus the arguments."""

    def __init__(self, *, dtype, B, Sq, Sk, Hq, Hkv, D, Dv=None, scale=None, causal=False,
                 q, k, v, cu_q=None, cu_k=None, max_q=None, max_k=None, seqused=None,
                 bias=None, num_splits=1, pack_gqa=-1, name="case", rel_r=None, rel_proj=None):
        self.dtype, self.B, self.Sq, self.Sk = dtype, B, Sq, Sk
        self.Hq, self.Hkv, self.D, self.Dv = Hq, Hkv, D, Dv or D
        self.scale = float(np.float32(scale if scale is not None else 1.0 / math.sqrt(D)))
        self.causal = causal
        self.q, self.k, self.v = q, k, v
        self.cu_q, self.cu_k, self.max_q, self.max_k = cu_q, cu_k, max_q, max_k
        self.seqused, self.bias = seqused, bias
        self.num_splits, self.pack_gqa, self.name = num_splits, pack_gqa, name
        # fused producer: the GPU gets r and rel_proj; the oracle gets the bias they make
        self.rel_r, self.rel_proj = rel_r, rel_proj
        if rel_r is not None:
            self.bias = oracle_mod.rel_bias_from_proj(rel_r, rel_proj, dtype)

    @property
    def varlen(self):
        return self.cu_q is not None

    def run_gpu(self, **over):
        """Run through the C ABI; returns (out tensor, lse tensor)."""
        kw = dict(causal=self.causal, scale=self.scale, num_splits=self.num_splits,
                  pack_gqa=self.pack_gqa)
        kw.update(over)
        if self.varlen:
            kw.update(cu_seqlens_q=dev_i32(self.cu_q), cu_seqlens_k=dev_i32(self.cu_k),
                      max_seqlen_q=int(self.max_q), max_seqlen_k=int(self.max_k))
        if self.seqused is not None:
            kw["seqused_k"] = dev_i32(self.seqused)
        if self.rel_r is not None:
            kw["rel_r"] = dev16(self.rel_r, self.dtype)
            kw["rel_proj"] = dev16(self.rel_proj, self.dtype)
        elif self.bias is not None:
            kw["rel_bias"] = dev16(self.bias, self.dtype)
        q = dev16(self.q, self.dtype)
        k = dev16(self.k, self.dtype)
        v = dev16(self.v, self.dtype)
        say(f"  GPU {self.name}: dtype={self.dtype} B={self.B} Sq={self.Sq} Sk={self.Sk} "
            f"Hq={self.Hq} Hkv={self.Hkv} D={self.D} causal={self.causal} varlen={self.varlen} "
            f"bias={self.bias is not None} seqused={self.seqused is not None} {over}")
        out, lse = fa.attn_fwd(q, k, v, **kw)
        torch.cuda.synchronize()
        return out, lse

    def oracle_kw(self):
        return dict(dtype=self.dtype, B=self.B, Sq=self.Sq, Sk=self.Sk, Hq=self.Hq, Hkv=self.Hkv,
                    D=self.D, Dv=self.Dv, scale=self.scale, causal=self.causal,
                    cu_seqlens_q=self.cu_q, cu_seqlens_k=self.cu_k, seqused_k=self.seqused,
                    rel_bias=self.bias)

    def oracle_full(self):
        return oracle_mod.attn_full(self.q, self.k, self.v, **self.oracle_kw())

    def oracle_rows(self, rows):
        return oracle_mod.attn_rows(self.q, self.k, self.v, rows=rows, **self.oracle_kw())

    def q_lens(self):
        ql, _ = oracle_mod.seq_lengths(self.B, self.Sq, self.Sk, self.cu_q, self.cu_k, self.seqused)
        return ql

    def gather(self, out: np.ndarray, lse: np.ndarray, rows: np.ndarray):
        """GPU results at (b, h, i) rows, from the full output arrays."""
        b, h, i = (rows[:, c].astype(np.int64) for c in range(3))
        if self.varlen:
            t = np.asarray(self.cu_q, dtype=np.int64)[b] + i
            return out[t, h], lse[h, t]
        return out[b, i, h], lse[b, h, i]


def random_case(rng_seed, *, dtype, B, Sq, Sk, Hq, Hkv, D, Dv=None, causal=False, varlen_lens=None,
                seqused=None, E=0, nan_pad=False, num_splits=1, pack_gqa=-1, name="case",
                q_std=1.0):
    """Seeded random inputs of the given shape (small test cases); Dv defaults to D."""
    Dv = Dv or D
    s = rng_seed
    cu_q = cu_k = max_q = max_k = None
    if varlen_lens is not None:
        qls, kls = varlen_lens
        cu_q, cu_k = gen.cu_seqlens(qls), gen.cu_seqlens(kls)
        Sq, Sk, B = int(cu_q[-1]), int(cu_k[-1]), len(qls)
        # the longest sequence of each side (0 when every sequence of that side is empty: the
        # library takes max_seqlen <= the total length)
        max_q, max_k = max(qls), max(kls)
        qshape, kshape, vshape = (Sq, Hq, D), (Sk, Hkv, D), (Sk, Hkv, Dv)
        rows_q = Sq
    else:
        qshape, kshape, vshape = (B, Sq, Hq, D), (B, Sk, Hkv, D), (B, Sk, Hkv, Dv)
        rows_q = B * Sq
    q = gen.stream_normal_bits(s, 1, qshape, dtype, q_std)
    k = gen.stream_normal_bits(s, 2, kshape, dtype)
    v = gen.stream_normal_bits(s, 3, vshape, dtype)
    bias = gen.stream_normal_bits(s, 4, (rows_q, Hq, E), dtype, 0.5) if E else None
    su = None if seqused is None else np.asarray(seqused, dtype=np.int32)
    if su is not None and nan_pad:
        for b in range(B):
            if varlen_lens is None:
                k[b, su[b]:] = NAN16[dtype]
                v[b, su[b]:] = NAN16[dtype]
    return Case(dtype=dtype, B=B, Sq=Sq, Sk=Sk, Hq=Hq, Hkv=Hkv, D=D, Dv=Dv, causal=causal, q=q, k=k,
                v=v, cu_q=cu_q, cu_k=cu_k, max_q=max_q, max_k=max_k, seqused=su, bias=bias,
                num_splits=num_splits, pack_gqa=pack_gqa, name=name)


def full_check(case: Case, out_lse=None, **over):
    """GPU vs the full oracle; returns (O max err, LSE max err). out_lse: results
    already computed (else the case runs here)."""
    out, lse = case.run_gpu(**over) if out_lse is None else out_lse
    O_ref, L_ref = case.oracle_full()
    o = host_f64(out, case.dtype)
    l = lse.cpu().numpy().astype(np.float64)
    return check_o(o, O_ref, case.dtype, case.name), check_lse(l, L_ref, case.name)


def sample_rows(case: Case, *, max_pairs=6, per_seq_rows=24, seed=0, tile=128):
    """Deterministic (b, h, i) sample: first/last batch and head plus seeded picks;
    rows at the start, around tile boundaries, the end, and seeded rows."""
    rng = gen.make_rng(10_000 + seed)
    ql = case.q_lens()
    bs = [b for b in range(case.B) if ql[b] > 0]
    if not bs:
        return np.zeros((0, 3), dtype=np.int32)
    pairs = {(bs[0], 0), (bs[-1], case.Hq - 1)}
    while len(pairs) < min(max_pairs, len(bs) * case.Hq):
        pairs.add((int(rng.choice(bs)), int(rng.integers(0, case.Hq))))
    rows = []
    for b, h in sorted(pairs):
        n = int(ql[b])
        cand = set(range(min(n, 4)))
        for t in range(tile, n, tile * max(1, n // (tile * 4) or 1)):
            cand.update({t - 1, t})
        cand.update(range(max(0, n - 3), n))
        while len(cand) < min(n, per_seq_rows):
            cand.add(int(rng.integers(0, n)))
        rows += [(b, h, i) for i in sorted(cand) if 0 <= i < n]
    return np.asarray(rows, dtype=np.int32)


def sampled_check(case: Case, rows=None, out_lse=None, **over):
    """GPU at full size vs the oracle on a row sample."""
    if out_lse is None:
        out, lse = case.run_gpu(**over)
    else:
        out, lse = out_lse
    if rows is None:
        rows = sample_rows(case)
    say(f"  oracle on {len(rows)} sampled rows")
    o_ref, l_ref = case.oracle_rows(rows)
    o_all = out.contiguous().view(torch.int16)
    lse_all = lse.cpu().numpy().astype(np.float64)
    b, h, i = (rows[:, c].astype(np.int64) for c in range(3))
    if case.varlen:
        t = torch.from_numpy(np.asarray(case.cu_q, dtype=np.int64)[b] + i)
        og = o_all[t.to(out.device), torch.from_numpy(h).to(out.device)]
        lg = lse_all[h, t.numpy()]
    else:
        og = o_all[torch.from_numpy(b).to(out.device), torch.from_numpy(i).to(out.device),
                   torch.from_numpy(h).to(out.device)]
        lg = lse_all[b, h, i]
    og = gen.bits_to_f32(og.cpu().numpy().view(np.uint16), case.dtype).astype(np.float64)
    return check_o(og, o_ref, case.dtype, case.name), check_lse(lg, l_ref, case.name)
