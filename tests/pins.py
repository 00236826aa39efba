"""Pins of the fp64 oracle against facts that do not come from the oracle itself.

Each ``pin_*`` takes a loaded oracle (``oracle.oracle.OracleLib``) and raises
AssertionError when the oracle disagrees with:
  * torch's scaled_dot_product_attention in float64 on the CPU (a library
    routine), with torch's own bottom-right causal mask and GQA head mapping;
  * scipy's logsumexp over a numpy-matmul score matrix (library routines);
  * closed forms (equal scores give the mean of V and LSE = ln n; causal row 0
    gives v0; a dominant score selects one V row; empty rows give (0, -inf));
  * the hand-written band fixture in tests/golden (tml-fa4 page);
  * invariances (varlen equals per-sequence dense; seqused_k equals truncation
    with NaN padding; GQA equals repeated-KV MHA; split + combine equals the
    unsplit result);
  * exhaustive widening of every finite 16-bit pattern by torch / numpy.

The same pins are run against deliberately broken copies of the oracle source
(tests/test_oracle_mutants.py) to show that each plausible mistake is caught.
"""
from __future__ import annotations

import math
import os

import numpy as np
import scipy.special
import torch
import torch.nn.functional as F
from torch.nn.attention.bias import causal_lower_right

from workloads import gen

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
NAN16 = {"bf16": 0x7FC0, "fp16": 0x7E00}


def widen(bits: np.ndarray, dtype: str) -> np.ndarray:
    """16-bit patterns -> float64 through torch / numpy conversions."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    if dtype == "bf16":
        t = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16)
        return t.to(torch.float64).numpy()
    return bits.view(np.float16).astype(np.float64)


def rand_bits(rng, shape, dtype, std=1.0):
    return gen.normal_bits(rng, shape, dtype, std)


def sdpa_rows(qf, kf, vf, scale, visible, add=None):
    """One sequence through torch SDPA (float64, CPU).

    qf [Sq, Hq, D], kf/vf [Sk, Hkv, *] float64; visible: bool [Sq, Sk] or None;
    add: float [Hq, Sq, Sk] additive score term or None.
    Returns O [Sq, Hq, Dv] and LSE [Hq, Sq] (scipy logsumexp of the masked scores).
    """
    Sq, Hq, _ = qf.shape
    Hkv = kf.shape[1]
    scale = float(np.float32(scale))  # the scale crosses the boundary as a float32
    q = torch.from_numpy(qf).permute(1, 0, 2)[None]
    k = torch.from_numpy(kf).permute(1, 0, 2)[None]
    v = torch.from_numpy(vf).permute(1, 0, 2)[None]
    Sk = kf.shape[0]
    if visible is None:
        visible = np.ones((Sq, Sk), dtype=bool)
    mask = np.where(visible[None], 0.0, -np.inf) * np.ones((Hq, 1, 1))
    if add is not None:
        mask = mask + add
    m = torch.from_numpy(mask)[None]
    o = F.scaled_dot_product_attention(q, k, v, attn_mask=m, scale=float(scale),
                                       enable_gqa=(Hq != Hkv))
    O = o[0].permute(1, 0, 2).numpy()
    G = Hq // Hkv
    kr = np.repeat(kf, G, axis=1)  # head h uses kv head h // G
    sc = float(scale) * np.einsum("ihd,jhd->hij", qf, kr) + mask
    with np.errstate(invalid="ignore"):
        L = scipy.special.logsumexp(sc, axis=-1)
    return O, L


def _check(a, b, tol, what):
    a = np.asarray(a)
    b = np.asarray(b)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    fin = np.isfinite(b)
    assert np.array_equal(np.isfinite(a), fin), f"{what}: finiteness differs"
    assert np.array_equal(a[~fin], b[~fin]), f"{what}: non-finite values differ"
    if fin.any():
        err = np.max(np.abs(a[fin] - b[fin]))
        assert err <= tol, f"{what}: max abs err {err:.3e} > {tol:.1e}"


def _dense_case(orc, rng, dtype, B, Sq, Sk, Hq, Hkv, D, Dv, scale, causal, tol=1e-12):
    q = rand_bits(rng, (B, Sq, Hq, D), dtype)
    k = rand_bits(rng, (B, Sk, Hkv, D), dtype)
    v = rand_bits(rng, (B, Sk, Hkv, Dv), dtype)
    O, L = orc.attn_full(q, k, v, dtype=dtype, B=B, Sq=Sq, Sk=Sk, Hq=Hq, Hkv=Hkv, D=D, Dv=Dv,
                         scale=scale, causal=causal, threads=2)
    vis = causal_lower_right(Sq, Sk)._materialize().numpy() if causal else None
    for b in range(B):
        Or, Lr = sdpa_rows(widen(q[b], dtype), widen(k[b], dtype), widen(v[b], dtype), scale, vis)
        _check(O[b], Or, tol, f"O dense b={b} causal={causal} {dtype}")
        _check(L[b], Lr, tol, f"LSE dense b={b} causal={causal} {dtype}")


def pin_sdpa_dense(orc):
    """Plain, causal (q_len <, =, > k_len) and GQA cases against SDPA + logsumexp."""
    rng = gen.make_rng(1001)
    for dtype in ("bf16", "fp16"):
        _dense_case(orc, rng, dtype, 2, 7, 11, 4, 2, 16, 8, 0.3, False)
        _dense_case(orc, rng, dtype, 2, 7, 11, 4, 2, 16, 8, 0.3, True)
        _dense_case(orc, rng, dtype, 1, 9, 9, 3, 3, 8, 8, 0.25, True)
        _dense_case(orc, rng, dtype, 1, 11, 6, 6, 2, 8, 12, 0.7, True)   # empty leading rows
        _dense_case(orc, rng, dtype, 1, 5, 13, 8, 1, 32, 16, 0.125, False)


def pin_varlen(orc):
    """varlen packing equals running each sequence alone (SDPA), including empty sequences."""
    rng = gen.make_rng(1002)
    dtype = "bf16"
    Hq, Hkv, D, Dv = 4, 2, 16, 16
    qlens = [5, 0, 9, 3, 4]
    klens = [8, 3, 9, 0, 2]
    cuq = gen.cu_seqlens(qlens)
    cuk = gen.cu_seqlens(klens)
    Tq, Tk = int(cuq[-1]), int(cuk[-1])
    q = rand_bits(rng, (Tq, Hq, D), dtype)
    k = rand_bits(rng, (Tk, Hkv, D), dtype)
    v = rand_bits(rng, (Tk, Hkv, Dv), dtype)
    for causal in (False, True):
        O, L = orc.attn_full(q, k, v, dtype=dtype, B=len(qlens), Sq=Tq, Sk=Tk, Hq=Hq, Hkv=Hkv,
                             D=D, Dv=Dv, scale=0.5, causal=causal, cu_seqlens_q=cuq,
                             cu_seqlens_k=cuk, threads=2)
        for b, (ql, kl) in enumerate(zip(qlens, klens)):
            if ql == 0:
                continue
            sq = slice(cuq[b], cuq[b + 1])
            sk = slice(cuk[b], cuk[b + 1])
            if kl == 0:
                assert np.all(O[sq] == 0.0) and np.all(L[:, sq] == -np.inf), "empty keys"
                continue
            vis = causal_lower_right(ql, kl)._materialize().numpy() if causal else None
            Or, Lr = sdpa_rows(widen(q[sq], dtype), widen(k[sk], dtype), widen(v[sk], dtype),
                               0.5, vis)
            _check(O[sq], Or, 1e-12, f"O varlen b={b} causal={causal}")
            _check(L[:, sq], Lr, 1e-12, f"LSE varlen b={b} causal={causal}")


def pin_seqused(orc):
    """seqused_k equals truncating K/V; NaN padding past it has no influence."""
    rng = gen.make_rng(1003)
    dtype = "fp16"
    B, Sq, Sk, Hq, Hkv, D, Dv = 3, 6, 12, 2, 1, 16, 16
    used = np.array([12, 5, 0], dtype=np.int32)
    q = rand_bits(rng, (B, Sq, Hq, D), dtype)
    k = rand_bits(rng, (B, Sk, Hkv, D), dtype)
    v = rand_bits(rng, (B, Sk, Hkv, Dv), dtype)
    for b in range(B):
        k[b, used[b]:] = NAN16[dtype]
        v[b, used[b]:] = NAN16[dtype]
    for causal in (False, True):
        O, L = orc.attn_full(q, k, v, dtype=dtype, B=B, Sq=Sq, Sk=Sk, Hq=Hq, Hkv=Hkv, D=D,
                             Dv=Dv, scale=0.25, causal=causal, seqused_k=used, threads=2)
        assert np.all(np.isfinite(O)), "NaN padding leaked"
        for b in range(B):
            kl = int(used[b])
            if kl == 0:
                assert np.all(O[b] == 0.0) and np.all(L[b] == -np.inf), "seqused_k = 0"
                continue
            vis = causal_lower_right(Sq, kl)._materialize().numpy() if causal else None
            Or, Lr = sdpa_rows(widen(q[b], dtype), widen(k[b, :kl], dtype),
                               widen(v[b, :kl], dtype), 0.25, vis)
            _check(O[b], Or, 1e-12, f"O seqused b={b} causal={causal}")
            _check(L[b], Lr, 1e-12, f"LSE seqused b={b} causal={causal}")


def _band_add(bias_f, q_len, k_len, E):
    """Additive score term [Hq, q_len, k_len] by enumerating every (i, j) pair of the band."""
    Hq = bias_f.shape[1]
    add = np.zeros((Hq, q_len, k_len))
    for i in range(q_len):
        for j in range(k_len):
            d = i + (k_len - q_len) - j
            if 0 <= d < E:
                add[:, i, j] = bias_f[i, :, d]
    return add


def pin_rel_bias_sdpa(orc):
    """rel_bias as an additive SDPA mask, causal and not, q_len <, =, > k_len, varlen."""
    rng = gen.make_rng(1004)
    dtype = "bf16"
    Hq, Hkv, D, Dv, E = 4, 2, 16, 8, 5
    qlens = [7, 9, 4]
    klens = [7, 4, 11]
    cuq = gen.cu_seqlens(qlens)
    cuk = gen.cu_seqlens(klens)
    Tq, Tk = int(cuq[-1]), int(cuk[-1])
    q = rand_bits(rng, (Tq, Hq, D), dtype)
    k = rand_bits(rng, (Tk, Hkv, D), dtype)
    v = rand_bits(rng, (Tk, Hkv, Dv), dtype)
    rb = rand_bits(rng, (Tq, Hq, E), dtype, 0.5)
    for causal in (False, True):
        O, L = orc.attn_full(q, k, v, dtype=dtype, B=3, Sq=Tq, Sk=Tk, Hq=Hq, Hkv=Hkv, D=D,
                             Dv=Dv, scale=0.35, causal=causal, cu_seqlens_q=cuq,
                             cu_seqlens_k=cuk, rel_bias=rb, threads=2)
        for b, (ql, kl) in enumerate(zip(qlens, klens)):
            sq = slice(cuq[b], cuq[b + 1])
            sk = slice(cuk[b], cuk[b + 1])
            vis = causal_lower_right(ql, kl)._materialize().numpy() if causal else None
            add = _band_add(widen(rb[sq], dtype), ql, kl, E)
            Or, Lr = sdpa_rows(widen(q[sq], dtype), widen(k[sk], dtype), widen(v[sk], dtype),
                               0.35, vis, add)
            _check(O[sq], Or, 1e-12, f"O bias b={b} causal={causal}")
            _check(L[:, sq], Lr, 1e-12, f"LSE bias b={b} causal={causal}")


def _read_band_golden():
    L = E = None
    index, extent = {}, {}
    with open(os.path.join(GOLDEN, "rel_bias_band_causal_self.txt")) as f:
        for line in f:
            line = line.split("#")[0].split()
            if not line:
                continue
            if line[0] == "L":
                L = int(line[1])
            elif line[0] == "E":
                E = int(line[1])
            elif line[0] == "index":
                index[(int(line[1]), int(line[2]))] = None if line[3] == "-" else int(line[3])
            elif line[0] == "extent":
                extent[int(line[1])] = sorted(int(x) for x in line[2:])
    return L, E, index, extent


def _boosted_keys(o_row, lse, n_vis):
    """Keys whose score carries the +30 probe bias.

    With q = k = 0 every unbiased score is 0; V rows are one-hot, so
    O[i, j] * exp(LSE) = exp(s_j) is 1 for an unbiased key and e^30 for a biased one.
    """
    es = np.asarray(o_row[:n_vis]) * math.exp(lse)
    return sorted(int(j) for j in np.nonzero(es > 1000.0)[0])


def pin_rel_bias_golden(orc):
    """The band's meaning in causal self-attention, from the hand-written fixture."""
    L, E, index, extent = _read_band_golden()
    dtype = "bf16"
    one = gen.f32_to_bf16_bits(np.float32(1.0)).item()
    thirty = gen.f32_to_bf16_bits(np.float32(30.0)).item()
    q = np.zeros((1, L, 1, 8), dtype=np.uint16)
    k = np.zeros((1, L, 1, 8), dtype=np.uint16)
    v = np.zeros((1, L, 1, L), dtype=np.uint16)
    for j in range(L):
        v[0, j, 0, j] = one
    rows = np.array([[0, 0, i] for i in range(L)], dtype=np.int32)
    kw = dict(dtype=dtype, B=1, Sq=L, Sk=L, Hq=1, Hkv=1, D=8, Dv=L, scale=1.0, causal=True,
              rows=rows, threads=1)
    for (i, d), j in index.items():
        rb = np.zeros((L, 1, E), dtype=np.uint16)
        rb[i, 0, d] = thirty
        O, lse = orc.attn_rows(q, k, v, rel_bias=rb, **kw)
        got = _boosted_keys(O[i], lse[i], i + 1)
        assert got == ([] if j is None else [j]), f"golden index: i={i} d={d} want {j} got {got}"
    rb = np.full((L, 1, E), thirty, dtype=np.uint16)
    O, lse = orc.attn_rows(q, k, v, rel_bias=rb, **kw)
    for i, keys in extent.items():
        got = _boosted_keys(O[i], lse[i], i + 1)
        assert got == keys, f"golden extent: i={i} want {keys} got {got}"


def pin_closed_forms(orc):
    """Equal scores, causal row 0, dominant score, empty rows."""
    rng = gen.make_rng(1005)
    for dtype in ("bf16", "fp16"):
        B, Sq, Sk, Hq, Hkv, D, Dv = 1, 6, 9, 2, 2, 16, 8
        # (i) q = 0: every visible score is 0 -> O = mean of visible V rows, LSE = ln n_vis
        q = np.zeros((B, Sq, Hq, D), dtype=np.uint16)
        k = rand_bits(rng, (B, Sk, Hkv, D), dtype)
        v = rand_bits(rng, (B, Sk, Hkv, Dv), dtype)
        for causal in (False, True):
            O, L = orc.attn_full(q, k, v, dtype=dtype, B=B, Sq=Sq, Sk=Sk, Hq=Hq, Hkv=Hkv, D=D,
                                 Dv=Dv, scale=0.5, causal=causal, threads=1)
            vf = widen(v[0], dtype)
            for i in range(Sq):
                n = (i + (Sk - Sq) + 1) if causal else Sk
                for h in range(Hq):
                    want = vf[:n, h].mean(axis=0)
                    assert np.max(np.abs(O[0, i, h] - want)) <= 1e-14, "mean-of-V closed form"
                    assert L[0, h, i] == math.log(n), "LSE = ln n closed form"
        # (ii) causal, q_len = k_len: row 0 sees only key 0 -> O = v0, LSE = s00
        q = rand_bits(rng, (B, 5, Hq, D), dtype)
        k = rand_bits(rng, (B, 5, Hkv, D), dtype)
        v = rand_bits(rng, (B, 5, Hkv, Dv), dtype)
        O, L = orc.attn_full(q, k, v, dtype=dtype, B=B, Sq=5, Sk=5, Hq=Hq, Hkv=Hkv, D=D, Dv=Dv,
                             scale=0.125, causal=True, threads=1)
        for h in range(Hq):
            assert np.array_equal(O[0, 0, h], widen(v[0, 0, h], dtype)), "causal row 0 = v0"
            s00 = 0.125 * float(np.dot(widen(q[0, 0, h], dtype), widen(k[0, 0, h], dtype)))
            assert abs(L[0, h, 0] - s00) <= 1e-13, "causal row 0 LSE = s00"
        # (iii) one dominant score selects one V row
        q = np.zeros((1, 4, 1, D), dtype=np.uint16)
        k = np.zeros((1, 7, 1, D), dtype=np.uint16)
        v = rand_bits(rng, (1, 7, 1, Dv), dtype)
        rb = np.zeros((4, 1, 3), dtype=np.uint16)
        big = gen.to_bits(np.float32(1000.0), dtype).item()
        rb[:, 0, 2] = big          # d = 2 -> key j = i + 3 - 2 = i + 1
        O, L = orc.attn_full(q, k, v, dtype=dtype, B=1, Sq=4, Sk=7, Hq=1, Hkv=1, D=D, Dv=Dv,
                             scale=1.0, causal=False, rel_bias=rb, threads=1)
        for i in range(4):
            assert np.array_equal(O[0, i, 0], widen(v[0, i + 1, 0], dtype)), "dominant score"
            assert abs(L[0, 0, i] - 1000.0) < 1e-9, "dominant LSE"
        # (v) empty rows: causal with q_len > k_len, rows i < q_len - k_len see nothing
        q = rand_bits(rng, (1, 8, 1, D), dtype)
        k = rand_bits(rng, (1, 3, 1, D), dtype)
        v = rand_bits(rng, (1, 3, 1, Dv), dtype)
        O, L = orc.attn_full(q, k, v, dtype=dtype, B=1, Sq=8, Sk=3, Hq=1, Hkv=1, D=D, Dv=Dv,
                             scale=0.3, causal=True, threads=1)
        assert np.all(O[0, :5] == 0.0) and np.all(L[0, 0, :5] == -np.inf), "empty rows"
        assert np.all(np.isfinite(L[0, 0, 5:])), "first visible row"
        assert np.array_equal(O[0, 5, 0], widen(v[0, 0, 0], dtype)), "first visible row sees k0"


def pin_gqa_repeat(orc):
    """GQA equals MHA with each KV head repeated for its G consecutive query heads."""
    rng = gen.make_rng(1006)
    dtype = "bf16"
    B, Sq, Sk, Hq, Hkv, D, Dv = 2, 5, 8, 6, 2, 16, 16
    G = Hq // Hkv
    q = rand_bits(rng, (B, Sq, Hq, D), dtype)
    k = rand_bits(rng, (B, Sk, Hkv, D), dtype)
    v = rand_bits(rng, (B, Sk, Hkv, Dv), dtype)
    kr = np.repeat(k, G, axis=2)
    vr = np.repeat(v, G, axis=2)
    kw = dict(dtype=dtype, B=B, Sq=Sq, Sk=Sk, Hq=Hq, D=D, Dv=Dv, scale=0.2, causal=True,
              threads=1)
    O1, L1 = orc.attn_full(q, k, v, Hkv=Hkv, **kw)
    O2, L2 = orc.attn_full(q, kr, vr, Hkv=Hq, **kw)
    assert np.array_equal(O1, O2) and np.array_equal(L1, L2), "GQA != repeated MHA"


def pin_split_combine(orc):
    """Key-range splits merged by LSE weights equal the unsplit result; combine closed forms."""
    rng = gen.make_rng(1007)
    dtype = "fp16"
    B, Sq, Sk, Hq, Hkv, D, Dv = 1, 6, 17, 2, 1, 16, 8
    q = rand_bits(rng, (B, Sq, Hq, D), dtype)
    k = rand_bits(rng, (B, Sk, Hkv, D), dtype)
    v = rand_bits(rng, (B, Sk, Hkv, Dv), dtype)
    rb = rand_bits(rng, (B * Sq, Hq, 4), dtype, 0.5)
    rows = np.array([[0, h, i] for h in range(Hq) for i in range(Sq)], dtype=np.int32)
    kw = dict(dtype=dtype, B=B, Sq=Sq, Sk=Sk, Hq=Hq, Hkv=Hkv, D=D, Dv=Dv, scale=0.4,
              causal=True, rows=rows, rel_bias=rb, threads=1)
    o_full, l_full = orc.attn_rows(q, k, v, **kw)
    bounds = [0, 3, 3, 10, 12, Sk]
    parts = [orc.attn_rows(q, k, v, key_lo=a, key_hi=b, **kw) for a, b in zip(bounds, bounds[1:])]
    o_parts = np.stack([p[0] for p in parts])
    l_parts = np.stack([p[1] for p in parts])
    assert np.all(l_parts[1] == -np.inf) and np.all(o_parts[1] == 0.0), "empty split"
    o_c, l_c = orc.combine(o_parts, l_parts)
    _check(o_c, o_full, 1e-12, "split+combine O")
    _check(l_c, l_full, 1e-12, "split+combine LSE")
    # merged LSE is numpy's logaddexp over the pieces
    with np.errstate(invalid="ignore"):
        want = np.logaddexp.reduce(l_parts, axis=0)
    _check(l_c, want, 1e-12, "combine LSE = logaddexp")
    # one split is the identity; all-empty gives (0, -inf)
    o1, l1 = orc.combine(o_full[None], l_full[None])
    assert np.array_equal(o1, o_full) and np.array_equal(l1, l_full), "combine of one split"
    oe, le = orc.combine(np.zeros((3, 2, Dv)), np.full((3, 2), -np.inf))
    assert np.all(oe == 0.0) and np.all(le == -np.inf), "all-empty combine"


def pin_widening(orc):
    """Every finite 16-bit value is widened exactly (Sk = 1 and zero scores give O = v0)."""
    for dtype in ("bf16", "fp16"):
        allbits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
        f = widen(allbits, dtype)
        fin = allbits[np.isfinite(f)]
        Dv = fin.size
        q = np.zeros((1, 1, 1, 8), dtype=np.uint16)
        k = np.zeros((1, 1, 1, 8), dtype=np.uint16)
        v = fin.reshape(1, 1, 1, Dv)
        O, L = orc.attn_full(q, k, v, dtype=dtype, B=1, Sq=1, Sk=1, Hq=1, Hkv=1, D=8, Dv=Dv,
                             scale=1.0, causal=False, threads=1)
        assert np.array_equal(O[0, 0, 0], widen(fin, dtype)), f"widening {dtype}"
        assert L[0, 0, 0] == 0.0


def pin_rel_proj(orc):
    """The rel_bias producer (r . rel_proj): torch's float64 einsum stored through
    float32 into the dtype; a one-hot r picks a row of rel_proj exactly."""
    from oracle.oracle import rel_bias_from_proj
    rng = gen.make_rng(1010)
    for dtype, tdt in (("bf16", torch.bfloat16), ("fp16", torch.float16)):
        r = rand_bits(rng, (7, 3, 24), dtype)
        pj = rand_bits(rng, (24, 128), dtype, 0.2)
        got = rel_bias_from_proj(r, pj, dtype)
        ref = torch.einsum("thd,de->the", torch.from_numpy(widen(r, dtype)),
                           torch.from_numpy(widen(pj, dtype))).to(torch.float32).to(tdt)
        ref_bits = ref.view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(got, ref_bits), f"rel_proj product {dtype}"
        one = np.zeros((2, 1, 24), dtype=np.float32)
        one[0, 0, 5] = 1.0
        one[1, 0, 23] = 1.0
        one_bits = torch.from_numpy(one).to(tdt).view(torch.int16).numpy().view(np.uint16)
        rows = rel_bias_from_proj(one_bits, pj, dtype)
        assert np.array_equal(rows[0, 0], pj[5]) and np.array_equal(rows[1, 0], pj[23]), "one-hot r"


ALL_PINS = [pin_sdpa_dense, pin_varlen, pin_seqused, pin_rel_bias_sdpa, pin_rel_bias_golden,
            pin_closed_forms, pin_gqa_repeat, pin_split_combine, pin_widening, pin_rel_proj]


def run_all(orc):
    """Run every pin; return the names of those that failed (used by the mutant test)."""
    failed = []
    for p in ALL_PINS:
        try:
            p(orc)
        except Exception:  # an assertion, or arithmetic blowing up on a broken oracle
            failed.append(p.__name__)
    return failed
