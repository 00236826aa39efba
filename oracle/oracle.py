"""ctypes front end of the fp64 CPU oracle (``attn_oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
benchmark's CPU-baseline leg, never by the library's product path. It shares
no code with the GPU library.

All 16-bit tensors are passed as numpy ``uint16`` bit patterns; ``dtype`` is
"bf16" or "fp16". Layouts are the attention forward's own:
  dense  q [B, Sq, Hq, D], k [B, Sk, Hkv, D], v [B, Sk, Hkv, Dv]
  varlen q [total_q, Hq, D], k [total_k, Hkv, D], v [total_k, Hkv, Dv]
  rel_bias [rows_q, Hq, E] flattened like q
Output rows are addressed by triples (b, h, i).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "attn_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

DTYPE_CODE = {"bf16": 0, "fp16": 1}


def build(force: bool = True, src: str = _SRC, out: str = _LIB) -> str:
    """Compile the oracle with gcc (-O2, OpenMP). Returns the library path."""
    if force or not os.path.exists(out) or os.path.getmtime(out) < os.path.getmtime(src):
        tmp = out + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                               "-Wall", "-Wextra", "-o", tmp, src, "-lm"])
        os.replace(tmp, out)
    return out


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def default_threads() -> int:
    return os.cpu_count() or 1


class OracleLib:
    """One loaded copy of the compiled oracle (the default one, or a test's variant)."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        P = ctypes.c_void_p
        i = ctypes.c_int
        ll = ctypes.c_longlong
        lib.oracle_attn_rows.argtypes = [P, P, P, i, i, i, i, i, i, i, i, ctypes.c_float, i,
                                         P, P, P, P, i, ll, ll, ll, P, P, P, i]
        lib.oracle_attn_rows.restype = i
        lib.oracle_combine.argtypes = [P, P, i, ll, i, P, P]
        lib.oracle_combine.restype = i
        self.lib = lib
        self.path = path

    def attn_rows(self, q, k, v, *, dtype: str, B: int, Sq: int, Sk: int, Hq: int, Hkv: int,
                  D: int, Dv: int, scale: float, causal: bool, rows: np.ndarray,
                  cu_seqlens_q=None, cu_seqlens_k=None, seqused_k=None, rel_bias=None,
                  key_lo: int = 0, key_hi: int = 1 << 62, threads: Optional[int] = None):
        """O (n x Dv, float64) and LSE (n, float64) of the given (b, h, i) rows."""
        q = np.ascontiguousarray(q, dtype=np.uint16)
        k = np.ascontiguousarray(k, dtype=np.uint16)
        v = np.ascontiguousarray(v, dtype=np.uint16)
        rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int32).reshape(-1, 3))
        cuq = None if cu_seqlens_q is None else np.ascontiguousarray(cu_seqlens_q, dtype=np.int32)
        cuk = None if cu_seqlens_k is None else np.ascontiguousarray(cu_seqlens_k, dtype=np.int32)
        su = None if seqused_k is None else np.ascontiguousarray(seqused_k, dtype=np.int32)
        rb = None if rel_bias is None else np.ascontiguousarray(rel_bias, dtype=np.uint16)
        E = 0 if rb is None else int(rb.shape[-1])
        n = rows.shape[0]
        o = np.zeros((n, Dv), dtype=np.float64)
        lse = np.zeros(n, dtype=np.float64)
        rc = self.lib.oracle_attn_rows(
            _ptr(q), _ptr(k), _ptr(v), DTYPE_CODE[dtype], B, Sq, Sk, Hq, Hkv, D, Dv,
            float(scale), int(bool(causal)), _ptr(cuq), _ptr(cuk), _ptr(su), _ptr(rb), E,
            int(key_lo), int(key_hi), n, _ptr(rows), _ptr(o), _ptr(lse),
            int(threads or default_threads()))
        if rc != 0:
            raise ValueError(f"oracle_attn_rows failed with code {rc}")
        return o, lse

    def combine(self, o_parts: np.ndarray, lse_parts: np.ndarray):
        """LSE-weighted merge of split partials: o_parts [ns, n, Dv], lse_parts [ns, n]."""
        o_parts = np.ascontiguousarray(o_parts, dtype=np.float64)
        lse_parts = np.ascontiguousarray(lse_parts, dtype=np.float64)
        ns, n, Dv = o_parts.shape
        o = np.zeros((n, Dv), dtype=np.float64)
        lse = np.zeros(n, dtype=np.float64)
        rc = self.lib.oracle_combine(_ptr(o_parts), _ptr(lse_parts), ns, n, Dv, _ptr(o),
                                     _ptr(lse))
        if rc != 0:
            raise ValueError(f"oracle_combine failed with code {rc}")
        return o, lse

    def attn_full(self, q, k, v, *, dtype, B, Sq, Sk, Hq, Hkv, D, Dv, scale, causal,
                  cu_seqlens_q=None, cu_seqlens_k=None, seqused_k=None, rel_bias=None,
                  threads=None):
        """The whole forward in the library's output layouts (float64).

        O: dense [B, Sq, Hq, Dv], varlen [total_q, Hq, Dv].
        LSE: dense [B, Hq, Sq], varlen [Hq, total_q].
        """
        ql, _ = seq_lengths(B, Sq, Sk, cu_seqlens_q, cu_seqlens_k, seqused_k)
        rows = all_rows(B, Hq, ql)
        o_rows, l_rows = self.attn_rows(q, k, v, dtype=dtype, B=B, Sq=Sq, Sk=Sk, Hq=Hq,
                                        Hkv=Hkv, D=D, Dv=Dv, scale=scale, causal=causal,
                                        rows=rows, cu_seqlens_q=cu_seqlens_q,
                                        cu_seqlens_k=cu_seqlens_k, seqused_k=seqused_k,
                                        rel_bias=rel_bias, threads=threads)
        b = rows[:, 0].astype(np.int64)
        h = rows[:, 1].astype(np.int64)
        i = rows[:, 2].astype(np.int64)
        if cu_seqlens_q is not None:
            T = int(np.asarray(cu_seqlens_q)[-1])
            t = np.asarray(cu_seqlens_q, dtype=np.int64)[b] + i
            O = np.zeros((T, Hq, Dv))
            O[t, h] = o_rows
            L = np.full((Hq, T), -np.inf)
            L[h, t] = l_rows
        else:
            O = np.zeros((B, Sq, Hq, Dv))
            O[b, i, h] = o_rows
            L = np.full((B, Hq, Sq), -np.inf)
            L[b, h, i] = l_rows
        return O, L


def default() -> OracleLib:
    """The oracle built from attn_oracle.c (compiled on first use)."""
    global _lib
    if _lib is None:
        _lib = OracleLib(build(force=False))
    return _lib


def attn_rows(*args, **kw):
    return default().attn_rows(*args, **kw)


def combine(*args, **kw):
    return default().combine(*args, **kw)


def attn_full(*args, **kw):
    return default().attn_full(*args, **kw)


def widen16(bits: np.ndarray, dtype: str) -> np.ndarray:
    """16-bit patterns -> float64 (exact)."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    if dtype == "bf16":
        return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return bits.view(np.float16).astype(np.float64)


def narrow16(x: np.ndarray, dtype: str) -> np.ndarray:
    """float64 -> float32 -> 16-bit patterns, each step rounding to nearest even (the
    path of a product accumulated in fp32 and stored in the 16-bit dtype)."""
    x32 = np.ascontiguousarray(np.asarray(x, dtype=np.float64).astype(np.float32))
    if dtype == "bf16":
        u = x32.view(np.uint32).astype(np.uint64)
        return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    return x32.astype(np.float16).view(np.uint16)


def rel_bias_from_proj(r: np.ndarray, rel_proj: np.ndarray, dtype: str) -> np.ndarray:
    """rel_bias [rows, H, E] = r [rows, H, d_rel] . rel_proj [d_rel, E], the einsum the
    tml-fa4 page applies before the call, summed in fp64 and stored in the dtype."""
    rows, H, d_rel = r.shape
    prod = widen16(r, dtype).reshape(rows * H, d_rel) @ widen16(rel_proj, dtype)
    return narrow16(prod.reshape(rows, H, rel_proj.shape[1]), dtype)


def seq_lengths(B, Sq, Sk, cu_seqlens_q=None, cu_seqlens_k=None, seqused_k=None):
    """Per-batch (q_len, k_len) lists under the oracle's length rules."""
    if cu_seqlens_q is not None:
        ql = np.diff(np.asarray(cu_seqlens_q, dtype=np.int64))
        kl = np.diff(np.asarray(cu_seqlens_k, dtype=np.int64))
    else:
        ql = np.full(B, Sq, dtype=np.int64)
        kl = np.full(B, Sk, dtype=np.int64)
    if seqused_k is not None:
        kl = np.asarray(seqused_k, dtype=np.int64).copy()
    return ql, kl


def all_rows(B, Hq, q_lens) -> np.ndarray:
    """Every (b, h, i) triple."""
    out = []
    for b in range(B):
        ql = int(q_lens[b])
        if ql == 0:
            continue
        bb = np.full(ql * Hq, b, dtype=np.int32)
        hh = np.repeat(np.arange(Hq, dtype=np.int32), ql)
        ii = np.tile(np.arange(ql, dtype=np.int32), Hq)
        out.append(np.stack([bb, hh, ii], axis=1))
    if not out:
        return np.zeros((0, 3), dtype=np.int32)
    return np.concatenate(out, axis=0)

