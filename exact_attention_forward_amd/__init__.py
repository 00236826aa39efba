"""MI355X exact attention forward: Python binding of the C ABI in include/attn.h.

Argument marshalling only. Every step of the forward runs in the gfx950 HIP
kernels of libmi355attn.so; torch supplies device memory and the stream.
There is no fallback: if the library is missing or a call is rejected, an
exception is raised.

    out, lse = attn_fwd(q, k, v, causal=True)                    # dense [B, S, H, D]
    out, lse = attn_fwd(q, k, v, cu_seqlens_q=cu, cu_seqlens_k=cu,
                        max_seqlen_q=m, max_seqlen_k=m, rel_bias=rb, causal=True)  # varlen
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmi355attn.so")

ATTN_BF16 = 0
ATTN_FP16 = 1
MAX_SPLITS = 256

STATUS = {
    0: "ATTN_OK", 1: "ATTN_ERR_NULL_POINTER", 2: "ATTN_ERR_BAD_SHAPE", 3: "ATTN_ERR_BAD_DTYPE",
    4: "ATTN_ERR_UNSUPPORTED_HEAD_DIM", 5: "ATTN_ERR_BAD_GQA", 6: "ATTN_ERR_BAD_REL_EXTENT",
    7: "ATTN_ERR_BAD_VARLEN", 8: "ATTN_ERR_MISALIGNED", 9: "ATTN_ERR_WORKSPACE",
    10: "ATTN_ERR_UNSUPPORTED_COMBO", 11: "ATTN_ERR_HIP", 12: "ATTN_ERR_BAD_SPLITS",
    13: "ATTN_ERR_BAD_SCALE", 14: "ATTN_ERR_BAD_ARG",
}
CODE = {v: k for k, v in STATUS.items()}

# The exported symbols and their C signatures (kept in step with include/attn.h).
_P = ctypes.c_void_p
_I = ctypes.c_int
_F = ctypes.c_float
_Z = ctypes.c_size_t
SIGNATURES = {
    "attn_fwd": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F, _I, _P, _P, _I, _I, _P,
                      _P, _I, _I, _I, _I, _P, _Z, _P]),
    "attn_fwd_rel_proj": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F, _I, _P, _P, _I, _I,
                               _P, _P, _P, _I, _I, _I, _I, _I, _P, _Z, _P]),
    "attn_check_args": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F, _I, _P, _P, _I, _I,
                             _P, _P, _I, _I, _I, _I, _P, _Z]),
    "attn_num_splits": (_I, [_I, _I, _I, _I, _I, _I, _I, _I, _I, _I, _I, _I]),
    "attn_fwd_workspace_size": (_Z, [_I, _I, _I, _I, _I, _I]),
    "attn_combine": (_I, [_P, _P, _I, _P, _P, _I, _I, _I, _I, _I, _I, _P]),
    "attn_status_string": (ctypes.c_char_p, [_I]),
    "attn_version": (ctypes.c_char_p, []),
}

_lib = None


class AttnError(RuntimeError):
    """A call rejected by the library (status != ATTN_OK)."""

    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


def load(path: str = LIB_PATH):
    """Load libmi355attn.so (built by exact_attention_forward_amd.build); raise if it is missing."""
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m exact_attention_forward_amd.build` "
                           "(there is no fallback implementation)")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if path == LIB_PATH:
        _lib = lib
    return lib


def status_string(code: int) -> str:
    return load().attn_status_string(code).decode()


def version() -> str:
    return load().attn_version().decode()


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return ATTN_BF16
    if t.dtype == torch.float16:
        return ATTN_FP16
    raise AttnError(CODE["ATTN_ERR_BAD_DTYPE"], f"dtype {t.dtype} is not bfloat16/float16")


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _check(status: int):
    if status != 0:
        raise AttnError(status, status_string(status))


def _stream_handle(stream, device):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream


def num_splits(B, Sq, Sk, Hq, Hkv, D, Dv, *, is_varlen=False, max_seqlen_q=0, max_seqlen_k=0,
               pack_gqa=-1, requested=0) -> int:
    """Split count attn_fwd uses (requested <= 0: the heuristic)."""
    return load().attn_num_splits(B, Sq, Sk, Hq, Hkv, D, Dv, int(bool(is_varlen)), max_seqlen_q,
                                  max_seqlen_k, pack_gqa, requested)


def workspace_size(B, Sq, Hq, Dv, *, is_varlen=False, splits=1) -> int:
    return load().attn_fwd_workspace_size(B, Sq, Hq, Dv, int(bool(is_varlen)), splits)


def attn_fwd(q, k, v, *, causal: bool = False, scale: Optional[float] = None,
             cu_seqlens_q=None, cu_seqlens_k=None, max_seqlen_q: Optional[int] = None,
             max_seqlen_k: Optional[int] = None, seqused_k=None, rel_bias=None,
             num_splits: int = 1, pack_gqa: int = -1, out=None, lse=None,
             return_lse: bool = True, workspace=None, stream=None, rel_r=None, rel_proj=None):
    """Fused attention forward. Returns (out, lse); lse is None if return_lse is False.

    Dense: q [B, Sq, Hq, D], k/v [B, Sk, Hkv, D]; lse [B, Hq, Sq].
    Varlen: q [total_q, Hq, D], k/v [total_k, Hkv, D], cu_seqlens int32 [B+1]; lse [Hq, total_q].
    rel_r [rows_q, Hq, d_rel] with rel_proj [d_rel, E] (instead of rel_bias): the bias is their
    product, formed inside the kernel (attn_fwd_rel_proj).
    out / lse / workspace are allocated with torch when not given (the allocation-free
    form passes all three, as forward_static does).
    """
    import torch
    lib = load()
    varlen = cu_seqlens_q is not None or cu_seqlens_k is not None
    if varlen:
        if q.dim() != 3:
            raise ValueError("varlen q must be [total_q, Hq, D]")
        Sq, Hq, D = q.shape
        Sk, Hkv, _ = k.shape
        Dv = v.shape[-1]
        B = (cu_seqlens_q if cu_seqlens_q is not None else cu_seqlens_k).numel() - 1
        if max_seqlen_q is None or max_seqlen_k is None:
            raise ValueError("varlen needs max_seqlen_q and max_seqlen_k")
        out_shape = (Sq, Hq, Dv)
        lse_shape = (Hq, Sq)
    else:
        if q.dim() != 4:
            raise ValueError("dense q must be [B, Sq, Hq, D]")
        B, Sq, Hq, D = q.shape
        _, Sk, Hkv, _ = k.shape
        Dv = v.shape[-1]
        max_seqlen_q = max_seqlen_q or 0
        max_seqlen_k = max_seqlen_k or 0
        out_shape = (B, Sq, Hq, Dv)
        lse_shape = (B, Hq, Sq)
    for name, t in (("q", q), ("k", k), ("v", v), ("rel_bias", rel_bias)):
        if t is not None and not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if k.dtype != q.dtype or v.dtype != q.dtype or (rel_bias is not None and rel_bias.dtype != q.dtype):
        raise AttnError(CODE["ATTN_ERR_BAD_DTYPE"], "q, k, v and rel_bias must share one dtype")
    dtype = _dtype_code(q)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty(out_shape, dtype=q.dtype, device=q.device)
    if lse is None and return_lse:
        lse = torch.empty(lse_shape, dtype=torch.float32, device=q.device)
    if rel_r is not None or rel_proj is not None:
        if rel_bias is not None or rel_r is None or rel_proj is None:
            raise ValueError("pass rel_r with rel_proj, or rel_bias, not both")
        for name, t in (("rel_r", rel_r), ("rel_proj", rel_proj)):
            if not t.is_contiguous() or t.dtype != q.dtype:
                raise ValueError(f"{name} must be contiguous and of q's dtype")
    E = 0 if rel_bias is None else int(rel_bias.shape[-1])
    if rel_proj is not None:
        E = int(rel_proj.shape[1])
    ns = lib.attn_num_splits(B, Sq, Sk, Hq, Hkv, D, Dv, int(varlen), max_seqlen_q, max_seqlen_k,
                             pack_gqa, num_splits)
    ws_bytes = 0
    if ns > 1:
        ws_bytes = lib.attn_fwd_workspace_size(B, Sq, Hq, Dv, int(varlen), ns)
        if workspace is None:
            workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
        else:
            ws_bytes = workspace.numel() * workspace.element_size()
    if rel_r is not None:
        st = lib.attn_fwd_rel_proj(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, Sq, Sk, Hq, Hkv, D,
                                   Dv, float(scale), int(bool(causal)), _ptr(cu_seqlens_q),
                                   _ptr(cu_seqlens_k), max_seqlen_q, max_seqlen_k, _ptr(seqused_k),
                                   _ptr(rel_r), _ptr(rel_proj), int(rel_proj.shape[0]), E, num_splits,
                                   pack_gqa, dtype, _ptr(workspace), ws_bytes,
                                   _stream_handle(stream, q.device))
    else:
        st = lib.attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, Sq, Sk, Hq, Hkv, D, Dv,
                          float(scale), int(bool(causal)), _ptr(cu_seqlens_q), _ptr(cu_seqlens_k),
                          max_seqlen_q, max_seqlen_k, _ptr(seqused_k), _ptr(rel_bias), E, num_splits,
                          pack_gqa, dtype, _ptr(workspace), ws_bytes, _stream_handle(stream, q.device))
    _check(st)
    return out, (lse if return_lse else None)


def attn_combine(o_partial, lse_partial, *, out, lse=None, B: int, Sq: int, is_varlen: bool = False,
                 stream=None):
    """LSE-weighted merge of split partials (fp32) into out (bf16/fp16) and lse (fp32)."""
    lib = load()
    ns = o_partial.shape[0]
    Hq = o_partial.shape[-2]
    Dv = o_partial.shape[-1]
    st = lib.attn_combine(_ptr(o_partial), _ptr(lse_partial), ns, _ptr(out), _ptr(lse), B, Sq, Hq, Dv,
                          int(bool(is_varlen)), _dtype_code(out), _stream_handle(stream, out.device))
    _check(st)
    return out, lse
