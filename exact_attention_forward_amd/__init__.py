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
    13: "ATTN_ERR_BAD_SCALE", 14: "ATTN_ERR_BAD_ARG", 15: "ATTN_ERR_SCRATCH",
}
SCRATCH_BYTES = 16 << 20  # ATTN_SCRATCH_BYTES: split partials attn_fwd_noalloc can hold
CODE = {v: k for k, v in STATUS.items()}

# The exported symbols and their C signatures (kept in step with include/attn.h).
_P = ctypes.c_void_p
_I = ctypes.c_int
_F = ctypes.c_float
_Z = ctypes.c_size_t
SIGNATURES = {
    "attn_fwd": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F, _I, _P, _P, _I, _I, _P,
                      _P, _I, _I, _I, _I, _P, _Z, _P]),
    "attn_fwd_noalloc": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F, _I, _P, _P, _I, _I, _P,
                              _P, _I, _I, _I, _I, _P]),
    "attn_fwd_rel_proj": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F, _I, _P, _P, _I, _I,
                               _P, _P, _P, _I, _I, _I, _I, _I, _P, _Z, _P]),
    "attn_check_args": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F, _I, _P, _P, _I, _I,
                             _P, _P, _I, _I, _I, _I, _P, _Z]),
    "attn_num_splits": (_I, [_I, _I, _I, _I, _I, _I, _I, _I, _I, _I, _I, _I, _I]),
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
        # torch's current stream on the device, as a raw handle (without building a Stream object)
        raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
        if raw is not None:
            return raw(device.index if device.index is not None else torch.cuda.current_device())
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream


def num_splits(B, Sq, Sk, Hq, Hkv, D, Dv, *, causal=False, is_varlen=False, max_seqlen_q=0,
               max_seqlen_k=0, pack_gqa=-1, requested=0) -> int:
    """Split count attn_fwd uses (requested <= 0: the heuristic)."""
    return load().attn_num_splits(B, Sq, Sk, Hq, Hkv, D, Dv, int(bool(causal)), int(bool(is_varlen)),
                                  max_seqlen_q, max_seqlen_k, pack_gqa, requested)


def workspace_size(B, Sq, Hq, Dv, *, is_varlen=False, splits=1) -> int:
    return load().attn_fwd_workspace_size(B, Sq, Hq, Dv, int(bool(is_varlen)), splits)


def _require(cond, msg):
    if not cond:
        raise ValueError(msg)


def _check_tensors(q, k, v, *, varlen, B, Sq, Hq, D, cu_seqlens_q, cu_seqlens_k, seqused_k, rel_bias,
                   rel_r, rel_proj, out, lse, workspace, out_shape, lse_shape):
    """Shape, dtype, layout and device checks done before any pointer reaches the library
    (the C entry points see only pointers and sizes, so a wrong tensor would be read or
    written out of bounds). Messages are formed only for a failing check: this runs on
    every call, and short calls are dominated by host time."""
    import torch
    nd = 3 if varlen else 4
    if k.dim() != nd or v.dim() != nd:
        raise ValueError(f"k and v must have q's rank ({nd})")
    ks, vs = k.shape, v.shape
    if varlen:
        if ks[2] != D:
            raise ValueError(f"k {tuple(ks)} must be [total_k, Hkv, D={D}]")
        if vs[:2] != ks[:2]:
            raise ValueError(f"v {tuple(vs)} must be [total_k, Hkv, Dv] like k")
    else:
        if ks[0] != B or ks[3] != D:
            raise ValueError(f"k {tuple(ks)} must be [B={B}, Sk, Hkv, D={D}]")
        if vs[:3] != ks[:3]:
            raise ValueError(f"v {tuple(vs)} must be [B, Sk, Hkv, Dv] like k")
    i32 = torch.int32
    for name, t in (("cu_seqlens_q", cu_seqlens_q), ("cu_seqlens_k", cu_seqlens_k)):
        if t is not None and not (t.dtype == i32 and t.dim() == 1 and t.numel() == B + 1 and t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous int32 tensor of B + 1 = {B + 1} elements")
    if seqused_k is not None and not (seqused_k.dtype == i32 and seqused_k.dim() == 1 and
                                      seqused_k.numel() == B and seqused_k.is_contiguous()):
        raise ValueError(f"seqused_k must be a contiguous int32 tensor of B = {B} elements")
    rows_q = Sq if varlen else B * Sq
    if rel_bias is not None:
        if not (rel_bias.dim() == 3 and rel_bias.shape[0] == rows_q and rel_bias.shape[1] == Hq):
            raise ValueError(f"rel_bias {tuple(rel_bias.shape)} must be [rows_q={rows_q}, Hq={Hq}, rel_extent]")
    if rel_r is not None:
        if not (rel_r.dim() == 3 and rel_r.shape[0] == rows_q and rel_r.shape[1] == Hq):
            raise ValueError(f"rel_r {tuple(rel_r.shape)} must be [rows_q={rows_q}, Hq={Hq}, d_rel]")
        if not (rel_proj.dim() == 2 and rel_proj.shape[0] == rel_r.shape[2]):
            raise ValueError(f"rel_proj {tuple(rel_proj.shape)} must be [d_rel={rel_r.shape[2]}, rel_extent]")
    if out is not None and not (out.shape == out_shape and out.dtype == q.dtype and out.is_contiguous()):
        raise ValueError(f"out must be a contiguous {q.dtype} tensor of shape {tuple(out_shape)}")
    if lse is not None and not (lse.shape == lse_shape and lse.dtype == torch.float32 and lse.is_contiguous()):
        raise ValueError(f"lse must be a contiguous float32 tensor of shape {tuple(lse_shape)}")
    if workspace is not None and not workspace.is_contiguous():
        raise ValueError("workspace must be contiguous")
    if not q.is_cuda:
        raise ValueError("q must be a CUDA (ROCm) tensor: the forward runs only on the GPU")
    dev = q.get_device()
    for t in (k, v, cu_seqlens_q, cu_seqlens_k, seqused_k, rel_bias, rel_r, rel_proj, out, lse, workspace):
        if t is not None and t.get_device() != dev:
            for name, u in (("k", k), ("v", v), ("cu_seqlens_q", cu_seqlens_q), ("cu_seqlens_k", cu_seqlens_k),
                            ("seqused_k", seqused_k), ("rel_bias", rel_bias), ("rel_r", rel_r),
                            ("rel_proj", rel_proj), ("out", out), ("lse", lse), ("workspace", workspace)):
                if u is t:
                    raise ValueError(f"{name} must be on {q.device} like q (it is on {t.device})")


def _fwd_shapes(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, rel_bias):
    """Sizes of a forward call from its tensors (dense or varlen), with the layout, contiguity
    and dtype checks both forward entry points share."""
    varlen = cu_seqlens_q is not None or cu_seqlens_k is not None
    if varlen:
        if q.dim() != 3:
            raise ValueError("varlen q must be [total_q, Hq, D]")
        _require(k.dim() == 3 and v.dim() == 3, "varlen k and v must be [total_k, Hkv, D] and [total_k, Hkv, Dv]")
        Sq, Hq, D = q.shape
        Sk, Hkv, _ = k.shape
        B = (cu_seqlens_q if cu_seqlens_q is not None else cu_seqlens_k).numel() - 1
        if max_seqlen_q is None or max_seqlen_k is None:
            raise ValueError("varlen needs max_seqlen_q and max_seqlen_k")
        out_shape, lse_shape = (Sq, Hq, v.shape[-1]), (Hq, Sq)
    else:
        if q.dim() != 4:
            raise ValueError("dense q must be [B, Sq, Hq, D]")
        _require(k.dim() == 4 and v.dim() == 4, "dense k and v must be [B, Sk, Hkv, D] and [B, Sk, Hkv, Dv]")
        B, Sq, Hq, D = q.shape
        _, Sk, Hkv, _ = k.shape
        max_seqlen_q = max_seqlen_q or 0
        max_seqlen_k = max_seqlen_k or 0
        out_shape, lse_shape = (B, Sq, Hq, v.shape[-1]), (B, Hq, Sq)
    for name, t in (("q", q), ("k", k), ("v", v), ("rel_bias", rel_bias)):
        if t is not None and not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if k.dtype != q.dtype or v.dtype != q.dtype or (rel_bias is not None and rel_bias.dtype != q.dtype):
        raise AttnError(CODE["ATTN_ERR_BAD_DTYPE"], "q, k, v and rel_bias must share one dtype")
    return (varlen, B, Sq, Sk, Hq, Hkv, D, v.shape[-1], int(max_seqlen_q), int(max_seqlen_k), out_shape,
            lse_shape)


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
    (varlen, B, Sq, Sk, Hq, Hkv, D, Dv, max_seqlen_q, max_seqlen_k, out_shape,
     lse_shape) = _fwd_shapes(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, rel_bias)
    dtype = _dtype_code(q)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if rel_r is not None or rel_proj is not None:
        if rel_bias is not None or rel_r is None or rel_proj is None:
            raise ValueError("pass rel_r with rel_proj, or rel_bias, not both")
        for name, t in (("rel_r", rel_r), ("rel_proj", rel_proj)):
            if not t.is_contiguous() or t.dtype != q.dtype:
                raise ValueError(f"{name} must be contiguous and of q's dtype")
    _check_tensors(q, k, v, varlen=varlen, B=B, Sq=Sq, Hq=Hq, D=D, cu_seqlens_q=cu_seqlens_q,
                   cu_seqlens_k=cu_seqlens_k, seqused_k=seqused_k, rel_bias=rel_bias, rel_r=rel_r,
                   rel_proj=rel_proj, out=out, lse=lse, workspace=workspace, out_shape=out_shape,
                   lse_shape=lse_shape)
    if out is None:
        out = torch.empty(out_shape, dtype=q.dtype, device=q.device)
    if lse is None and return_lse:
        lse = torch.empty(lse_shape, dtype=torch.float32, device=q.device)
    E = 0 if rel_bias is None else int(rel_bias.shape[-1])
    if rel_proj is not None:
        E = int(rel_proj.shape[1])
    if workspace is not None:
        # the library checks that the given workspace holds the split partials it needs
        ws_bytes = workspace.numel() * workspace.element_size()
    else:
        ns = lib.attn_num_splits(B, Sq, Sk, Hq, Hkv, D, Dv, int(bool(causal)), int(varlen), max_seqlen_q,
                                 max_seqlen_k, pack_gqa, num_splits)
        ws_bytes = 0
        if ns > 1:
            ws_bytes = lib.attn_fwd_workspace_size(B, Sq, Hq, Dv, int(varlen), ns)
            workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
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


def attn_fwd_noalloc(q, k, v, *, out, lse=None, causal: bool = False, scale: Optional[float] = None,
                     cu_seqlens_q=None, cu_seqlens_k=None, max_seqlen_q: Optional[int] = None,
                     max_seqlen_k: Optional[int] = None, seqused_k=None, rel_bias=None, num_splits: int = 1,
                     pack_gqa: int = -1, stream=None):
    """attn_fwd through attn_fwd_noalloc: no workspace; out (and lse, if wanted) are given by
    the caller, so neither this wrapper nor the library allocates. Returns (out, lse)."""
    lib = load()
    (varlen, B, Sq, Sk, Hq, Hkv, D, Dv, max_seqlen_q, max_seqlen_k, out_shape,
     lse_shape) = _fwd_shapes(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, rel_bias)
    _require(out is not None, "attn_fwd_noalloc needs a caller-given out")
    _check_tensors(q, k, v, varlen=varlen, B=B, Sq=Sq, Hq=Hq, D=D, cu_seqlens_q=cu_seqlens_q,
                   cu_seqlens_k=cu_seqlens_k, seqused_k=seqused_k, rel_bias=rel_bias, rel_r=None,
                   rel_proj=None, out=out, lse=lse, workspace=None, out_shape=out_shape, lse_shape=lse_shape)
    E = 0 if rel_bias is None else int(rel_bias.shape[-1])
    st = lib.attn_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, Sq, Sk, Hq, Hkv, D, Dv,
                              float(1.0 / math.sqrt(D) if scale is None else scale), int(bool(causal)),
                              _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), max_seqlen_q, max_seqlen_k, _ptr(seqused_k),
                              _ptr(rel_bias), E, num_splits, pack_gqa, _dtype_code(q),
                              _stream_handle(stream, q.device))
    _check(st)
    return out, lse


def attn_combine(o_partial, lse_partial, *, out, lse=None, B: int, Sq: int, is_varlen: bool = False,
                 stream=None):
    """LSE-weighted merge of split partials (fp32) into out (bf16/fp16) and lse (fp32).

    Dense: o_partial [ns, B*Sq, Hq, Dv], lse_partial [ns, B, Hq, Sq], out [B, Sq, Hq, Dv], lse [B, Hq, Sq].
    Varlen (Sq = total_q): o_partial [ns, Sq, Hq, Dv], lse_partial [ns, Hq, Sq], out [Sq, Hq, Dv],
    lse [Hq, Sq]. These are the layouts attn_fwd leaves in its workspace.
    """
    import torch
    lib = load()
    _require(o_partial.dim() == 4, "o_partial must be [num_splits, rows_q, Hq, Dv]")
    ns, rows_q, Hq, Dv = (int(x) for x in o_partial.shape)
    _require(rows_q == (Sq if is_varlen else B * Sq), f"o_partial has {rows_q} rows, expected "
             f"{Sq if is_varlen else B * Sq}")
    lse_p_shape = (ns, Hq, Sq) if is_varlen else (ns, B, Hq, Sq)
    out_shape = (Sq, Hq, Dv) if is_varlen else (B, Sq, Hq, Dv)
    lse_shape = lse_p_shape[1:]
    _require(o_partial.dtype == torch.float32 and o_partial.is_contiguous(), "o_partial must be contiguous float32")
    _require(tuple(lse_partial.shape) == lse_p_shape and lse_partial.dtype == torch.float32 and
             lse_partial.is_contiguous(), f"lse_partial must be a contiguous float32 tensor of shape {lse_p_shape}")
    _require(tuple(out.shape) == out_shape and out.is_contiguous(), f"out must be contiguous, shape {out_shape}")
    if lse is not None:
        _require(tuple(lse.shape) == lse_shape and lse.dtype == torch.float32 and lse.is_contiguous(),
                 f"lse must be a contiguous float32 tensor of shape {lse_shape}")
    dev = out.device
    _require(dev.type == "cuda", "out must be a CUDA (ROCm) tensor: the combine runs only on the GPU")
    for name, t in (("o_partial", o_partial), ("lse_partial", lse_partial), ("lse", lse)):
        if t is not None:
            _require(t.device == dev, f"{name} must be on {dev} like out (it is on {t.device})")
    st = lib.attn_combine(_ptr(o_partial), _ptr(lse_partial), ns, _ptr(out), _ptr(lse), B, Sq, Hq, Dv,
                          int(bool(is_varlen)), _dtype_code(out), _stream_handle(stream, out.device))
    _check(st)
    return out, lse


def split_partials(workspace, num_splits: int, *, B: int, Sq: int, Hq: int, Dv: int, is_varlen: bool = False):
    """Views of attn_fwd's workspace as (o_partial, lse_partial) for attn_combine: fp32 O
    [num_splits, rows_q, Hq, Dv] followed by fp32 LSE [num_splits, <lse layout>]."""
    import torch
    rows_q = Sq if is_varlen else B * Sq
    n_o = num_splits * rows_q * Hq * Dv
    n_l = num_splits * rows_q * Hq
    flat = workspace.view(torch.uint8)[: (n_o + n_l) * 4].view(torch.float32)
    o_p = flat[:n_o].view(num_splits, rows_q, Hq, Dv)
    l_p = flat[n_o:].view((num_splits, Hq, Sq) if is_varlen else (num_splits, B, Hq, Sq))
    return o_p, l_p
