"""The C-ABI library loads on the CPU, exports every declared symbol, and validates arguments.

No GPU call is made here: attn_check_args, attn_num_splits, attn_fwd_workspace_size,
attn_status_string and attn_version are pure host functions. Pointers are fake
addresses that are only checked for NULL and alignment.
"""
import os
import re

import pytest

import exact_attention_forward_amd as fa
from exact_attention_forward_amd import CODE

REPO = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
A = 0x10000  # a fake, 16-byte aligned device address


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(fa.LIB_PATH):
        from exact_attention_forward_amd import build
        build.build()
    return fa.load()


def declared_functions():
    with open(os.path.join(REPO, "include", "attn.h")) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_]+\s*\*?\s*(attn_[a-z_]+)\s*\(", text, re.M)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == set(fa.SIGNATURES), (names, sorted(fa.SIGNATURES))
    for n in names:
        assert hasattr(lib, n), f"missing export {n}"


def test_version_and_status_strings(lib):
    assert "gfx950" in fa.version()
    for code in range(0, 16):
        s = fa.status_string(code)
        assert s and s != "unknown status"
    assert fa.status_string(99) == "unknown status"


def args(**over):
    a = dict(q=A, k=A, v=A, out=A, lse=A, B=1, Sq=257, Sk=257, Hq=8, Hkv=8, D=128, Dv=128,
             scale=0.0883883, causal=0, cu_q=None, cu_k=None, max_q=0, max_k=0, seqused=None,
             bias=None, E=0, ns=1, pack=-1, dtype=0, ws=None, ws_bytes=0)
    a.update(over)
    return a


def check(lib, **over):
    a = args(**over)
    return lib.attn_check_args(a["q"], a["k"], a["v"], a["out"], a["lse"], a["B"], a["Sq"], a["Sk"],
                               a["Hq"], a["Hkv"], a["D"], a["Dv"], a["scale"], a["causal"], a["cu_q"],
                               a["cu_k"], a["max_q"], a["max_k"], a["seqused"], a["bias"], a["E"],
                               a["ns"], a["pack"], a["dtype"], a["ws"], a["ws_bytes"])


def test_valid_calls(lib):
    assert check(lib) == 0
    for D in range(8, 257, 8):  # the head-dim family: multiples of 8 up to 256
        assert check(lib, D=D, Dv=D) == 0
    for D, Dv in ((128, 64), (64, 128), (192, 128), (72, 72), (48, 48), (8, 256), (256, 8)):
        assert check(lib, D=D, Dv=Dv) == 0
    assert check(lib, dtype=1) == 0
    assert check(lib, Hq=32, Hkv=8, causal=1) == 0
    assert check(lib, cu_q=A, cu_k=A, max_q=100, max_k=100, B=3, Sq=257, Sk=257) == 0
    assert check(lib, bias=A, E=256) == 0
    assert check(lib, lse=None) == 0
    assert check(lib, seqused=A) == 0
    # nothing to compute: NULL tensors are fine
    assert check(lib, B=0, q=None, k=None, v=None, out=None) == 0
    assert check(lib, Sk=0, k=None, v=None) == 0


@pytest.mark.parametrize("over,code", [
    (dict(dtype=2), "ATTN_ERR_BAD_DTYPE"),
    (dict(B=-1), "ATTN_ERR_BAD_SHAPE"),
    (dict(Sq=-3), "ATTN_ERR_BAD_SHAPE"),
    (dict(Hq=0), "ATTN_ERR_BAD_SHAPE"),
    (dict(D=100, Dv=100), "ATTN_ERR_UNSUPPORTED_HEAD_DIM"),
    (dict(D=128, Dv=60), "ATTN_ERR_UNSUPPORTED_HEAD_DIM"),
    (dict(D=4, Dv=4), "ATTN_ERR_UNSUPPORTED_HEAD_DIM"),
    (dict(D=264, Dv=264), "ATTN_ERR_UNSUPPORTED_HEAD_DIM"),
    (dict(D=512, Dv=512), "ATTN_ERR_UNSUPPORTED_HEAD_DIM"),
    (dict(D=0, Dv=64), "ATTN_ERR_BAD_SHAPE"),
    (dict(Hq=8, Hkv=3), "ATTN_ERR_BAD_GQA"),
    (dict(bias=A, E=100), "ATTN_ERR_BAD_REL_EXTENT"),
    (dict(bias=A, E=0), "ATTN_ERR_BAD_REL_EXTENT"),
    (dict(bias=None, E=128), "ATTN_ERR_BAD_REL_EXTENT"),
    (dict(cu_q=A), "ATTN_ERR_BAD_VARLEN"),
    (dict(cu_k=A), "ATTN_ERR_BAD_VARLEN"),
    (dict(cu_q=A, cu_k=A, max_q=0, max_k=10), "ATTN_ERR_BAD_VARLEN"),
    (dict(cu_q=A, cu_k=A, max_q=300, max_k=10), "ATTN_ERR_BAD_VARLEN"),
    (dict(q=None), "ATTN_ERR_NULL_POINTER"),
    (dict(out=None), "ATTN_ERR_NULL_POINTER"),
    (dict(k=None), "ATTN_ERR_NULL_POINTER"),
    (dict(q=A + 8), "ATTN_ERR_MISALIGNED"),
    (dict(v=A + 2), "ATTN_ERR_MISALIGNED"),
    (dict(lse=A + 2), "ATTN_ERR_MISALIGNED"),
    (dict(bias=A + 1, E=128), "ATTN_ERR_MISALIGNED"),
    (dict(ns=4, Sk=100000, ws=None), "ATTN_ERR_WORKSPACE"),
    (dict(ns=4, Sk=100000, ws=A, ws_bytes=16), "ATTN_ERR_WORKSPACE"),
    (dict(scale=float("nan")), "ATTN_ERR_BAD_SCALE"),
    (dict(scale=float("inf")), "ATTN_ERR_BAD_SCALE"),
    (dict(pack=2), "ATTN_ERR_BAD_ARG"),
    (dict(B=1 << 30, Sq=1 << 30, Hq=1 << 20), "ATTN_ERR_BAD_SHAPE"),
])
def test_invalid_calls(lib, over, code):
    assert check(lib, **over) == CODE[code]


def test_workspace_and_splits(lib):
    # split with a large enough workspace is accepted
    ns = lib.attn_num_splits(1, 257, 100000, 8, 8, 128, 128, 0, 0, 0, 0, -1, 4)
    assert ns == 4
    need = lib.attn_fwd_workspace_size(1, 257, 8, 128, 0, 4)
    assert need == 4 * 257 * 8 * 129 * 4
    assert check(lib, ns=4, Sk=100000, ws=A, ws_bytes=need) == 0
    assert check(lib, ns=4, Sk=100000, ws=A + 4, ws_bytes=need) == CODE["ATTN_ERR_MISALIGNED"]
    assert lib.attn_fwd_workspace_size(1, 257, 8, 128, 0, 1) == 0
    # requested splits are clamped to the number of key blocks and to 256
    assert lib.attn_num_splits(1, 10, 200, 1, 1, 64, 64, 0, 0, 0, 0, -1, 50) == ceil_div(200, bn(64))
    assert lib.attn_num_splits(1, 10, 10**6, 1, 1, 64, 64, 0, 0, 0, 0, -1, 1000) == 256
    # heuristic: no split when the grid already covers the chip
    assert lib.attn_num_splits(1, 20480, 20480, 56, 56, 128, 128, 0, 0, 0, 0, -1, 0) == 1
    assert lib.attn_num_splits(1, 1024, 20480, 4, 4, 128, 128, 0, 0, 0, 0, -1, 0) == \
        heuristic(4 * ceil_div(1024, bm(128)), 20480, 128)
    assert lib.attn_num_splits(1, 2048, 20480, 2, 1, 256, 256, 0, 0, 0, 0, -1, 0) == heuristic(32, 20480, 256)
    # decode B=32, one KV head, 8:1 packed into one row tile: 32 work-groups
    assert lib.attn_num_splits(32, 1, 131072, 8, 1, 256, 256, 0, 0, 0, 0, -1, 0) == heuristic(32, 131072, 256)
    # short query, long keys: 6 heads x ceil(1000 / rows per work-group) row tiles
    wg = 6 * ceil_div(1000, bm(64))
    assert lib.attn_num_splits(1, 1000, 10**6, 6, 6, 64, 64, 0, 0, 0, 0, -1, 0) == heuristic(wg, 10**6, 64)
    # never fewer than 4 key blocks per split
    assert lib.attn_num_splits(1, 1, 640, 1, 1, 64, 64, 0, 0, 0, 0, -1, 0) == ceil_div(640, bn(64)) // 4
    assert lib.attn_num_splits(1, 1, 640, 1, 1, 256, 256, 0, 0, 0, 0, -1, 0) == ceil_div(640, bn(256)) // 4
    # a head-dim pair plans like the class of the larger dim
    assert lib.attn_num_splits(1, 1, 640, 1, 1, 72, 72, 0, 0, 0, 0, -1, 0) == ceil_div(640, bn(128)) // 4
    assert lib.attn_num_splits(1, 1, 640, 1, 1, 128, 200, 0, 0, 0, 0, -1, 0) == ceil_div(640, bn(256)) // 4
    # varlen sizes come from max_seqlen
    assert lib.attn_num_splits(4, 400, 400000, 8, 8, 128, 128, 0, 1, 100, 100000, -1, 0) == \
        heuristic(4 * 8 * ceil_div(100, bm(128)), 100000, 128)



def bn(D):
    """Keys per key block of the forward kernel: 128 at head-dim class 16, 64 above."""
    return 128 if D <= 16 else 64


def ceil_div(a, b):
    return -(-a // b)


def resident(D):
    """Work-groups that fit on the chip at once: 256 CUs x 2 (head-dim class up to 64) or
    x 1 (classes 128 and 256)."""
    return 256 * (2 if D <= 64 else 1)


def bm(D):
    """Rows per work-group: 256 at head-dim class 128 (eight waves), 128 elsewhere."""
    return 256 if 64 < D <= 128 else 128


def heuristic(work_groups, k_len, D):
    """The documented split rule: floor(resident / work-groups), times up to 8 waves while each
    split keeps 64 key blocks, at least 4 key blocks per split."""
    if work_groups >= resident(D):
        return 1
    nkb = ceil_div(k_len, bn(D))
    n = resident(D) // work_groups
    rounds = min(8, nkb // n // 64)
    if rounds > 1:
        n *= rounds
    return max(1, min(n, max(1, nkb // 4), 256))


def test_python_binding_rejects_bad_dtype():
    import torch
    x = torch.zeros((1, 4, 1, 64), dtype=torch.float32)
    with pytest.raises(fa.AttnError):
        fa.attn_fwd(x, x, x)


def check_rel_proj(lib, r=A, proj=A, d_rel=16, E=256, **over):
    """attn_fwd_rel_proj with arguments its validation rejects (or B = 0): no GPU call."""
    a = args(**over)
    return lib.attn_fwd_rel_proj(a["q"], a["k"], a["v"], a["out"], a["lse"], a["B"], a["Sq"], a["Sk"],
                                 a["Hq"], a["Hkv"], a["D"], a["Dv"], a["scale"], a["causal"], a["cu_q"],
                                 a["cu_k"], a["max_q"], a["max_k"], a["seqused"], r, proj, d_rel, E,
                                 a["ns"], a["pack"], a["dtype"], a["ws"], a["ws_bytes"], None)


def test_rel_proj_validation(lib):
    C = CODE
    assert check_rel_proj(lib, B=0) == 0  # nothing to compute
    assert check_rel_proj(lib, B=0, E=384) == 0
    assert check_rel_proj(lib, proj=None) == C["ATTN_ERR_NULL_POINTER"]
    assert check_rel_proj(lib, r=None) == C["ATTN_ERR_NULL_POINTER"]
    assert check_rel_proj(lib, d_rel=12) == C["ATTN_ERR_BAD_ARG"]
    assert check_rel_proj(lib, d_rel=0) == C["ATTN_ERR_BAD_ARG"]
    assert check_rel_proj(lib, d_rel=264) == C["ATTN_ERR_BAD_ARG"]
    assert check_rel_proj(lib, r=A + 2) == C["ATTN_ERR_MISALIGNED"]
    assert check_rel_proj(lib, E=100) == C["ATTN_ERR_BAD_REL_EXTENT"]
    # any rel_extent: LDS holds one key tile's bias values per row, whatever E is
    assert check_rel_proj(lib, B=0, E=512) == 0
    assert check_rel_proj(lib, B=0, D=256, Dv=256, E=256) == 0
    assert check_rel_proj(lib, B=0, D=256, Dv=256, E=1024) == 0


@pytest.mark.parametrize("D,hkv_max", [(8, 1 << 19), (16, 1 << 18), (64, 1 << 17), (128, 1 << 16), (256, 1 << 15)])
def test_tile_bytes_bound_per_class(lib, D, hkv_max):
    """One K or V tile (128 keys at head-dim class 16, 64 above) of Hkv heads must span at
    most 2^30 bytes, the fixed out-of-range load offset of the columns past the head dim."""
    keys = 128 if D <= 16 else 64
    assert keys * hkv_max * D * 2 == 1 << 30
    assert check(lib, B=1, Sq=1, Sk=1, Hq=hkv_max, Hkv=hkv_max, D=D, Dv=D) == 0
    over = hkv_max + 1
    assert check(lib, B=1, Sq=1, Sk=1, Hq=over, Hkv=over, D=D, Dv=D) == CODE["ATTN_ERR_BAD_SHAPE"]
    # the larger of D and Dv decides
    assert check(lib, B=1, Sq=1, Sk=1, Hq=over, Hkv=over, D=8, Dv=D) == CODE["ATTN_ERR_BAD_SHAPE"]


def noalloc(lib, **over):
    """attn_fwd_noalloc with arguments it rejects before any HIP call: no GPU call."""
    a = args(**over)
    return lib.attn_fwd_noalloc(a["q"], a["k"], a["v"], a["out"], a["lse"], a["B"], a["Sq"], a["Sk"], a["Hq"],
                                a["Hkv"], a["D"], a["Dv"], a["scale"], a["causal"], a["cu_q"], a["cu_k"],
                                a["max_q"], a["max_k"], a["seqused"], a["bias"], a["E"], a["ns"], a["pack"],
                                a["dtype"], None)


def test_noalloc_rejections(lib):
    # attn_fwd's own errors, in attn_fwd's order
    assert noalloc(lib, dtype=7) == CODE["ATTN_ERR_BAD_DTYPE"]
    assert noalloc(lib, Dv=100) == CODE["ATTN_ERR_UNSUPPORTED_HEAD_DIM"]
    assert noalloc(lib, q=None) == CODE["ATTN_ERR_NULL_POINTER"]
    assert noalloc(lib, out=A + 8, ns=4) == CODE["ATTN_ERR_MISALIGNED"]
    assert noalloc(lib, pack=3) == CODE["ATTN_ERR_BAD_ARG"]
    # partials beyond the 16 MiB array: the largest split count that fits (256 rows x 16
    # heads x 129 floats per split), and one more that does not
    rows, per = 256 * 16, 129 * 4
    fit = fa.SCRATCH_BYTES // (rows * per)
    assert fit == 7
    assert fa.workspace_size(1, 256, 16, 128, splits=fit) <= fa.SCRATCH_BYTES
    assert fa.workspace_size(1, 256, 16, 128, splits=fit + 1) > fa.SCRATCH_BYTES
    assert noalloc(lib, Sq=256, Sk=65536, Hq=16, Hkv=16, ns=fit + 1) == CODE["ATTN_ERR_SCRATCH"]
    assert noalloc(lib, Sq=256, Sk=65536, Hq=16, Hkv=16, ns=64) == CODE["ATTN_ERR_SCRATCH"]
    # the heuristic's own choice counts: 64 rows x 8 heads over 2^20 keys split 256 ways
    ns = fa.num_splits(1, 64, 1 << 20, 8, 8, 128, 128)
    assert fa.workspace_size(1, 64, 8, 128, splits=ns) > fa.SCRATCH_BYTES
    assert noalloc(lib, Sq=64, Sk=1 << 20, ns=0) == CODE["ATTN_ERR_SCRATCH"]


def combine(lib, o=A, l=A, ns=2, out=A, lse=A, B=1, Sq=16, Hq=8, Dv=128, varlen=0, dtype=0):
    """attn_combine with arguments its validation rejects (or no rows): no GPU call."""
    return lib.attn_combine(o, l, ns, out, lse, B, Sq, Hq, Dv, varlen, dtype, None)


@pytest.mark.parametrize("over,code", [
    (dict(dtype=5), "ATTN_ERR_BAD_DTYPE"),
    (dict(B=-1), "ATTN_ERR_BAD_SHAPE"),
    (dict(Sq=-1), "ATTN_ERR_BAD_SHAPE"),
    (dict(Hq=0), "ATTN_ERR_BAD_SHAPE"),
    (dict(Dv=100), "ATTN_ERR_UNSUPPORTED_HEAD_DIM"),
    (dict(Dv=0), "ATTN_ERR_UNSUPPORTED_HEAD_DIM"),
    (dict(Dv=264), "ATTN_ERR_UNSUPPORTED_HEAD_DIM"),
    (dict(ns=0), "ATTN_ERR_BAD_SPLITS"),
    (dict(ns=257), "ATTN_ERR_BAD_SPLITS"),
    (dict(o=None), "ATTN_ERR_NULL_POINTER"),
    (dict(l=None), "ATTN_ERR_NULL_POINTER"),
    (dict(out=None), "ATTN_ERR_NULL_POINTER"),
    (dict(o=A + 4), "ATTN_ERR_MISALIGNED"),
    (dict(l=A + 2), "ATTN_ERR_MISALIGNED"),
    (dict(out=A + 8), "ATTN_ERR_MISALIGNED"),
    (dict(lse=A + 1), "ATTN_ERR_MISALIGNED"),
    (dict(B=1 << 20, Sq=1 << 20, Hq=1 << 20), "ATTN_ERR_BAD_SHAPE"),
    (dict(B=1 << 16, Sq=1 << 16, Hq=8, Dv=8), "ATTN_ERR_BAD_SHAPE"),  # one work-group per (row, head): > 2^31
])
def test_combine_invalid_calls(lib, over, code):
    assert combine(lib, **over) == CODE[code]


def test_combine_nothing_to_do(lib):
    # no rows: accepted without a launch, NULL buffers included
    assert combine(lib, B=0, o=None, l=None, out=None, lse=None) == 0
    assert combine(lib, Sq=0, varlen=1, o=None, l=None, out=None) == 0


def _cpu(shape, dtype=None):
    import torch
    return torch.zeros(shape, dtype=dtype or torch.bfloat16)


@pytest.mark.parametrize("case,match", [
    (dict(k=(1, 64, 2, 64)), "k"),                       # head dim differs from q
    (dict(k=(2, 64, 2, 128)), "k"),                      # batch differs
    (dict(v=(1, 32, 2, 128)), "v"),                      # keys differ from k
    (dict(k=(64, 2, 128)), "rank|k and v"),              # rank differs
    (dict(out=(1, 16, 8, 64)), "out"),
    (dict(lse=(1, 16, 8)), "lse"),
    (dict(lse_dtype="bf16"), "lse"),
    (dict(seqused=(2,)), "seqused_k"),
    (dict(seqused_dtype="int64"), "seqused_k"),
    (dict(rel_bias=(15, 8, 256)), "rel_bias"),              # rows differ from B * Sq
    (dict(), "CUDA"),                                    # all shapes right: the CPU tensors are refused
])
def test_binding_rejects_bad_tensors(case, match):
    """Checks in the Python binding that run before any pointer reaches the library."""
    import torch
    q = _cpu((1, 16, 8, 128))
    k = _cpu(case.get("k", (1, 64, 2, 128)))
    v = _cpu(case.get("v", (1, 64, 2, 128)))
    kw = {}
    if "out" in case:
        kw["out"] = _cpu(case["out"])
    if "lse" in case:
        kw["lse"] = _cpu(case["lse"], torch.float32)
    if "lse_dtype" in case:
        kw["lse"] = _cpu((1, 8, 16))
    if "seqused" in case:
        kw["seqused_k"] = torch.zeros(case["seqused"], dtype=torch.int32)
    if "seqused_dtype" in case:
        kw["seqused_k"] = torch.zeros((1,), dtype=torch.int64)
    if "rel_bias" in case:
        kw["rel_bias"] = _cpu(case["rel_bias"])
    with pytest.raises(ValueError, match=match):
        fa.attn_fwd(q, k, v, **kw)


def test_binding_rejects_bad_varlen_metadata():
    import torch
    q = _cpu((30, 8, 64))
    k = _cpu((40, 8, 64))
    good = torch.tensor([0, 10, 30], dtype=torch.int32)
    for cu_q, cu_k, match in (
            (torch.tensor([0, 10, 30]), good, "cu_seqlens_q"),             # int64 by default
            (good, torch.tensor([0, 40], dtype=torch.int32), "cu_seqlens_k"),  # B + 1 differs
            (good, good.view(1, 3), "cu_seqlens_k")):                     # not 1-D
        with pytest.raises(ValueError, match=match):
            fa.attn_fwd(q, k, k, cu_seqlens_q=cu_q, cu_seqlens_k=cu_k, max_seqlen_q=20, max_seqlen_k=30)


def test_binding_combine_rejects_bad_tensors():
    import torch
    o_p = torch.zeros((3, 16, 8, 64), dtype=torch.float32)
    l_p = torch.zeros((3, 1, 8, 16), dtype=torch.float32)
    out = _cpu((1, 16, 8, 64))
    with pytest.raises(ValueError, match="lse_partial"):
        fa.attn_combine(o_p, l_p[:, :, :4], out=out, B=1, Sq=16)
    with pytest.raises(ValueError, match="rows"):
        fa.attn_combine(o_p, l_p, out=out, B=2, Sq=16)
    with pytest.raises(ValueError, match="out"):
        fa.attn_combine(o_p, l_p, out=_cpu((1, 16, 8, 128)), B=1, Sq=16)
    with pytest.raises(ValueError, match="CUDA"):
        fa.attn_combine(o_p, l_p, out=out, B=1, Sq=16)
