"""Seeded synthetic inputs shared by the HIP path's tests/bench and the CPU oracle.

This module only draws random numbers and stores them in the 16-bit formats the
attention forward consumes. It holds none of the attention arithmetic: no dot
products, masks, softmax or bias rule. Both sides read the exact 16-bit values
produced here, so they see identical inputs.

Recipe:
  * every workload has a seed; each tensor has a stream number (0 = integer
    metadata such as sequence lengths and seqused_k, 1 = q, 2 = k, 3 = v,
    4 = rel_bias);
  * a tensor is cut into fixed blocks of 2^22 elements (row-major order); block
    n is drawn from its own numpy PCG64 generator seeded with
    SeedSequence([seed, stream, n]), so blocks can be drawn in parallel and the
    values do not depend on the thread count;
  * values: float32 standard normal draws, multiplied by the tensor's standard
    deviation in float32, then rounded to nearest-even into bfloat16 or float16;
  * integer ranges "uniform in [lo, hi]" include both ends (stream 0, drawn in
    the order: sequence lengths, then seqused_k).
"""
from __future__ import annotations

import numpy as np

BF16 = "bf16"
FP16 = "fp16"
DTYPES = (BF16, FP16)

_CHUNK = 1 << 22  # float32 draws per chunk of the sequential helper
BLOCK = 1 << 22   # elements per independently seeded block of a workload tensor

STREAM_META, STREAM_Q, STREAM_K, STREAM_V, STREAM_BIAS = 0, 1, 2, 3, 4
STREAM_REL_R, STREAM_REL_PROJ = 5, 6  # inputs of the fused rel_bias producer


def make_rng(seed: int, stream: int = None, block: int = None) -> np.random.Generator:
    """PCG64 generator: plain seed, or SeedSequence([seed, stream(, block)])."""
    if stream is None:
        return np.random.Generator(np.random.PCG64(int(seed)))
    key = [int(seed), int(stream)] + ([] if block is None else [int(block)])
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(key)))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to nearest-even bfloat16; return the uint16 bit patterns.

    NaN inputs map to a quiet NaN; finite values that round past the largest
    bfloat16 become infinity, as IEEE round-to-nearest-even prescribes.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    r = (u >> 16) & 1
    r += 0x7FFF
    r += u            # no overflow: only NaN patterns reach the top of the range
    r >>= 16
    out = r.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def f32_to_fp16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to nearest-even IEEE half; return the uint16 bit patterns."""
    return np.asarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def fp16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return np.asarray(b, dtype=np.uint16).view(np.float16).astype(np.float32)


def to_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == BF16:
        return f32_to_bf16_bits(x)
    if dtype == FP16:
        return f32_to_fp16_bits(x)
    raise ValueError(f"unknown dtype {dtype!r}")


def bits_to_f32(b: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == BF16:
        return bf16_bits_to_f32(b)
    if dtype == FP16:
        return fp16_bits_to_f32(b)
    raise ValueError(f"unknown dtype {dtype!r}")


def normal_f32(rng: np.random.Generator, shape, std: float = 1.0,
               chunk: int = _CHUNK) -> np.ndarray:
    """float32 N(0, std^2) draws in a fixed chunked order (chunk size does not change values)."""
    n = int(np.prod(shape, dtype=np.int64))
    out = np.empty(n, dtype=np.float32)
    pos = 0
    while pos < n:
        m = min(chunk, n - pos)
        rng.standard_normal(m, dtype=np.float32, out=out[pos:pos + m])
        pos += m
    if std != 1.0:
        out *= np.float32(std)
    return out.reshape(shape)


def normal_bits(rng: np.random.Generator, shape, dtype: str, std: float = 1.0,
                chunk: int = _CHUNK) -> np.ndarray:
    """Draw N(0, std^2) in float32 and round to the 16-bit dtype (chunked, memory-bounded)."""
    n = int(np.prod(shape, dtype=np.int64))
    out = np.empty(n, dtype=np.uint16)
    buf = np.empty(min(chunk, max(n, 1)), dtype=np.float32)
    pos = 0
    s = np.float32(std)
    while pos < n:
        m = min(chunk, n - pos)
        b = buf[:m]
        rng.standard_normal(m, dtype=np.float32, out=b)
        if std != 1.0:
            b *= s
        out[pos:pos + m] = to_bits(b, dtype)
        pos += m
    return out.reshape(shape)


def stream_normal_bits(seed: int, stream: int, shape, dtype: str, std: float = 1.0,
                       threads: int = None) -> np.ndarray:
    """A workload tensor: N(0, std^2) in float32 per independently seeded block, rounded to dtype."""
    import concurrent.futures
    import os
    n = int(np.prod(shape, dtype=np.int64))
    out = np.empty(n, dtype=np.uint16)
    nblocks = (n + BLOCK - 1) // BLOCK
    s = np.float32(std)

    def fill(bi):
        lo = bi * BLOCK
        m = min(BLOCK, n - lo)
        x = make_rng(seed, stream, bi).standard_normal(m, dtype=np.float32)
        if std != 1.0:
            x *= s
        out[lo:lo + m] = to_bits(x, dtype)

    workers = threads or min(16, os.cpu_count() or 1)
    if workers <= 1 or nblocks <= 1:
        for bi in range(nblocks):
            fill(bi)
    else:
        with concurrent.futures.ThreadPoolExecutor(max_workers=workers) as ex:
            list(ex.map(fill, range(nblocks)))
    return out.reshape(shape)


def uniform_ints(rng: np.random.Generator, lo: int, hi: int, n: int) -> np.ndarray:
    """n integers uniform in [lo, hi], both ends included, as int32."""
    return rng.integers(lo, hi + 1, size=n, dtype=np.int64).astype(np.int32)


def cu_seqlens(lengths) -> np.ndarray:
    """Prefix offsets [0, l0, l0+l1, ...] as int32 (packing metadata, not attention math)."""
    lengths = np.asarray(lengths, dtype=np.int64)
    c = np.zeros(len(lengths) + 1, dtype=np.int64)
    np.cumsum(lengths, out=c[1:])
    return c.astype(np.int32)
