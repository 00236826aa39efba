"""The seeded input generator: stream stability, rounding, integer ranges."""
import numpy as np
import torch

from workloads import configs, gen


def test_chunked_equals_one_shot():
    a = gen.normal_bits(gen.make_rng(7), (3, 1000, 7), "bf16", chunk=997)
    b = gen.normal_bits(gen.make_rng(7), (3, 1000, 7), "bf16", chunk=1 << 22)
    assert np.array_equal(a, b)
    c = gen.normal_bits(gen.make_rng(7), (21000,), "fp16", std=0.5, chunk=64)
    d = gen.normal_bits(gen.make_rng(7), (21000,), "fp16", std=0.5)
    assert np.array_equal(c, d)


def test_block_streams_independent_of_threads():
    a = gen.stream_normal_bits(9, gen.STREAM_K, (3 * gen.BLOCK + 12345,), "bf16", threads=1)
    b = gen.stream_normal_bits(9, gen.STREAM_K, (3 * gen.BLOCK + 12345,), "bf16", threads=5)
    assert np.array_equal(a, b)
    # block n is its own stream
    first = gen.make_rng(9, gen.STREAM_K, 1).standard_normal(10, dtype=np.float32)
    assert np.array_equal(a[gen.BLOCK:gen.BLOCK + 10], gen.f32_to_bf16_bits(first))
    # different streams differ
    c = gen.stream_normal_bits(9, gen.STREAM_V, (1000,), "bf16")
    assert not np.array_equal(a[:1000], c)


def test_bf16_rounding_matches_torch():
    rng = gen.make_rng(3)
    x = np.concatenate([
        rng.standard_normal(100000, dtype=np.float32) * 10,
        # exact ties between two bfloat16 values, both parities
        (np.arange(1, 2000, dtype=np.uint32) << 16 | 0x8000).view(np.float32),
        np.array([0.0, -0.0, 1e-40, -1e-40, 3.0e38, np.inf, -np.inf], dtype=np.float32),
    ])
    ours = gen.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert gen.f32_to_bf16_bits(np.array([np.nan], dtype=np.float32))[0] == 0x7FC0


def test_fp16_rounding_matches_torch():
    x = gen.make_rng(4).standard_normal(100000, dtype=np.float32) * 100
    ours = gen.f32_to_fp16_bits(x)
    ref = torch.from_numpy(x).to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_uniform_ints_inclusive():
    v = gen.uniform_ints(gen.make_rng(5), 3, 6, 4000)
    assert v.dtype == np.int32 and v.min() == 3 and v.max() == 6


def test_workload_inputs_deterministic_and_shaped():
    s1 = configs.workload("c1")
    a = configs.make_inputs(s1)
    b = configs.make_inputs(configs.workload("c1"))
    assert a["q"].shape == (1, 257, 8, 128) and a["q"].dtype == np.uint16
    for key in ("q", "k", "v"):
        assert np.array_equal(a[key], b[key])
    # q, k and v are distinct draws
    assert not np.array_equal(a["q"], a["k"])
    f = gen.bf16_bits_to_f32(a["q"])
    assert abs(float(f.mean())) < 0.02 and abs(float(f.std()) - 1.0) < 0.02


def test_varlen_metadata():
    s = configs.Spec("t", "bf16", 8, 0, 0, 32, 8, 128, 128, True, 0.0883883461356163, 3,
                     varlen=True, len_range=(512, 8192), rel_extent=256)
    lens = gen.uniform_ints(gen.make_rng(3), 512, 8192, 8)
    cu = gen.cu_seqlens(lens)
    assert cu[0] == 0 and cu[-1] == lens.sum() and np.all(np.diff(cu) == lens)
    assert cu.dtype == np.int32
