"""Seeded input generation: reproducible, correctly rounded, shaped as named."""
import numpy as np
import pytest

from io_aware_tiled_06_amd.workloads import (WORKLOADS, Workload, make_inputs, round_to_bf16,
                                             round_to_dtype, sample_rows)


def test_workload_table():
    w = WORKLOADS
    assert [(x.B, x.H, x.N, x.d, x.dtype, x.seed) for x in w.values()] == [
        (1, 1, 256, 64, "fp32", 0),
        (1, 8, 4096, 128, "bf16", 1),
        (1, 8, 10000, 128, "fp16", 2),
        (32, 16, 512, 64, "bf16", 3),
        (1, 16, 32768, 128, "bf16", 4),
    ]
    assert w["n32768_d128_bf16"].qk_sigma == 3.0
    assert w["n10000_d128_fp16"].N % 128 == 16  # ragged tail
    assert w["n4096_d128_bf16"].scale == float(np.float32(1 / np.sqrt(128)))


def test_inputs_reproducible_and_rounded():
    w = Workload("t", 2, 3, 50, 16, "bf16", 7, 3.0)
    a = make_inputs(w)
    b = make_inputs(w)
    for x, y in zip(a, b):
        assert x.shape == (2, 3, 50, 16) and x.dtype == np.float32
        assert np.array_equal(x, y)
    for x in a:
        # bf16 values have 16 zero low bits
        assert np.all((x.view(np.uint32) & 0xFFFF) == 0)
    # sigma scales q and k only
    assert a[0].std() > 2.0 and a[2].std() < 1.5


def test_bf16_rounding_matches_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(10000) * np.exp(rng.uniform(-20, 20, 10000))).astype(np.float32)
    ours = round_to_bf16(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(ours, ref)


def test_fp16_rounding():
    x = np.array([1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11], dtype=np.float32)
    # ties to even: 1+2^-11 -> 1.0, 1+3*2^-11 -> 1+2^-9
    assert np.array_equal(round_to_dtype(x, "fp16"), np.array([1.0, 1.0 + 2.0 ** -9], np.float32))


def test_sample_rows():
    r = sample_rows(10000, 64)
    assert r[0] == 0 and r[-1] == 9999 and len(r) == 64 and np.all(np.diff(r) > 0)
    assert np.array_equal(sample_rows(10, 64), np.arange(10))
