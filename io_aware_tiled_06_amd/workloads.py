"""Named attention workloads and their seeded synthetic inputs.

This module holds no attention arithmetic. It only names shapes and draws
inputs, so the CPU oracle (``oracle/``), the HIP path, the tests and the
benchmark can all be fed the same values without sharing any of the method.

The sequence lengths follow the pages' cases: N = 4096 and N = 32K in
"FlashAttention, simplified" (section "The problem") and the 10,000-token
example in "FlashAttention" (interactiveprimer, "A concrete example: 10,000
tokens"), at 2 bytes per element for the half-precision cases. The pages name
no dataset; every input is i.i.d. normal from a fixed seed.

Input recipe (one per workload):
  rng = numpy.random.default_rng(seed)
  q, k, v = three draws of rng.standard_normal((B, H, N, d), float32), in
            that order; q and k are then multiplied by ``qk_sigma``
  each is rounded to the workload's element type (round to nearest even)
The rounded values, held exactly in float32 arrays, are what both the GPU and
the oracle consume.
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np

DTYPES = ("fp32", "fp16", "bf16")
# element codes shared with the C interface (fa_dtype)
DTYPE_CODE = {"fp32": 0, "fp16": 1, "bf16": 2}
DTYPE_BYTES = {"fp32": 4, "fp16": 2, "bf16": 2}


@dataclass(frozen=True)
class Workload:
    """One non-causal attention problem: [B, H, N, d] inputs of ``dtype``."""

    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str
    seed: int
    qk_sigma: float = 1.0

    def __post_init__(self):
        if self.dtype not in DTYPES:
            raise ValueError(f"unknown dtype {self.dtype!r}")
        if min(self.B, self.H, self.N, self.d) < 0:
            raise ValueError("negative size")

    @property
    def scale(self) -> float:
        """1/sqrt(d) rounded to float32: the exact value passed to the kernels."""
        return float(np.float32(1.0 / np.sqrt(self.d)))

    @property
    def shape(self) -> tuple:
        return (self.B, self.H, self.N, self.d)

    @property
    def elem_bytes(self) -> int:
        return DTYPE_BYTES[self.dtype]

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


# The five workloads: a small fp32 parity case, the two pages' long cases at
# d=128 in half precision (one with a ragged tail: 10000 = 78*128 + 16), a
# short-sequence batch, and the 32K long-context case with peaky scores.
WORKLOADS = {
    "n256_d64_fp32": Workload("n256_d64_fp32", 1, 1, 256, 64, "fp32", 0),
    "n4096_d128_bf16": Workload("n4096_d128_bf16", 1, 8, 4096, 128, "bf16", 1),
    "n10000_d128_fp16": Workload("n10000_d128_fp16", 1, 8, 10000, 128, "fp16", 2),
    "b32_n512_d64_bf16": Workload("b32_n512_d64_bf16", 32, 16, 512, 64, "bf16", 3),
    "n32768_d128_bf16": Workload("n32768_d128_bf16", 1, 16, 32768, 128, "bf16", 4, 3.0),
}
WORKLOAD_ORDER = list(WORKLOADS)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); finite inputs.

    Returns float32 values that are exactly representable in bfloat16.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    if not np.all(np.isfinite(x)):
        raise ValueError("round_to_bf16 expects finite values")
    u = x.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).reshape(x.shape)


def round_to_dtype(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float32 values to ``dtype`` (nearest even); result held in float32."""
    if dtype == "fp32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "fp16":
        return np.asarray(x, dtype=np.float32).astype(np.float16).astype(np.float32)
    if dtype == "bf16":
        return round_to_bf16(x)
    raise ValueError(f"unknown dtype {dtype!r}")


def make_inputs(w: Workload):
    """Draw (q, k, v) for ``w`` per the recipe above, as float32 arrays [B,H,N,d].

    The values are already rounded to ``w.dtype``; converting them to that
    element type is exact.
    """
    rng = np.random.default_rng(w.seed)
    shape = w.shape
    q = rng.standard_normal(shape, dtype=np.float32)
    k = rng.standard_normal(shape, dtype=np.float32)
    v = rng.standard_normal(shape, dtype=np.float32)
    if w.qk_sigma != 1.0:
        s = np.float32(w.qk_sigma)
        q *= s
        k *= s
    return (round_to_dtype(q, w.dtype), round_to_dtype(k, w.dtype),
            round_to_dtype(v, w.dtype))


def sample_rows(N: int, count: int, seed: int = 12345) -> np.ndarray:
    """Sorted query-row indices for sampled checks: both ends plus random rows."""
    if count >= N:
        return np.arange(N)
    rng = np.random.default_rng(seed)
    ends = np.array([0, 1, N - 2, N - 1])
    mid = rng.choice(N, size=max(count - len(ends), 0), replace=False)
    return np.unique(np.concatenate([ends, mid]))
