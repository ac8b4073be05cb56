"""The race-guard build (libflashattn_poison.so, FA_DEBUG_POISON) against the
float64 oracle.

In that build every global-to-LDS copy first fills its destination with NaN
(the all-ones pattern, a NaN in fp32, fp16 and bf16) and waits for the write.
A ring slot therefore holds NaN from the moment it is refilled (after the
barrier that follows its last read) until the new tile lands. A read of a
slot that is not ordered after its copy's wait and barrier, or a copy issued
into a slot that is still being read, turns into NaN in the outputs instead
of into stale or early data that could happen to pass. The cases run every
copy path: the named half-precision workloads, the four launch shapes of the
forward kernel (key split, whole rounds of 4-wave workgroups, rounds plus a
split remainder, 8-wave 256-row workgroups) with both signs of the scale,
causal and not, and the backward kernels (4-wave dQ and dK/dV, 8-wave dQ and
dK/dV) causal and not. Tolerances are those of the parity tests.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import io_aware_tiled_06_amd as fa  # noqa: E402
from io_aware_tiled_06_amd.workloads import WORKLOADS, Workload, make_inputs, sample_rows  # noqa: E402
from oracle import attention_backward_reference, attention_reference  # noqa: E402
from test_gpu_backward import check, upstream  # noqa: E402
from test_gpu_parity import LAUNCH_SHAPES, assert_close, causal_rows_reference, dev  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def poison():
    with fa.using_library(fa.POISON_LIB_PATH) as L:
        yield L


@pytest.mark.parametrize("name", ["n4096_d128_bf16", "n10000_d128_fp16", "b32_n512_d64_bf16"])
@pytest.mark.parametrize("causal", [False, True])
def test_race_guard_workloads(poison, name, causal):
    w = WORKLOADS[name]
    print(f"[race-guard] {name} causal={causal}", flush=True)
    q, k, v = make_inputs(w)
    o, lse = fa.flash_attn_fwd(dev(q, w.dtype), dev(k, w.dtype), dev(v, w.dtype), w.scale, causal=causal)
    torch.cuda.synchronize()
    o = o.float().cpu().numpy().astype(np.float64)
    lse = lse.cpu().numpy().astype(np.float64)
    if w.N <= 4096:
        o_ref, lse_ref = attention_reference(q, k, v, w.scale, causal=causal)
        assert_close(o, lse, o_ref, lse_ref, w.dtype, f"race guard {name}")
    else:
        assert np.all(np.isfinite(o)), "non-finite O"
        rows = np.unique(np.concatenate([sample_rows(w.N, 24), np.arange(0, w.N, 1024), [w.N - 16, w.N - 1]]))
        if causal:
            o_ref, lse_ref = causal_rows_reference(q, k, v, w.scale, rows)
        else:
            o_ref, lse_ref = attention_reference(q[:, :, rows], k, v, w.scale)
        assert_close(o[:, :, rows], lse[:, :, rows], o_ref, lse_ref, w.dtype, f"race guard {name} sampled")


def test_race_guard_long_context_head(poison):
    """The 32K workload's 8-wave launch: one whole head against the oracle,
    every other head checked for NaN."""
    w = WORKLOADS["n32768_d128_bf16"]
    q, k, v = make_inputs(w)
    print("[race-guard] n32768_d128_bf16", flush=True)
    o, lse = fa.flash_attn_fwd(dev(q, w.dtype), dev(k, w.dtype), dev(v, w.dtype), w.scale)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(lse).all())
    o_h = o[0, 7].float().cpu().numpy().astype(np.float64)
    lse_h = lse[0, 7].cpu().numpy().astype(np.float64)
    o_ref, lse_ref = attention_reference(q[0, 7], k[0, 7], v[0, 7], w.scale)
    assert_close(o_h, lse_h, o_ref, lse_ref, w.dtype, "race guard n32768 head 7")


@pytest.mark.parametrize("d", [128, 64])
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("shape", list(LAUNCH_SHAPES))
def test_race_guard_launch_shapes(poison, shape, dtype, d):
    B, H, N = LAUNCH_SHAPES[shape]
    w = Workload(f"guard-{shape}", B, H, N, d, dtype, 190 + N % 7, 2.0)
    q, k, v = make_inputs(w)
    tq, tk, tv = dev(q, dtype), dev(k, dtype), dev(v, dtype)
    edges = [0, 31, 32, 127, 128, 255, 256, N - 33, N - 32, N - 2, N - 1]
    rows = np.unique(np.concatenate([sample_rows(N, 12), [r for r in edges if 0 <= r < N]]))
    for scale in (w.scale, -0.6 * w.scale):
        s = float(np.float32(scale))
        for causal in (False, True):
            what = f"race guard {shape} B{B} H{H} N{N} d{d} {dtype} scale={s:+.4f} causal={causal}"
            print(f"[race-guard] {what}", flush=True)
            o, lse = fa.flash_attn_fwd(tq, tk, tv, s, causal=causal)
            torch.cuda.synchronize()
            assert bool(torch.isfinite(o).all()), f"{what}: non-finite O"
            o_s = o[:, :, rows].float().cpu().numpy().astype(np.float64)
            lse_s = lse[:, :, rows].cpu().numpy().astype(np.float64)
            if causal:
                o_ref, lse_ref = causal_rows_reference(q, k, v, s, rows)
            else:
                o_ref, lse_ref = attention_reference(q[:, :, rows], k, v, s)
            assert_close(o_s, lse_s, o_ref, lse_ref, dtype, what)


# Backward grids: 4-wave dQ and dK/dV (small grids, d = 64, causal), and the
# 8-wave dQ and dK/dV (at least two 256-row workgroups per CU, d = 128).
BWD_CASES = [(1, 2, 1000, 128, "bf16"), (1, 4, 1000, 64, "fp16"), (4, 32, 1000, 128, "bf16"),
             (2, 64, 1000, 128, "fp16"), (1, 2, 33, 128, "bf16")]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,H,N,d,dtype", BWD_CASES)
def test_race_guard_backward(poison, B, H, N, d, dtype, causal):
    w = Workload("guard-bwd", B, H, N, d, dtype, 3100 + N + d + H, 2.0)
    q, k, v = make_inputs(w)
    do = upstream(w, 4100 + N + H)
    dt = {"bf16": torch.bfloat16, "fp16": torch.float16}[dtype]
    t = [torch.from_numpy(np.ascontiguousarray(x)).to(dt).cuda() for x in (q, k, v, do)]
    print(f"[race-guard] backward B{B} H{H} N{N} d{d} {dtype} causal={causal}", flush=True)
    o, lse = fa.flash_attn_fwd(t[0], t[1], t[2], w.scale, causal=causal)
    grads = fa.flash_attn_bwd(t[0], t[1], t[2], o, lse, t[3], w.scale, causal=causal)
    torch.cuda.synchronize()
    got = tuple(g.double().cpu().numpy() for g in grads)
    # compare only the first heads in the big grids (every head checked for NaN)
    hmax = min(H, 4)
    assert all(np.all(np.isfinite(g)) for g in got)
    ref = attention_backward_reference(q[:, :hmax], k[:, :hmax], v[:, :hmax], do[:, :hmax], w.scale, causal=causal)
    check(tuple(g[:, :hmax] for g in got), ref, f"race guard B{B} H{H} N{N} d{d} {dtype} causal={causal}", dtype)


# Many back-to-back launches of the loops whose wait leaves the newest copies
# in flight: every output bitwise equal to the first launch's and free of NaN.
# (Short steps give a late copy the least slack: the 512-token batch at d = 64,
# 16 steps per workgroup; the key split at 4096; the 8-wave launch at B2 H16
# N = 8192, four rounds of 256-row workgroups.)
MANY_CASES = [("b32_n512_d64_bf16", False, 300), ("b32_n512_d64_bf16", True, 300),
              ("n4096_d128_bf16", False, 200), (Workload("guard-wide", 2, 16, 8192, 128, "bf16", 77), False, 20)]


@pytest.mark.parametrize("name,causal,reps", MANY_CASES, ids=lambda x: getattr(x, "name", str(x)))
def test_race_guard_many_launches(poison, name, causal, reps):
    w = WORKLOADS[name] if isinstance(name, str) else name
    q, k, v = (dev(x, w.dtype) for x in make_inputs(w))
    g = torch.Generator(device="cpu").manual_seed(11)
    do = torch.randn(q.shape, generator=g).to(q.dtype).to(q.device)
    print(f"[race-guard] {reps} launches of {w.name} causal={causal}", flush=True)
    o0, lse0 = fa.flash_attn_fwd(q, k, v, w.scale, causal=causal)
    g0 = fa.flash_attn_bwd(q, k, v, o0, lse0, do, w.scale, causal=causal)
    o = torch.empty_like(o0)
    differ = torch.zeros((), dtype=torch.int64, device=q.device)
    nan = torch.zeros((), dtype=torch.int64, device=q.device)
    for i in range(reps):
        _, lse = fa.flash_attn_fwd(q, k, v, w.scale, causal=causal, out=o)
        differ += ((o != o0).any() | (lse != lse0).any()).long()
        nan += (torch.isnan(o).any() | torch.isnan(lse).any()).long()
        if i % 4 == 0:  # the backward pass is slower: a quarter as many
            gr = fa.flash_attn_bwd(q, k, v, o0, lse0, do, w.scale, causal=causal)
            differ += torch.stack([(a != b).any() for a, b in zip(gr, g0)]).any().long()
            nan += torch.stack([torch.isnan(a).any() for a in gr]).any().long()
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o0).all()) and all(bool(torch.isfinite(x).all()) for x in g0)
    assert int(nan) == 0, f"{int(nan)} launches with NaN"
    assert int(differ) == 0, f"{int(differ)} launches differ from the first"


def test_race_guard_library_is_the_poison_build(poison):
    """The fixture really switched libraries (both export the same names)."""
    assert fa.lib()._name == fa.POISON_LIB_PATH
