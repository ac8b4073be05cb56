"""Backward pass on the GPU against the float64 gradient oracle (float32,
float16 and bfloat16 inputs).

The GPU forward pass supplies O and LSE (as a caller would); the oracle
differentiates exact attention at the same (rounded) inputs. The pages fix no
tolerance for gradients; the bound follows the arithmetic. With u the unit
roundoff of the element type (the largest relative error of rounding to
nearest: 2^-8 for bf16, 8 significant bits; 2^-11 for fp16, 11 bits), per
gradient tensor G with reference R:
  relative RMS  ||G - R|| / ||R||            <= 2.5 u
  max abs       max|G - R| / max|R|          <= 5 u
Sources of error: P and dS are rounded to the input type before their
products (relative error up to u each, about u/sqrt(3) on average), D = dO . O
uses the forward's rounded O, and the gradients themselves are rounded to the
input type. Measured: dV ~0.6 u RMS, dQ and dK ~1 u RMS and at most 1.9 u
(bf16) or 2 u (fp16) in the max column, since dS = P (dP - D) has vanishing
row sums and amplifies the error of D; on the 32768-token rows (peaky,
sigma 3) dQ reaches 1.4 u RMS and 1.8 u max.
float32 inputs round nothing to a narrower type; their error is set by the
float32 rounding of the exponent argument c*s - LSE*log2(e), whose magnitude
reaches about 20 (log2 units) on these inputs: about 20 u_fp32 ~ 1.2e-6
absolute, so about 1e-6 relative in every P, which the gradients inherit.
Bound: relative RMS <= 1e-5, max <= 5e-5 of max|R|. Measured: at most
1.7e-6 RMS and 3.5e-6 max.
"""
import math

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import io_aware_tiled_06_amd as fa  # noqa: E402
from io_aware_tiled_06_amd.workloads import WORKLOADS, Workload, make_inputs, sample_rows  # noqa: E402
from oracle import attention_backward_cols, attention_backward_reference, attention_backward_rows  # noqa: E402

pytestmark = pytest.mark.gpu

TORCH_DT = {"fp32": torch.float32, "fp16": torch.float16, "bf16": torch.bfloat16}
UNIT = {"bf16": 2.0 ** -8, "fp16": 2.0 ** -11}  # unit roundoff
# (relative RMS, max over max|R|) per element type
TOL = {dt: (2.5 * u, 5 * u) for dt, u in UNIT.items()}
TOL["fp32"] = (1e-5, 5e-5)


def upstream(w, seed):
    """dL/dO: i.i.d. N(0,1), rounded to the element type (the same values feed
    GPU and oracle)."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((w.B, w.H, w.N, w.d), dtype=np.float32)
    return torch.from_numpy(x).to(TORCH_DT[w.dtype]).float().numpy()


def run_backward(w, q, k, v, do, scale, causal):
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(TORCH_DT[w.dtype]).cuda()  # noqa: E731
    tq, tk, tv, tdo = dev(q), dev(k), dev(v), dev(do)
    o, lse = fa.flash_attn_fwd(tq, tk, tv, scale, causal=causal)
    dq, dk, dv = fa.flash_attn_bwd(tq, tk, tv, o, lse, tdo, scale, causal=causal)
    torch.cuda.synchronize()
    return tuple(t.float().cpu().numpy().astype(np.float64) for t in (dq, dk, dv))


def check(got, ref, what, dtype):
    rel_rms_tol, rel_max_tol = TOL[dtype]
    for name, g, r in zip(("dQ", "dK", "dV"), got, ref):
        assert np.all(np.isfinite(g)), f"{what} {name}: non-finite"
        err = g - r
        rel = float(np.linalg.norm(err) / max(np.linalg.norm(r), 1e-300))
        mx = float(np.max(np.abs(err)) / max(np.max(np.abs(r)), 1e-300))
        print(f"[bwd] {what} {name}: rel_rms={rel:.2e} rel_max={mx:.2e}", flush=True)
        assert rel <= rel_rms_tol, f"{what} {name}: relative RMS {rel:.3e} > {rel_rms_tol:.2e}"
        assert mx <= rel_max_tol, f"{what} {name}: max error {mx:.3e} of max |ref| > {rel_max_tol:.2e}"


CASES = [
    (1, 2, 256, 64, "bf16"),
    (1, 2, 300, 128, "bf16"),
    (2, 3, 129, 128, "fp16"),
    (1, 4, 1000, 64, "fp16"),
    (1, 2, 2048, 128, "bf16"),
    (1, 1, 1, 128, "bf16"),
    (1, 2, 33, 64, "bf16"),
    (1, 2, 300, 128, "fp32"),
    (2, 3, 129, 64, "fp32"),
    (1, 2, 1000, 128, "fp32"),
    (1, 1, 1, 64, "fp32"),
    (1, 2, 33, 128, "fp32"),
]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,H,N,d,dtype", CASES)
def test_backward_matches_oracle(B, H, N, d, dtype, causal):
    w = Workload("bwd", B, H, N, d, dtype, 3000 + N + d, 2.0)
    q, k, v = make_inputs(w)
    do = upstream(w, 4000 + N)
    got = run_backward(w, q, k, v, do, w.scale, causal)
    ref = attention_backward_reference(q, k, v, do, w.scale, causal=causal)
    check(got, ref, f"B{B} H{H} N{N} d{d} {dtype} causal={causal}", dtype)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_named_workload_4096(causal):
    """The 4096-token bf16 workload (B=1, H=8, d=128)."""
    w = WORKLOADS["n4096_d128_bf16"]
    q, k, v = make_inputs(w)
    do = upstream(w, 41)
    got = run_backward(w, q, k, v, do, w.scale, causal)
    ref = attention_backward_reference(q, k, v, do, w.scale, causal=causal)
    check(got, ref, f"n4096 causal={causal}", w.dtype)


@pytest.mark.parametrize("scale", [0.0, -0.2])
def test_backward_scales(scale):
    w = Workload("bwds", 1, 2, 200, 64, "bf16", 51, 1.5)
    q, k, v = make_inputs(w)
    do = upstream(w, 52)
    got = run_backward(w, q, k, v, do, scale, False)
    ref = attention_backward_reference(q, k, v, do, scale)
    if scale == 0.0:  # dQ = dK = 0 exactly
        assert np.all(got[0] == 0.0) and np.all(got[1] == 0.0)
        err = float(np.linalg.norm(got[2] - ref[2]) / np.linalg.norm(ref[2]))
        assert err <= 2.5 * UNIT["bf16"]
    else:
        check(got, ref, f"scale={scale}", "bf16")


def test_backward_deterministic():
    w = Workload("bwdd", 1, 2, 700, 128, "bf16", 61)
    q, k, v = make_inputs(w)
    do = upstream(w, 62)
    a = run_backward(w, q, k, v, do, w.scale, False)
    b = run_backward(w, q, k, v, do, w.scale, False)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_named_workload_256_fp32(causal):
    """The 256-token float32 workload (B=1, H=1, d=64)."""
    w = WORKLOADS["n256_d64_fp32"]
    q, k, v = make_inputs(w)
    do = upstream(w, 43)
    got = run_backward(w, q, k, v, do, w.scale, causal)
    ref = attention_backward_reference(q, k, v, do, w.scale, causal=causal)
    check(got, ref, f"n256 fp32 causal={causal}", w.dtype)


def test_backward_fp32_deterministic():
    w = Workload("bwdd32", 1, 2, 300, 128, "fp32", 63)
    q, k, v = make_inputs(w)
    do = upstream(w, 64)
    a = run_backward(w, q, k, v, do, w.scale, True)
    b = run_backward(w, q, k, v, do, w.scale, True)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_long_context(causal):
    """The 32768-token workload (B=1, H=16, d=128, bf16, q and k with sigma 3)
    in the launches `bench.py --backward` times.

    dQ: sampled rows against the row-wise oracle, to the bf16 bounds above.
    dK, dV: one key of every 256-key tile of head 0 (and tile edges) against
    the column-wise oracle, to the same bounds.
    dV: the identity sum_j dV_j = sum_i dO_i (every probability row sums to
    1, causal rows too), which holds at any size. Its error has two sources:
    the rounded probabilities of a row sum to 1 within about u/(2 sqrt 3)
    (relative, random over rows), and each dV_j is rounded to bf16 (about
    u/(2 sqrt 3) relative, random over keys). Each is about 0.3 u of
    ||sum_i dO_i|| for random dO, so the bound is the dV RMS bound, 2.5 u.
    """
    w = WORKLOADS["n32768_d128_bf16"]
    q, k, v = make_inputs(w)
    do = upstream(w, 45)
    dt = TORCH_DT[w.dtype]
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(dt).cuda()  # noqa: E731
    tq, tk, tv, tdo = dev(q), dev(k), dev(v), dev(do)
    print(f"[bwd] n32768 causal={causal}: forward + backward", flush=True)
    o, lse = fa.flash_attn_fwd(tq, tk, tv, w.scale, causal=causal)
    dq, dk, dv = fa.flash_attn_bwd(tq, tk, tv, o, lse, tdo, w.scale, causal=causal)
    torch.cuda.synchronize()
    for name, g in (("dQ", dq), ("dK", dk), ("dV", dv)):
        assert bool(torch.isfinite(g).all()), f"{name}: non-finite"

    rows = np.unique(np.concatenate([sample_rows(w.N, 12), [31, 32, 255, 256, 16384]]))
    got = dq[:, :, torch.from_numpy(rows).cuda()].double().cpu().numpy()
    ref = attention_backward_rows(q, k, v, do, w.scale, rows, causal=causal)
    rel_rms_tol, rel_max_tol = TOL[w.dtype]
    err = got - ref
    rel = float(np.linalg.norm(err) / np.linalg.norm(ref))
    mx = float(np.max(np.abs(err)) / np.max(np.abs(ref)))
    print(f"[bwd] n32768 causal={causal} dQ rows: rel_rms={rel:.2e} rel_max={mx:.2e}", flush=True)
    assert rel <= rel_rms_tol and mx <= rel_max_tol

    # dK and dV of head 0 at one key per 256-key workgroup tile (a different
    # offset in each tile) plus tile edges, element by element against the
    # column-wise oracle (every query row of the head gathered per key)
    h = 0
    cols = np.unique(np.concatenate([np.arange(0, w.N, 256) + (np.arange(w.N // 256) * 37) % 256,
                                     [0, 31, 32, 255, 256, w.N - 1]]))
    got_k = dk[0, h, torch.from_numpy(cols).cuda()].double().cpu().numpy()
    got_v = dv[0, h, torch.from_numpy(cols).cuda()].double().cpu().numpy()
    print(f"[bwd] n32768 causal={causal} dK/dV of {len(cols)} keys of head {h}: oracle", flush=True)
    ref_k, ref_v = attention_backward_cols(q[:, h:h + 1], k[:, h:h + 1], v[:, h:h + 1], do[:, h:h + 1], w.scale,
                                           cols, causal=causal)
    for name, g, r in (("dK", got_k, ref_k[0, 0]), ("dV", got_v, ref_v[0, 0])):
        e = g - r
        rel = float(np.linalg.norm(e) / np.linalg.norm(r))
        mx = float(np.max(np.abs(e)) / np.max(np.abs(r)))
        print(f"[bwd] n32768 causal={causal} {name} keys: rel_rms={rel:.2e} rel_max={mx:.2e}", flush=True)
        assert rel <= rel_rms_tol and mx <= rel_max_tol, name

    lhs = dv.double().sum(dim=2).cpu().numpy()
    rhs = do.astype(np.float64).sum(axis=2)
    rel_dv = float(np.linalg.norm(lhs - rhs) / np.linalg.norm(rhs))
    print(f"[bwd] n32768 causal={causal} sum_j dV_j vs sum_i dO_i: rel={rel_dv:.2e}", flush=True)
    assert rel_dv <= 2.5 * UNIT[w.dtype]


@pytest.mark.parametrize("B,H,dtype", [(4, 32, "bf16"), (2, 64, "fp16")])
def test_backward_wide_key_workgroups(B, H, dtype):
    """Grids with at least two 256-key workgroups per CU of a 256-CU MI355X
    (B * H * ceil(N / 256) = 512), which take the 8-wave dK/dV kernel at
    d = 128 (non-causal), with a ragged length (1000 = 31 * 32 + 8); all three
    gradients against the oracle."""
    w = Workload("bwdw", B, H, 1000, 128, dtype, 71, 2.0)
    q, k, v = make_inputs(w)
    do = upstream(w, 72)
    got = run_backward(w, q, k, v, do, w.scale, False)
    ref = attention_backward_reference(q, k, v, do, w.scale)
    check(got, ref, f"wide B{B} H{H} N1000 {dtype}", dtype)
