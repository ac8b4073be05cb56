"""Tensors past 2 GiB: every offset of the forward and backward kernels is 64-bit.

Two layouts, d=128 bf16, each of q, k, v, o, dO, dQ, dK, dV over 2^31 bytes:

- long heads: B=1, H=260, N=32768 (head 256 starts at byte 2^31). The
  benchmark's launches: 8-wave forward, 8-wave dQ and dK/dV kernels.
- short heads: B=1, H=4100, N=2048 (head 4096 starts at byte 2^31). The
  4-wave forward; the same 8-wave backward kernels. Heads this short let the
  oracle compute every gradient of a checked head.

In both layouts a few heads hold seeded random data and every other head is
zero. In the long layout q and k have sigma 3, as in the 32K workload; in the
short one sigma 1, as in the other full-gradient checks.

- Checked heads: O, LSE, dQ, dK and dV against the float64 oracle. Long heads
  use sampled rows for O, LSE and dQ. For dV they use the identity
  sum_j dV_j = sum_i dO_i, which holds at any size and fails if a head's dV
  was written elsewhere.
- Zero heads: O = 0, LSE = ln(visible keys) and zero gradients, so no write
  meant for another head landed in them.

Tolerances are those of the other parity tests: forward max|dO| <= 2e-2,
relative RMS <= 1e-2, max|dLSE| <= 1e-3. Backward: relative RMS <= 2.5 u and
max error <= 5 u of max|reference|, with u = 2^-8.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import io_aware_tiled_06_amd as fa  # noqa: E402
from io_aware_tiled_06_amd.workloads import WORKLOADS, make_inputs, sample_rows  # noqa: E402
from oracle import attention_backward_reference, attention_backward_rows, attention_reference  # noqa: E402

pytestmark = pytest.mark.gpu

UNIT_BF16 = 2.0 ** -8
LAYOUTS = {
    # name: (H, N, seeded heads, zero heads checked)
    "long": (260, 32768, (0, 256, 259), (1, 128, 255, 257, 258)),
    "short": (4100, 2048, (0, 4096, 4099), (1, 2048, 4095, 4097, 4098)),
}


def build(layout, seed):
    H, N, heads, zeros = LAYOUTS[layout]
    base = WORKLOADS["n32768_d128_bf16"]
    # long heads: q and k with sigma 3 as in the 32K workload; short heads:
    # sigma 1, as in the other full-gradient checks
    sigma = base.qk_sigma if layout == "long" else 1.0
    w = base.with_(name=f"offsets_{layout}", H=len(heads), N=N, seed=seed, qk_sigma=sigma)
    q3, k3, v3 = make_inputs(w)
    rng = np.random.default_rng(seed + 40)
    do3 = torch.from_numpy(rng.standard_normal(q3.shape, dtype=np.float32)).to(torch.bfloat16).float().numpy()
    shape = (1, H, N, w.d)
    assert H * N * w.d * 2 > 2 ** 31 and heads[1] * N * w.d * 2 >= 2 ** 31
    t = {}
    for name, x in (("q", q3), ("k", k3), ("v", v3), ("do", do3)):
        full = torch.zeros(shape, dtype=torch.bfloat16, device="cuda")
        for i, h in enumerate(heads):
            full[0, h] = torch.from_numpy(np.ascontiguousarray(x[0, i])).to(torch.bfloat16).cuda()
        t[name] = full
    return w, (q3, k3, v3, do3), t, torch.tensor(heads, device="cuda"), torch.tensor(zeros, device="cuda")


def causal_rows_reference(q, k, v, scale, rows):
    """Oracle rows of causal attention: query i over keys 0..i, row by row."""
    lead = q.shape[:-2]
    o = np.empty(lead + (len(rows), v.shape[-1]))
    lse = np.empty(lead + (len(rows),))
    for t, i in enumerate(rows):
        oi, li = attention_reference(q[..., i:i + 1, :], k[..., :i + 1, :], v[..., :i + 1, :], scale)
        o[..., t, :] = oi[..., 0, :]
        lse[..., t] = li[..., 0]
    return o, lse


def check_forward(o_s, lse_s, o_ref, lse_ref, what):
    err = o_s - o_ref
    mx = float(np.max(np.abs(err)))
    rel = float(np.linalg.norm(err) / np.linalg.norm(o_ref))
    dl = float(np.max(np.abs(lse_s - lse_ref)))
    print(f"[offsets] {what}: max|dO|={mx:.2e} rel_rms={rel:.2e} max|dLSE|={dl:.2e}", flush=True)
    assert mx <= 2e-2 and rel <= 1e-2 and dl <= 1e-3


def check_grad(got, ref, what):
    err = got - ref
    rel = float(np.linalg.norm(err) / np.linalg.norm(ref))
    mx = float(np.max(np.abs(err)) / np.max(np.abs(ref)))
    print(f"[offsets] {what}: rel_rms={rel:.2e} rel_max={mx:.2e}", flush=True)
    assert np.all(np.isfinite(got)), what
    assert rel <= 2.5 * UNIT_BF16 and mx <= 5 * UNIT_BF16, what


def check_zero_heads(o, lse, zh, rows, n, causal):
    assert float(o[:, zh].abs().max()) == 0.0
    lz = lse[:, zh][:, :, torch.from_numpy(rows).cuda()].double().cpu().numpy()
    visible = (rows + 1) if causal else np.full(rows.shape, n)
    assert float(np.max(np.abs(lz - np.log(visible)))) <= 1e-3


@pytest.mark.parametrize("causal", [False, True])
def test_long_heads_forward(causal):
    w, (q3, k3, v3, _), t, hh, zh = build("long", 7)
    print(f"[offsets] long heads H=260 N=32768 forward causal={causal}", flush=True)
    o, lse = fa.flash_attn_fwd(t["q"], t["k"], t["v"], w.scale, causal=causal)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([sample_rows(w.N, 24), [127, 128, 255, 256]]))
    idx = torch.from_numpy(rows).cuda()
    o_s = o[:, hh][:, :, idx].double().cpu().numpy()
    lse_s = lse[:, hh][:, :, idx].double().cpu().numpy()
    if causal:
        o_ref, lse_ref = causal_rows_reference(q3, k3, v3, w.scale, rows)
    else:
        o_ref, lse_ref = attention_reference(q3[:, :, rows], k3, v3, w.scale)
    check_forward(o_s, lse_s, o_ref, lse_ref, f"long causal={causal}")
    check_zero_heads(o, lse, zh, rows, w.N, causal)


def test_long_heads_backward():
    w, (q3, k3, v3, do3), t, hh, zh = build("long", 7)
    print("[offsets] long heads H=260 N=32768 backward", flush=True)
    o, lse = fa.flash_attn_fwd(t["q"], t["k"], t["v"], w.scale)
    dq, dk, dv = fa.flash_attn_bwd(t["q"], t["k"], t["v"], o, lse, t["do"], w.scale)
    torch.cuda.synchronize()
    for name, g in (("dQ", dq), ("dK", dk), ("dV", dv)):
        assert bool(torch.isfinite(g[:, hh]).all()), f"{name}: non-finite"
        assert float(g[:, hh].abs().max()) > 0.0, f"{name}: zero in a seeded head"
        assert float(g[:, zh].abs().max()) == 0.0, f"{name}: nonzero in a zero head"
    rows = np.unique(np.concatenate([sample_rows(w.N, 8), [255, 256]]))
    got = dq[:, hh][:, :, torch.from_numpy(rows).cuda()].double().cpu().numpy()
    check_grad(got, attention_backward_rows(q3, k3, v3, do3, w.scale, rows), "long dQ rows")
    dv_sum = dv[:, hh].double().sum(dim=2).cpu().numpy()
    do_sum = do3.astype(np.float64).sum(axis=2)
    rel_dv = float(np.linalg.norm(dv_sum - do_sum) / np.linalg.norm(do_sum))
    print(f"[offsets] long sum_j dV_j vs sum_i dO_i: rel={rel_dv:.2e}", flush=True)
    assert rel_dv <= 2.5 * UNIT_BF16


@pytest.mark.parametrize("causal", [False, True])
def test_short_heads_forward_backward(causal):
    w, (q3, k3, v3, do3), t, hh, zh = build("short", 8)
    print(f"[offsets] short heads H=4100 N=2048 causal={causal}", flush=True)
    o, lse = fa.flash_attn_fwd(t["q"], t["k"], t["v"], w.scale, causal=causal)
    dq, dk, dv = fa.flash_attn_bwd(t["q"], t["k"], t["v"], o, lse, t["do"], w.scale, causal=causal)
    torch.cuda.synchronize()
    o_ref, lse_ref = attention_reference(q3, k3, v3, w.scale, causal=causal)
    check_forward(o[:, hh].double().cpu().numpy(), lse[:, hh].double().cpu().numpy(), o_ref, lse_ref,
                  f"short causal={causal}")
    check_zero_heads(o, lse, zh, np.arange(w.N), w.N, causal)
    ref = attention_backward_reference(q3, k3, v3, do3, w.scale, causal=causal)
    for name, g, r in zip(("dQ", "dK", "dV"), (dq, dk, dv), ref):
        check_grad(g[:, hh].double().cpu().numpy(), r, f"short causal={causal} {name}")
        assert float(g[:, zh].abs().max()) == 0.0, f"{name}: nonzero in a zero head"
