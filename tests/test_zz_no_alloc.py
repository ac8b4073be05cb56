"""The allocation-free backward entry point (flash_attn_bwd_noalloc) against
flash_attn_bwd, through the C interface, on the GPU.

Two calls in a row share the library's fixed scratch: the first at the largest
size it accepts (B*H*N = NOALLOC_MAX_ROWS), the second smaller, so the second
reads a scratch array that still holds the first call's statistics. Each must
give bitwise the gradients of flash_attn_bwd with a caller-owned scratch (the
same kernels on the same inputs), and the small case is also compared with the
float64 gradient oracle to the bf16/fp16 bounds of the backward tests
(relative RMS <= 2.5 u, max <= 5 u of max|ref|, u the unit roundoff).
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import io_aware_tiled_06_amd as fa  # noqa: E402
from io_aware_tiled_06_amd.workloads import Workload, make_inputs  # noqa: E402
from oracle import attention_backward_reference  # noqa: E402

pytestmark = pytest.mark.gpu

TORCH_DT = {"fp16": torch.float16, "bf16": torch.bfloat16}
UNIT = {"bf16": 2.0 ** -8, "fp16": 2.0 ** -11}


def _inputs(w, seed):
    q, k, v = make_inputs(w)
    rng = np.random.default_rng(seed)
    do = rng.standard_normal(w.shape, dtype=np.float32)
    dt = TORCH_DT[w.dtype]
    t = [torch.from_numpy(x).to(dt).cuda() for x in (q, k, v, do)]
    return (q, k, v), t


def _both(tq, tk, tv, tdo, scale):
    o, lse = fa.flash_attn_fwd(tq, tk, tv, scale)
    ref = fa.flash_attn_bwd(tq, tk, tv, o, lse, tdo, scale)
    outs = [torch.empty_like(tq) for _ in range(3)]
    got = fa.flash_attn_bwd_noalloc(tq, tk, tv, o, lse, tdo, *outs, scale)
    torch.cuda.synchronize()
    return ref, got


def test_noalloc_matches_backward_two_calls():
    # call 1: the largest accepted size (B*H*N = 4194304), d = 64, bf16;
    # inputs drawn on the GPU (the values do not matter for bitwise equality)
    B, H, N, d = 1, 128, 32768, 64
    assert B * H * N == fa.NOALLOC_MAX_ROWS
    print(f"[noalloc] call 1: B={B} H={H} N={N} d={d} bf16", flush=True)
    gen = torch.Generator(device="cuda").manual_seed(21)
    tq, tk, tv, tdo = (torch.randn((B, H, N, d), generator=gen, device="cuda").to(torch.bfloat16)
                       for _ in range(4))
    ref, got = _both(tq, tk, tv, tdo, 0.125)
    for name, r, g in zip(("dQ", "dK", "dV"), ref, got):
        assert torch.equal(r, g), f"call 1 {name} differs from flash_attn_bwd"
    del tq, tk, tv, tdo, ref, got
    torch.cuda.empty_cache()

    # call 2: smaller, ragged, fp16, d = 128; also against the float64 oracle
    w = Workload("noalloc", 1, 3, 1000, 128, "fp16", 22, 2.0)
    print(f"[noalloc] call 2: B={w.B} H={w.H} N={w.N} d={w.d} {w.dtype}", flush=True)
    (q, k, v), (tq, tk, tv, tdo) = _inputs(w, 23)
    ref, got = _both(tq, tk, tv, tdo, w.scale)
    for name, r, g in zip(("dQ", "dK", "dV"), ref, got):
        assert torch.equal(r, g), f"call 2 {name} differs from flash_attn_bwd"
    do = tdo.float().cpu().numpy().astype(np.float64)
    oracle = attention_backward_reference(q, k, v, do, w.scale)
    u = UNIT[w.dtype]
    for name, g, r in zip(("dQ", "dK", "dV"), got, oracle):
        g = g.double().cpu().numpy()
        rel = float(np.linalg.norm(g - r) / np.linalg.norm(r))
        mx = float(np.max(np.abs(g - r)) / np.max(np.abs(r)))
        print(f"[noalloc] call 2 {name}: rel_rms={rel:.2e} rel_max={mx:.2e}", flush=True)
        assert rel <= 2.5 * u and mx <= 5 * u, name


def test_noalloc_rejects_oversize_on_gpu():
    """Beyond the fixed scratch: an error before any launch, outputs untouched."""
    x = torch.zeros((1, 1, fa.NOALLOC_MAX_ROWS + 32, 64), dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros((1, 1, x.shape[2]), dtype=torch.float32, device="cuda")
    outs = [torch.full_like(x, 7.0) for _ in range(3)]
    with pytest.raises(fa.FlashAttnError) as e:
        fa.flash_attn_bwd_noalloc(x, x, x, x, lse, x, *outs)
    assert e.value.status == fa.FA_ERR_TOO_LARGE
    torch.cuda.synchronize()
    assert all(bool((t == 7.0).all()) for t in outs)
