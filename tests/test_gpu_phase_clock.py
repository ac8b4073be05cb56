"""The phase-clock build (libflashattn_clock.so, FA_DEBUG_CLOCK): one record
per workgroup of the forward kernel, with consistent fields, and results
bitwise those of the library proper (the build adds timing only)."""
import ctypes

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import io_aware_tiled_06_amd as fa  # noqa: E402
from io_aware_tiled_06_amd.workloads import Workload, make_inputs  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("B,H,N,d,nw,split,n_wg", [(2, 8, 1024, 128, 4, 2, 128), (4, 32, 1000, 64, 4, 1, 1024)])
def test_phase_clock_records(B, H, N, d, nw, split, n_wg):
    w = Workload("clock", B, H, N, d, "bf16", 21)
    q, k, v = (torch.from_numpy(x).to(torch.bfloat16).cuda() for x in make_inputs(w))
    print(f"[phase-clock] B{B} H{H} N{N} d{d}", flush=True)
    o_ref, lse_ref = fa.flash_attn_fwd(q, k, v, w.scale)
    with fa.using_library(fa.CLOCK_LIB_PATH) as L:
        L.fa_clock_clear.restype = ctypes.c_int
        L.fa_clock_read.argtypes = [ctypes.POINTER(ctypes.c_ulonglong), ctypes.c_int]
        L.fa_clock_read.restype = ctypes.c_int
        torch.cuda.synchronize()
        assert L.fa_clock_clear() == 0
        o, lse = fa.flash_attn_fwd(q, k, v, w.scale)
        torch.cuda.synchronize()
        buf = (ctypes.c_ulonglong * (8 * 4096))()
        n = L.fa_clock_read(buf, 4096)
    assert torch.equal(o, o_ref) and torch.equal(lse, lse_ref)
    assert n == n_wg
    a = np.frombuffer(buf, dtype=np.uint64).reshape(-1, 8)[:n]
    tag = a[:, 7]
    assert np.all(tag & 0xFF == 1)
    assert np.all((tag >> 8) & 0xFF == nw) and np.all((tag >> 16) & 0xFF == split) and np.all((tag >> 24) & 0xFF == d)
    assert sorted((tag >> 32).tolist()) == list(range(n_wg))  # every workgroup once
    assert np.all(a[:, 1] > a[:, 0])  # realtime end after start
    assert np.all((0 < a[:, 2]) & (a[:, 2] <= a[:, 3]) & (a[:, 3] <= a[:, 4]))  # prologue, loop, stores in order
    assert len(set((a[:, 6] & 0xF).tolist())) == 8  # every XCD ran some
