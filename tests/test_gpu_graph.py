"""HIP graph capture of the library's calls (torch.cuda.CUDAGraph).

The entry points only launch kernels on the caller's stream: no allocation,
memset or synchronisation. A captured call therefore replays the same
kernels on the same buffers.

Each case:
1. runs one call eagerly and keeps its outputs;
2. captures the same call into a graph;
3. replays the graph three times. Before each replay the outputs are
   overwritten with NaN. Between replays the program does eager work of its
   own (another library call, a torch op) and synchronises.
4. Every replay must equal the eager result bitwise; the kernels are
   deterministic.

The shapes reach every launch path of the forward pass, plus the causal
form, float32, and the allocation-free backward.
"""
import ctypes
import math

import pytest
import torch

import io_aware_tiled_06_amd as fa
from io_aware_tiled_06_amd.workloads import Workload, make_inputs

pytestmark = pytest.mark.gpu

DTYPE_CODE = {"fp32": 0, "fp16": 1, "bf16": 2}  # fa_dtype in include/flash_attn.h
TORCH_DTYPE = {"fp32": torch.float32, "fp16": torch.float16, "bf16": torch.bfloat16}

# (label, B, H, N, d, dtype, causal); paths for a 256-CU device
FWD_CASES = [
    ("rounds, two 4-wave workgroups per CU", 4, 16, 1024, 128, "bf16", False),
    ("key split in the workgroup", 1, 2, 2048, 128, "bf16", False),
    ("full rounds plus the 64-row remainder launch", 1, 4, 16640, 128, "fp16", False),
    ("8-wave 256-row workgroups", 1, 32, 8192, 128, "bf16", False),
    ("rounds at d = 64, three workgroups per CU", 4, 32, 512, 64, "bf16", False),
    ("causal", 1, 8, 3000, 128, "bf16", True),
    ("float32", 1, 2, 300, 64, "fp32", False),
]


def _inputs(B, H, N, d, dtype, seed):
    w = Workload(f"graph_b{B}_h{H}_n{N}_d{d}_{dtype}", B, H, N, d, dtype, seed)
    dev = torch.device("cuda:0")
    return [torch.from_numpy(x).to(TORCH_DTYPE[dtype]).to(dev) for x in make_inputs(w)]


def _replay_and_check(graph, outputs, refs, eager_other):
    for rep in range(3):
        for t in outputs:
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        eager_other()
        torch.cuda.synchronize()
        for i, (t, r) in enumerate(zip(outputs, refs)):
            assert torch.equal(t, r), f"replay {rep}: output {i} differs from the eager call"


def _other_work():
    """Eager work of the program between replays: a different library call
    (its own buffers) and a torch op."""
    q, k, v = _inputs(1, 2, 700, 64, "fp16", 11)
    o, lse = fa.flash_attn_fwd(q, k, v)
    o.mul_(2.0)
    return o, lse


@pytest.mark.parametrize("label,B,H,N,d,dtype,causal", FWD_CASES, ids=[c[0] for c in FWD_CASES])
def test_forward_graph_replays(label, B, H, N, d, dtype, causal):
    print(f"[graph] forward {label}: B{B} H{H} N{N} d{d} {dtype} causal={causal}", flush=True)
    q, k, v = _inputs(B, H, N, d, dtype, 21)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    scale = 1.0 / math.sqrt(d)
    L = fa.lib()
    fn = L.flash_attn_fwd_causal if causal else L.flash_attn_fwd

    def call():
        st = fn(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, N, d,
                ctypes.c_float(scale), DTYPE_CODE[dtype], ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        assert st == 0, f"status {st}"

    call()  # eager: the reference, and any per-device set-up before capture
    torch.cuda.synchronize()
    refs = [o.clone(), lse.clone()]
    assert torch.isfinite(refs[0].float()).all() and torch.isfinite(refs[1]).all()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    _replay_and_check(g, [o, lse], refs, _other_work)


def test_noalloc_backward_graph_replays():
    B, H, N, d, dtype = 1, 4, 1024, 128, "bf16"
    print(f"[graph] flash_attn_bwd_noalloc B{B} H{H} N{N} d{d} {dtype}", flush=True)
    q, k, v = _inputs(B, H, N, d, dtype, 31)
    gen = torch.Generator(device="cpu").manual_seed(32)
    dout = torch.randn(q.shape, generator=gen).to(q.dtype).to(q.device)
    o, lse = fa.flash_attn_fwd(q, k, v)
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))

    def call():
        fa.flash_attn_bwd_noalloc(q, k, v, o, lse, dout, dq, dk, dv)

    call()
    torch.cuda.synchronize()
    refs = [dq.clone(), dk.clone(), dv.clone()]
    assert all(torch.isfinite(r.float()).all() for r in refs)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    _replay_and_check(g, [dq, dk, dv], refs, _other_work)
