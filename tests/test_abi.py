"""The C interface without a GPU: the library loads, exports every function the
header declares, and rejects bad arguments before any HIP call."""
import ctypes
import math
import os
import re

import pytest

import io_aware_tiled_06_amd as fa

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "flash_attn.h")

# Fake, 16-byte aligned "device" addresses: validation errors return before
# any of them is touched or passed to HIP.
P = 0x10000
P2 = 0x20000
P3 = 0x30000
PO = 0x40000
PL = 0x50000


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(fa.LIB_PATH):
        import __graft_entry__

        __graft_entry__.build()
    return fa.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?(?:int|size_t|char\s*\*|void)\s*\**\s*(\w+)\s*\(", text, re.M)))


def test_header_declares_expected_entry_points():
    assert declared_functions() == sorted(fa.EXPORTED_SYMBOLS)


def test_library_exports_every_declared_symbol(L):
    for name in declared_functions():
        assert hasattr(L, name), name
    # and they are C symbols (unmangled) in the dynamic symbol table
    import subprocess

    out = subprocess.run(["nm", "-D", "--defined-only", fa.LIB_PATH], capture_output=True, text=True).stdout
    for name in declared_functions():
        assert re.search(rf"\bT {name}$", out, re.M), name


def test_race_guard_library_exports_every_declared_symbol(L):
    """The race-guard build (FA_DEBUG_POISON) of the same sources loads and
    exports the same interface."""
    if not os.path.exists(fa.POISON_LIB_PATH):
        import __graft_entry__

        __graft_entry__.build()
    P_ = ctypes.CDLL(fa.POISON_LIB_PATH)
    for name in declared_functions():
        assert hasattr(P_, name), name


def test_strerror(L):
    for st in range(8):
        assert isinstance(fa.strerror(st), str) and fa.strerror(st)
    assert fa.strerror(0) == "success"
    assert fa.strerror(99) == "unknown status"


def call(L, q=P, k=P2, v=P3, o=PO, lse=PL, B=1, H=1, N=16, d=64, scale=0.125, dtype=2):
    return L.flash_attn_fwd(q, k, v, o, lse, B, H, N, d, scale, dtype, None)


def call_causal(L, q=P, k=P2, v=P3, o=PO, lse=PL, B=1, H=1, N=16, d=64, scale=0.125, dtype=2):
    return L.flash_attn_fwd_causal(q, k, v, o, lse, B, H, N, d, scale, dtype, None)


def naive(L, ws=0x60000, ws_bytes=1 << 20, **kw):
    args = dict(q=P, k=P2, v=P3, o=PO, lse=PL, B=1, H=1, N=16, d=64, scale=0.125, dtype=2)
    args.update(kw)
    a = args
    return L.attn_naive_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["N"], a["d"],
                            a["scale"], a["dtype"], ws, ws_bytes, None)


@pytest.mark.parametrize("entry", [call, call_causal, naive])
def test_validation_errors(L, entry):
    assert entry(L, B=-1) == fa.FA_ERR_SHAPE
    assert entry(L, N=-5) == fa.FA_ERR_SHAPE
    assert entry(L, d=96) == fa.FA_ERR_UNSUPPORTED
    assert entry(L, d=0) == fa.FA_ERR_UNSUPPORTED
    assert entry(L, dtype=3) == fa.FA_ERR_UNSUPPORTED
    assert entry(L, scale=math.inf) == fa.FA_ERR_SCALE
    assert entry(L, scale=math.nan) == fa.FA_ERR_SCALE
    assert entry(L, q=None) == fa.FA_ERR_NULL
    assert entry(L, k=None) == fa.FA_ERR_NULL
    assert entry(L, v=None) == fa.FA_ERR_NULL
    assert entry(L, o=None) == fa.FA_ERR_NULL
    assert entry(L, q=P + 8) == fa.FA_ERR_ALIGN
    assert entry(L, o=PO + 2) == fa.FA_ERR_ALIGN
    assert entry(L, lse=PL + 4) == fa.FA_ERR_ALIGN
    # an absurd grid is rejected as a shape error
    assert entry(L, B=1 << 20, H=1 << 10, N=1 << 20) == fa.FA_ERR_SHAPE


@pytest.mark.parametrize("entry", [call, call_causal, naive])
def test_empty_problems_are_noops(L, entry):
    # nothing is launched and pointers are not looked at
    assert entry(L, B=0, q=None, k=None, v=None, o=None, lse=None) == fa.FA_OK
    assert entry(L, H=0, q=None) == fa.FA_OK
    assert entry(L, N=0, o=None) == fa.FA_OK


def test_naive_workspace_rules(L):
    need = 16 * 16 * (4 + 2)
    assert naive(L, ws_bytes=need - 1) == fa.FA_ERR_WORKSPACE
    assert naive(L, ws=None) == fa.FA_ERR_NULL
    assert naive(L, ws=0x60008) == fa.FA_ERR_ALIGN


def test_naive_workspace_bytes(L):
    assert fa.attn_naive_workspace_bytes(2, 3, 100, "bf16") == 2 * 3 * 100 * 100 * 6
    assert fa.attn_naive_workspace_bytes(1, 1, 100, "fp32") == 100 * 100 * 8
    assert fa.attn_naive_workspace_bytes(1, 8, 4096, "fp16") == 8 * 4096 * 4096 * 6
    assert L.attn_naive_workspace_bytes(1, 1, 10, 7) == 0
    assert L.attn_naive_workspace_bytes(-1, 1, 10, 2) == 0
    assert L.attn_naive_workspace_bytes(1 << 30, 1 << 30, 1 << 30, 2) == 0  # overflow


def test_binding_refuses_cpu_tensors():
    torch = pytest.importorskip("torch")
    x = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        fa.flash_attn_fwd(x, x, x)
    with pytest.raises(ValueError, match="GPU"):
        fa.attn_naive_fwd(x, x, x)


def test_binding_refuses_bad_naive_workspace():
    """The three-pass path writes S and P through the workspace address: a
    workspace on the host (or another device), or a strided one, must raise
    before any call."""
    torch = pytest.importorskip("torch")
    gpu = torch.device("cuda:0")  # a device object only; nothing is allocated on it
    with pytest.raises(ValueError, match="device"):
        fa._check_workspace(torch.empty(64, dtype=torch.uint8), gpu)
    with pytest.raises(ValueError, match="device"):
        fa._check_workspace(torch.empty(64, dtype=torch.uint8), torch.device("cuda:1"))
    with pytest.raises(TypeError):
        fa._check_workspace(bytearray(64), gpu)
    strided = torch.empty(128, dtype=torch.uint8)[::2]
    with pytest.raises(ValueError, match="contiguous"):
        fa._check_workspace(strided, strided.device)
    fa._check_workspace(torch.empty(64, dtype=torch.uint8), torch.device("cpu"))  # accepted as such


def bwd(L, ptrs=None, B=1, H=1, N=16, d=64, scale=0.125, dtype=2, causal=False):
    base = [P, P2, P3, 0x70000, 0x80000, PL, 0x90000, 0xA0000, 0xB0000, 0xC0000]
    if ptrs:
        for i, val in ptrs.items():
            base[i] = val
    fn = L.flash_attn_bwd_causal if causal else L.flash_attn_bwd
    return fn(*base, B, H, N, d, scale, dtype, None)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_validation(L, causal):
    assert bwd(L, B=-1, causal=causal) == fa.FA_ERR_SHAPE
    assert bwd(L, d=96, causal=causal) == fa.FA_ERR_UNSUPPORTED
    assert bwd(L, dtype=7, causal=causal) == fa.FA_ERR_UNSUPPORTED
    assert bwd(L, scale=math.nan, causal=causal) == fa.FA_ERR_SCALE
    for i in range(10):  # every pointer is required
        assert bwd(L, {i: None}, causal=causal) == fa.FA_ERR_NULL, i
    for i in (0, 3, 4, 6, 7, 8, 9):
        assert bwd(L, {i: [P, P2, P3, 0x70000, 0x80000, PL, 0x90000, 0xA0000, 0xB0000, 0xC0000][i] + 2},
                   causal=causal) == fa.FA_ERR_ALIGN, i
    assert bwd(L, N=0, causal=causal) == fa.FA_OK


def bwd_noalloc(L, ptrs=None, B=1, H=1, N=16, d=64, scale=0.125, dtype=2):
    base = [P, P2, P3, 0x70000, 0x80000, PL, 0x90000, 0xA0000, 0xB0000]
    if ptrs:
        for i, val in ptrs.items():
            base[i] = val
    return L.flash_attn_bwd_noalloc(*base, B, H, N, d, scale, dtype, None)


def test_noalloc_backward_validation(L):
    """The allocation-free backward pass validates like flash_attn_bwd and
    rejects problems beyond its fixed scratch, all before any HIP call."""
    assert bwd_noalloc(L, B=-1) == fa.FA_ERR_SHAPE
    assert bwd_noalloc(L, d=96) == fa.FA_ERR_UNSUPPORTED
    assert bwd_noalloc(L, dtype=7) == fa.FA_ERR_UNSUPPORTED
    assert bwd_noalloc(L, scale=math.inf) == fa.FA_ERR_SCALE
    for i in range(9):
        assert bwd_noalloc(L, {i: None}) == fa.FA_ERR_NULL, i
    for i in (0, 3, 4, 6, 7, 8):
        assert bwd_noalloc(L, {i: [P, P2, P3, 0x70000, 0x80000, PL, 0x90000, 0xA0000, 0xB0000][i] + 2}) == \
            fa.FA_ERR_ALIGN, i
    assert bwd_noalloc(L, N=0) == fa.FA_OK
    # one row past the limit, in several shapes
    assert bwd_noalloc(L, B=1, H=1, N=fa.NOALLOC_MAX_ROWS + 1) == fa.FA_ERR_TOO_LARGE
    assert bwd_noalloc(L, B=2, H=64, N=32769) == fa.FA_ERR_TOO_LARGE
    assert bwd_noalloc(L, B=1 << 20, H=1 << 20, N=1 << 20) in (fa.FA_ERR_SHAPE, fa.FA_ERR_TOO_LARGE)
    assert "scratch" in fa.strerror(fa.FA_ERR_TOO_LARGE)

