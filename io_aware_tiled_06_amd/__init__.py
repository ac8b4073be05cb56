"""MI355X (gfx950) attention forward pass: thin Python binding of libflashattn.so.

The binding only marshals arguments: every step of the computation runs in
the HIP kernels of ``libflashattn.so`` (built by ``io_aware_tiled_06_amd.build``).
There is no CPU fallback; without the built library, or with tensors that are
not on a GPU, calls raise.

    o, lse = flash_attn_fwd(q, k, v)            # q, k, v: [B, H, N, d] on the GPU
    o, lse = attn_naive_fwd(q, k, v)            # three-pass comparator
"""
from __future__ import annotations

import ctypes
import math
import os

__all__ = [
    "FlashAttnError",
    "flash_attn_fwd",
    "flash_attn_bwd",
    "attn_naive_fwd",
    "attn_naive_workspace_bytes",
    "lib",
    "LIB_PATH",
    "POISON_LIB_PATH",
    "CLOCK_LIB_PATH",
    "using_library",
    "EXPORTED_SYMBOLS",
    "DTYPE_CODE",
    "FA_OK",
    "FA_ERR_NULL",
    "FA_ERR_SHAPE",
    "FA_ERR_UNSUPPORTED",
    "FA_ERR_ALIGN",
    "FA_ERR_WORKSPACE",
    "FA_ERR_SCALE",
    "FA_ERR_HIP",
    "FA_ERR_TOO_LARGE",
    "NOALLOC_MAX_ROWS",
    "flash_attn_bwd_noalloc",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libflashattn.so")
# The race-guard build of the same sources (every LDS slot a copy refills
# holds NaN until the copy lands); see using_library().
POISON_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libflashattn_poison.so")
# The phase-clock build (the forward kernel records each workgroup's phase
# times and CU; it also exports fa_clock_clear and fa_clock_read); for
# bench.py --phase-clock.
CLOCK_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libflashattn_clock.so")
EXPORTED_SYMBOLS = ("flash_attn_fwd", "flash_attn_fwd_causal", "flash_attn_bwd", "flash_attn_bwd_causal",
                    "flash_attn_bwd_noalloc", "attn_naive_workspace_bytes", "attn_naive_fwd", "fa_strerror")

# fa_status values (include/flash_attn.h)
FA_OK, FA_ERR_NULL, FA_ERR_SHAPE, FA_ERR_UNSUPPORTED = 0, 1, 2, 3
FA_ERR_ALIGN, FA_ERR_WORKSPACE, FA_ERR_SCALE, FA_ERR_HIP = 4, 5, 6, 7
FA_ERR_TOO_LARGE = 8
# largest B*H*N of flash_attn_bwd_noalloc (FA_NOALLOC_MAX_ROWS)
NOALLOC_MAX_ROWS = 4194304
# fa_dtype values
DTYPE_CODE = {"fp32": 0, "fp16": 1, "bf16": 2}

_lib = None


class FlashAttnError(RuntimeError):
    """A non-zero fa_status returned by the library."""

    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {strerror(status)} (status {status})")


def lib() -> ctypes.CDLL:
    """The loaded libflashattn.so (or the library selected by using_library)
    with argument types declared."""
    global _lib
    if _lib is None:
        _lib = _load(LIB_PATH)
    return _lib


_loaded = {}


def using_library(path: str):
    """Context manager: every call of this module inside the block goes to the
    library at `path` (a build of the same sources, e.g. POISON_LIB_PATH),
    then back to the one before. Not thread-safe; meant for tests."""
    import contextlib

    @contextlib.contextmanager
    def _ctx():
        global _lib
        prev = _lib
        _lib = _load(path)
        try:
            yield _lib
        finally:
            _lib = prev

    return _ctx()


def _load(path: str) -> ctypes.CDLL:
    if path in _loaded:
        return _loaded[path]
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -m io_aware_tiled_06_amd.build all` (needs hipcc)")
    L = ctypes.CDLL(path)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    L.flash_attn_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, vp]
    L.flash_attn_fwd.restype = i
    L.flash_attn_fwd_causal.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, vp]
    L.flash_attn_fwd_causal.restype = i
    for name in ("flash_attn_bwd", "flash_attn_bwd_causal"):
        fn = getattr(L, name)
        fn.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, vp]
        fn.restype = i
    L.flash_attn_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, vp]
    L.flash_attn_bwd_noalloc.restype = i
    L.attn_naive_workspace_bytes.argtypes = [i, i, i, i]
    L.attn_naive_workspace_bytes.restype = sz
    L.attn_naive_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, vp, sz, vp]
    L.attn_naive_fwd.restype = i
    L.fa_strerror.argtypes = [i]
    L.fa_strerror.restype = ctypes.c_char_p
    _loaded[path] = L
    return L


def strerror(status: int) -> str:
    return lib().fa_strerror(int(status)).decode()


def _dtype_code(t) -> int:
    import torch

    codes = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}
    if t.dtype not in codes:
        raise TypeError(f"unsupported dtype {t.dtype}; expected float32, float16 or bfloat16")
    return codes[t.dtype]


def _check_inputs(q, k, v):
    import torch

    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        if t.device.type != "cuda":
            raise ValueError(f"{name} must be on the GPU (got {t.device}); there is no CPU path")
        if t.dim() != 4:
            raise ValueError(f"{name} must be [B, H, N, d]")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if not (q.shape == k.shape == v.shape):
        raise ValueError(f"q, k, v shapes differ: {tuple(q.shape)}, {tuple(k.shape)}, {tuple(v.shape)}")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v dtypes differ")
    if not (q.device == k.device == v.device):
        raise ValueError("q, k, v are on different devices")


def _default_scale(d: int) -> float:
    import numpy as np

    return float(np.float32(1.0 / math.sqrt(d)))


def _outputs(q, out, return_lse):
    import torch

    B, H, N, _ = q.shape
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype or out.device != q.device or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor of q's shape, dtype and device")
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if return_lse else None
    return out, lse


def _stream_ptr(q, stream):
    import torch

    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    return ctypes.c_void_p(stream.cuda_stream)


def flash_attn_fwd(q, k, v, scale=None, *, causal=False, out=None, return_lse=True, stream=None):
    """Fused tiled attention forward pass on the GPU.

    q, k, v: contiguous [B, H, N, d] tensors (float32, float16 or bfloat16) on
    one GPU; d in {64, 128}. scale defaults to 1/sqrt(d) rounded to float32.
    causal=True calls flash_attn_fwd_causal (query i sees keys 0..i).
    Returns (o, lse): o like q, lse float32 [B, H, N] (None if not requested).
    The call is asynchronous on ``stream`` (default: the current stream).
    """
    import torch

    _check_inputs(q, k, v)
    B, H, N, d = q.shape
    s = _default_scale(d) if scale is None else float(scale)
    o, lse = _outputs(q, out, return_lse)
    fn = lib().flash_attn_fwd_causal if causal else lib().flash_attn_fwd
    with torch.cuda.device(q.device):
        st = fn(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr() if lse is not None else None,
                B, H, N, d, s, _dtype_code(q), _stream_ptr(q, stream))
    if st != FA_OK:
        raise FlashAttnError(st, "flash_attn_fwd_causal" if causal else "flash_attn_fwd")
    return o, lse


def flash_attn_bwd(q, k, v, o, lse, dout, scale=None, *, causal=False, dq=None, dk=None, dv=None, delta=None,
                   stream=None):
    """Gradients of the fused forward pass (dQ, dK, dV) on the GPU.

    q, k, v, o, dout: contiguous [B, H, N, d] float32, float16 or bfloat16
    tensors on one GPU; lse: the float32 [B, H, N] LSE that flash_attn_fwd returned for these
    inputs (and the same `causal`). dq, dk, dv default to new tensors like q;
    delta (float32 scratch of 2 * B * H * N elements) to a new tensor. Returns
    (dq, dk, dv).
    """
    import torch

    _check_inputs(q, k, v)
    for name, t in (("o", o), ("dout", dout)):
        if t.shape != q.shape or t.dtype != q.dtype or t.device != q.device or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous tensor of q's shape, dtype and device")
    B, H, N, d = q.shape
    if lse.shape != (B, H, N) or lse.dtype != torch.float32 or lse.device != q.device or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [B, H, N] tensor on q's device")
    s = _default_scale(d) if scale is None else float(scale)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        if t.shape != q.shape or t.dtype != q.dtype or t.device != q.device or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous tensor of q's shape, dtype and device")
    if delta is None:
        delta = torch.empty((2, B, H, N), dtype=torch.float32, device=q.device)
    elif (delta.dtype != torch.float32 or delta.device != q.device or not delta.is_contiguous()
          or delta.numel() < 2 * B * H * N):
        raise ValueError("delta must be a contiguous float32 tensor of at least 2*B*H*N elements on q's device")
    fn = lib().flash_attn_bwd_causal if causal else lib().flash_attn_bwd
    with torch.cuda.device(q.device):
        st = fn(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(), lse.data_ptr(),
                dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), delta.data_ptr(), B, H, N, d, s, _dtype_code(q),
                _stream_ptr(q, stream))
    if st != FA_OK:
        raise FlashAttnError(st, "flash_attn_bwd_causal" if causal else "flash_attn_bwd")
    return dq, dk, dv


def flash_attn_bwd_noalloc(q, k, v, o, lse, dout, dq, dk, dv, scale=None, *, stream=None):
    """flash_attn_bwd (non-causal) through the entry point that allocates
    nothing: the row statistics live in the library's fixed device scratch
    (B*H*N <= NOALLOC_MAX_ROWS). The caller supplies every output (dq, dk, dv
    like q). Calls that overlap on one GPU share that scratch and race."""
    import torch

    _check_inputs(q, k, v)
    B, H, N, d = q.shape
    for name, t in (("o", o), ("dout", dout), ("dq", dq), ("dk", dk), ("dv", dv)):
        if (not isinstance(t, torch.Tensor) or t.shape != q.shape or t.dtype != q.dtype or t.device != q.device
                or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous tensor of q's shape, dtype and device")
    if lse.shape != (B, H, N) or lse.dtype != torch.float32 or lse.device != q.device or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [B, H, N] tensor on q's device")
    s = _default_scale(d) if scale is None else float(scale)
    with torch.cuda.device(q.device):
        st = lib().flash_attn_bwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(),
                                          lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, N, d, s,
                                          _dtype_code(q), _stream_ptr(q, stream))
    if st != FA_OK:
        raise FlashAttnError(st, "flash_attn_bwd_noalloc")
    return dq, dk, dv


def _check_workspace(workspace, device) -> None:
    """A caller's workspace must be a contiguous tensor on the inputs' GPU: its
    address is handed to the kernels, which write S and P through it."""
    import torch

    if not isinstance(workspace, torch.Tensor):
        raise TypeError("workspace must be a torch.Tensor")
    if workspace.device != device:
        raise ValueError(f"workspace must be on the inputs' device {device} (got {workspace.device})")
    if not workspace.is_contiguous():
        raise ValueError("workspace must be contiguous")


def attn_naive_workspace_bytes(B: int, H: int, N: int, dtype: str) -> int:
    """Workspace for the three-pass path to process all heads at once."""
    return int(lib().attn_naive_workspace_bytes(B, H, N, DTYPE_CODE[dtype]))


def attn_naive_fwd(q, k, v, scale=None, *, out=None, return_lse=True, workspace=None, stream=None):
    """Three-pass materialising attention (S and P through device memory).

    Same arguments and results as ``flash_attn_fwd``. ``workspace`` is a
    uint8 GPU tensor of at least one head's N*N*(4 + element size) bytes; by
    default one large enough for every head is allocated.
    """
    import torch

    _check_inputs(q, k, v)
    B, H, N, d = q.shape
    s = _default_scale(d) if scale is None else float(scale)
    o, lse = _outputs(q, out, return_lse)
    if workspace is None:
        nbytes = int(lib().attn_naive_workspace_bytes(B, H, N, _dtype_code(q)))
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=q.device)
    _check_workspace(workspace, q.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    with torch.cuda.device(q.device):
        st = lib().attn_naive_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                  lse.data_ptr() if lse is not None else None,
                                  B, H, N, d, s, _dtype_code(q), workspace.data_ptr(), ws_bytes,
                                  _stream_ptr(q, stream))
    if st != FA_OK:
        raise FlashAttnError(st, "attn_naive_fwd")
    return o, lse
