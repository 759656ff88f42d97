"""Python binding of libssd.so (ctypes).  Argument marshalling only.

Every step of the layer runs in the HIP kernels of libssd.so; torch is used
for device memory and the current stream.  If the library is not built (or
cannot be loaded), every call raises -- there is no fallback path.

    y, final_state = chunk_scan_fwd(x, dt, A, B, C, D=None, chunk_len=256,
                                    init_state=None, cu_seqlens=None)
    y = decode_step(state, x, dt, A, B, C, D=None)      # updates state in place

Both take optional step-size preprocessing (dt_bias=[nheads] fp32,
dt_softplus=bool, dt_limit=(lo, hi)): dt = clamp(softplus(dt + dt_bias)).

Shapes (row-major, contiguous):
    x, y        [batch, seqlen, nheads, headdim]   bf16 or fp32 ("io" dtype)
    dt          [batch, seqlen, nheads]            fp32 (final positive step)
    A, D        [nheads]                           fp32
    B, C        [batch, seqlen, ngroups, dstate]   io dtype
    init_state, final_state [nseq, nheads, headdim, dstate] fp32
    cu_seqlens  [nseq + 1] int32 (packed batch: batch == 1)
"""
from __future__ import annotations

import contextlib
import ctypes
import os
import re

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libssd.so")
RACE_WIDEN_LIB_PATH = os.path.join(_HERE, "libssd_racewiden.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "ssd.h")

SSD_F32, SSD_BF16 = 0, 1
_STATUS = {
    0: "SSD_OK", 1: "SSD_ERR_NULL_PTR", 2: "SSD_ERR_SHAPE", 3: "SSD_ERR_DTYPE",
    4: "SSD_ERR_UNSUPPORTED", 5: "SSD_ERR_ALIGNMENT", 6: "SSD_ERR_ALIAS",
    7: "SSD_ERR_WORKSPACE", 8: "SSD_ERR_HIP", 9: "SSD_ERR_DEVICE",
}


class SsdError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {_STATUS.get(code, code)} ({code})")


class SsdDims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("batch", "seqlen", "nheads", "headdim", "dstate", "ngroups", "nseq")]


class SsdDtOpts(ctypes.Structure):
    _fields_ = [("dt_bias", ctypes.c_void_p), ("softplus", ctypes.c_int32),
                ("dt_min", ctypes.c_float), ("dt_max", ctypes.c_float)]


_lib = None
_VP = ctypes.c_void_p


def load_library(path: str = LIB_PATH):
    """Load libssd.so (raises if it is missing: build it with
    ``python -m selective_state_space_71_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"libssd.so is not built ({path}); run "
                           "`python -m selective_state_space_71_amd.build`")
    lib = ctypes.CDLL(path)
    lib.ssd_status_string.restype = ctypes.c_char_p
    lib.ssd_status_string.argtypes = [ctypes.c_int]
    lib.ssd_abi_version.restype = ctypes.c_int32
    lib.ssd_abi_version.argtypes = []
    lib.ssd_chunk_scan_fwd_workspace_size.restype = ctypes.c_size_t
    lib.ssd_chunk_scan_fwd_workspace_size.argtypes = [ctypes.POINTER(SsdDims), ctypes.c_int32, ctypes.c_int]
    lib.ssd_chunk_scan_fwd.restype = ctypes.c_int
    lib.ssd_chunk_scan_fwd.argtypes = [
        ctypes.POINTER(SsdDims), ctypes.c_int, ctypes.c_int32,
        _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP,
        _VP, ctypes.c_size_t, _VP,
    ]
    lib.ssd_chunk_scan_fwd_ex.restype = ctypes.c_int
    lib.ssd_chunk_scan_fwd_ex.argtypes = [
        ctypes.POINTER(SsdDims), ctypes.c_int, ctypes.c_int32, ctypes.POINTER(SsdDtOpts),
        _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP,
        _VP, ctypes.c_size_t, _VP,
    ]
    lib.ssd_chunk_scan_fwd_noalloc.restype = ctypes.c_int
    lib.ssd_chunk_scan_fwd_noalloc.argtypes = [
        ctypes.POINTER(SsdDims), ctypes.c_int, ctypes.c_int32, ctypes.POINTER(SsdDtOpts),
        _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP,
    ]
    lib.ssd_decode_step_ex.restype = ctypes.c_int
    lib.ssd_decode_step_ex.argtypes = [
        ctypes.POINTER(SsdDims), ctypes.c_int, ctypes.POINTER(SsdDtOpts),
        _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP,
    ]
    lib.ssd_chunk_scan_fwd_check.restype = ctypes.c_int
    lib.ssd_chunk_scan_fwd_check.argtypes = [_VP, _VP]
    lib.ssd_decode_step.restype = ctypes.c_int
    lib.ssd_decode_step.argtypes = [
        ctypes.POINTER(SsdDims), ctypes.c_int,
        _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP,
    ]
    lib.ssd_causal_conv1d_fwd.restype = ctypes.c_int
    lib.ssd_causal_conv1d_fwd.argtypes = [
        ctypes.POINTER(SsdDims), ctypes.c_int, ctypes.c_int32, _VP, _VP, _VP, ctypes.c_int32, _VP, _VP,
        _VP, _VP, _VP, _VP, _VP,
    ]
    lib.ssd_chunk_scan_bwd_workspace_size.restype = ctypes.c_size_t
    lib.ssd_chunk_scan_bwd_workspace_size.argtypes = [ctypes.POINTER(SsdDims), ctypes.c_int]
    lib.ssd_chunk_scan_bwd.restype = ctypes.c_int
    lib.ssd_chunk_scan_bwd.argtypes = [ctypes.POINTER(SsdDims), ctypes.c_int] + [_VP] * 18 + [ctypes.c_size_t, _VP]
    lib.ssd_gated_rmsnorm_fwd.restype = ctypes.c_int
    lib.ssd_gated_rmsnorm_fwd.argtypes = [
        ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int, _VP, _VP, _VP, ctypes.c_float,
        ctypes.c_int32, _VP, _VP,
    ]
    _lib = lib
    return lib


@contextlib.contextmanager
def using_library(path: str):
    """Route every call of this binding through another build of the library
    (such as the race-widening debug build at RACE_WIDEN_LIB_PATH) inside the
    block; the previous library is restored on exit."""
    global _lib
    prev = _lib
    _lib = None
    try:
        yield load_library(path)
    finally:
        _lib = prev


def header_functions(path: str = HEADER_PATH):
    """Names of the functions declared in include/ssd.h."""
    text = open(path).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ssd_[a-z0-9_]+)\s*\(", text)))


def _io_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return SSD_BF16
    if t.dtype == torch.float32:
        return SSD_F32
    raise TypeError(f"io tensors must be bfloat16 or float32, got {t.dtype}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t, name, dtype=None, shape=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _dt_opts(dt_bias, dt_softplus, dt_limit, H, dev):
    """ssd_dt_opts_t for the given preprocessing, or None when there is none."""
    if dt_bias is None and not dt_softplus and dt_limit is None:
        return None
    if dt_bias is not None:
        _need(dt_bias, "dt_bias", torch.float32, (H,), dev)
    lo, hi = dt_limit if dt_limit is not None else (-float("inf"), float("inf"))
    return SsdDtOpts(None if dt_bias is None else dt_bias.data_ptr(), 1 if dt_softplus else 0, lo, hi)


def fwd_dims(x, B, cu_seqlens=None) -> SsdDims:
    b, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    nseq = b if cu_seqlens is None else cu_seqlens.numel() - 1
    return SsdDims(b, L, H, P, N, G, nseq)


def workspace_size(dims: SsdDims, chunk_len: int, io: int) -> int:
    return int(load_library().ssd_chunk_scan_fwd_workspace_size(ctypes.byref(dims), chunk_len, io))


def chunk_scan_fwd(x, dt, A, B, C, D=None, chunk_len: int = 256, init_state=None,
                   cu_seqlens=None, return_final_state: bool = True, y=None, final_state=None,
                   workspace=None, dt_bias=None, dt_softplus: bool = False, dt_limit=None,
                   check: bool = False):
    """SSD forward through ``ssd_chunk_scan_fwd_ex``.  Returns (y, final_state).

    The call only enqueues the kernels.  Failures the device detects (a broken
    ``cu_seqlens``, a chain wait that gave up, an XCD whose work list was not
    drained) leave y and final_state invalid without an error here; with
    ``check=True`` the binding synchronises and raises ``SsdError`` for them
    (through ``ssd_chunk_scan_fwd_check``)."""
    lib = load_library()
    dev = x.device
    _need(x, "x", device=dev)
    io = _io_code(x)
    b, L, H, P = x.shape
    if B.dim() != 4 or B.shape[:2] != (b, L):
        raise ValueError("B must be [batch, seqlen, ngroups, dstate]")
    G, N = B.shape[2], B.shape[3]
    _need(dt, "dt", torch.float32, (b, L, H), dev)
    _need(A, "A", torch.float32, (H,), dev)
    _need(B, "B", x.dtype, (b, L, G, N), dev)
    _need(C, "C", x.dtype, (b, L, G, N), dev)
    if D is not None:
        _need(D, "D", torch.float32, (H,), dev)
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", torch.int32, None, dev)
        if b != 1:
            raise ValueError("packed varlen input needs batch == 1")
    dims = fwd_dims(x, B, cu_seqlens)
    nseq = dims.nseq
    if init_state is not None:
        _need(init_state, "init_state", torch.float32, (nseq, H, P, N), dev)
    if y is None:
        y = torch.empty_like(x)
    else:
        _need(y, "y", x.dtype, x.shape, dev)
    if final_state is None and return_final_state:
        final_state = torch.empty((nseq, H, P, N), dtype=torch.float32, device=dev)
    elif final_state is not None:
        _need(final_state, "final_state", torch.float32, (nseq, H, P, N), dev)
    ws_bytes = workspace_size(dims, chunk_len, io)
    if ws_bytes == 0:
        # the call itself names the reason (shape checks come before pointer
        # checks); cu_seqlens decides between the dense and the packed rules
        code = lib.ssd_chunk_scan_fwd(ctypes.byref(dims), io, chunk_len, *([None] * 7), _ptr(cu_seqlens),
                                      None, None, None, 0, None)
        raise SsdError(code, "ssd_chunk_scan_fwd (size query)")
    if workspace is None or workspace.numel() < ws_bytes:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    opts = _dt_opts(dt_bias, dt_softplus, dt_limit, H, dev)
    code = lib.ssd_chunk_scan_fwd_ex(
        ctypes.byref(dims), io, int(chunk_len), None if opts is None else ctypes.byref(opts),
        _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(init_state),
        _ptr(cu_seqlens), _ptr(y), _ptr(final_state),
        _ptr(workspace), ctypes.c_size_t(workspace.numel()), _stream(dev))
    if code != 0:
        raise SsdError(code, "ssd_chunk_scan_fwd_ex")
    chunk_scan_fwd.last_workspace = workspace
    if check:
        code = lib.ssd_chunk_scan_fwd_check(_ptr(workspace), _stream(dev))
        if code != 0:
            raise SsdError(code, "ssd_chunk_scan_fwd_check")
    return y, final_state


def chunk_scan_fwd_noalloc(x, dt, A, B, C, D=None, chunk_len: int = 256, init_state=None,
                           cu_seqlens=None, y=None, final_state=None, dt_bias=None,
                           dt_softplus: bool = False, dt_limit=None):
    """SSD forward through ``ssd_chunk_scan_fwd_noalloc``: no workspace; the
    library's per-device scratch array holds the schedule (and the boundary
    states when ``final_state`` is None).  Returns (y, final_state or None).
    With ``y`` (and ``final_state``) passed in, nothing is allocated here
    either.  Calls that overlap in time on one device race (they share the
    scratch array)."""
    lib = load_library()
    dev = x.device
    _need(x, "x", device=dev)
    io = _io_code(x)
    b, L, H, P = x.shape
    if B.dim() != 4 or B.shape[:2] != (b, L):
        raise ValueError("B must be [batch, seqlen, ngroups, dstate]")
    G, N = B.shape[2], B.shape[3]
    _need(dt, "dt", torch.float32, (b, L, H), dev)
    _need(A, "A", torch.float32, (H,), dev)
    _need(B, "B", x.dtype, (b, L, G, N), dev)
    _need(C, "C", x.dtype, (b, L, G, N), dev)
    if D is not None:
        _need(D, "D", torch.float32, (H,), dev)
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", torch.int32, None, dev)
    dims = fwd_dims(x, B, cu_seqlens)
    if init_state is not None:
        _need(init_state, "init_state", torch.float32, (dims.nseq, H, P, N), dev)
    if y is None:
        y = torch.empty_like(x)
    _need(y, "y", x.dtype, x.shape, dev)
    if final_state is not None:
        _need(final_state, "final_state", torch.float32, (dims.nseq, H, P, N), dev)
    opts = _dt_opts(dt_bias, dt_softplus, dt_limit, H, dev)
    code = lib.ssd_chunk_scan_fwd_noalloc(
        ctypes.byref(dims), io, int(chunk_len), None if opts is None else ctypes.byref(opts),
        _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(init_state),
        _ptr(cu_seqlens), _ptr(y), _ptr(final_state), _stream(dev))
    if code != 0:
        raise SsdError(code, "ssd_chunk_scan_fwd_noalloc")
    return y, final_state


def check_workspace(workspace, device=None) -> int:
    """Synchronise and read the forward kernel's failure word (0 = fine)."""
    lib = load_library()
    dev = workspace.device if device is None else device
    return int(lib.ssd_chunk_scan_fwd_check(_ptr(workspace), _stream(dev)))


def decode_step(state, x, dt, A, B, C, D=None, y=None, dt_bias=None, dt_softplus: bool = False,
                dt_limit=None):
    """One decode step through ``ssd_decode_step_ex``; ``state`` is updated in place."""
    lib = load_library()
    dev = x.device
    _need(x, "x", device=dev)
    io = _io_code(x)
    b, H, P = x.shape
    G, N = B.shape[1], B.shape[2]
    _need(state, "state", torch.float32, (b, H, P, N), dev)
    _need(dt, "dt", torch.float32, (b, H), dev)
    _need(A, "A", torch.float32, (H,), dev)
    _need(B, "B", x.dtype, (b, G, N), dev)
    _need(C, "C", x.dtype, (b, G, N), dev)
    if D is not None:
        _need(D, "D", torch.float32, (H,), dev)
    if y is None:
        y = torch.empty_like(x)
    dims = SsdDims(b, 1, H, P, N, G, b)
    opts = _dt_opts(dt_bias, dt_softplus, dt_limit, H, dev)
    code = lib.ssd_decode_step_ex(ctypes.byref(dims), io, None if opts is None else ctypes.byref(opts),
                                  _ptr(state), _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
                                  _ptr(y), _stream(dev))
    if code != 0:
        raise SsdError(code, "ssd_decode_step_ex")
    return y


def causal_conv1d_fwd(xbc, weight, nheads: int, headdim: int, ngroups: int, dstate: int, bias=None,
                      silu: bool = True, conv_state=None, cu_seqlens=None, return_final_state: bool = False,
                      x=None, B=None, C=None, conv_state_out=None):
    """Block prologue through ``ssd_causal_conv1d_fwd``: depthwise causal
    convolution of the fused x | B | C projection ``xbc`` [batch, seqlen,
    channels] with ``weight`` [channels, width] (fp32), split into x [batch,
    seqlen, nheads, headdim] and B, C [batch, seqlen, ngroups, dstate].
    Returns (x, B, C) or (x, B, C, conv_state_out)."""
    lib = load_library()
    dev = xbc.device
    _need(xbc, "xbc", device=dev)
    io = _io_code(xbc)
    if xbc.dim() != 3:
        raise ValueError("xbc must be [batch, seqlen, channels]")
    b, L, Cc = xbc.shape
    HP, GN = nheads * headdim, ngroups * dstate
    if Cc != HP + 2 * GN:
        raise ValueError(f"xbc has {Cc} channels, expected {HP + 2 * GN}")
    if weight.dim() != 2:
        raise ValueError("weight must be [channels, width]")
    W = weight.shape[1]
    _need(weight, "weight", torch.float32, (Cc, W), dev)
    if bias is not None:
        _need(bias, "bias", torch.float32, (Cc,), dev)
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", torch.int32, None, dev)
    nseq = b if cu_seqlens is None else cu_seqlens.numel() - 1
    if conv_state is not None:
        _need(conv_state, "conv_state", xbc.dtype, (nseq, W - 1, Cc), dev)
    x = torch.empty((b, L, nheads, headdim), dtype=xbc.dtype, device=dev) if x is None else x
    B = torch.empty((b, L, ngroups, dstate), dtype=xbc.dtype, device=dev) if B is None else B
    C = torch.empty((b, L, ngroups, dstate), dtype=xbc.dtype, device=dev) if C is None else C
    _need(x, "x", xbc.dtype, (b, L, nheads, headdim), dev)
    _need(B, "B", xbc.dtype, (b, L, ngroups, dstate), dev)
    _need(C, "C", xbc.dtype, (b, L, ngroups, dstate), dev)
    if conv_state_out is None and return_final_state:
        conv_state_out = torch.empty((nseq, W - 1, Cc), dtype=xbc.dtype, device=dev)
    elif conv_state_out is not None:
        _need(conv_state_out, "conv_state_out", xbc.dtype, (nseq, W - 1, Cc), dev)
    dims = SsdDims(b, L, nheads, headdim, dstate, ngroups, nseq)
    code = lib.ssd_causal_conv1d_fwd(ctypes.byref(dims), io, W, _ptr(xbc), _ptr(weight), _ptr(bias),
                                     1 if silu else 0, _ptr(conv_state), _ptr(cu_seqlens), _ptr(x), _ptr(B),
                                     _ptr(C), _ptr(conv_state_out), _stream(dev))
    if code != 0:
        raise SsdError(code, "ssd_causal_conv1d_fwd")
    return (x, B, C, conv_state_out) if return_final_state else (x, B, C)


def gated_rmsnorm_fwd(y, z, weight, eps: float = 1e-5, group_size=None, norm_before_gate: bool = False,
                      out=None):
    """Block epilogue through ``ssd_gated_rmsnorm_fwd``: RMSNorm over groups of
    ``group_size`` channels of the last axis of y * silu(z) (or of y, gated
    after the norm), times ``weight``.  ``y`` may be [..., nheads, headdim]:
    the channels are its last two axes.  ``out`` may be ``y`` (in place)."""
    lib = load_library()
    dev = y.device
    _need(y, "y", device=dev)
    io = _io_code(y)
    dim = weight.numel()
    if y.numel() % dim != 0 or y.shape[-1] > dim or dim % y.shape[-1] != 0:
        raise ValueError("the trailing axes of y must hold the weight's channels")
    rows = y.numel() // dim
    _need(weight, "weight", torch.float32, None, dev)
    if z is not None:
        _need(z, "z", y.dtype, tuple(y.shape), dev)
    out = torch.empty_like(y) if out is None else out
    _need(out, "out", y.dtype, tuple(y.shape), dev)
    gs = dim if group_size is None else int(group_size)
    code = lib.ssd_gated_rmsnorm_fwd(rows, dim, gs, io, _ptr(y), _ptr(z), _ptr(weight), float(eps),
                                     1 if norm_before_gate else 0, _ptr(out), _stream(dev))
    if code != 0:
        raise SsdError(code, "ssd_gated_rmsnorm_fwd")
    return out


def chunk_scan_bwd(x, dt, A, B, C, dy, D=None, init_state=None, cu_seqlens=None, dfinal_state=None,
                   want_dinit: bool = True, workspace=None):
    """Backward of ``chunk_scan_fwd`` through ``ssd_chunk_scan_bwd``: gradients
    of <dy, y> + <dfinal_state, final_state>.  Returns a dict with dx (io
    dtype), ddt, dA, dB, dC, dD and dinit (fp32; dinit None unless wanted)."""
    lib = load_library()
    dev = x.device
    _need(x, "x", device=dev)
    io = _io_code(x)
    b, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    _need(dt, "dt", torch.float32, (b, L, H), dev)
    _need(A, "A", torch.float32, (H,), dev)
    _need(B, "B", x.dtype, (b, L, G, N), dev)
    _need(C, "C", x.dtype, (b, L, G, N), dev)
    _need(dy, "dy", x.dtype, (b, L, H, P), dev)
    if D is not None:
        _need(D, "D", torch.float32, (H,), dev)
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", torch.int32, None, dev)
    dims = fwd_dims(x, B, cu_seqlens)
    nseq = dims.nseq
    for name, t in (("init_state", init_state), ("dfinal_state", dfinal_state)):
        if t is not None:
            _need(t, name, torch.float32, (nseq, H, P, N), dev)
    f32 = dict(dtype=torch.float32, device=dev)
    out = dict(dx=torch.empty_like(x), ddt=torch.empty((b, L, H), **f32), dA=torch.empty(H, **f32),
               dB=torch.empty((b, L, G, N), **f32), dC=torch.empty((b, L, G, N), **f32),
               dD=torch.empty(H, **f32), dinit=torch.empty((nseq, H, P, N), **f32) if want_dinit else None)
    n = int(lib.ssd_chunk_scan_bwd_workspace_size(ctypes.byref(dims), io))
    if n == 0:
        code = lib.ssd_chunk_scan_bwd(ctypes.byref(dims), io, *([None] * 7), _ptr(cu_seqlens), *([None] * 10),
                                      0, None)
        raise SsdError(code, "ssd_chunk_scan_bwd (size query)")
    if workspace is None or workspace.numel() < n:
        workspace = torch.empty(n, dtype=torch.uint8, device=dev)
    code = lib.ssd_chunk_scan_bwd(ctypes.byref(dims), io, _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
                                  _ptr(init_state), _ptr(cu_seqlens), _ptr(dy), _ptr(dfinal_state),
                                  _ptr(out["dx"]), _ptr(out["ddt"]), _ptr(out["dA"]), _ptr(out["dB"]),
                                  _ptr(out["dC"]), _ptr(out["dD"]), _ptr(out["dinit"]), _ptr(workspace),
                                  ctypes.c_size_t(workspace.numel()), _stream(dev))
    if code != 0:
        raise SsdError(code, "ssd_chunk_scan_bwd")
    chunk_scan_bwd.last_workspace = workspace
    return out
