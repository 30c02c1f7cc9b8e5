"""libselscan: the selective state-space scan of Mamba on AMD MI355X (gfx950).

Thin Python binding over the C ABI in ``include/selscan.h``.  It only
marshals arguments: torch tensors provide device memory and the current HIP
stream; every step of the scan runs in the HIP kernels of ``libselscan.so``.
There is no fallback: if the library is missing the import of a kernel entry
point raises.

    y, last_state = selscan.fwd(u, delta, A, B, C, D, z, delta_bias, softplus=True)
    y, last_state = selscan.mamba2_fwd(x, dt, A, B, C, D, z, dt_bias, softplus=True)
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libselscan.so")

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_NO_DEVICE, ERR_LAUNCH, ERR_WORKSPACE = range(6)
F32, BF16 = 0, 1

_STATUS_NAMES = {0: "OK", 1: "INVALID_ARG", 2: "UNSUPPORTED", 3: "NO_DEVICE", 4: "LAUNCH", 5: "WORKSPACE"}


class SelscanError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"libselscan {_STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


class Shape(ctypes.Structure):
    """selscan_shape_t (Mamba-1)."""
    _fields_ = [("batch", ctypes.c_int64), ("dim", ctypes.c_int64), ("dstate", ctypes.c_int64),
                ("seqlen", ctypes.c_int64), ("in_dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t)]


class M2Shape(ctypes.Structure):
    """selscan_m2_shape_t (Mamba-2)."""
    _fields_ = [("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64), ("nheads", ctypes.c_int64),
                ("headdim", ctypes.c_int64), ("ngroups", ctypes.c_int64), ("dstate", ctypes.c_int64),
                ("in_dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t)]


_lib = None

EXPORTED = ("selscan_fwd", "selscan_mamba2_fwd", "selscan_workspace_bytes", "selscan_mamba2_workspace_bytes",
            "selscan_fwd_h0", "selscan_mamba2_fwd_h0", "selscan_step", "selscan_mamba2_step", "selscan_conv1d",
            "selscan_bwd", "selscan_bwd_workspace_bytes", "selscan_fwd_noalloc",
            "selscan_mamba2_bwd", "selscan_mamba2_bwd_workspace_bytes",
            "selscan_last_error", "selscan_version", "selscan_timing_enable", "selscan_timing_collect")


class ConvShape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("dim", ctypes.c_int64), ("seqlen", ctypes.c_int64),
                ("width", ctypes.c_int64), ("in_dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32)]


class KernelTime(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char_p), ("launches", ctypes.c_int64), ("total_ms", ctypes.c_double),
                ("min_ms", ctypes.c_double), ("max_ms", ctypes.c_double)]


def lib() -> ctypes.CDLL:
    """The loaded libselscan.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m selective_state_space_25_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, fp, i32 = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int
        L.selscan_fwd.argtypes = [ctypes.POINTER(Shape), vp, vp, fp, vp, vp, fp, vp, fp, i32, vp, fp, vp]
        L.selscan_fwd.restype = i32
        L.selscan_mamba2_fwd.argtypes = [ctypes.POINTER(M2Shape), vp, vp, fp, vp, vp, fp, vp, fp, i32, vp, fp, vp]
        L.selscan_mamba2_fwd.restype = i32
        L.selscan_fwd_h0.argtypes = [ctypes.POINTER(Shape), vp, vp, fp, vp, vp, fp, vp, fp, i32, fp, vp, fp, vp]
        L.selscan_fwd_h0.restype = i32
        L.selscan_mamba2_fwd_h0.argtypes = [ctypes.POINTER(M2Shape), vp, vp, fp, vp, vp, fp, vp, fp, i32, fp, vp, fp,
                                            vp]
        L.selscan_mamba2_fwd_h0.restype = i32
        L.selscan_fwd_noalloc.argtypes = [ctypes.POINTER(Shape), vp, vp, fp, vp, vp, fp, vp, fp, i32, fp, vp, fp,
                                          vp]
        L.selscan_fwd_noalloc.restype = i32
        L.selscan_step.argtypes = [ctypes.POINTER(Shape), fp, vp, vp, fp, vp, vp, fp, vp, fp, i32, vp, vp]
        L.selscan_step.restype = i32
        L.selscan_mamba2_step.argtypes = [ctypes.POINTER(M2Shape), fp, vp, vp, fp, vp, vp, fp, vp, fp, i32, vp, vp]
        L.selscan_mamba2_step.restype = i32
        L.selscan_conv1d.argtypes = [ctypes.POINTER(ConvShape), vp, fp, fp, i32, vp, vp]
        L.selscan_conv1d.restype = i32
        L.selscan_bwd.argtypes = [ctypes.POINTER(Shape), vp, vp, fp, vp, vp, fp, vp, fp, i32, fp, vp] + [fp] * 9 + [vp]
        L.selscan_bwd.restype = i32
        L.selscan_mamba2_bwd.argtypes = [ctypes.POINTER(M2Shape), vp, vp, fp, vp, vp, fp, vp, fp, i32, fp, vp] + \
            [fp] * 9 + [vp]
        L.selscan_mamba2_bwd.restype = i32
        L.selscan_mamba2_bwd_workspace_bytes.argtypes = [ctypes.POINTER(M2Shape)]
        L.selscan_mamba2_bwd_workspace_bytes.restype = ctypes.c_size_t
        L.selscan_bwd_workspace_bytes.argtypes = [ctypes.POINTER(Shape)]
        L.selscan_bwd_workspace_bytes.restype = ctypes.c_size_t
        L.selscan_workspace_bytes.argtypes = [ctypes.POINTER(Shape)]
        L.selscan_workspace_bytes.restype = ctypes.c_size_t
        L.selscan_mamba2_workspace_bytes.argtypes = [ctypes.POINTER(M2Shape)]
        L.selscan_mamba2_workspace_bytes.restype = ctypes.c_size_t
        L.selscan_last_error.restype = ctypes.c_char_p
        L.selscan_version.restype = ctypes.c_char_p
        L.selscan_timing_enable.argtypes = [i32]
        L.selscan_timing_enable.restype = i32
        L.selscan_timing_collect.argtypes = [ctypes.POINTER(KernelTime), i32]
        L.selscan_timing_collect.restype = i32
        _lib = L
    return _lib


def version() -> str:
    return lib().selscan_version().decode()


def last_error() -> str:
    return lib().selscan_last_error().decode()


def _check(status: int) -> None:
    if status != OK:
        raise SelscanError(status, last_error())


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"unsupported dtype {t.dtype}: use float32 or bfloat16")


def _ptr(t, name, shape=None, dtype=None, device=None):
    """Device pointer of a dense tensor after checking shape/dtype/device."""
    if t is None:
        return None
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    return t.data_ptr()


def _stream_handle(device):
    torch = _torch()
    return torch.cuda.current_stream(device).cuda_stream


def m1_shape(batch, dim, dstate, seqlen, in_dtype=BF16, out_dtype=None, workspace=None, workspace_bytes=0):
    return Shape(batch, dim, dstate, seqlen, in_dtype, in_dtype if out_dtype is None else out_dtype,
                 workspace, workspace_bytes)


def fwd(u, delta, A, B, C, D=None, z=None, delta_bias=None, softplus=True, out=None, last_state=None,
        return_last_state=True, workspace=None, out_dtype=None, h0=None):
    """Mamba-1 selective scan on the GPU.

    u, delta, z: [batch, dim, L]; B, C: [batch, N, L] (float32 or bfloat16, one
    dtype for all five); A: [dim, N], D, delta_bias: [dim] float32.
    Returns (y [batch, dim, L] float32 unless out_dtype says otherwise,
    last_state [batch, dim, N] float32 or None).  y defaults to float32, the
    precision of the state: a bfloat16 y carries up to 2^-8 relative rounding.
    h0 [batch, dim, N] float32: initial state (None: zero).
    """
    torch = _torch()
    dev = u.device
    if dev.type != "cuda":
        raise ValueError("selscan.fwd needs tensors on a GPU device")
    batch, dim, L = u.shape
    N = A.shape[1]
    dt = u.dtype
    code = _dtype_code(u)
    odt = (out.dtype if out is not None else torch.float32) if out_dtype is None else out_dtype
    if out is None:
        out = torch.empty((batch, dim, L), dtype=odt, device=dev)
    if last_state is None and return_last_state:
        last_state = torch.empty((batch, dim, N), dtype=torch.float32, device=dev)
    ws_ptr, ws_bytes = (None, 0) if workspace is None else (workspace.data_ptr(), workspace.numel() * workspace.element_size())
    s = Shape(batch, dim, N, L, code, _dtype_code(out), ws_ptr, ws_bytes)
    args = (
        _ptr(u, "u", (batch, dim, L), dt, dev), _ptr(delta, "delta", (batch, dim, L), dt, dev),
        _ptr(A, "A", (dim, N), torch.float32, dev), _ptr(B, "B", (batch, N, L), dt, dev),
        _ptr(C, "C", (batch, N, L), dt, dev), _ptr(D, "D", (dim,), torch.float32, dev),
        _ptr(z, "z", (batch, dim, L), dt, dev), _ptr(delta_bias, "delta_bias", (dim,), torch.float32, dev),
        int(bool(softplus)), _ptr(out, "out", (batch, dim, L), odt, dev),
        _ptr(last_state, "last_state", (batch, dim, N), torch.float32, dev), _stream_handle(dev))
    if h0 is None:
        _check(lib().selscan_fwd(ctypes.byref(s), *args))
    else:
        h0p = _ptr(h0, "h0", (batch, dim, N), torch.float32, dev)
        _check(lib().selscan_fwd_h0(ctypes.byref(s), *args[:9], h0p, *args[9:]))
    return out, last_state


def step(state, u, delta, A, B, C, D=None, z=None, delta_bias=None, softplus=True, out=None, out_dtype=None):
    """One-token Mamba-1 update (decoding).  state [batch, dim, N] float32 is
    updated in place; u, delta, z [batch, dim]; B, C [batch, N] (float32 or
    bfloat16); A [dim, N], D, delta_bias [dim] float32.  Returns y [batch, dim]
    (float32 unless out_dtype or out says otherwise)."""
    torch = _torch()
    dev = u.device
    if dev.type != "cuda":
        raise ValueError("selscan.step needs tensors on a GPU device")
    batch, dim = u.shape
    N = A.shape[1]
    dt = u.dtype
    odt = (out.dtype if out is not None else torch.float32) if out_dtype is None else out_dtype
    if out is None:
        out = torch.empty((batch, dim), dtype=odt, device=dev)
    s = Shape(batch, dim, N, 1, _dtype_code(u), _dtype_code(out), None, 0)
    _check(lib().selscan_step(
        ctypes.byref(s), _ptr(state, "state", (batch, dim, N), torch.float32, dev),
        _ptr(u, "u", (batch, dim), dt, dev), _ptr(delta, "delta", (batch, dim), dt, dev),
        _ptr(A, "A", (dim, N), torch.float32, dev), _ptr(B, "B", (batch, N), dt, dev),
        _ptr(C, "C", (batch, N), dt, dev), _ptr(D, "D", (dim,), torch.float32, dev),
        _ptr(z, "z", (batch, dim), dt, dev), _ptr(delta_bias, "delta_bias", (dim,), torch.float32, dev),
        int(bool(softplus)), _ptr(out, "out", (batch, dim), odt, dev), _stream_handle(dev)))
    return out


class _BoundCall:
    """A C-ABI call with its arguments marshalled once: calling it enqueues
    the kernel again on the same buffers (whose contents the caller may
    change in place between calls, as a decoding loop does)."""

    def __init__(self, fn, shape, args):
        self._fn, self._shape, self._args = fn, shape, args

    def __call__(self):
        st = self._fn(ctypes.byref(self._shape), *self._args)
        if st != OK:
            raise SelscanError(st, last_error())


def bind_step(state, u, delta, A, B, C, D=None, z=None, delta_bias=None, softplus=True, out=None, out_dtype=None):
    """selscan_step with its arguments checked and marshalled once: returns
    (call, y).  Each call() updates `state` in place with the token currently
    held in u, delta, B, C, z and writes y, on the stream that was current at
    binding time."""
    torch = _torch()
    dev = u.device
    if dev.type != "cuda":
        raise ValueError("selscan.bind_step needs tensors on a GPU device")
    batch, dim = u.shape
    N = A.shape[1]
    dt = u.dtype
    odt = (out.dtype if out is not None else torch.float32) if out_dtype is None else out_dtype
    if out is None:
        out = torch.empty((batch, dim), dtype=odt, device=dev)
    s = Shape(batch, dim, N, 1, _dtype_code(u), _dtype_code(out), None, 0)
    args = (_ptr(state, "state", (batch, dim, N), torch.float32, dev),
            _ptr(u, "u", (batch, dim), dt, dev), _ptr(delta, "delta", (batch, dim), dt, dev),
            _ptr(A, "A", (dim, N), torch.float32, dev), _ptr(B, "B", (batch, N), dt, dev),
            _ptr(C, "C", (batch, N), dt, dev), _ptr(D, "D", (dim,), torch.float32, dev),
            _ptr(z, "z", (batch, dim), dt, dev), _ptr(delta_bias, "delta_bias", (dim,), torch.float32, dev),
            int(bool(softplus)), _ptr(out, "out", (batch, dim), odt, dev), _stream_handle(dev))
    return _BoundCall(lib().selscan_step, s, args), out


def bind_mamba2_step(state, x, dt, A, B, C, D=None, z=None, dt_bias=None, softplus=True, out=None,
                     out_dtype=None):
    """selscan_mamba2_step with its arguments checked and marshalled once:
    returns (call, y); see bind_step."""
    torch = _torch()
    dev = x.device
    if dev.type != "cuda":
        raise ValueError("selscan.bind_mamba2_step needs tensors on a GPU device")
    batch, H, P = x.shape
    G, N = B.shape[1], B.shape[2]
    dtp = x.dtype
    odt = (out.dtype if out is not None else torch.float32) if out_dtype is None else out_dtype
    if out is None:
        out = torch.empty((batch, H, P), dtype=odt, device=dev)
    s = M2Shape(batch, 1, H, P, G, N, _dtype_code(x), _dtype_code(out), None, 0)
    args = (_ptr(state, "state", (batch, H, P, N), torch.float32, dev),
            _ptr(x, "x", (batch, H, P), dtp, dev), _ptr(dt, "dt", (batch, H), dtp, dev),
            _ptr(A, "A", (H,), torch.float32, dev), _ptr(B, "B", (batch, G, N), dtp, dev),
            _ptr(C, "C", (batch, G, N), dtp, dev), _ptr(D, "D", (H,), torch.float32, dev),
            _ptr(z, "z", (batch, H, P), dtp, dev), _ptr(dt_bias, "dt_bias", (H,), torch.float32, dev),
            int(bool(softplus)), _ptr(out, "out", (batch, H, P), odt, dev), _stream_handle(dev))
    return _BoundCall(lib().selscan_mamba2_step, s, args), out


def bwd(u, delta, A, B, C, D=None, z=None, delta_bias=None, dout=None, softplus=True, h0=None,
        want_dh0=False, workspace=None):
    """Gradients of the Mamba-1 scan on the GPU.

    Inputs as for fwd; dout [batch, dim, L] (float32 or bfloat16: the dtype
    of the forward's y) is the gradient of the loss with respect to y.
    Returns a dict of float32 tensors: du, ddelta, dz (when z is given)
    [batch, dim, L]; dA [dim, N]; dB, dC [batch, N, L]; dD (when D is given)
    and ddelta_bias (when delta_bias is given) [dim]; dh0 [batch, dim, N]
    (when h0 is given or want_dh0).
    """
    torch = _torch()
    dev = u.device
    if dev.type != "cuda":
        raise ValueError("selscan.bwd needs tensors on a GPU device")
    if dout is None:
        raise ValueError("dout is required")
    batch, dim, L = u.shape
    N = A.shape[1]
    dt = u.dtype
    f32 = torch.float32
    new = lambda *shape: torch.empty(shape, dtype=f32, device=dev)
    g = {"du": new(batch, dim, L), "ddelta": new(batch, dim, L), "dA": new(dim, N),
         "dB": new(batch, N, L), "dC": new(batch, N, L)}
    if z is not None:
        g["dz"] = new(batch, dim, L)
    if D is not None:
        g["dD"] = new(dim)
    if delta_bias is not None:
        g["ddelta_bias"] = new(dim)
    if h0 is not None or want_dh0:
        g["dh0"] = new(batch, dim, N)
    ws_ptr, ws_bytes = (None, 0) if workspace is None else (workspace.data_ptr(), workspace.numel() * workspace.element_size())
    s = Shape(batch, dim, N, L, _dtype_code(u), _dtype_code(dout), ws_ptr, ws_bytes)
    gp = lambda k: g[k].data_ptr() if k in g else None
    _check(lib().selscan_bwd(
        ctypes.byref(s), _ptr(u, "u", (batch, dim, L), dt, dev), _ptr(delta, "delta", (batch, dim, L), dt, dev),
        _ptr(A, "A", (dim, N), f32, dev), _ptr(B, "B", (batch, N, L), dt, dev), _ptr(C, "C", (batch, N, L), dt, dev),
        _ptr(D, "D", (dim,), f32, dev), _ptr(z, "z", (batch, dim, L), dt, dev),
        _ptr(delta_bias, "delta_bias", (dim,), f32, dev), int(bool(softplus)),
        _ptr(h0, "h0", (batch, dim, N), f32, dev), _ptr(dout, "dout", (batch, dim, L), None, dev),
        gp("du"), gp("ddelta"), gp("dA"), gp("dB"), gp("dC"), gp("dD"), gp("dz"), gp("ddelta_bias"), gp("dh0"),
        _stream_handle(dev)))
    return g


def bwd_workspace_bytes(batch, dim, dstate, seqlen, in_dtype=BF16, out_dtype=None) -> int:
    s = m1_shape(batch, dim, dstate, seqlen, in_dtype, out_dtype)
    return int(lib().selscan_bwd_workspace_bytes(ctypes.byref(s)))


def workspace_bytes(batch, dim, dstate, seqlen, in_dtype=BF16, out_dtype=None) -> int:
    s = m1_shape(batch, dim, dstate, seqlen, in_dtype, out_dtype)
    return int(lib().selscan_workspace_bytes(ctypes.byref(s)))


def mamba2_fwd(x, dt, A, B, C, D=None, z=None, dt_bias=None, softplus=True, out=None, last_state=None,
               return_last_state=True, workspace=None, out_dtype=None, h0=None):
    """Mamba-2 multi-head selective scan on the GPU.

    x, z: [batch, L, H, P]; dt: [batch, L, H]; B, C: [batch, L, G, N]
    (float32 or bfloat16); A, D, dt_bias: [H] float32.
    Returns (y [batch, L, H, P] float32 unless out_dtype says otherwise,
    last_state [batch, H, P, N] float32 or None).  h0 [batch, H, P, N]
    float32: initial state (None: zero).
    """
    torch = _torch()
    dev = x.device
    if dev.type != "cuda":
        raise ValueError("selscan.mamba2_fwd needs tensors on a GPU device")
    batch, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    dtp = x.dtype
    odt = (out.dtype if out is not None else torch.float32) if out_dtype is None else out_dtype
    if out is None:
        out = torch.empty((batch, L, H, P), dtype=odt, device=dev)
    if last_state is None and return_last_state:
        last_state = torch.empty((batch, H, P, N), dtype=torch.float32, device=dev)
    ws_ptr, ws_bytes = (None, 0) if workspace is None else (workspace.data_ptr(), workspace.numel() * workspace.element_size())
    s = M2Shape(batch, L, H, P, G, N, _dtype_code(x), _dtype_code(out), ws_ptr, ws_bytes)
    args = (
        _ptr(x, "x", (batch, L, H, P), dtp, dev), _ptr(dt, "dt", (batch, L, H), dtp, dev),
        _ptr(A, "A", (H,), torch.float32, dev), _ptr(B, "B", (batch, L, G, N), dtp, dev),
        _ptr(C, "C", (batch, L, G, N), dtp, dev), _ptr(D, "D", (H,), torch.float32, dev),
        _ptr(z, "z", (batch, L, H, P), dtp, dev), _ptr(dt_bias, "dt_bias", (H,), torch.float32, dev),
        int(bool(softplus)), _ptr(out, "out", (batch, L, H, P), odt, dev),
        _ptr(last_state, "last_state", (batch, H, P, N), torch.float32, dev), _stream_handle(dev))
    if h0 is None:
        _check(lib().selscan_mamba2_fwd(ctypes.byref(s), *args))
    else:
        h0p = _ptr(h0, "h0", (batch, H, P, N), torch.float32, dev)
        _check(lib().selscan_mamba2_fwd_h0(ctypes.byref(s), *args[:9], h0p, *args[9:]))
    return out, last_state


def mamba2_step(state, x, dt, A, B, C, D=None, z=None, dt_bias=None, softplus=True, out=None, out_dtype=None):
    """One-token Mamba-2 update (decoding).  state [batch, H, P, N] float32 is
    updated in place; x, z [batch, H, P]; dt [batch, H]; B, C [batch, G, N]
    (float32 or bfloat16); A, D, dt_bias [H] float32.  Returns y [batch, H, P]."""
    torch = _torch()
    dev = x.device
    if dev.type != "cuda":
        raise ValueError("selscan.mamba2_step needs tensors on a GPU device")
    batch, H, P = x.shape
    G, N = B.shape[1], B.shape[2]
    dtp = x.dtype
    odt = (out.dtype if out is not None else torch.float32) if out_dtype is None else out_dtype
    if out is None:
        out = torch.empty((batch, H, P), dtype=odt, device=dev)
    s = M2Shape(batch, 1, H, P, G, N, _dtype_code(x), _dtype_code(out), None, 0)
    _check(lib().selscan_mamba2_step(
        ctypes.byref(s), _ptr(state, "state", (batch, H, P, N), torch.float32, dev),
        _ptr(x, "x", (batch, H, P), dtp, dev), _ptr(dt, "dt", (batch, H), dtp, dev),
        _ptr(A, "A", (H,), torch.float32, dev), _ptr(B, "B", (batch, G, N), dtp, dev),
        _ptr(C, "C", (batch, G, N), dtp, dev), _ptr(D, "D", (H,), torch.float32, dev),
        _ptr(z, "z", (batch, H, P), dtp, dev), _ptr(dt_bias, "dt_bias", (H,), torch.float32, dev),
        int(bool(softplus)), _ptr(out, "out", (batch, H, P), odt, dev), _stream_handle(dev)))
    return out


def mamba2_bwd(x, dt, A, B, C, D=None, z=None, dt_bias=None, dout=None, softplus=True, h0=None,
               want_dh0=False, workspace=None):
    """Gradients of the Mamba-2 scan on the GPU (headdim 64).

    Inputs as for mamba2_fwd; dout [batch, L, nheads, headdim] (float32 or
    bfloat16) is the gradient of the loss with respect to y.  Returns a dict
    of float32 tensors: dx, dz (when z is given) [batch, L, nheads, headdim];
    ddt [batch, L, nheads]; dA [nheads]; dB, dC [batch, L, ngroups, N]; dD
    (when D is given) and ddt_bias (when dt_bias is given) [nheads]; dh0
    [batch, nheads, headdim, N] (when h0 is given or want_dh0).
    """
    torch = _torch()
    dev = x.device
    if dev.type != "cuda":
        raise ValueError("selscan.mamba2_bwd needs tensors on a GPU device")
    if dout is None:
        raise ValueError("dout is required")
    batch, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    dt_ = x.dtype
    f32 = torch.float32
    new = lambda *shape: torch.empty(shape, dtype=f32, device=dev)
    g = {"dx": new(batch, L, H, P), "ddt": new(batch, L, H), "dA": new(H), "dB": new(batch, L, G, N),
         "dC": new(batch, L, G, N)}
    if z is not None:
        g["dz"] = new(batch, L, H, P)
    if D is not None:
        g["dD"] = new(H)
    if dt_bias is not None:
        g["ddt_bias"] = new(H)
    if h0 is not None or want_dh0:
        g["dh0"] = new(batch, H, P, N)
    ws_ptr, ws_bytes = (None, 0) if workspace is None else (workspace.data_ptr(), workspace.numel() * workspace.element_size())
    s = M2Shape(batch, L, H, P, G, N, _dtype_code(x), _dtype_code(dout), ws_ptr, ws_bytes)
    gp = lambda k: g[k].data_ptr() if k in g else None
    _check(lib().selscan_mamba2_bwd(
        ctypes.byref(s), _ptr(x, "x", (batch, L, H, P), dt_, dev), _ptr(dt, "dt", (batch, L, H), dt_, dev),
        _ptr(A, "A", (H,), f32, dev), _ptr(B, "B", (batch, L, G, N), dt_, dev), _ptr(C, "C", (batch, L, G, N), dt_, dev),
        _ptr(D, "D", (H,), f32, dev), _ptr(z, "z", (batch, L, H, P), dt_, dev),
        _ptr(dt_bias, "dt_bias", (H,), f32, dev), int(bool(softplus)),
        _ptr(h0, "h0", (batch, H, P, N), f32, dev), _ptr(dout, "dout", (batch, L, H, P), None, dev),
        gp("dx"), gp("ddt"), gp("dA"), gp("dB"), gp("dC"), gp("dD"), gp("dz"), gp("ddt_bias"), gp("dh0"),
        _stream_handle(dev)))
    return g


def mamba2_bwd_workspace_bytes(batch, seqlen, nheads, headdim, ngroups, dstate, in_dtype=BF16, out_dtype=None) -> int:
    s = M2Shape(batch, seqlen, nheads, headdim, ngroups, dstate, in_dtype, in_dtype if out_dtype is None else out_dtype,
                None, 0)
    return int(lib().selscan_mamba2_bwd_workspace_bytes(ctypes.byref(s)))


def mamba2_workspace_bytes(batch, seqlen, nheads, headdim, ngroups, dstate, in_dtype=BF16, out_dtype=None) -> int:
    s = M2Shape(batch, seqlen, nheads, headdim, ngroups, dstate, in_dtype,
                in_dtype if out_dtype is None else out_dtype, None, 0)
    return int(lib().selscan_mamba2_workspace_bytes(ctypes.byref(s)))


def conv1d(x, weight, bias=None, silu=True, out=None, out_dtype=None):
    """Causal depthwise convolution: x [batch, dim, L] (float32 or bfloat16),
    weight [dim, K] and bias [dim] float32.  out[t] = act(bias + sum_k
    weight[k] x[t - (K - 1) + k]), act = silu or identity.  Returns out
    [batch, dim, L] in x's dtype unless out_dtype or out says otherwise."""
    torch = _torch()
    dev = x.device
    if dev.type != "cuda":
        raise ValueError("selscan.conv1d needs tensors on a GPU device")
    batch, dim, L = x.shape
    K = weight.shape[1]
    odt = (out.dtype if out is not None else x.dtype) if out_dtype is None else out_dtype
    if out is None:
        out = torch.empty((batch, dim, L), dtype=odt, device=dev)
    s = ConvShape(batch, dim, L, K, _dtype_code(x), _dtype_code(out))
    _check(lib().selscan_conv1d(
        ctypes.byref(s), _ptr(x, "x", (batch, dim, L), x.dtype, dev),
        _ptr(weight, "weight", (dim, K), torch.float32, dev), _ptr(bias, "bias", (dim,), torch.float32, dev),
        int(bool(silu)), _ptr(out, "out", (batch, dim, L), odt, dev), _stream_handle(dev)))
    return out


def timing_enable(on: bool) -> None:
    """Bracket every later kernel launch with HIP events on its own stream."""
    _check(lib().selscan_timing_enable(int(bool(on))))


def timing_collect() -> dict:
    """Wait for the bracketed launches so far; {kernel: {launches, total_ms,
    avg_ms, min_ms, max_ms}} in order of first launch."""
    cap = 32
    buf = (KernelTime * cap)()
    n = lib().selscan_timing_collect(buf, cap)
    if n < 0:
        raise SelscanError(n, "selscan_timing_collect failed")
    res = {}
    for k in buf[:min(n, cap)]:
        res[k.name.decode()] = {"launches": k.launches, "total_ms": k.total_ms,
                                "avg_ms": k.total_ms / max(k.launches, 1), "min_ms": k.min_ms, "max_ms": k.max_ms}
    return res


__all__ = ["bind_step", "bind_mamba2_step", "bwd", "bwd_workspace_bytes", "conv1d", "ConvShape", "step", "mamba2_step", "timing_enable", "timing_collect", "KernelTime", "fwd", "mamba2_fwd", "workspace_bytes", "mamba2_workspace_bytes", "version", "last_error", "lib",
           "SelscanError", "Shape", "M2Shape", "m1_shape", "EXPORTED", "LIB_PATH"]
