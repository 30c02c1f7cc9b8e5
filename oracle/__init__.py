"""fp64 CPU oracle of the selective state-space scan (test infrastructure).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The product library never touches it, and it shares no
code with the HIP path: the arithmetic lives in ``oracle.c`` (plain C, double
precision, host libm), and this module only widens inputs to float64,
allocates outputs and calls it.

What the scan computes, and where the pages define it, is documented at the
top of ``oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None


def build(force: bool = True) -> str:
    """Compile ``oracle.c`` into ``liboracle.so`` with gcc (no fast-math, no
    FMA contraction, OpenMP over independent rows)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.run(
            ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
             "-ffp-contract=off", "-fno-fast-math", _SRC, "-o", tmp, "-lm"],
            check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            path = os.environ.get("SELSCAN_ORACLE_LIB")  # a deliberately broken copy, in tests
            if not path:
                if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                    build(force=True)
                path = _LIB
            lib = ctypes.CDLL(path)
            dp = ctypes.POINTER(ctypes.c_double)
            i64 = ctypes.c_int64
            lib.oracle_m1_f64.argtypes = [i64, i64, i64, i64] + [dp] * 8 + [ctypes.c_int, dp, dp, dp]
            lib.oracle_m1_f64.restype = ctypes.c_int
            lib.oracle_m2_f64.argtypes = [i64] * 6 + [dp] * 8 + [ctypes.c_int, dp, dp, dp]
            lib.oracle_m2_f64.restype = ctypes.c_int
            lib.oracle_m1_bwd_f64.argtypes = [i64] * 4 + [dp] * 8 + [ctypes.c_int] + [dp] * 11
            lib.oracle_m1_bwd_f64.restype = ctypes.c_int
            lib.oracle_m2_bwd_f64.argtypes = [i64] * 6 + [dp] * 8 + [ctypes.c_int] + [dp] * 11
            lib.oracle_m2_bwd_f64.restype = ctypes.c_int
            lib.oracle_conv1d_f64.argtypes = [i64] * 4 + [dp] * 3 + [ctypes.c_int, dp]
            lib.oracle_conv1d_f64.restype = ctypes.c_int
            lib.oracle_version.restype = ctypes.c_char_p
            lib.oracle_set_threads.argtypes = [ctypes.c_int]
            lib.oracle_set_threads.restype = None
            _lib = lib
    return _lib


def _f64(a, shape=None):
    """Widen to a C-contiguous float64 array (exact for bf16/fp16/fp32)."""
    if a is None:
        return None
    if hasattr(a, "detach"):  # a torch tensor: widen on the CPU
        a = a.detach().to("cpu").double().numpy()
    a = np.ascontiguousarray(np.asarray(a, dtype=np.float64))
    if shape is not None and a.shape != tuple(shape):
        raise ValueError(f"expected shape {tuple(shape)}, got {a.shape}")
    return a


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def set_threads(n: int | None) -> None:
    """Set the OpenMP thread count used by later oracle calls (from this
    Python thread)."""
    if n is not None:
        os.environ["OMP_NUM_THREADS"] = str(int(n))
        _load().oracle_set_threads(int(n))


def m1(u, delta, A, B, C, D=None, z=None, delta_bias=None, softplus=True, h0=None):
    """Mamba-1 selective scan in fp64.

    Shapes: u, delta, z [batch, dim, L]; A [dim, N]; B, C [batch, N, L];
    D, delta_bias [dim]; h0 [batch, dim, N].
    Returns (y [batch, dim, L] float64, last_state [batch, dim, N] float64).
    """
    u = _f64(u)
    nb, nd, nl = u.shape
    A = _f64(A)
    nn = A.shape[1]
    delta = _f64(delta, (nb, nd, nl))
    A = _f64(A, (nd, nn))
    B = _f64(B, (nb, nn, nl))
    C = _f64(C, (nb, nn, nl))
    D = _f64(D, (nd,))
    z = _f64(z, (nb, nd, nl))
    delta_bias = _f64(delta_bias, (nd,))
    h0 = _f64(h0, (nb, nd, nn))
    y = np.empty((nb, nd, nl), np.float64)
    last = np.empty((nb, nd, nn), np.float64)
    rc = _load().oracle_m1_f64(nb, nd, nn, nl, _ptr(u), _ptr(delta), _ptr(A), _ptr(B),
                               _ptr(C), _ptr(D), _ptr(z), _ptr(delta_bias), int(bool(softplus)),
                               _ptr(h0), _ptr(y), _ptr(last))
    if rc != 0:
        raise RuntimeError(f"oracle_m1_f64 failed with status {rc}")
    return y, last


def m2(x, dt, A, B, C, D=None, z=None, dt_bias=None, softplus=True, h0=None):
    """Mamba-2 multi-head selective scan in fp64.

    Shapes: x, z [batch, L, H, P]; dt [batch, L, H]; A, D, dt_bias [H];
    B, C [batch, L, G, N]; h0 [batch, H, P, N].
    Returns (y [batch, L, H, P], last_state [batch, H, P, N]), float64.
    """
    x = _f64(x)
    nb, nl, nh, npd = x.shape
    B = _f64(B)
    ng, nn = B.shape[2], B.shape[3]
    B = _f64(B, (nb, nl, ng, nn))
    C = _f64(C, (nb, nl, ng, nn))
    dt = _f64(dt, (nb, nl, nh))
    A = _f64(A, (nh,))
    D = _f64(D, (nh,))
    z = _f64(z, (nb, nl, nh, npd))
    dt_bias = _f64(dt_bias, (nh,))
    h0 = _f64(h0, (nb, nh, npd, nn))
    y = np.empty((nb, nl, nh, npd), np.float64)
    last = np.empty((nb, nh, npd, nn), np.float64)
    rc = _load().oracle_m2_f64(nb, nl, nh, npd, ng, nn, _ptr(x), _ptr(dt), _ptr(A), _ptr(B),
                               _ptr(C), _ptr(D), _ptr(z), _ptr(dt_bias), int(bool(softplus)),
                               _ptr(h0), _ptr(y), _ptr(last))
    if rc != 0:
        raise RuntimeError(f"oracle_m2_f64 failed with status {rc}")
    return y, last


def m1_bwd(u, delta, A, B, C, D, z, delta_bias, dout, softplus=True, h0=None):
    """Gradients of the Mamba-1 scan output (y gated by silu(z)) in fp64 from
    the initial state h0 [batch, dim, N] (None = zero).  Returns a dict: du,
    ddelta, dz [batch, dim, L]; dA [dim, N]; dB, dC [batch, N, L]; dD,
    ddelta_bias [dim]; dh0 [batch, dim, N]."""
    u = _f64(u)
    nb, nd, nl = u.shape
    A = _f64(A)
    nn = A.shape[1]
    delta = _f64(delta, (nb, nd, nl))
    B = _f64(B, (nb, nn, nl))
    C = _f64(C, (nb, nn, nl))
    D = _f64(D, (nd,))
    z = _f64(z, (nb, nd, nl))
    delta_bias = _f64(delta_bias, (nd,))
    h0 = _f64(h0, (nb, nd, nn))
    dout = _f64(dout, (nb, nd, nl))
    g = {k: np.empty(s, np.float64) for k, s in (("du", (nb, nd, nl)), ("ddelta", (nb, nd, nl)), ("dA", (nd, nn)),
                                                  ("dB", (nb, nn, nl)), ("dC", (nb, nn, nl)), ("dD", (nd,)),
                                                  ("dz", (nb, nd, nl)), ("ddelta_bias", (nd,)),
                                                  ("dh0", (nb, nd, nn)))}
    rc = _load().oracle_m1_bwd_f64(nb, nd, nn, nl, _ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
                                   _ptr(z), _ptr(delta_bias), int(bool(softplus)), _ptr(h0), _ptr(dout),
                                   _ptr(g["du"]), _ptr(g["ddelta"]), _ptr(g["dA"]), _ptr(g["dB"]), _ptr(g["dC"]),
                                   _ptr(g["dD"]), _ptr(g["dz"]), _ptr(g["ddelta_bias"]), _ptr(g["dh0"]))
    if rc != 0:
        raise RuntimeError(f"oracle_m1_bwd_f64 failed with status {rc}")
    return g


def m2_bwd(x, dt, A, B, C, D, z, dt_bias, dout, softplus=True, h0=None):
    """Gradients of the Mamba-2 scan output (gated by silu(z)) in fp64 from
    the initial state h0 [batch, nheads, headdim, N] (None = zero).  Returns a
    dict: dx, dz [batch, L, nheads, headdim]; ddt [batch, L, nheads]; dA, dD,
    ddt_bias [nheads]; dB, dC [batch, L, ngroups, N]; dh0 [batch, nheads,
    headdim, N]."""
    x = _f64(x)
    nb, nl, nh, np_ = x.shape
    B = _f64(B)
    ng, nn = B.shape[2], B.shape[3]
    dt = _f64(dt, (nb, nl, nh))
    A = _f64(A, (nh,))
    C = _f64(C, (nb, nl, ng, nn))
    D = _f64(D, (nh,))
    z = _f64(z, (nb, nl, nh, np_))
    dt_bias = _f64(dt_bias, (nh,))
    h0 = _f64(h0, (nb, nh, np_, nn))
    dout = _f64(dout, (nb, nl, nh, np_))
    g = {k: np.empty(s, np.float64) for k, s in (("dx", (nb, nl, nh, np_)), ("ddt", (nb, nl, nh)), ("dA", (nh,)),
                                                  ("dB", (nb, nl, ng, nn)), ("dC", (nb, nl, ng, nn)), ("dD", (nh,)),
                                                  ("dz", (nb, nl, nh, np_)), ("ddt_bias", (nh,)),
                                                  ("dh0", (nb, nh, np_, nn)))}
    rc = _load().oracle_m2_bwd_f64(nb, nl, nh, np_, ng, nn, _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
                                   _ptr(z), _ptr(dt_bias), int(bool(softplus)), _ptr(h0), _ptr(dout),
                                   _ptr(g["dx"]), _ptr(g["ddt"]), _ptr(g["dA"]), _ptr(g["dB"]), _ptr(g["dC"]),
                                   _ptr(g["dD"]), _ptr(g["dz"]), _ptr(g["ddt_bias"]), _ptr(g["dh0"]))
    if rc != 0:
        raise RuntimeError(f"oracle_m2_bwd_f64 failed with status {rc}")
    return g


def conv1d(x, w, bias=None, silu=True):
    """Causal depthwise convolution in fp64: x [batch, dim, L], w [dim, K],
    bias [dim]; out[t] = act(bias + sum_k w[k] x[t - (K - 1) + k]), zero
    before the first token.  Returns out [batch, dim, L] float64."""
    x = _f64(x)
    nb, nd, nl = x.shape
    w = _f64(w)
    nk = w.shape[1]
    w = _f64(w, (nd, nk))
    bias = _f64(bias, (nd,))
    out = np.empty((nb, nd, nl), np.float64)
    rc = _load().oracle_conv1d_f64(nb, nd, nl, nk, _ptr(x), _ptr(w), _ptr(bias), int(bool(silu)), _ptr(out))
    if rc != 0:
        raise RuntimeError(f"oracle_conv1d_f64 failed with status {rc}")
    return out


def version() -> str:
    return _load().oracle_version().decode()
