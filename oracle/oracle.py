"""ctypes wrapper around the plain-C fp64 oracle (``ssm_oracle.c``).

Test infrastructure only (see the package docstring). Arrays are numpy
float64, C-contiguous, in the layouts documented in ``ssm_oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ORACLE_SRC = os.path.join(HERE, "ssm_oracle.c")
ORACLE_LIB = os.path.join(HERE, "liboracle.so")

_dp = ctypes.POINTER(ctypes.c_double)
_i64 = ctypes.c_int64


def build_oracle(src: str = ORACLE_SRC, out: str = ORACLE_LIB) -> str:
    """Compile the oracle with gcc (fp64, -O2, OpenMP, no fast-math)."""
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-std=c99", "-O2", "-fopenmp", "-fPIC", "-shared",
           "-fno-fast-math", "-ffp-contract=off", "-o", tmp, src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(_dp)


def _f64(a, shape=None):
    if a is None:
        return None
    a = np.ascontiguousarray(np.asarray(a, dtype=np.float64))
    if shape is not None and a.shape != tuple(shape):
        a = a.reshape(shape)
    return a


def _groups(B):
    """Number of channel groups of a (batch, L, N) or (batch, L, G, N) B."""
    shp = np.asarray(B).shape
    return shp[2] if len(shp) == 4 else 1


class Oracle:
    """Thin handle on one compiled oracle library (the real one or a test
    mutant built from an edited copy of the source)."""

    def __init__(self, lib_path: str = ORACLE_LIB):
        self.path = lib_path
        lib = ctypes.CDLL(lib_path)
        lib.oracle_scan_f64.restype = ctypes.c_int
        lib.oracle_scan_f64.argtypes = [_i64] * 5 + [_dp] * 9 + [ctypes.c_int, _dp, _dp, ctypes.c_int]
        lib.oracle_state_update_f64.restype = ctypes.c_int
        lib.oracle_state_update_f64.argtypes = [_i64] * 4 + [_dp] * 9 + [ctypes.c_int, _dp, ctypes.c_int]
        lib.oracle_scan_bwd_f64.restype = ctypes.c_int
        lib.oracle_scan_bwd_f64.argtypes = [_i64] * 5 + [_dp] * 20 + [ctypes.c_int]
        lib.oracle_ssd_f64.restype = ctypes.c_int
        lib.oracle_ssd_f64.argtypes = [_i64] * 6 + [_dp] * 10 + [ctypes.c_int]
        lib.oracle_conv1d_silu_f64.restype = ctypes.c_int
        lib.oracle_conv1d_silu_f64.argtypes = [_i64] * 4 + [_dp] * 6 + [ctypes.c_int]
        lib.oracle_conv1d_update_f64.restype = ctypes.c_int
        lib.oracle_conv1d_update_f64.argtypes = [_i64] * 3 + [_dp] * 5 + [ctypes.c_int]
        self.lib = lib

    def scan(self, x, delta, A, B, C, D=None, z=None, delta_bias=None, h0=None,
             zoh=False, nthreads=None):
        """Full-sequence scan. x, delta, z: (batch, L, dim); A: (dim, N);
        B, C: (batch, L, N), or (batch, L, G, N) for G groups of channels;
        D, delta_bias: (dim,); h0: (batch, dim, N). Returns (out (batch, L,
        dim), last_state (batch, dim, N)) in fp64."""
        x = _f64(x)
        batch, L, dim = x.shape
        A = _f64(A)
        N = A.shape[1]
        delta = _f64(delta, x.shape)
        G = _groups(B)
        B = _f64(B, (batch, L, G, N))
        C = _f64(C, (batch, L, G, N))
        D = _f64(D, (dim,))
        z = _f64(z, x.shape)
        delta_bias = _f64(delta_bias, (dim,))
        h0 = _f64(h0, (batch, dim, N))
        out = np.empty((batch, L, dim), dtype=np.float64)
        last = np.empty((batch, dim, N), dtype=np.float64)
        nt = nthreads if nthreads else (os.cpu_count() or 1)
        rc = self.lib.oracle_scan_f64(batch, L, dim, N, G, _ptr(x), _ptr(delta), _ptr(A),
                                      _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(delta_bias),
                                      _ptr(h0), int(bool(zoh)), _ptr(out), _ptr(last), nt)
        if rc != 0:
            raise ValueError("oracle_scan_f64 returned %d" % rc)
        return out, last

    def state_update(self, state, x, delta, A, B, C, D=None, z=None, delta_bias=None,
                     zoh=False, nthreads=None):
        """One decode token. state: (batch, dim, N), updated copy returned;
        x, delta, z: (batch, dim); B, C: (batch, N), or (batch, G, N) for G
        groups of channels. Returns (out, new_state)."""
        x = _f64(x)
        batch, dim = x.shape
        A = _f64(A)
        N = A.shape[1]
        st = np.array(_f64(state, (batch, dim, N)), dtype=np.float64, copy=True)
        delta = _f64(delta, x.shape)
        G = np.asarray(B).shape[1] if np.asarray(B).ndim == 3 else 1
        B = _f64(B, (batch, G, N))
        C = _f64(C, (batch, G, N))
        D = _f64(D, (dim,))
        z = _f64(z, x.shape)
        delta_bias = _f64(delta_bias, (dim,))
        out = np.empty((batch, dim), dtype=np.float64)
        nt = nthreads if nthreads else (os.cpu_count() or 1)
        rc = self.lib.oracle_state_update_f64(batch, dim, N, G, _ptr(st), _ptr(x), _ptr(delta),
                                              _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                                              _ptr(delta_bias), int(bool(zoh)), _ptr(out), nt)
        if rc != 0:
            raise ValueError("oracle_state_update_f64 returned %d" % rc)
        return out, st


    def scan_bwd(self, x, delta, A, B, C, dout, D=None, z=None, delta_bias=None, h0=None,
                 dlast=None, nthreads=None):
        """Gradients of the scan (first-order B-bar) for dLoss/dout and
        optionally dLoss/dlast_state. Returns a dict with dx, ddelta, dz
        (batch, L, dim), dA (dim, N), dB, dC (the shape of B: (batch, L, N) or
        (batch, L, G, N)), dD, dbias (dim,) and dh0 (batch, dim, N), all fp64."""
        x = _f64(x)
        batch, L, dim = x.shape
        A = _f64(A)
        N = A.shape[1]
        delta = _f64(delta, x.shape)
        bshape = np.asarray(B).shape
        G = _groups(B)
        B = _f64(B, (batch, L, G, N))
        C = _f64(C, (batch, L, G, N))
        D = _f64(D, (dim,))
        z = _f64(z, x.shape)
        delta_bias = _f64(delta_bias, (dim,))
        h0 = _f64(h0, (batch, dim, N))
        dout = _f64(dout, x.shape)
        dlast = _f64(dlast, (batch, dim, N))
        g = {"dx": np.empty(x.shape), "ddelta": np.empty(x.shape), "dA": np.empty((dim, N)),
             "dB": np.empty(bshape), "dC": np.empty(bshape), "dD": np.empty(dim),
             "dz": np.empty(x.shape), "dbias": np.empty(dim), "dh0": np.empty((batch, dim, N))}
        nt = nthreads if nthreads else (os.cpu_count() or 1)
        rc = self.lib.oracle_scan_bwd_f64(
            batch, L, dim, N, G, _ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
            _ptr(delta_bias), _ptr(h0), _ptr(dout), _ptr(dlast), _ptr(g["dx"]), _ptr(g["ddelta"]),
            _ptr(g["dA"]), _ptr(g["dB"]), _ptr(g["dC"]), _ptr(g["dD"]), _ptr(g["dz"]),
            _ptr(g["dbias"]), _ptr(g["dh0"]), nt)
        if rc != 0:
            raise ValueError("oracle_scan_bwd_f64 returned %d" % rc)
        return g

    def ssd(self, x, dt, A, B, C, D=None, dt_bias=None, h0=None, nthreads=None):
        """Mamba-2 SSD layer by its recurrence. x: (batch, L, H, P); dt: (batch,
        L, H); A, D, dt_bias: (H,); B, C: (batch, L, G, N); h0: (batch, H, N,
        P). Returns (out (batch, L, H, P), last_state (batch, H, N, P)), fp64."""
        x = _f64(x)
        batch, L, H, P = x.shape
        dt = _f64(dt, (batch, L, H))
        A = _f64(A, (H,))
        G, N = np.asarray(B).shape[2], np.asarray(B).shape[3]
        B = _f64(B, (batch, L, G, N))
        C = _f64(C, (batch, L, G, N))
        D = _f64(D, (H,))
        dt_bias = _f64(dt_bias, (H,))
        h0 = _f64(h0, (batch, H, N, P))
        out = np.empty((batch, L, H, P))
        last = np.empty((batch, H, N, P))
        nt = nthreads if nthreads else (os.cpu_count() or 1)
        rc = self.lib.oracle_ssd_f64(batch, L, H, P, N, G, _ptr(x), _ptr(dt), _ptr(A), _ptr(B),
                                     _ptr(C), _ptr(D), _ptr(dt_bias), _ptr(h0), _ptr(out),
                                     _ptr(last), nt)
        if rc != 0:
            raise ValueError("oracle_ssd_f64 returned %d" % rc)
        return out, last

    def conv1d(self, xin, weight, bias=None, state_in=None, nthreads=None):
        """Causal depthwise convolution + SiLU. xin: (batch, L, dim); weight:
        (dim, width); bias: (dim,); state_in: (batch, dim, width - 1). Returns
        (out (batch, L, dim), state_out (batch, dim, width - 1))."""
        xin = _f64(xin)
        batch, L, dim = xin.shape
        weight = _f64(weight)
        width = weight.shape[1]
        bias = _f64(bias, (dim,))
        state_in = _f64(state_in, (batch, dim, width - 1))
        out = np.empty((batch, L, dim), dtype=np.float64)
        st = np.empty((batch, dim, width - 1), dtype=np.float64)
        nt = nthreads if nthreads else (os.cpu_count() or 1)
        rc = self.lib.oracle_conv1d_silu_f64(batch, L, dim, width, _ptr(xin), _ptr(weight),
                                             _ptr(bias), _ptr(state_in), _ptr(out), _ptr(st), nt)
        if rc != 0:
            raise ValueError("oracle_conv1d_silu_f64 returned %d" % rc)
        return out, st

    def conv1d_update(self, state, xin, weight, bias=None, nthreads=None):
        """One token: state (batch, dim, width - 1), updated copy returned; xin
        (batch, dim). Returns (out (batch, dim), new_state)."""
        xin = _f64(xin)
        batch, dim = xin.shape
        weight = _f64(weight)
        width = weight.shape[1]
        st = np.array(_f64(state, (batch, dim, width - 1)), dtype=np.float64, copy=True)
        bias = _f64(bias, (dim,))
        out = np.empty((batch, dim), dtype=np.float64)
        nt = nthreads if nthreads else (os.cpu_count() or 1)
        rc = self.lib.oracle_conv1d_update_f64(batch, dim, width, _ptr(st), _ptr(xin),
                                               _ptr(weight), _ptr(bias), _ptr(out), nt)
        if rc != 0:
            raise ValueError("oracle_conv1d_update_f64 returned %d" % rc)
        return out, st


_default = None
_lock = threading.Lock()


def default_oracle() -> Oracle:
    """The oracle built from ``ssm_oracle.c``; compiled on first use if the
    library is missing or older than its source."""
    global _default
    with _lock:
        if _default is None:
            if (not os.path.exists(ORACLE_LIB)
                    or os.path.getmtime(ORACLE_LIB) < os.path.getmtime(ORACLE_SRC)):
                build_oracle()
            _default = Oracle(ORACLE_LIB)
        return _default
