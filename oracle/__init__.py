"""fp64 CPU oracles for the selective scan and the causal conv1d + SiLU --
TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It wraps ``oracle_scan.c`` and
``oracle_conv.c`` (plain C, double precision, sequential in time) through ctypes
and shares no code with the HIP library.  Every function here is pinned by the
CPU tests in ``tests/test_oracle_pins.py`` and ``tests/test_oracle_conv_pins.py``
(brute force, closed forms, exact decay, split/decode invariances, special cases,
planted-mistake checks).

Inputs are float64 numpy arrays (callers expand stored fp32/bf16 values exactly
before the call); outputs are float64 and never rounded to a storage type.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "oracle_scan.c")
LIBRARY = os.path.join(_HERE, "liboracle_scan.so")
CONV_SOURCE = os.path.join(_HERE, "oracle_conv.c")
CONV_LIBRARY = os.path.join(_HERE, "liboracle_conv.so")

CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-fno-fast-math", "-ffp-contract=off",
          "-pthread"]


def build(source: str = SOURCE, output: str = LIBRARY, extra_flags=()) -> str:
    """Compile the oracle with gcc (no fast-math, no FMA contraction)."""
    cmd = ["gcc", *CFLAGS, *extra_flags, source, "-o", output, "-lm"]
    subprocess.run(cmd, check=True)
    return output


_dp = ctypes.POINTER(ctypes.c_double)
_i64 = ctypes.c_int64


class Oracle:
    """A loaded oracle library (the committed one, or a test build of a variant)."""

    def __init__(self, path: str = LIBRARY):
        self.path = path
        lib = ctypes.CDLL(path)
        lib.oracle_scan.restype = ctypes.c_int
        lib.oracle_scan.argtypes = [_dp] * 11 + [_i64] * 4 + [ctypes.c_int, ctypes.c_int]
        lib.oracle_step.restype = ctypes.c_int
        lib.oracle_step.argtypes = [_dp] * 10 + [_i64] * 3 + [ctypes.c_int]
        lib.oracle_scan_ext.restype = ctypes.c_int
        lib.oracle_scan_ext.argtypes = ([_dp] * 11 + [_i64] * 4 + [ctypes.c_int, ctypes.c_int] +
                                        [_dp] * 4)
        lib.oracle_step_ext.restype = ctypes.c_int
        lib.oracle_step_ext.argtypes = [_dp] * 10 + [_i64] * 3 + [ctypes.c_int] + [_dp] * 4
        lib.oracle_scan_bwd.restype = ctypes.c_int
        lib.oracle_scan_bwd.argtypes = [_dp] * 20 + [_i64] * 4 + [ctypes.c_int]
        lib.oracle_scan_bwd_ext.restype = ctypes.c_int
        lib.oracle_scan_bwd_ext.argtypes = ([_dp] * 11 + [ctypes.c_int] + [_dp] * 17 +
                                            [_i64] * 4 + [ctypes.c_int])
        lib.oracle_softplus.restype = ctypes.c_double
        lib.oracle_softplus.argtypes = [ctypes.c_double]
        lib.oracle_silu.restype = ctypes.c_double
        lib.oracle_silu.argtypes = [ctypes.c_double]
        self._lib = lib

    # -- scalar helpers -------------------------------------------------------
    def softplus(self, x: float) -> float:
        return self._lib.oracle_softplus(float(x))

    def silu(self, z: float) -> float:
        return self._lib.oracle_silu(float(z))

    # -- full scan ------------------------------------------------------------
    def scan(self, u, delta, A, B, C, D=None, z=None, bias=None, h0=None,
             nthreads: Optional[int] = None, zoh: bool = False, lam=None, u_prev=None,
             B_prev=None, theta=None) -> Tuple[np.ndarray, np.ndarray]:
        """Return (y, h_last) in float64 (zoh: zero-order-hold Bbar instead of Euler's).

        u, delta, z: (batch, L, d_inner); B, C: (batch, L, d_state);
        A: (d_inner, d_state); D, bias: (d_inner,); h0: (batch, d_inner, d_state).
        lam (batch, L, d_inner): exponential-trapezoidal mixing coefficients, with the input
        before t = 0 in u_prev (batch, d_inner) and B_prev (batch, d_state); theta
        (batch, L, d_state / 2): rotation rates of the state pairs.
        """
        u = _c64(u)
        batch, L, d_inner = u.shape
        A = _c64(A)
        d_state = A.shape[1]
        delta, B, C = _c64(delta), _c64(B), _c64(C)
        D, z, bias, h0 = _c64(D), _c64(z), _c64(bias), _c64(h0)
        _check(delta, u.shape, "delta")
        _check(B, (batch, L, d_state), "B")
        _check(C, (batch, L, d_state), "C")
        _check(A, (d_inner, d_state), "A")
        _check(D, (d_inner,), "D")
        _check(bias, (d_inner,), "bias")
        _check(z, u.shape, "z")
        _check(h0, (batch, d_inner, d_state), "h0")
        lam, u_prev, B_prev, theta = _c64(lam), _c64(u_prev), _c64(B_prev), _c64(theta)
        _check(lam, u.shape, "lam")
        _check(u_prev, (batch, d_inner), "u_prev")
        _check(B_prev, (batch, d_state), "B_prev")
        _check(theta, (batch, L, d_state // 2), "theta")
        y = np.empty(u.shape, dtype=np.float64)
        h_last = np.empty((batch, d_inner, d_state), dtype=np.float64)
        if nthreads is None:
            nthreads = default_threads()
        rc = self._lib.oracle_scan_ext(_p(u), _p(delta), _p(A), _p(B), _p(C), _p(D), _p(z),
                                       _p(bias), _p(h0), _p(y), _p(h_last), batch, L, d_inner,
                                       d_state, int(nthreads), int(bool(zoh)), _p(lam),
                                       _p(u_prev), _p(B_prev), _p(theta))
        if rc != 0:
            raise ValueError("oracle_scan rejected its arguments")
        return y, h_last

    # -- gradients ------------------------------------------------------------
    def scan_bwd(self, u, delta, A, B, C, dy, D=None, z=None, bias=None, h0=None,
                 dh_last=None, nthreads: Optional[int] = None) -> dict:
        """Gradients of sum(dy * y) + sum(dh_last * h_last) (Euler scan) with respect to
        every input: keys du, ddelta, dA, dB, dC, dD, dz, dbias, dh0 (float64; dD, dz,
        dbias are returned even when D, z, bias are absent: the gradient at zero / no gate)."""
        u = _c64(u)
        batch, L, d_inner = u.shape
        A = _c64(A)
        d_state = A.shape[1]
        delta, B, C, dy = _c64(delta), _c64(B), _c64(C), _c64(dy)
        D, z, bias, h0, dh_last = _c64(D), _c64(z), _c64(bias), _c64(h0), _c64(dh_last)
        for a, shp, name in ((delta, u.shape, "delta"), (dy, u.shape, "dy"),
                             (B, (batch, L, d_state), "B"), (C, (batch, L, d_state), "C"),
                             (D, (d_inner,), "D"), (bias, (d_inner,), "bias"),
                             (z, u.shape, "z"), (h0, (batch, d_inner, d_state), "h0"),
                             (dh_last, (batch, d_inner, d_state), "dh_last")):
            _check(a, shp, name)
        out = dict(du=np.zeros(u.shape), ddelta=np.zeros(u.shape), dA=np.zeros(A.shape),
                   dB=np.zeros((batch, L, d_state)), dC=np.zeros((batch, L, d_state)),
                   dD=np.zeros(d_inner), dz=np.zeros(u.shape), dbias=np.zeros(d_inner),
                   dh0=np.zeros((batch, d_inner, d_state)))
        if nthreads is None:
            nthreads = default_threads()
        rc = self._lib.oracle_scan_bwd(
            _p(u), _p(delta), _p(A), _p(B), _p(C), _p(D), _p(z), _p(bias), _p(h0), _p(dy),
            _p(dh_last), _p(out["du"]), _p(out["ddelta"]), _p(out["dA"]), _p(out["dB"]),
            _p(out["dC"]), _p(out["dD"]), _p(out["dz"]), _p(out["dbias"]), _p(out["dh0"]),
            batch, L, d_inner, d_state, int(nthreads))
        if rc != 0:
            raise ValueError("oracle_scan_bwd rejected its arguments")
        return out

    def scan_bwd_ext(self, u, delta, A, B, C, dy, D=None, z=None, bias=None, h0=None,
                     dh_last=None, zoh: bool = False, lam=None, u_prev=None, B_prev=None,
                     theta=None, nthreads: Optional[int] = None) -> dict:
        """Gradients of sum(dy * y) + sum(dh_last * h_last) for the scan with the
        zero-order hold, the trapezoid (lam, u_prev, B_prev) or the rotation (theta): the
        keys of scan_bwd plus dlam, du_prev, dB_prev (trapezoid) and dtheta (rotation)."""
        u = _c64(u)
        batch, L, d_inner = u.shape
        A = _c64(A)
        d_state = A.shape[1]
        delta, B, C, dy = _c64(delta), _c64(B), _c64(C), _c64(dy)
        D, z, bias, h0, dh_last = _c64(D), _c64(z), _c64(bias), _c64(h0), _c64(dh_last)
        lam, u_prev, B_prev, theta = _c64(lam), _c64(u_prev), _c64(B_prev), _c64(theta)
        for a, shp, name in ((delta, u.shape, "delta"), (dy, u.shape, "dy"),
                             (B, (batch, L, d_state), "B"), (C, (batch, L, d_state), "C"),
                             (D, (d_inner,), "D"), (bias, (d_inner,), "bias"),
                             (z, u.shape, "z"), (h0, (batch, d_inner, d_state), "h0"),
                             (dh_last, (batch, d_inner, d_state), "dh_last"),
                             (lam, u.shape, "lam"), (u_prev, (batch, d_inner), "u_prev"),
                             (B_prev, (batch, d_state), "B_prev"),
                             (theta, (batch, L, d_state // 2), "theta")):
            _check(a, shp, name)
        out = dict(du=np.zeros(u.shape), ddelta=np.zeros(u.shape), dA=np.zeros(A.shape),
                   dB=np.zeros((batch, L, d_state)), dC=np.zeros((batch, L, d_state)),
                   dD=np.zeros(d_inner), dz=np.zeros(u.shape), dbias=np.zeros(d_inner),
                   dh0=np.zeros((batch, d_inner, d_state)), dlam=np.zeros(u.shape),
                   du_prev=np.zeros((batch, d_inner)), dB_prev=np.zeros((batch, d_state)),
                   dtheta=np.zeros((batch, L, d_state // 2)))
        if nthreads is None:
            nthreads = default_threads()
        rc = self._lib.oracle_scan_bwd_ext(
            _p(u), _p(delta), _p(A), _p(B), _p(C), _p(D), _p(z), _p(bias), _p(h0), _p(dy),
            _p(dh_last), int(bool(zoh)), _p(lam), _p(u_prev), _p(B_prev), _p(theta),
            _p(out["du"]), _p(out["ddelta"]), _p(out["dA"]), _p(out["dB"]), _p(out["dC"]),
            _p(out["dD"]), _p(out["dz"]), _p(out["dbias"]), _p(out["dh0"]), _p(out["dlam"]),
            _p(out["du_prev"]), _p(out["dB_prev"]), _p(out["dtheta"]),
            batch, L, d_inner, d_state, int(nthreads))
        if rc != 0:
            raise ValueError("oracle_scan_bwd_ext rejected its arguments")
        return out

    # -- one decode step ------------------------------------------------------
    def step(self, h, u, delta, A, B, C, D=None, z=None, bias=None, zoh: bool = False,
             lam=None, u_prev=None, B_prev=None, theta=None) -> Tuple[np.ndarray, np.ndarray]:
        """Return (y, h_new); h is not modified.  u, delta, z, lam, u_prev: (batch, d_inner);
        B, C, B_prev: (batch, d_state); theta: (batch, d_state / 2);
        h: (batch, d_inner, d_state)."""
        h_new = np.array(h, dtype=np.float64, copy=True, order="C")
        u = _c64(u)
        batch, d_inner = u.shape
        A = _c64(A)
        d_state = A.shape[1]
        delta, B, C, D, z, bias = (_c64(delta), _c64(B), _c64(C), _c64(D), _c64(z),
                                   _c64(bias))
        _check(h_new, (batch, d_inner, d_state), "h")
        _check(delta, u.shape, "delta")
        _check(B, (batch, d_state), "B")
        _check(C, (batch, d_state), "C")
        _check(z, u.shape, "z")
        lam, u_prev, B_prev, theta = _c64(lam), _c64(u_prev), _c64(B_prev), _c64(theta)
        _check(lam, u.shape, "lam")
        _check(u_prev, u.shape, "u_prev")
        _check(B_prev, (batch, d_state), "B_prev")
        _check(theta, (batch, d_state // 2), "theta")
        y = np.empty(u.shape, dtype=np.float64)
        rc = self._lib.oracle_step_ext(_p(h_new), _p(u), _p(delta), _p(A), _p(B), _p(C), _p(D),
                                       _p(z), _p(bias), _p(y), batch, d_inner, d_state,
                                       int(bool(zoh)), _p(lam), _p(u_prev), _p(B_prev),
                                       _p(theta))
        if rc != 0:
            raise ValueError("oracle_step rejected its arguments")
        return y, h_new


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def _c64(a):
    if a is None:
        return None
    return np.ascontiguousarray(a, dtype=np.float64)


def _p(a):
    if a is None:
        return None
    return a.ctypes.data_as(_dp)


def _check(a, shape, name):
    if a is not None and tuple(a.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(a.shape)}")


class ConvOracle:
    """The causal depthwise conv1d + SiLU oracle (oracle_conv.c)."""

    def __init__(self, path: str = CONV_LIBRARY):
        self.path = path
        lib = ctypes.CDLL(path)
        lib.oracle_conv1d_silu.restype = ctypes.c_int
        lib.oracle_conv1d_silu.argtypes = [_dp] * 7 + [_i64] * 4
        lib.oracle_conv1d_step.restype = ctypes.c_int
        lib.oracle_conv1d_step.argtypes = [_dp] * 6 + [_i64] * 3
        self._lib = lib

    def conv(self, x, w, bias=None, state_in=None):
        """Return (pre, u, state_out) in float64.  x: (batch, L, D); w: (D, K);
        bias: (D,); state_in: (batch, D, K - 1)."""
        x, w = _c64(x), _c64(w)
        batch, L, D = x.shape
        K = w.shape[1]
        bias, state_in = _c64(bias), _c64(state_in)
        _check(w, (D, K), "w")
        _check(bias, (D,), "bias")
        _check(state_in, (batch, D, K - 1), "state_in")
        pre = np.empty(x.shape, dtype=np.float64)
        u = np.empty(x.shape, dtype=np.float64)
        state_out = np.empty((batch, D, K - 1), dtype=np.float64)
        rc = self._lib.oracle_conv1d_silu(_p(x), _p(w), _p(bias), _p(state_in), _p(pre),
                                          _p(u), _p(state_out), batch, L, D, K)
        if rc != 0:
            raise ValueError("oracle_conv1d_silu rejected its arguments")
        return pre, u, state_out

    def step(self, state, x, w, bias=None):
        """One decode step: return (pre, u, state_new); state is not modified.
        state: (batch, D, K - 1); x: (batch, D)."""
        x, w = _c64(x), _c64(w)
        batch, D = x.shape
        K = w.shape[1]
        st = np.array(state, dtype=np.float64, copy=True, order="C")
        _check(st, (batch, D, K - 1), "state")
        bias = _c64(bias)
        _check(bias, (D,), "bias")
        pre = np.empty(x.shape, dtype=np.float64)
        u = np.empty(x.shape, dtype=np.float64)
        rc = self._lib.oracle_conv1d_step(_p(st), _p(x), _p(w), _p(bias), _p(pre), _p(u),
                                          batch, D, K)
        if rc != 0:
            raise ValueError("oracle_conv1d_step rejected its arguments")
        return pre, u, st


_default: Optional[Oracle] = None
_default_conv: Optional[ConvOracle] = None


def _stale(lib, src):
    return not os.path.exists(lib) or os.path.getmtime(lib) < os.path.getmtime(src)


def load() -> Oracle:
    """The committed oracle, compiled on first use if it has not been built."""
    global _default
    if _default is None:
        if _stale(LIBRARY, SOURCE):
            build()
        _default = Oracle(LIBRARY)
    return _default


def load_conv() -> ConvOracle:
    """The committed conv1d + SiLU oracle, compiled on first use."""
    global _default_conv
    if _default_conv is None:
        if _stale(CONV_LIBRARY, CONV_SOURCE):
            build(CONV_SOURCE, CONV_LIBRARY)
        _default_conv = ConvOracle(CONV_LIBRARY)
    return _default_conv
