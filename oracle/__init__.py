"""hqml oracle -- TEST INFRASTRUCTURE ONLY.

Python access to the plain fp64 gate-by-gate CPU simulation in
``hqml_oracle.c`` (forward, adjoint gradient, training step) and to the
independent dense-matrix checker in ``dense.py``.  Only the tests, the smoke
check and the benchmark's CPU-baseline leg use this package; the GPU product
path never imports it, and it imports nothing from the product path.

Every function takes the fp32 arrays the GPU path sees and promotes them to
fp64, so both sides start from identical values.  ``entangler`` selects the
block that ends each layer: 0 = the CZ chain, 1 = the CNOT chain CNOT(q, q+1)
for q = 0..n-2 in that order.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "hqml_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_default = None


def compile_source(src: str, out: str) -> str:
    """gcc -O2 (IEEE arithmetic, no fast-math) with OpenMP."""
    tmp = out + f".tmp{os.getpid()}"
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=gnu11",
                           "-Wall", "-o", tmp, src, "-lm"])
    os.replace(tmp, out)
    return out


def build(force: bool = False) -> str:
    """Compile the oracle library next to its source if it is missing or stale."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(SOURCE):
        compile_source(SOURCE, _LIB)
    return _LIB


def _d(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _f64(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


class Oracle:
    """One loaded copy of the oracle library (the default build, or a variant
    compiled from modified source by a test)."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        d = ctypes.POINTER(ctypes.c_double)
        i = ctypes.c_int
        u = ctypes.c_uint32
        lib.oracle_forward.argtypes = [i, i, i, u, u, i, d, d, d]
        lib.oracle_backward.argtypes = [i, i, i, u, u, i, d, d, d, d, d]
        lib.oracle_train_step.argtypes = [i, i, i, u, u, i, d, d, d, d, d, d]
        lib.oracle_state.argtypes = [i, i, i, d, d, d]
        lib.oracle_max_norm_drift.argtypes = [i, i, i, d, d]
        lib.oracle_max_norm_drift.restype = ctypes.c_double
        lib.oracle_set_num_threads.argtypes = [i]
        lib.oracle_get_max_threads.restype = i
        for f in (lib.oracle_forward, lib.oracle_backward, lib.oracle_train_step, lib.oracle_state):
            f.restype = i
        self.lib = lib
        self.path = path

    def set_num_threads(self, t: int) -> None:
        self.lib.oracle_set_num_threads(int(t))

    def max_threads(self) -> int:
        return int(self.lib.oracle_get_max_threads())

    def state(self, x, theta, entangler: int = 0) -> np.ndarray:
        """Final complex128 state [2^n] of one sample (x: [n], theta: [L][n][3])."""
        x = _f64(x).ravel()
        n = x.size
        theta = np.ascontiguousarray(_f64(theta).reshape(-1, n, 3))
        L = theta.shape[0]
        out = np.zeros(2 * (1 << n), dtype=np.float64)
        rc = self.lib.oracle_state(n, L, int(entangler), _d(x), _d(theta), _d(out))
        if rc != 0:
            raise ValueError("oracle_state rejected its arguments")
        return out.view(np.complex128)

    def forward(self, x, theta, zmask: int = 1, xmask: int = 0, entangler: int = 0) -> np.ndarray:
        """E_b = <O> per sample, fp64 [B].  O is the Pauli string with factor Z on the
        qubits of zmask only, X on those of xmask only and Y on those of both (default
        Z_0).  x: [B][n], theta: [L][n][3]."""
        x = _f64(x)
        B, n = x.shape
        theta = np.ascontiguousarray(_f64(theta).reshape(-1, n, 3))
        out = np.zeros(B, dtype=np.float64)
        rc = self.lib.oracle_forward(n, theta.shape[0], B, int(zmask), int(xmask), int(entangler), _d(x),
                                     _d(theta), _d(out))
        if rc != 0:
            raise ValueError("oracle_forward rejected its arguments")
        return out

    def backward(self, x, theta, dLdE, zmask: int = 1, xmask: int = 0, entangler: int = 0):
        """(grad [L][n][3], E [B]) for upstream derivatives dLdE [B]."""
        x = _f64(x)
        B, n = x.shape
        theta = np.ascontiguousarray(_f64(theta).reshape(-1, n, 3))
        L = theta.shape[0]
        g = _f64(dLdE).ravel()
        grad = np.zeros((L, n, 3), dtype=np.float64)
        e = np.zeros(B, dtype=np.float64)
        rc = self.lib.oracle_backward(n, L, B, int(zmask), int(xmask), int(entangler), _d(x), _d(theta), _d(g),
                                      _d(grad), _d(e))
        if rc != 0:
            raise ValueError("oracle_backward rejected its arguments")
        return grad, e

    def train_step(self, x, theta, y, zmask: int = 1, xmask: int = 0, entangler: int = 0):
        """(E [B], loss, grad [L][n][3]) for the mean-squared-error loss on <O>."""
        x = _f64(x)
        B, n = x.shape
        theta = np.ascontiguousarray(_f64(theta).reshape(-1, n, 3))
        L = theta.shape[0]
        y = _f64(y).ravel()
        e = np.zeros(B, dtype=np.float64)
        loss = np.zeros(1, dtype=np.float64)
        grad = np.zeros((L, n, 3), dtype=np.float64)
        rc = self.lib.oracle_train_step(n, L, B, int(zmask), int(xmask), int(entangler), _d(x), _d(theta), _d(y),
                                        _d(e), _d(loss), _d(grad))
        if rc != 0:
            raise ValueError("oracle_train_step rejected its arguments")
        return e, float(loss[0]), grad

    def max_norm_drift(self, x, theta, entangler: int = 0) -> float:
        """Largest |1 - ||psi||^2| seen after any single gate (one sample)."""
        x = _f64(x).ravel()
        n = x.size
        theta = np.ascontiguousarray(_f64(theta).reshape(-1, n, 3))
        return float(self.lib.oracle_max_norm_drift(n, theta.shape[0], int(entangler), _d(x), _d(theta)))


def default() -> Oracle:
    global _default
    with _lock:
        if _default is None:
            _default = Oracle(build())
    return _default


def set_num_threads(t: int) -> None:
    default().set_num_threads(t)


def max_threads() -> int:
    return default().max_threads()


def state(x, theta, entangler: int = 0) -> np.ndarray:
    return default().state(x, theta, entangler)


def forward(x, theta, zmask: int = 1, xmask: int = 0, entangler: int = 0) -> np.ndarray:
    return default().forward(x, theta, zmask, xmask, entangler)


def backward(x, theta, dLdE, zmask: int = 1, xmask: int = 0, entangler: int = 0):
    return default().backward(x, theta, dLdE, zmask, xmask, entangler)


def train_step(x, theta, y, zmask: int = 1, xmask: int = 0, entangler: int = 0):
    return default().train_step(x, theta, y, zmask, xmask, entangler)


def max_norm_drift(x, theta, entangler: int = 0) -> float:
    return default().max_norm_drift(x, theta, entangler)
