"""Helpers shared by the GPU parity tests."""
from __future__ import annotations

import sys

import numpy as np


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def tol_e(e_ref, n):
    """Parity bound on <Z_0>: 1e-5 relative, measured against max(|E_ref|, 2^(-n/2))
    (the observable's natural scale for a deep random circuit)."""
    return 1e-5 * np.maximum(np.abs(e_ref), 2.0 ** (-n / 2))


def assert_e_close(e_gpu, e_ref, n, scale=1.0):
    e_gpu = np.asarray(e_gpu, dtype=np.float64)
    bound = scale * tol_e(e_ref, n)
    err = np.abs(e_gpu - e_ref)
    assert np.all(err <= bound), f"<Z_0> mismatch: max err {err.max():.3e}, worst ratio {(err / bound).max():.3f}"


def assert_grad_close(g_gpu, g_ref, atol=1e-4):
    g_gpu = np.asarray(g_gpu, dtype=np.float64)
    err = np.abs(g_gpu - g_ref)
    assert err.max() <= atol, f"gradient mismatch: max abs err {err.max():.3e} (bound {atol})"
