"""Helpers shared by the GPU parity tests."""
from __future__ import annotations

import sys

import numpy as np


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


EPS32 = 2.0 ** -24


def tol_e(e_ref, n, L=1):
    """Parity bound on <O>: 1e-5 relative, measured against max(|E_ref|, 2^(-n/2)) (the
    observable's natural scale for a deep random circuit), or, where larger, 1e-5 |E_ref|
    plus five standard deviations of the fp32 rounding noise of E: an fp32 state takes
    about L (n + 2) roundings per amplitude (n rotations and the diagonal per layer), each
    a relative error of eps32, and E = sum s_i |psi_i|^2 then deviates by about
    2 sqrt(2) eps32 sqrt(L (n + 2)) 2^(-n/2) for a spread state (sum |psi_i|^4 ~ 2 / 2^n)."""
    e = np.abs(e_ref)
    sigma = 2.0 * np.sqrt(2.0) * EPS32 * np.sqrt(L * (n + 2)) * 2.0 ** (-n / 2)
    return np.maximum(1e-5 * np.maximum(e, 2.0 ** (-n / 2)), 1e-5 * e + 5.0 * sigma)


def assert_e_close(e_gpu, e_ref, n, L=1, scale=1.0):
    e_gpu = np.asarray(e_gpu, dtype=np.float64)
    bound = scale * tol_e(e_ref, n, L)
    err = np.abs(e_gpu - e_ref)
    assert np.all(err <= bound), f"<Z_0> mismatch: max err {err.max():.3e}, worst ratio {(err / bound).max():.3f}"


def assert_grad_close(g_gpu, g_ref, atol=1e-4):
    g_gpu = np.asarray(g_gpu, dtype=np.float64)
    err = np.abs(g_gpu - g_ref)
    assert err.max() <= atol, f"gradient mismatch: max abs err {err.max():.3e} (bound {atol})"
