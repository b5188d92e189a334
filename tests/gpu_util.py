"""Helpers shared by the GPU parity tests: parity bounds and the stored oracle values."""
from __future__ import annotations

import os
import sys

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


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


def assert_grad_rel(g_gpu, g_ref, rel, what="gradient"):
    """The bound that binds where gradients are small (deep random circuits): the
    largest error is at most `rel` times the largest reference entry."""
    g_gpu = np.asarray(g_gpu, dtype=np.float64)
    err = np.abs(g_gpu - g_ref).max()
    scale = np.abs(g_ref).max()
    assert err <= rel * scale, f"{what}: max|dg| {err:.3e} > {rel:g} x max|g_ref| {scale:.3e}"
    return err / scale


# ---- bf16 storage: a bound from the rounding of the stored states ----

BF16_HALF_ULP = 2.0 ** -9   # bf16 keeps 8 significant bits: round-to-nearest error <= 2^-9 relative


def bf16_sigma(n, passes, grad=False):
    """rms error of E (grad=False) or of a gradient entry (grad=True) caused by storing
    every pass output in bf16.

    E: each of the `passes` roundings multiplies every amplitude by (1 + e_i), e_i uniform
    in [-2^-9, 2^-9] (rms 2^-9 / sqrt 3); carried to the end by the rest of the circuit,
    a rounding moves E = <psi|O|psi> by 2 Re<phi|delta> with ||phi|| = 1, whose rms is
    2 (2^-9 / sqrt 3) sqrt(sum_i |phi_i|^2 |psi_i|^2), about 2 (2^-9 / sqrt 3) 2^(-n/2)
    for spread states; independent roundings add in quadrature.

    Gradient entry: a statistic Im<lam|s|psi> (||lam|| = 2 for a one-hot dL/dE) sees the
    same rounding twice, through the stored psi it reads and through lambda, which the
    adjoint seeds from the rounded final state (a factor sqrt 2), and an entry combines
    the three Pauli statistics of its qubit through the gradient map, |H| <= 1 (a factor
    up to sqrt 3): sigma_grad = sqrt 6 sigma_E."""
    s = 2.0 * BF16_HALF_ULP / np.sqrt(3.0) * np.sqrt(passes) * 2.0 ** (-n / 2)
    return s * np.sqrt(6.0) if grad else s


def bf16_bound(n, passes, k=5.0, grad=False):
    """Absolute bound k sigma (k = 5) on E (or on every gradient entry, grad=True) in
    bf16 storage, orders of magnitude inside the stated 2e-2 envelope at the full
    workload sizes."""
    return k * bf16_sigma(n, passes, grad)


def golden_sample(name, b):
    """Stored oracle values of sample b of a workload's first batch: (E [1], grad
    [L][n][3]) for dL/dE_b = 1 (written by tests/golden/make_golden.py from the oracle)."""
    path = os.path.join(GOLDEN, f"{name}_golden.npz")
    if not os.path.exists(path):
        return None
    d = np.load(path)
    k = int(np.nonzero(d["samples"] == b)[0][0])
    return d["expz"][k:k + 1], d["grad"][k]
