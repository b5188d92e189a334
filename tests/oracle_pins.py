"""Pins of the CPU oracle to facts other than itself.

Each ``pin_*`` takes an ``oracle.Oracle`` and raises AssertionError when the
oracle disagrees with a fact fixed by the mathematics or by the independent
dense-matrix checker (``oracle/dense.py``).  ``test_oracle_pins.py`` runs them on
the real oracle; ``test_oracle_mutants.py`` runs them on deliberately broken
copies of the oracle source to show that a plausible mistake is caught.

Sources of the facts:
  * E(theta) = <psi_M|O|psi_M>, adjoint gradient and recursion: hugo-pages page
    "深度解析：正向与反向门融合驱动的高效量子机器学习仿真", section 1.2.
  * parameter-shift rule (the pages' memory-light gradient, same page section
    1.1, citing Mitarai et al. 2018): for a gate exp(-i t s/2) the exact
    derivative is [E(t + pi/2) - E(t - pi/2)] / 2.
  * Ry(t)|0> has <Z> = cos t (textbook).
  * CNOT entangler (same page, section 3.2: CNOT gates permute amplitude indices):
    the chain CNOT(0,1), CNOT(1,2), ..., CNOT(n-2,n-1) maps |i> to |P(i)>, bit k of
    P(i) being the parity of bits 0..k of i.  Conjugating Pauli strings by it
    (textbook Clifford algebra): P^dag Z_k P = Z_0 Z_1 ... Z_k and
    P^dag X_q P = X_q X_(q+1) (q < n-1), P^dag X_(n-1) P = X_(n-1).
"""
from __future__ import annotations

import math

import numpy as np

from oracle import dense


def _rand(n, L, B, seed):
    r = np.random.default_rng([7919, seed])
    x = r.random((B, n)) * math.pi
    th = r.random((L, n, 3)) * 2 * math.pi
    return x, th


def pin_ry_closed_form(o):
    """No layers: E = cos(x_0) for any width (Ry(x)|0> has <Z> = cos x)."""
    for n in (1, 2, 5):
        x, _ = _rand(n, 0, 4, n)
        e = o.forward(x, np.zeros((0, n, 3)))
        assert np.max(np.abs(e - np.cos(x[:, 0]))) < 1e-14, (n, e)


def pin_one_layer_closed_form(o):
    """One layer, any width: only qubit 0's rotations reach <Z_0> (the CZ chain
    and Rz commute with Z_0), so with (a, b) = theta[0][0][0:2]
        E = cos x0 cos a cos b - sin x0 sin b,
        dE/da = -cos x0 sin a cos b,  dE/db = -cos x0 cos a sin b - sin x0 cos b,
    and every other derivative is 0."""
    for n in (1, 3, 7, 20):
        x, th = _rand(n, 1, 5 if n < 20 else 2, 10 + n)
        a, b = th[0, 0, 0], th[0, 0, 1]
        x0 = x[:, 0]
        e_ref = np.cos(x0) * np.cos(a) * np.cos(b) - np.sin(x0) * np.sin(b)
        e = o.forward(x, th)
        assert np.max(np.abs(e - e_ref)) < 1e-13, (n, e, e_ref)
        w = np.linspace(-1.0, 1.5, x.shape[0])
        g, e2 = o.backward(x, th, w)
        assert np.max(np.abs(e2 - e_ref)) < 1e-13
        ga = np.sum(w * (-np.cos(x0) * np.sin(a) * np.cos(b)))
        gb = np.sum(w * (-np.cos(x0) * np.cos(a) * np.sin(b) - np.sin(x0) * np.cos(b)))
        ref = np.zeros_like(g)
        ref[0, 0, 0], ref[0, 0, 1] = ga, gb
        assert np.max(np.abs(g - ref)) < 1e-13, (n, g, ref)


def pin_norm_preserved(o):
    """Every gate is unitary: ||psi|| = 1 after each gate."""
    x, th = _rand(6, 3, 1, 3)
    assert o.max_norm_drift(x[0], th) < 1e-13


def pin_dense_state_and_gradient(o):
    """Gate-by-gate oracle == dense 2^n x 2^n product (state, E, gradient), n <= 4."""
    for n, L in ((1, 1), (2, 2), (3, 2), (4, 2), (4, 3)):
        x, th = _rand(n, L, 2, 100 + 10 * n + L)
        for b in range(2):
            s = o.state(x[b], th)
            sd = dense.state(x[b], th)
            assert np.max(np.abs(s - sd)) < 1e-12, (n, L)
        e = o.forward(x, th)
        ed = np.array([dense.expz(x[b], th) for b in range(2)])
        assert np.max(np.abs(e - ed)) < 1e-12, (n, L)
        w = np.array([0.7, -1.3])
        g, _ = o.backward(x, th, w)
        gd = sum(w[b] * dense.grad_expz(x[b], th) for b in range(2))
        assert np.max(np.abs(g - gd)) < 1e-12, (n, L, np.max(np.abs(g - gd)))


def pin_parameter_shift(o):
    """Adjoint gradient == exact parameter-shift derivative, every parameter."""
    for n, L in ((4, 3), (6, 2)):
        x, th = _rand(n, L, 2, 200 + n)
        w = np.array([1.0, -0.5])
        g, _ = o.backward(x, th, w)
        ref = np.zeros_like(th)
        for idx in np.ndindex(th.shape):
            tp, tm = th.copy(), th.copy()
            tp[idx] += math.pi / 2
            tm[idx] -= math.pi / 2
            ref[idx] = np.sum(w * (o.forward(x, tp) - o.forward(x, tm)) / 2)
        assert np.max(np.abs(g - ref)) < 1e-12, (n, L, np.max(np.abs(g - ref)))


def pin_finite_differences(o):
    """Adjoint gradient == central finite differences (h = 1e-5, error ~1e-10)."""
    n, L = 3, 2
    x, th = _rand(n, L, 1, 300)
    g, _ = o.backward(x, th, np.ones(1))
    h = 1e-5
    for idx in np.ndindex(th.shape):
        tp, tm = th.copy(), th.copy()
        tp[idx] += h
        tm[idx] -= h
        fd = (o.forward(x, tp)[0] - o.forward(x, tm)[0]) / (2 * h)
        assert abs(fd - g[idx]) < 1e-8, (idx, fd, g[idx])


def pin_light_cone(o):
    """For L < n, <Z_0> only sees qubits 0..L-1 (Z_0 spreads one qubit per
    layer through the CZ chain), and dE/dtheta[l][q] = 0 unless q <= L-1-l."""
    n, L = 9, 3
    x, th = _rand(n, L, 2, 400)
    e = o.forward(x, th)
    e_small = o.forward(x[:, :L], th[:, :L, :])
    assert np.max(np.abs(e - e_small)) < 1e-13
    g, _ = o.backward(x, th, np.array([1.0, 0.25]))
    for l in range(L):
        for q in range(n):
            if q > L - 1 - l:
                assert np.max(np.abs(g[l, q])) < 1e-14, (l, q, g[l, q])
    g_small, _ = o.backward(x[:, :L], th[:, :L, :], np.array([1.0, 0.25]))
    assert np.max(np.abs(g[:, :L, :] - g_small)) < 1e-13


def pin_last_layer_rz_zero(o):
    """The last layer's Rz is followed only by diagonal gates and Z_0, so its
    derivative is exactly 0."""
    x, th = _rand(5, 3, 3, 500)
    g, _ = o.backward(x, th, np.ones(3))
    assert np.max(np.abs(g[-1, :, 2])) < 1e-15
    assert np.max(np.abs(g[-1, :, :2])) > 1e-6   # the other last-layer terms are not all 0


def pin_trig_degree_one(o):
    """E is 2 pi periodic and a degree-1 trigonometric polynomial in each angle:
    E(t+pi/2) + E(t-pi/2) = E(t) + E(t+pi) (= twice the constant term)."""
    n, L = 4, 2
    x, th = _rand(n, L, 2, 600)
    for idx in [(0, 0, 0), (1, 2, 1), (0, 3, 2), (1, 0, 1)]:
        def E(shift, idx=idx):
            t = th.copy()
            t[idx] += shift
            return o.forward(x, t)
        assert np.max(np.abs(E(2 * math.pi) - E(0.0))) < 1e-13
        lhs = E(math.pi / 2) + E(-math.pi / 2)
        rhs = E(0.0) + E(math.pi)
        assert np.max(np.abs(lhs - rhs)) < 1e-13, idx
    for q in range(n):            # same for the encoding angles
        def Ex(shift, q=q):
            xx = x.copy()
            xx[:, q] += shift
            return o.forward(xx, th)
        assert np.max(np.abs(Ex(math.pi / 2) + Ex(-math.pi / 2) - Ex(0.0) - Ex(math.pi))) < 1e-13


def pin_train_step_is_mse(o):
    """train_step = forward, loss = mean (E - y)^2, backward with dL/dE = 2(E - y)/B,
    and the batch gradient is the sum of single-sample gradients."""
    n, L, B = 4, 2, 5
    x, th = _rand(n, L, B, 700)
    y = np.array([1.0, -1.0, -1.0, 1.0, 1.0])
    e, loss, g = o.train_step(x, th, y)
    e_ref = np.array([dense.expz(x[b], th) for b in range(B)])
    assert np.max(np.abs(e - e_ref)) < 1e-12
    assert abs(loss - np.mean((e_ref - y) ** 2)) < 1e-12
    dl = 2 * (e_ref - y) / B
    g_ref = sum(dl[b] * dense.grad_expz(x[b], th) for b in range(B))
    assert np.max(np.abs(g - g_ref)) < 1e-12
    g_sum = sum(o.backward(x[b:b + 1], th, dl[b:b + 1])[0] for b in range(B))
    assert np.max(np.abs(g - g_sum)) < 1e-13


def pin_zstring_product_state(o):
    """No layers, O = prod_{q in S} Z_q: the state is a product of Ry(x_q)|0>, so
    E = prod_{q in S} cos x_q (section 1.2's E(theta) with a Z-string O)."""
    n = 5
    x, _ = _rand(n, 0, 3, 800)
    for mask in (1, 2, 5, 0b01011, 0b11111):
        e = o.forward(x, np.zeros((0, n, 3)), mask)
        ref = np.prod([np.cos(x[:, q]) for q in range(n) if (mask >> q) & 1], axis=0)
        assert np.max(np.abs(e - ref)) < 1e-14, (mask, e, ref)


def pin_zstring_dense_and_parameter_shift(o):
    """Z-string observables: E and the adjoint gradient equal the dense checker's
    (n <= 4) and the exact parameter-shift derivative (n = 5)."""
    for n, L, mask in ((2, 2, 3), (3, 2, 0b110), (4, 2, 0b1010)):
        x, th = _rand(n, L, 2, 900 + n)
        e = o.forward(x, th, mask)
        ed = np.array([dense.expz(x[b], th, mask) for b in range(2)])
        assert np.max(np.abs(e - ed)) < 1e-12, (n, mask)
        w = np.array([0.4, -1.1])
        g, _ = o.backward(x, th, w, mask)
        gd = sum(w[b] * dense.grad_expz(x[b], th, mask) for b in range(2))
        assert np.max(np.abs(g - gd)) < 1e-12, (n, mask)
    n, L, mask = 5, 2, 0b10110
    x, th = _rand(n, L, 2, 950)
    w = np.array([1.0, 0.3])
    g, _ = o.backward(x, th, w, mask)
    ref = np.zeros_like(th)
    for idx in np.ndindex(th.shape):
        tp, tm = th.copy(), th.copy()
        tp[idx] += math.pi / 2
        tm[idx] -= math.pi / 2
        ref[idx] = np.sum(w * (o.forward(x, tp, mask) - o.forward(x, tm, mask)) / 2)
    assert np.max(np.abs(g - ref)) < 1e-12, np.max(np.abs(g - ref))
    y = np.array([1.0, -1.0])
    e, loss, gt = o.train_step(x, th, y, mask)
    gb, _ = o.backward(x, th, 2 * (e - y) / 2, mask)
    assert np.max(np.abs(gt - gb)) < 1e-13


def pin_pauli_product_state(o):
    """No layers, O a Pauli string: on Ry(x)|0> a qubit has <Z> = cos x, <X> = sin x
    and <Y> = 0, and the product state makes E the product of the factors."""
    n = 4
    x, _ = _rand(n, 0, 3, 1000)
    f = {"Z": np.cos, "X": np.sin, "Y": lambda v: 0.0 * v}
    for zm, xm in ((0, 1), (0, 0b0110), (0b1001, 0b0110), (0b0001, 0b0001), (0b0100, 0b1011)):
        ref = np.ones(x.shape[0])
        for q in range(n):
            z, xb = (zm >> q) & 1, (xm >> q) & 1
            if z or xb:
                ref = ref * f["Y" if (z and xb) else "Z" if z else "X"](x[:, q])
        e = o.forward(x, np.zeros((0, n, 3)), zm, xm)
        assert np.max(np.abs(e - ref)) < 1e-14, (zm, xm, e, ref)


def pin_pauli_dense_and_parameter_shift(o):
    """Pauli strings with X and Y factors: E and the adjoint gradient equal the dense
    checker's (n <= 4) and the exact parameter-shift derivative (n = 5)."""
    for n, L, zm, xm in ((1, 2, 1, 1), (2, 2, 0, 3), (3, 2, 0b101, 0b011), (4, 2, 0b0110, 0b1100)):
        x, th = _rand(n, L, 2, 1100 + n)
        e = o.forward(x, th, zm, xm)
        ed = np.array([dense.expz(x[b], th, zm, xm) for b in range(2)])
        assert np.max(np.abs(e - ed)) < 1e-12, (n, zm, xm)
        w = np.array([0.9, -0.4])
        g, _ = o.backward(x, th, w, zm, xm)
        gd = sum(w[b] * dense.grad_expz(x[b], th, zm, xm) for b in range(2))
        assert np.max(np.abs(g - gd)) < 1e-12, (n, zm, xm)
    n, L, zm, xm = 5, 2, 0b01010, 0b11000
    x, th = _rand(n, L, 2, 1150)
    w = np.array([1.0, -0.7])
    g, _ = o.backward(x, th, w, zm, xm)
    ref = np.zeros_like(th)
    for idx in np.ndindex(th.shape):
        tp, tm = th.copy(), th.copy()
        tp[idx] += math.pi / 2
        tm[idx] -= math.pi / 2
        ref[idx] = np.sum(w * (o.forward(x, tp, zm, xm) - o.forward(x, tm, zm, xm)) / 2)
    assert np.max(np.abs(g - ref)) < 1e-12, np.max(np.abs(g - ref))


def _single_qubit_bloch(xq, th_q):
    """<X>, <Y>, <Z> of Rz Ry Rx Ry(xq)|0> (one qubit, gates from the matrix exponential)."""
    v = dense.rot("Y", xq) @ np.array([1.0, 0.0], dtype=np.complex128)
    for a, ax in enumerate(dense.AXES):
        v = dense.rot(ax, th_q[a]) @ v
    return {s: float(np.real(np.vdot(v, dense.PAULI[s] @ v))) for s in dense.AXES}


def pin_cnot_one_layer_product_closed_form(o):
    """One layer with the CNOT chain: the state is P applied to a product state, so
    for a Pauli string O, E = <prod| P^dag O P |prod> factors into single-qubit
    expectations: <Z_k> = prod_{q <= k} <Z>_q, <X_q> = <X>_q <X>_(q+1), <X_(n-1)> =
    <X>_(n-1), <Y_0> = <Y>_0 <X>_1 (Y_0 = i X_0 Z_0).  A reversed chain, swapped
    control and target or a missing gate gives different products."""
    n = 4
    x, th = _rand(n, 1, 3, 1200)
    for b in range(x.shape[0]):
        bl = [_single_qubit_bloch(x[b, q], th[0, q]) for q in range(n)]
        cases = [(1 << k, 0, np.prod([bl[q]["Z"] for q in range(k + 1)])) for k in range(n)]
        cases += [(0, 1 << q, bl[q]["X"] * bl[q + 1]["X"]) for q in range(n - 1)]
        cases += [(0, 1 << (n - 1), bl[n - 1]["X"]), (1, 1, bl[0]["Y"] * bl[1]["X"])]
        for zm, xm, ref in cases:
            e = o.forward(x[b:b + 1], th, zm, xm, entangler=1)[0]
            assert abs(e - ref) < 1e-13, (b, zm, xm, e, ref)


def pin_cnot_dense_and_parameter_shift(o):
    """CNOT entangler: state, E and the adjoint gradient equal the dense checker's
    (n <= 4; CNOT there is |0><0| x I + |1><1| x X), and the exact parameter-shift
    derivative (n = 5); every gate stays unitary."""
    for n, L, zm, xm in ((2, 2, 1, 0), (3, 2, 0b100, 0), (3, 3, 0b101, 0b011), (4, 2, 0b0110, 0b1100), (4, 3, 1, 0)):
        x, th = _rand(n, L, 2, 1300 + 10 * n + L)
        s = o.state(x[0], th, entangler=1)
        assert np.max(np.abs(s - dense.state(x[0], th, entangler=1))) < 1e-12, (n, L)
        e = o.forward(x, th, zm, xm, entangler=1)
        ed = np.array([dense.expz(x[b], th, zm, xm, entangler=1) for b in range(2)])
        assert np.max(np.abs(e - ed)) < 1e-12, (n, L, zm, xm)
        w = np.array([0.8, -1.2])
        g, _ = o.backward(x, th, w, zm, xm, entangler=1)
        gd = sum(w[b] * dense.grad_expz(x[b], th, zm, xm, entangler=1) for b in range(2))
        assert np.max(np.abs(g - gd)) < 1e-12, (n, L, zm, xm)
    n, L, zm, xm = 5, 2, 0b00100, 0b00001
    x, th = _rand(n, L, 2, 1350)
    w = np.array([1.0, -0.6])
    g, _ = o.backward(x, th, w, zm, xm, entangler=1)
    ref = np.zeros_like(th)
    for idx in np.ndindex(th.shape):
        tp, tm = th.copy(), th.copy()
        tp[idx] += math.pi / 2
        tm[idx] -= math.pi / 2
        ref[idx] = np.sum(w * (o.forward(x, tp, zm, xm, entangler=1) - o.forward(x, tm, zm, xm, entangler=1)) / 2)
    assert np.max(np.abs(g - ref)) < 1e-12, np.max(np.abs(g - ref))
    assert o.max_norm_drift(x[0], th, entangler=1) < 1e-13


def pin_cnot_light_cone(o):
    """CNOT entangler, O = Z_0: qubit 0 is only ever a control, so Z_0 passes the last
    chain unchanged, and each earlier chain widens the cone by one qubit upward
    (X_q -> X_q X_(q+1)): for L < n, E and the gradient only involve qubits 0..L-1."""
    n, L = 8, 3
    x, th = _rand(n, L, 2, 1400)
    e = o.forward(x, th, entangler=1)
    assert np.max(np.abs(e - o.forward(x[:, :L], th[:, :L, :], entangler=1))) < 1e-13
    g, _ = o.backward(x, th, np.array([0.6, -1.0]), entangler=1)
    for l in range(L):
        for q in range(n):
            if q > L - 1 - l:
                assert np.max(np.abs(g[l, q])) < 1e-14, (l, q, g[l, q])
    g_small, _ = o.backward(x[:, :L], th[:, :L, :], np.array([0.6, -1.0]), entangler=1)
    assert np.max(np.abs(g[:, :L, :] - g_small)) < 1e-13


ALL_PINS = [
    pin_ry_closed_form,
    pin_one_layer_closed_form,
    pin_norm_preserved,
    pin_dense_state_and_gradient,
    pin_parameter_shift,
    pin_finite_differences,
    pin_light_cone,
    pin_last_layer_rz_zero,
    pin_trig_degree_one,
    pin_train_step_is_mse,
    pin_zstring_product_state,
    pin_zstring_dense_and_parameter_shift,
    pin_pauli_product_state,
    pin_pauli_dense_and_parameter_shift,
    pin_cnot_one_layer_product_closed_form,
    pin_cnot_dense_and_parameter_shift,
    pin_cnot_light_cone,
]
