"""The CPU oracle against facts other than itself (closed forms, the dense
checker, parameter shift, finite differences, light cone, invariants)."""
import numpy as np
import pytest

import oracle
import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(oracle.default())


def test_one_layer_closed_form_at_20_qubits():
    """The one-layer closed form at the headline width (n = 20)."""
    r = np.random.default_rng(11)
    x = r.random((1, 20)) * np.pi
    th = r.random((1, 20, 3)) * 2 * np.pi
    a, b = th[0, 0, 0], th[0, 0, 1]
    e_ref = np.cos(x[0, 0]) * np.cos(a) * np.cos(b) - np.sin(x[0, 0]) * np.sin(b)
    assert abs(oracle.forward(x, th)[0] - e_ref) < 1e-12


def test_results_independent_of_thread_count():
    r = np.random.default_rng(12)
    x = r.random((6, 5)) * np.pi
    th = r.random((3, 5, 3)) * 2 * np.pi
    y = np.array([1, -1, 1, 1, -1, -1.0])
    o = oracle.default()
    t0 = o.max_threads()
    try:
        o.set_num_threads(1)
        a = o.train_step(x, th, y)
        o.set_num_threads(4)
        b = o.train_step(x, th, y)
    finally:
        o.set_num_threads(t0)
    assert np.array_equal(a[0], b[0]) and a[1] == b[1] and np.array_equal(a[2], b[2])


def test_rejects_bad_arguments():
    with pytest.raises(ValueError):
        oracle.forward(np.zeros((2, 31)), np.zeros((1, 31, 3)))
