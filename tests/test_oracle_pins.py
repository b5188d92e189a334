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


@pytest.mark.parametrize("n, L, B", [(5, 3, 6), (14, 2, 1), (14, 1, 3)])
def test_results_independent_of_thread_count(n, L, B):
    """Bitwise the same results on 1, 3 and 4 threads: threads over samples (n = 5)
    and threads over the amplitude loops (n = 14 with a batch smaller than the thread
    count, the mode of the full-size stored values, which use one sample per call)."""
    r = np.random.default_rng(12 + n + B)
    x = r.random((B, n)) * np.pi
    th = r.random((L, n, 3)) * 2 * np.pi
    y = np.where(r.random(B) < 0.5, -1.0, 1.0)
    o = oracle.default()
    t0 = o.max_threads()
    runs = []
    try:
        for t in (1, 3, 4):
            o.set_num_threads(t)
            runs.append(o.train_step(x, th, y))
            runs.append(o.backward(x[:1], th, np.ones(1)))
    finally:
        o.set_num_threads(t0)
    a = runs[0]
    for b in runs[2::2]:
        assert np.array_equal(a[0], b[0]) and a[1] == b[1] and np.array_equal(a[2], b[2])
    for b in runs[3::2]:
        assert np.array_equal(runs[1][0], b[0]) and np.array_equal(runs[1][1], b[1])


def test_rejects_bad_arguments():
    with pytest.raises(ValueError):
        oracle.forward(np.zeros((2, 31)), np.zeros((1, 31, 3)))
