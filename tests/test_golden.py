"""The oracle still reproduces its stored expected values (tests/golden/)."""
import json
import os

import numpy as np

import hqml_inputs
import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_hea4q2l_golden():
    ref = json.load(open(os.path.join(GOLDEN, "hea4q2l.json")))
    x, th, y = hqml_inputs.workload_inputs("hea4q2l")
    e, loss, g = oracle.train_step(x, th, y)
    assert np.max(np.abs(e - np.array(ref["expz"]))) < 1e-13
    assert abs(loss - ref["loss"]) < 1e-13
    assert np.max(np.abs(g.ravel() - np.array(ref["grad"]))) < 1e-13


def test_full_size_golden_values_and_bounds_that_bind():
    """The stored full-size oracle values: shapes, last-layer Rz derivatives 0 to rounding
    (Rz, the CZ chain and Z_0 are diagonal), and bounds that bind: an all-zero or a
    sign-flipped result fails the bf16 bound and the fp32 relative gradient bound for
    every stored sample."""
    import numpy as np

    from gpu_util import bf16_bound, golden_sample

    for name, samples, (n, L) in (("hea20q100l", range(32), (20, 100)),
                                   ("hea20q1000l", (0, 17, 42, 59, 84), (20, 1000))):
        bf = max(bf16_bound(n, L), bf16_bound(n, L, grad=True))
        for b in samples:
            e, g = golden_sample(name, b)
            assert e.shape == (1,) and g.shape == (L, n, 3)
            assert np.abs(g[L - 1, :, 2]).max() < 1e-15
            assert abs(e[0]) <= 1.0
            gmax = np.abs(g).max()
            for wrong in (np.zeros_like(g), -g):
                assert np.abs(wrong - g).max() > max(bf, 1e-3 * gmax)
            assert 2 * gmax > bf
