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
