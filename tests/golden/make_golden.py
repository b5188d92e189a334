"""Write the stored expected values under tests/golden/.

Calls only the CPU oracle (``oracle/``) on the seeded inputs of
``hqml_inputs``; nothing here comes from the GPU path.  Re-run after a change
to the oracle's arithmetic that a passage of the pages justifies:
    python tests/golden/make_golden.py
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import numpy as np  # noqa: E402

import hqml_inputs  # noqa: E402
import oracle  # noqa: E402


def main():
    for name in ("hea4q2l",):
        x, th, y = hqml_inputs.workload_inputs(name)
        e, loss, g = oracle.train_step(x, th, y)
        out = {
            "workload": name,
            "source": "oracle/hqml_oracle.c train_step (fp64) on hqml_inputs.workload_inputs",
            "expz": [float(v) for v in e],
            "loss": float(loss),
            "grad": np.asarray(g).ravel().tolist(),
        }
        with open(os.path.join(HERE, f"{name}.json"), "w") as f:
            json.dump(out, f, indent=1)


if __name__ == "__main__":
    main()
