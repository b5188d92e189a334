"""Write the stored expected values under tests/golden/.

Calls only the CPU oracle (``oracle/``) on the seeded inputs of
``hqml_inputs``; nothing here comes from the GPU path.  Re-run after a change
to the oracle's arithmetic that a passage of the pages justifies:
    python tests/golden/make_golden.py          # small fixtures (seconds)
    python tests/golden/make_golden.py full     # full-size single samples (minutes)
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import numpy as np  # noqa: E402

import hqml_inputs  # noqa: E402
import oracle  # noqa: E402


def single_sample(name, b, batch_index=0):
    """E and gradient of one sample (dL/dE = 1) of a named workload."""
    x, th, _ = hqml_inputs.workload_inputs(name, batch_index=batch_index)
    g, e = oracle.backward(x[b:b + 1], th, np.ones(1))
    path = os.path.join(HERE, f"{name}_b{batch_index}_s{b}.npz")
    np.savez_compressed(path, expz=e, grad=g.astype(np.float64),
                        source=np.array("oracle/hqml_oracle.c backward (fp64), dL/dE = 1, "
                                        f"sample {b} of batch {batch_index} of hqml_inputs.workload_inputs('{name}')"))
    print("wrote", path, flush=True)


def main():
    which = sys.argv[1:] or ["small"]
    if "full" in which:
        single_sample("hea20q100l", 0)
        single_sample("hea20q100l", 31)
        single_sample("hea20q1000l", 0)
    if "small" not in which:
        return
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
