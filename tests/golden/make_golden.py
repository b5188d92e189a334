"""Write the stored expected values under tests/golden/.

Calls only the CPU oracle (``oracle/``) on the seeded inputs of
``hqml_inputs``; nothing here comes from the GPU path.  Re-run after a change
to the oracle's arithmetic that a passage of the pages justifies:
    python tests/golden/make_golden.py          # small fixtures (seconds)
    python tests/golden/make_golden.py full     # full-size samples (about half an
                                                # hour on 7 cores)

Full-size values are per-sample: E_b and the gradient of E_b alone (dL/dE_b = 1),
from which a test forms any batch quantity (the training step's gradient is
sum_b 2 (E_b - y_b) / B * grad_b).  Each sample is one single-threaded oracle call
in its own worker process; finished samples are kept under ``_parts/`` (not
committed) so an interrupted run resumes, and the per-workload files are written
once every sample is done.
"""
import concurrent.futures as cf
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import numpy as np  # noqa: E402

import hqml_inputs  # noqa: E402
import oracle  # noqa: E402

PARTS = os.path.join(HERE, "_parts")

# (workload, first-batch sample indices).  hea20q100l: the whole batch the benchmark
# times.  hea20q1000l: samples of the first mini-batch of the 1,000-sample set; 0..59
# are in the fp32 batch (60) and all five in the bf16 batch (85), which starts with
# the same samples.
FULL = [
    ("hea20q1000l", (0, 17, 42, 59, 84)),
    ("hea20q100l", tuple(range(32))),
]


def _part_path(name, b):
    return os.path.join(PARTS, f"{name}_s{b}.npz")


def _one_sample(job):
    name, b = job
    path = _part_path(name, b)
    if os.path.exists(path):
        return path
    oracle.set_num_threads(1)
    w = hqml_inputs.WORKLOADS[name]
    # the 1000-layer set is sliced by a batch of 85 so that sample 84 exists
    x, th, _ = hqml_inputs.workload_inputs(name, batch=85 if w.n_layers >= 1000 else None)
    g, e = oracle.backward(x[b:b + 1], th, np.ones(1))
    tmp = path + f".tmp{os.getpid()}.npz"
    np.savez(tmp, expz=e, grad=g.astype(np.float64))
    os.replace(tmp, path)
    return path


def full(workers):
    os.makedirs(PARTS, exist_ok=True)
    jobs = [(name, b) for name, samples in FULL for b in samples]
    with cf.ProcessPoolExecutor(max_workers=workers) as pool:
        for path in pool.map(_one_sample, jobs):
            print("done", os.path.basename(path), flush=True)
    for name, samples in FULL:
        parts = [np.load(_part_path(name, b)) for b in samples]
        out = os.path.join(HERE, f"{name}_golden.npz")
        np.savez_compressed(
            out,
            samples=np.array(samples, dtype=np.int64),
            expz=np.concatenate([p["expz"] for p in parts]),
            grad=np.stack([p["grad"] for p in parts]),
            source=np.array("oracle/hqml_oracle.c backward (fp64), one call per sample with dL/dE = 1, "
                            f"samples {list(samples)} of hqml_inputs.workload_inputs('{name}')"))
        print("wrote", out, flush=True)


def small():
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


def main():
    which = sys.argv[1:] or ["small"]
    if "full" in which:
        full(int(os.environ.get("GOLDEN_WORKERS", "7")))
    if "small" in which:
        small()


if __name__ == "__main__":
    main()
