"""Throughput of the fused training step (forward + adjoint backward) on one GPU.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload hea20q100l]

A step is one hqml_train_step over one batch of seeded synthetic input (the
20-qubit, 100-layer hardware-efficient ansatz at batch 32 by default): every
fused forward pass, the fused adjoint passes and all reductions, with inputs
already resident in device memory.  Prints one JSON line.

Besides the throughput, the line carries:
  roofline      the dominant kernel (the fused adjoint tile pass): algorithmic
                bytes per launch / its mean launch time, from HIP events recorded
                around every launch in a separate instrumented loop, against the
                8 TB/s HBM peak; "traffic" is the measured HBM bytes per launch from
                rocprofv3 counters when the kernel source still matches them;
  roofline_fwd  the same for the fused forward tile pass;
  cpu_baseline  the CPU oracle (fp64, gate by gate) timed on this host for a
                bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
PROFILES = os.path.join(ROOT, "profiles")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in ("hqml_kernels.hip", "hqml_internal.hpp"):
        with open(os.path.join(ROOT, "qml_gradients_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def algorithmic_bytes(plan: dict, B: int, storage: str):
    """Bytes of state each fused kernel must move at minimum (per train step).

    Per amplitude and sample: forward pass = read input + write output (no read
    for the product-state pass); adjoint pass = read the saved pass output + read
    lambda + write lambda (the fused last pass reads the previous output and writes
    lambda; a layer-0 statistics pass reads lambda only).  lambda is fp32 complex
    (8 B); saved states are 8 B (fp32) or 4 B (bf16).
    """
    N = 1 << plan["n"]
    s = 4 if storage == "bf16" else 8
    P = len(plan["passes"])
    fwd = bwd = 0
    for k, ps in enumerate(plan["passes"]):
        if k == P - 1:
            # fused forward+adjoint of the last pass: counted with the adjoint kernels
            bwd += ((0 if ps["init"] else s) + 8) * N * B
            continue
        fwd += ((0 if ps["init"] else s) + s) * N * B
        bwd += (s + 8 + 8) * N * B
    bwd += 8 * N * B * len(plan["stats_only"])
    return fwd, bwd


def traffic_record(kernel: str, workload: str):
    path = os.path.join(PROFILES, f"traffic_{kernel}_{workload}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("kernel_source_sha") != kernel_source_hash():
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(workload: str, timeout_s: float = 60.0):
    import numpy as np  # noqa: F401

    import hqml_inputs
    import oracle
    x, th, y = hqml_inputs.workload_inputs(workload)
    o = oracle.default()
    threads = o.max_threads()
    t0 = time.perf_counter()
    o.train_step(x[:1], th, y[:1])
    dt = time.perf_counter() - t0
    return {"value": 1.0 / dt, "unit": "samples/s", "cores": threads, "kind": "oracle",
            "sample": f"1 of the {x.shape[0]} samples of {workload} (full circuit, fp64 train step), "
                      f"{dt:.1f} s on {threads} OpenMP threads"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="hea20q100l")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--instrumented-steps", type=int, default=3)
    ap.add_argument("--overlap", type=int, default=0,
                    help="batch chunks pipelined over two streams (0 = library default, 1 = off)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a 1 GiB device-to-device copy 5 times (HBM counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU; --gpus must be 1 "
                                   "(the data-parallel sharding over GPUs is described in DESIGN.md)"}))
        sys.exit(2)

    import torch

    import hqml_inputs
    import qml_gradients_amd as hq

    if args.copy_calibration:
        src = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        src.fill_(1.0)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read_per_launch": src.numel() * 4,
                          "copy_bytes_written_per_launch": src.numel() * 4}), flush=True)
        return

    w = hqml_inputs.WORKLOADS[args.workload]
    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)
    x, th, y = hqml_inputs.workload_inputs(args.workload)
    X = torch.from_numpy(x).to(dev)
    TH = torch.from_numpy(th).to(dev)
    Y = torch.from_numpy(y).to(dev)
    B = X.shape[0]
    ctx = hq.Context(w.n_qubits, w.n_layers, B, storage=w.storage, ckpt_block=w.ckpt_block)
    ctx.set_overlap(args.overlap)
    plan = json.loads(hq.hqml_describe_plan(ctx.cfg))
    expz = torch.empty(B, device=dev)
    loss = torch.empty(1, device=dev)
    grad = torch.empty((w.n_layers, w.n_qubits, 3), device=dev)

    def step():
        hq.hqml_train_step(ctx.handle, B, X.data_ptr(), TH.data_ptr(), Y.data_ptr(), expz.data_ptr(),
                           loss.data_ptr(), grad.data_ptr())

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms_total = ev0.elapsed_time(ev1)
    ms_per_step = ms_total / args.steps
    value = B / (ms_per_step / 1e3)

    # Instrumented loop: HIP events around every launch (same workload).
    ctx.set_timing(True)
    ctx.kernel_times(reset=True)
    for _ in range(args.instrumented_steps):
        step()
    ms_k, cnt_k = ctx.kernel_times(reset=True)
    ctx.set_timing(False)
    fwd_b, bwd_b = algorithmic_bytes(plan, B, w.storage)
    n_steps = args.instrumented_steps

    def roof(kind, total_bytes_per_step, kernel_name):
        if n_steps == 0 or cnt_k[kind] == 0:
            return None
        launches = cnt_k[kind] / n_steps
        per_launch_bytes = total_bytes_per_step / launches
        avg_ms = ms_k[kind] / cnt_k[kind]
        achieved = per_launch_bytes / (avg_ms / 1e3) / 1e9
        return {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBPS, 4),
                "traffic": traffic_record(kernel_name, args.workload),
                "kernel": kernel_name, "avg_launch_ms": round(avg_ms, 4),
                "launches_per_step": launches, "algorithmic_bytes_per_launch": int(per_launch_bytes)}

    roof_bwd = roof(hq.HQML_K_BWD_PASS, bwd_b, "k_tile_bwd")
    roof_fwd = roof(hq.HQML_K_FWD_PASS, fwd_b, "k_tile_fwd")
    step_bytes = fwd_b + bwd_b
    out = {
        "metric": "train samples/sec (fwd+adjoint bwd) 20q HEA 100L; achieved HBM GB/s vs peak",
        "value": round(value, 2),
        "unit": "samples/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded x~U[0,pi), theta~U[0,2pi), y in {-1,+1})",
        "config": {"workload": args.workload, "n_qubits": w.n_qubits, "n_layers": w.n_layers,
                   "batch": B, "state_storage": w.storage, "ckpt_block": w.ckpt_block,
                   "overlap_chunks": args.overlap, "parallelism": "single GPU"},
        "step_state_bytes": step_bytes,
        "step_hbm_GBps": round(step_bytes / (ms_per_step / 1e3) / 1e9, 1),
        "step_hbm_frac": round(step_bytes / (ms_per_step / 1e3) / 1e9 / HBM_PEAK_GBPS, 4),
        "passes": {"fwd": len(plan["passes"]), "bwd": len(plan["passes"]) + len(plan["stats_only"]),
                   "per_layer": round(len(plan["passes"]) / w.n_layers, 3)},
        "roofline": roof_bwd if roof_bwd else roof_fwd,
        "roofline_fwd": roof_fwd,
        "kernel_ms_per_step": {k: round(ms_k[i] / max(n_steps, 1), 3) for i, k in
                               enumerate(["fwd_pass", "bwd_pass", "small", "other"])},
    }
    ctx.close()
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(args.workload)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
