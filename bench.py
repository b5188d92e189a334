"""Throughput of the fused training step (forward + adjoint backward) on one GPU.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload hea20q100l]

A step is one hqml_train_step over one batch of seeded synthetic input (the
20-qubit, 100-layer hardware-efficient ansatz at batch 32 by default): every
fused forward pass, the fused adjoint passes and all reductions, with inputs
already resident in device memory.  Prints one JSON line.

Besides the throughput, the line carries:
  roofline      the dominant kernel (the fused adjoint tile pass: k_tile_bwdh, the
                half-tile general shape, for all adjoint launches but the fused last
                pass and the product-state pass of the fp32 CZ-chain plan) against the
                published HBM peak of 8 TB/s: the adjoint launches' algorithmic state
                bytes per launch (read the saved pass output, read and write lambda: 24 B
                per amplitude and sample in fp32) / their mean launch time, from HIP
                events recorded on the launch stream around every launch in a
                separate instrumented loop (batch chunking off); "traffic" is the
                measured HBM bytes per launch from rocprofv3 counters while the
                kernel source still matches them;
  roofline_alu  the same kernel's arithmetic rate (algorithmic flops per launch /
                time) against a plain (non-packed) fp32 FMA peak derived from the
                unit counts and clock, and as a fraction of the published 157.3
                TFLOP/s (which counts packed FP32, excluded from this build);
  roofline_fwd  the fused forward tile pass (memory-bound) against 8 TB/s;
  cpu_baseline  the CPU oracle (fp64, gate by gate) timed on this host for a
                bounded sample of the same workload, with the host's CPU model,
                logical and physical core counts and the threads it used.
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
# Plain (non-packed) fp32 FMA rate: 256 CUs x 4 SIMDs x 16 lanes x 2 flops x 2.4 GHz.
# Packed-FP32 instructions are excluded from the build, so this is the ALU peak the
# kernels can reach (the published 157.3 TFLOP/s counts packed FP32).
ALU_PEAK_TFLOPS = 256 * 4 * 16 * 2 * 2.4e9 / 1e12
FP32_PUBLISHED_TFLOPS = 157.3
PROFILES = os.path.join(ROOT, "profiles")
L2_POSITIONS = (0, 1, 9, 10, 11)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    # what the tile kernels are built from: their sources and the build's compile flags
    for f in ("hqml_kernels.hip", "hqml_half.hpp", "hqml_device.hpp", "hqml_internal.hpp"):
        with open(os.path.join(ROOT, "qml_gradients_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    from qml_gradients_amd import build as hq_build
    h.update(repr((hq_build.FLAGS[:-1], hq_build.UNITS)).encode())   # FLAGS[-1]: the include path
    return h.hexdigest()[:16]


def algorithmic_bytes(plan: dict, B: int, storage: str, compute: str = "fp32"):
    """Bytes of state each fused kernel must move at minimum (per train step).

    Per amplitude and sample: forward pass = read input + write output (no read
    for the product-state pass); adjoint pass = read the saved pass output + read
    lambda + write lambda (the fused last pass reads the previous output and writes
    lambda; a layer-0 statistics pass reads lambda only).  lambda is complex in the
    compute type (8 B fp32, 16 B fp64); saved states are 8 B (fp32), 4 B (bf16) or
    16 B (fp64).
    """
    N = 1 << plan["n"]
    s = {"bf16": 4, "fp32": 8, "fp64": 16}[storage]
    lb = 16 if compute == "fp64" else 8
    P = len(plan["passes"])
    fwd = bwd = 0
    for k, ps in enumerate(plan["passes"]):
        if plan.get("cnot"):
            # CNOT-chain plan: no fused last pass; pass 0's backward reads lambda only
            # (and writes it once for a one-layer circuit)
            fwd += ((0 if ps["init"] else s) + s) * N * B
            bwd += (lb * (2 if P == 1 else 1) if ps["init"] else s + lb + lb) * N * B
            continue
        if k == P - 1:
            # fused forward+adjoint of the last pass: counted with the adjoint kernels
            bwd += ((0 if ps["init"] else s) + lb) * N * B
            continue
        fwd += ((0 if ps["init"] else s) + s) * N * B
        bwd += (s + lb + lb) * N * B
    bwd += lb * N * B * len(plan["stats_only"])
    # checkpointing: every block but the last is recomputed from its checkpoint
    # (the block's last output is itself the next checkpoint, kept from the forward)
    c = plan["c"]
    if c:
        for k in range(plan["nblocks"] - 1):
            for p in range(k * c, min(P, (k + 1) * c) - 1):
                fwd += ((0 if plan["passes"][p]["init"] else s) + s) * N * B
    return fwd, bwd


def half_tiles(plan: dict, compute: str = "fp32") -> bool:
    """Whether the adjoint passes run on half tiles (k_tile_bwdh): a tile plan with a half
    view for every view (either compute type, either entangler)."""
    return bool(plan.get("half"))


def algorithmic_flops_bwd(plan: dict, B: int, compute: str = "fp32"):
    """Floating-point operations the fused adjoint kernels perform per train step
    (FMA = 2, multiply or add = 1), per amplitude and sample of each launch:
      rotation (scaled tan form) on one state: 4 per qubit;
      X and Y statistics of one qubit: 8; Z statistics of a register layout: 5;
      merged diagonal applied to lambda: 9 (to psi and lambda: 18); final lambda scale: 2.
    g = qubits the pass's view rotates, g1 / g2 = those at L1 / L2 register positions.
    The general and product-state shapes take both layers' statistics from one set of
    sums (merged statistics) and rotate psi only by the L1 half of the later layer; on
    half tiles every statistic is taken at the pass output and psi is not rotated."""
    N = 1 << plan["n"]
    P = len(plan["passes"])
    half = half_tiles(plan, compute)
    total = 0
    for k, ps in enumerate(plan["passes"]):
        gm = plan["views"][ps["view"]]["group_mask"]
        g = bin(gm).count("1")
        g2 = sum((gm >> p) & 1 for p in L2_POSITIONS)
        g1 = g - g2
        if half and k != P - 1 and ps["rotA"] >= 0 and ps["diag"] >= 0 and ps["rotB"] >= 0 and not ps["init"]:
            g1 = 0
        if k == P - 1 and not ps["init"]:
            # forward rotations, E, seed, statistics, un-rotations, scale
            f = 4 * g + 3 + 8 * g + 10 + 4 * g2 + 4 * g + 2
        elif ps["rotB"] >= 0 and ps["init"]:
            f = 8 * g + 10 + 4 * g1 + 4 * g + 9 + 2
        elif ps["rotB"] >= 0:
            f = 8 * g + 10 + 4 * g1 + 8 * g + 9 + 2
        elif ps["rotA"] >= 0:
            f = 8 * g + 10 + 4 * g + 2
        else:
            f = 8 * g + 10
        total += f * N * B
    for v in plan["stats_only"]:
        g = bin(plan["views"][v]["group_mask"]).count("1")
        total += (8 * g + 10) * N * B
    return total


def algorithmic_flops_small(n: int, L: int, B: int):
    """Floating-point operations of the whole-circuit kernel per train step (FMA = 2,
    multiply or add = 1), per amplitude and sample: each of the L - 1 forward steps applies
    a merged diagonal (6) and rotates n qubits in tan form (4 per qubit); the adjoint takes
    X and Y statistics of every qubit at each of the L points (8 per qubit), the Z
    statistics (1 per qubit and 2 per amplitude for Im(conj(lambda) psi)), and each of its
    L - 1 steps applies the conjugate diagonal to psi and lambda (12) and un-rotates both
    (8 per qubit)."""
    per_amp = (L - 1) * (6 + 4 * n) + L * (9 * n + 2) + (L - 1) * (12 + 8 * n)
    return per_amp * (1 << n) * B


def small_kernel_name(n: int, entangler: str, compute: str) -> str:
    """The whole-circuit kernel a context runs: the register-resident one at 12 qubits with
    the CZ chain in fp32 compute, the register-round one otherwise."""
    return "k_small12" if n == 12 and entangler == "cz" and compute == "fp32" else "k_small"


def traffic_record(kernel: str, workload: str, entangler: str = "cz"):
    """Counter-measured HBM bytes per launch (CZ-chain plan), while the source matches."""
    if entangler != "cz":
        return None
    path = os.path.join(PROFILES, f"traffic_{kernel}_{workload}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("kernel_source_sha") != kernel_source_hash():
        return None
    return rec.get("bytes_per_launch")


def host_cpu():
    """CPU model, logical CPUs this process may use, and physical cores (distinct
    (package, core) pairs in /proc/cpuinfo)."""
    model, cores = None, set()
    phys = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                k, _, v = line.partition(":")
                k, v = k.strip(), v.strip()
                if k == "model name" and model is None:
                    model = v
                elif k == "physical id":
                    phys = v
                elif k == "core id":
                    cores.add((phys, v))
    except OSError:
        pass
    try:
        logical = len(os.sched_getaffinity(0))
    except AttributeError:
        logical = os.cpu_count()
    return {"cpu_model": model, "nproc": logical, "logical_cpus_host": os.cpu_count(),
            "physical_cores": len(cores) or None}


def cpu_baseline(workload: str, entangler: str = "cz"):
    """The oracle's train step on one sample of the workload (its full circuit, fp64).
    With one sample the oracle runs its OpenMP threads over the amplitude loops; the
    whole batch of the workload would take tens of minutes of host time."""
    import hqml_inputs
    import oracle
    x, th, y = hqml_inputs.workload_inputs(workload)
    o = oracle.default()
    threads = o.max_threads()
    t0 = time.perf_counter()
    o.train_step(x[:1], th, y[:1], entangler=1 if entangler == "cnot" else 0)
    dt = time.perf_counter() - t0
    out = {"value": round(1.0 / dt, 5), "unit": "samples/s", "cores": threads, "kind": "oracle",
           "sample": f"1 of the {x.shape[0]} samples of {workload}: its full fp64 forward, loss and "
                     f"gate-by-gate adjoint, {dt:.1f} s with {threads} OpenMP threads over the "
                     f"amplitude loops (threads over samples need a batch of at least {threads})",
           "parallel_over": "amplitudes", "threads": threads}
    out.update(host_cpu())
    return out


def gate_by_gate(w, X, TH, Y, steps, entangler="cz"):
    """The same train step on the comparator without fusion (one kernel per gate,
    gate-by-gate adjoint): one untimed step, then `steps` timed ones."""
    import torch

    import qml_gradients_amd as hq
    B = X.shape[0]
    ctx = hq.Context(w.n_qubits, w.n_layers, B, fusion="gate_by_gate", entangler=entangler)
    info = ctx.plan_info()
    ctx.train_step(X, TH, Y)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(steps):
        ctx.train_step(X, TH, Y)
    ev1.record()
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / steps
    ctx.close()
    return {"value": round(B / (ms / 1e3), 3), "unit": "samples/s", "ms_per_step": round(ms, 2), "steps": steps,
            "gate_kernels_per_step": info["fwd_passes"] + info["bwd_passes"]}


def run_epoch(args, w, ctx, dev, memory):
    """One epoch over the deep model's fixed 1000-sample set: mini-batches of the
    workload's batch size in order (the last one smaller), each a full train step,
    with a plain SGD update of theta on the device between steps.  One untimed
    warm-up step on the first batch precedes the timed epoch."""
    import torch

    import hqml_inputs
    import qml_gradients_amd as hq
    total = 1000
    nb = (total + w.batch - 1) // w.batch
    batches = []
    for i in range(nb):
        x, th, y = hqml_inputs.workload_inputs(w.name, batch_index=i)
        batches.append((torch.from_numpy(x).to(dev), torch.from_numpy(y).to(dev)))
    TH = torch.from_numpy(th).to(dev)
    expz = torch.empty(w.batch, device=dev)
    loss = torch.empty(1, device=dev)
    grad = torch.empty((w.n_layers, w.n_qubits, 3), device=dev)

    def step(X, Y):
        hq.hqml_train_step(ctx.handle, X.shape[0], X.data_ptr(), TH.data_ptr(), Y.data_ptr(),
                           expz.data_ptr(), loss.data_ptr(), grad.data_ptr())
        TH.sub_(args.lr * grad)

    step(*batches[0])
    torch.cuda.synchronize()
    TH.copy_(torch.from_numpy(th).to(dev))
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    losses = torch.empty(nb, device=dev)
    ev0.record(stream)
    for i, (X, Y) in enumerate(batches):
        step(X, Y)
        losses[i] = loss[0]
    ev1.record(stream)
    torch.cuda.synchronize()
    sec = ev0.elapsed_time(ev1) / 1e3
    return {"metric": "seconds per 1000-sample epoch (train steps + SGD update)", "value": round(sec, 3),
            "unit": "s/epoch", "higher_is_better": False, "samples_per_s": round(total / sec, 2),
            "n_gpus": 1, "dtype": "f32", "data": "synthetic 1000-sample set (seeded)",
            "config": {"workload": w.name, "n_qubits": w.n_qubits, "n_layers": w.n_layers,
                       "batch": w.batch, "batches": nb, "state_storage": w.storage,
                       "ckpt_block": w.ckpt_block, "lr": args.lr},
            "memory": memory, "first_last_loss": [float(losses[0]), float(losses[-1])]}


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
    ap.add_argument("--epoch", action="store_true",
                    help="deep model only: time one epoch over its 1000-sample set, applying "
                         "theta -= lr * grad between steps (lr = --lr)")
    ap.add_argument("--lr", type=float, default=0.01)
    ap.add_argument("--compute", choices=["fp32", "fp64"], default="fp32",
                    help="arithmetic type (fp64: the fp64-compute mode, fp64 arrays)")
    ap.add_argument("--storage", choices=["fp32", "bf16", "fp64"], default=None,
                    help="saved-state storage (default: the workload's)")
    ap.add_argument("--ckpt-block", type=int, default=None,
                    help="layers per checkpoint block (default: the workload's; 0 = keep every pass output)")
    ap.add_argument("--gbg-steps", type=int, default=2,
                    help="timed steps of the gate-by-gate comparator on the same workload (0 = skip)")
    ap.add_argument("--entangler", choices=["cz", "cnot"], default="cz",
                    help="the block ending each layer: the CZ chain (the pages' ansatz) or the CNOT chain")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a 1 GiB device-to-device copy 5 times (HBM counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "the library runs on one GPU; --gpus must be 1 (samples shard over "
                                   "GPUs by batch with an all-gather of the per-rank fp64 gradient; "
                                   "that multi-GPU layer is not implemented)"}))
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
    if args.storage is not None or args.compute != "fp32" or args.ckpt_block is not None:
        import dataclasses
        st = args.storage or ("fp64" if args.compute == "fp64" else w.storage)
        ck = w.ckpt_block if args.ckpt_block is None else args.ckpt_block
        w = dataclasses.replace(w, storage=st, ckpt_block=ck)
    f64 = args.compute == "fp64"
    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)
    dt = torch.float64 if f64 else torch.float32
    x, th, y = hqml_inputs.workload_inputs(args.workload)
    X = torch.from_numpy(x).to(dev, dt)
    TH = torch.from_numpy(th).to(dev, dt)
    Y = torch.from_numpy(y).to(dev, dt)
    B = X.shape[0]
    free0 = torch.cuda.mem_get_info(0)[0]
    ctx = hq.Context(w.n_qubits, w.n_layers, B, storage=w.storage, ckpt_block=w.ckpt_block, compute=args.compute,
                     entangler=args.entangler)
    torch.cuda.synchronize()
    memory = {"workspace_bytes": hq.hqml_workspace_bytes(ctx.cfg),
              "device_mem_delta_bytes": int(free0 - torch.cuda.mem_get_info(0)[0])}
    if args.epoch:
        print(json.dumps(run_epoch(args, w, ctx, dev, memory)), flush=True)
        ctx.close()
        return
    ctx.set_overlap(args.overlap)
    plan = json.loads(hq.hqml_describe_plan(ctx.cfg))
    expz = torch.empty(B, device=dev, dtype=dt)
    loss = torch.empty(1, device=dev, dtype=dt)
    grad = torch.empty((w.n_layers, w.n_qubits, 3), device=dev, dtype=dt)
    train = hq.hqml_train_step_f64 if f64 else hq.hqml_train_step

    def step():
        train(ctx.handle, B, X.data_ptr(), TH.data_ptr(), Y.data_ptr(), expz.data_ptr(), loss.data_ptr(),
              grad.data_ptr())

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    ev0.record(stream)
    marks[0].record(stream)
    for i in range(args.steps):
        step()
        marks[i + 1].record(stream)
    ev1.record(stream)
    torch.cuda.synchronize()
    ms_total = ev0.elapsed_time(ev1)
    ms_per_step = ms_total / args.steps
    value = B / (ms_per_step / 1e3)
    per_step = sorted(marks[i].elapsed_time(marks[i + 1]) for i in range(args.steps))

    # Instrumented loop: HIP events around every launch (same workload).
    ctx.set_timing(True)
    ctx.kernel_times(reset=True)
    for _ in range(args.instrumented_steps):
        step()
    ms_k, cnt_k = ctx.kernel_times(reset=True)
    ctx.set_timing(False)
    fwd_b, bwd_b = algorithmic_bytes(plan, B, w.storage, args.compute)
    n_steps = args.instrumented_steps

    bwd_flops = algorithmic_flops_bwd(plan, B, args.compute)
    # the adjoint launches: half-tile general passes (all but the fused last pass and the
    # product-state pass) when the plan has them, else the full-tile kernel
    bwd_kernel = "k_tile_bwdh" if half_tiles(plan, args.compute) else "k_tile_bwd"

    def launches_and_ms(kind):
        if n_steps == 0 or cnt_k[kind] == 0:
            return None, None
        return cnt_k[kind] / n_steps, ms_k[kind] / cnt_k[kind]

    def roof_hbm(kind, total_bytes_per_step, kernel_name):
        launches, avg_ms = launches_and_ms(kind)
        if launches is None:
            return None
        per_launch_bytes = total_bytes_per_step / launches
        achieved = per_launch_bytes / (avg_ms / 1e3) / 1e9
        return {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBPS, 4),
                "traffic": traffic_record(kernel_name, args.workload, args.entangler),
                "kernel": kernel_name, "avg_launch_ms": round(avg_ms, 4),
                "launches_per_step": launches, "algorithmic_bytes_per_launch": int(per_launch_bytes)}

    def roof_alu(kind, flops_per_step, bytes_per_step, kernel_name):
        launches, avg_ms = launches_and_ms(kind)
        if launches is None:
            return None
        per_launch = flops_per_step / launches
        achieved = per_launch / (avg_ms / 1e3) / 1e12
        hbm = bytes_per_step / launches / (avg_ms / 1e3) / 1e9
        return {"bound": "alu", "achieved": round(achieved, 2), "peak": round(ALU_PEAK_TFLOPS, 1),
                "unit": "TFLOP/s", "frac": round(achieved / ALU_PEAK_TFLOPS, 4),
                "traffic": traffic_record(kernel_name, args.workload, args.entangler),
                "kernel": kernel_name, "avg_launch_ms": round(avg_ms, 4), "launches_per_step": launches,
                "algorithmic_flops_per_launch": int(per_launch),
                "algorithmic_bytes_per_launch": int(bytes_per_step / launches),
                "hbm_achieved_GBps": round(hbm, 1), "hbm_frac": round(hbm / HBM_PEAK_GBPS, 4),
                "frac_of_published_fp32_peak": round(achieved / FP32_PUBLISHED_TFLOPS, 4)}

    # dominant kernel against the published HBM peak; its arithmetic rate beside it (the
    # CNOT plan's adjoint passes each rotate one qubit group, so no ALU figure there)
    roof_bwd = roof_hbm(hq.HQML_K_BWD_PASS, bwd_b, bwd_kernel)
    roof_bwd_alu = None if plan.get("cnot") else roof_alu(hq.HQML_K_BWD_PASS, bwd_flops, bwd_b, bwd_kernel)
    if roof_bwd_alu:
        roof_bwd_alu["peak_basis"] = ("non-packed fp32 FMA: 256 CUs x 4 SIMDs x 16 lanes x 2 flops x 2.4 GHz "
                                      "(self-derived; packed FP32 is excluded from the build)")
    roof_fwd = roof_hbm(hq.HQML_K_FWD_PASS, fwd_b, "k_tile_fwd")
    roof_small = None
    if plan.get("small"):   # the whole circuit in one kernel: the state never leaves the chip
        roof_small = roof_alu(hq.HQML_K_SMALL, algorithmic_flops_small(w.n_qubits, w.n_layers, B), 0,
                              small_kernel_name(w.n_qubits, args.entangler, args.compute))
        if roof_small:
            roof_small["peak_basis"] = ("non-packed fp32 FMA: 256 CUs x 4 SIMDs x 16 lanes x 2 flops x 2.4 GHz "
                                        "(self-derived); one workgroup per sample (at 12 qubits up to four, which "
                                        "repeat the forward pass and the un-computation: work the algorithmic "
                                        "count leaves out), so a batch of B keeps at most B (4B) compute units busy")
    step_bytes = fwd_b + bwd_b
    out = {
        "metric": "train samples/sec (fwd+adjoint bwd) 20q HEA 100L; achieved HBM GB/s vs peak",
        "value": round(value, 2),
        "unit": "samples/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "ms_per_step_median": round(per_step[len(per_step) // 2], 4) if per_step else None,
        "ms_per_step_min": round(per_step[0], 4) if per_step else None,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f64" if f64 else "f32",
        "data": "synthetic (seeded x~U[0,pi), theta~U[0,2pi), y in {-1,+1})",
        "config": {"workload": args.workload, "n_qubits": w.n_qubits, "n_layers": w.n_layers,
                   "batch": B, "state_storage": w.storage, "compute": args.compute, "ckpt_block": w.ckpt_block,
                   "entangler": args.entangler,
                   "overlap_chunks": args.overlap, "parallelism": "single GPU"},
        "memory": memory,
        "step_state_bytes": step_bytes,
        "step_hbm_GBps": round(step_bytes / (ms_per_step / 1e3) / 1e9, 1),
        "step_hbm_frac": round(step_bytes / (ms_per_step / 1e3) / 1e9 / HBM_PEAK_GBPS, 4),
        "passes": {"fwd": len(plan["passes"]), "bwd": len(plan["passes"]) + len(plan["stats_only"]),
                   "per_layer": round(len(plan["passes"]) / w.n_layers, 3)},
        "roofline": roof_bwd if roof_bwd else roof_fwd if roof_fwd else roof_small,
        "roofline_alu": roof_bwd_alu,
        "roofline_fwd": roof_fwd,
        "kernel_ms_per_step": {k: round(ms_k[i] / max(n_steps, 1), 3) for i, k in
                               enumerate(["fwd_pass", "bwd_pass", "small", "other"])},
    }
    ctx.close()
    if args.gbg_steps > 0 and w.storage == "fp32" and w.ckpt_block == 0 and not f64:
        g = gate_by_gate(w, X, TH, Y, args.gbg_steps, args.entangler)
        g["fused_speedup"] = round(value / g["value"], 2)
        out["gate_by_gate"] = g
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(args.workload, entangler=args.entangler)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
