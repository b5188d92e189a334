"""Seeded synthetic inputs for the hardware-efficient-ansatz training step.

This module is shared by the CPU oracle's tests, the GPU parity tests and the
benchmark.  It draws random numbers only; it holds none of the simulation's
arithmetic.

Recipe (one NumPy PCG64 stream per array, keyed by ``[seed, stream]``):
  * stream 1: angle-encoding inputs x ~ U[0, pi), shape [B][n]
  * stream 2: circuit parameters theta ~ U[0, 2*pi), shape [L][n][3]
    (last axis: the Rx, Ry, Rz angle of qubit q in layer l)
  * stream 3: labels y in {-1, +1} with probability 1/2 each, shape [B]
Draws are fp64 and rounded to fp32; every consumer sees the same fp32 values.

The named workloads follow the five circuit sizes the method is measured on:
a 4-qubit toy, a 12-qubit/20-layer model, the 20-qubit/100-layer headline
model, the 20-qubit/1000-layer deep model (checkpointed, fp32 and bf16
storage) and a 29-qubit/4-layer wide model.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    n_qubits: int
    n_layers: int
    batch: int
    storage: str = "fp32"      # "fp32" or "bf16" state storage
    ckpt_block: int = 0        # 0: keep every pass output; b>0: checkpoint every b layers
    seed: int = 0


WORKLOADS = {
    "hea4q2l": Workload("hea4q2l", 4, 2, 8, seed=1),
    "hea12q20l": Workload("hea12q20l", 12, 20, 64, seed=2),
    "hea20q100l": Workload("hea20q100l", 20, 100, 32, seed=3),
    "hea20q1000l": Workload("hea20q1000l", 20, 1000, 60, ckpt_block=20, seed=4),
    "hea20q1000l_bf16": Workload("hea20q1000l_bf16", 20, 1000, 85, storage="bf16",
                                 ckpt_block=20, seed=4),
    "hea29q4l": Workload("hea29q4l", 29, 4, 1, ckpt_block=1, seed=5),
}


def _rng(seed: int, stream: int) -> np.random.Generator:
    return np.random.default_rng([int(seed), int(stream)])


def make_x(n: int, B: int, seed: int) -> np.ndarray:
    """Encoding angles, [B][n] fp32, uniform in [0, pi)."""
    return (_rng(seed, 1).random((B, n)) * math.pi).astype(np.float32)


def make_theta(n: int, L: int, seed: int) -> np.ndarray:
    """Circuit parameters, [L][n][3] fp32, uniform in [0, 2 pi)."""
    return (_rng(seed, 2).random((L, n, 3)) * (2.0 * math.pi)).astype(np.float32)


def make_y(B: int, seed: int) -> np.ndarray:
    """Labels, [B] fp32, each -1 or +1 with probability 1/2."""
    bits = _rng(seed, 3).integers(0, 2, size=B)
    return (2.0 * bits - 1.0).astype(np.float32)


def make_inputs(n: int, L: int, B: int, seed: int):
    """(x, theta, y) for an n-qubit, L-layer circuit and a batch of B samples."""
    return make_x(n, B, seed), make_theta(n, L, seed), make_y(B, seed)


def workload_inputs(name: str, batch: int | None = None, batch_index: int = 0):
    """Inputs of a named workload.

    ``batch_index`` selects a later mini-batch of an epoch: the samples are the
    ``batch_index``-th slice of a fixed 1000-sample set (deep model) or of a set
    of exactly one batch (other models).  theta is shared by all batches.
    """
    w = WORKLOADS[name]
    B = w.batch if batch is None else batch
    if w.n_layers >= 1000:
        total = 1000
        xs = make_x(w.n_qubits, total, w.seed)
        ys = make_y(total, w.seed)
        lo = batch_index * B
        hi = min(lo + B, total)
        x, y = xs[lo:hi].copy(), ys[lo:hi].copy()
    else:
        x, y = make_x(w.n_qubits, B, w.seed), make_y(B, w.seed)
    return x, make_theta(w.n_qubits, w.n_layers, w.seed), y
