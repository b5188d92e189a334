"""Z-string observables O = prod_{q in S} Z_q (obs_mask) on the GPU vs the oracle.

The observable enters the last fused pass (E and the adjoint seed lambda = 2 g O psi)
and, through the tile layouts, depends on where the qubits of S sit in a tile:
at lane positions (qubits 0..3), register positions, wave positions or tile-index
bits.  Each case runs the fused train step (last pass fused with the first adjoint
pass), the forward/backward split (seed formed from the saved final state) and the
gate-by-gate comparator.  Tolerances as for Z_0.
"""
import numpy as np
import pytest

import hqml_inputs
import oracle
from gpu_util import assert_e_close, assert_grad_close, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

CASES = [
    (5, 3, 3, 0b10110),
    (5, 2, 2, 0b11111),
    (13, 2, 2, (1 << 12) | (1 << 7) | 1),
    (14, 2, 2, (1 << 13) | (1 << 5) | 1),
    (15, 3, 2, 0b111111111111111),
    (16, 3, 2, (1 << 15) | (1 << 2)),
    (17, 4, 2, (1 << 16) | (1 << 13) | (1 << 9) | (1 << 4)),
    (21, 2, 1, (1 << 20) | (1 << 12) | (1 << 3) | 1),
]


def _run(n, L, B, mask, seed, **kw):
    import qml_gradients_amd as hq
    x, th, y = hqml_inputs.make_inputs(n, L, B, seed)
    X, TH, Y = (torch.from_numpy(a) for a in (x, th, y))
    ctx = hq.Context(n, L, B, obs_mask=mask, **kw)
    e, loss, g = (t.cpu().numpy() for t in ctx.train_step(X, TH, Y))
    out = {"train": (e, float(loss[0]), g)}
    if kw.get("fusion", "fused") == "fused":
        e2 = ctx.forward(X, TH).cpu().numpy()
        w = np.linspace(-1.0, 1.0, B).astype(np.float32)
        g2 = ctx.backward(torch.from_numpy(w)).cpu().numpy()
        out["split"] = (e2, w, g2)
    ctx.close()
    return (x, th, y), out


@pytest.mark.parametrize("n,L,B,mask", CASES)
def test_zstring_fused(n, L, B, mask):
    say(f"[gpu] Z-string n={n} L={L} B={B} mask={mask:#x}")
    (x, th, y), out = _run(n, L, B, mask, seed=500 + n)
    e_ref, loss_ref, g_ref = oracle.train_step(x, th, y, mask)
    e, loss, g = out["train"]
    assert_e_close(e, e_ref, n, L)
    assert abs(loss - loss_ref) <= 1e-5 * max(1.0, loss_ref)
    assert_grad_close(g, g_ref)
    e2, w, g2 = out["split"]
    g2_ref, _ = oracle.backward(x, th, w.astype(np.float64), mask)
    assert_e_close(e2, e_ref, n, L)
    assert_grad_close(g2, g2_ref)


@pytest.mark.parametrize("n,L,B,mask", [CASES[0], CASES[4], CASES[6]])
def test_zstring_gate_by_gate(n, L, B, mask):
    say(f"[gpu] Z-string gate-by-gate n={n} mask={mask:#x}")
    (x, th, y), out = _run(n, L, B, mask, seed=600 + n, fusion="gate_by_gate")
    e_ref, loss_ref, g_ref = oracle.train_step(x, th, y, mask)
    e, loss, g = out["train"]
    assert_e_close(e, e_ref, n, L)
    assert_grad_close(g, g_ref)


@pytest.mark.parametrize("storage,ckpt", [("fp32", 2), ("bf16", 0)])
def test_zstring_checkpoint_and_bf16(storage, ckpt):
    n, L, B, mask = 16, 5, 2, (1 << 14) | (1 << 6) | 0b11
    say(f"[gpu] Z-string {storage} ckpt={ckpt}")
    (x, th, y), out = _run(n, L, B, mask, seed=700, storage=storage, ckpt_block=ckpt)
    e_ref, loss_ref, g_ref = oracle.train_step(x, th, y, mask)
    e, loss, g = out["train"]
    if storage == "fp32":
        assert_e_close(e, e_ref, n, L)
        assert_grad_close(g, g_ref)
    else:
        assert np.max(np.abs(e - e_ref)) <= 2e-2
        assert_grad_close(g, g_ref, atol=2e-2)


# Pauli strings with X / Y factors: (n, L, B, z mask, x mask); Y where both masks hold a qubit.
PAULI_CASES = [
    (3, 2, 3, 0, 0b001),                                  # X_0, whole-circuit kernel
    (5, 3, 2, 0b01010, 0b11000),                          # Z_1 Y_3 X_4
    (12, 3, 2, (1 << 11) | 1, (1 << 11) | (1 << 6)),      # Z_0 X_6 Y_11
    (14, 2, 2, 0, 1),                                     # X_0: lane position
    (14, 3, 2, 1 << 13, 1 << 13),                         # Y_13: a high qubit
    (16, 3, 2, (1 << 9) | (1 << 2), (1 << 15) | (1 << 9) | (1 << 2)),   # Y_2 Y_9 X_15
    (17, 2, 2, 0b10, sum(1 << q for q in range(8, 17))),  # Z_1 and X on the 9 qubits 8..16
    (21, 2, 1, 1 << 20, (1 << 20) | (1 << 12) | (1 << 5) | 1),          # X_0 X_5 X_12 Y_20
]


@pytest.mark.parametrize("n,L,B,zm,xm", PAULI_CASES)
def test_pauli_string_fused(n, L, B, zm, xm):
    import qml_gradients_amd as hq
    say(f"[gpu] Pauli string n={n} L={L} z={zm:#x} x={xm:#x}")
    x, th, y = hqml_inputs.make_inputs(n, L, B, seed=1200 + n)
    X, TH, Y = (torch.from_numpy(a) for a in (x, th, y))
    ctx = hq.Context(n, L, B, obs_mask=zm, obs_x_mask=xm)
    e, loss, g = (t.cpu().numpy() for t in ctx.train_step(X, TH, Y))
    e_ref, loss_ref, g_ref = oracle.train_step(x, th, y, zm, xm)
    assert_e_close(e, e_ref, n, L)
    assert abs(float(loss[0]) - loss_ref) <= 1e-5 * max(1.0, loss_ref)
    assert_grad_close(g, g_ref)
    w = np.linspace(-1.0, 1.0, B).astype(np.float32)
    e2 = ctx.forward(X, TH).cpu().numpy()
    g2 = ctx.backward(torch.from_numpy(w)).cpu().numpy()
    g2_ref, _ = oracle.backward(x, th, w.astype(np.float64), zm, xm)
    assert_e_close(e2, e_ref, n, L)
    assert_grad_close(g2, g2_ref)
    ctx.close()


@pytest.mark.parametrize("mode", ["ckpt", "bf16", "fp64", "gate_by_gate", "overlap"])
def test_pauli_string_modes(mode):
    import qml_gradients_amd as hq
    n, L, B = 16, 4, 3
    zm, xm = (1 << 14) | 0b100, (1 << 14) | (1 << 7) | 1     # X_0 Z_2 X_7 Y_14
    say(f"[gpu] Pauli string mode={mode}")
    x, th, y = hqml_inputs.make_inputs(n, L, B, seed=1300)
    kw = {"ckpt": dict(ckpt_block=2), "bf16": dict(storage="bf16"), "fp64": dict(compute="fp64", storage="fp64"),
          "gate_by_gate": dict(fusion="gate_by_gate"), "overlap": {}}[mode]
    ctx = hq.Context(n, L, B, obs_mask=zm, obs_x_mask=xm, **kw)
    if mode == "overlap":
        ctx.set_overlap(3)
    dt = np.float64 if mode == "fp64" else np.float32
    e, loss, g = (t.cpu().numpy() for t in ctx.train_step(*(torch.from_numpy(a.astype(dt)) for a in (x, th, y))))
    ctx.close()
    e_ref, loss_ref, g_ref = oracle.train_step(x, th, y, zm, xm)
    if mode == "bf16":
        assert np.max(np.abs(e - e_ref)) <= 2e-2
        assert_grad_close(g, g_ref, atol=2e-2)
    elif mode == "fp64":
        assert np.max(np.abs(e - e_ref)) <= 1e-10
        assert np.max(np.abs(g - g_ref)) <= 1e-10
    else:
        assert_e_close(e, e_ref, n, L)
        assert_grad_close(g, g_ref)
