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
    assert_e_close(e, e_ref, n)
    assert abs(loss - loss_ref) <= 1e-5 * max(1.0, loss_ref)
    assert_grad_close(g, g_ref)
    e2, w, g2 = out["split"]
    g2_ref, _ = oracle.backward(x, th, w.astype(np.float64), mask)
    assert_e_close(e2, e_ref, n)
    assert_grad_close(g2, g2_ref)


@pytest.mark.parametrize("n,L,B,mask", [CASES[0], CASES[4], CASES[6]])
def test_zstring_gate_by_gate(n, L, B, mask):
    say(f"[gpu] Z-string gate-by-gate n={n} mask={mask:#x}")
    (x, th, y), out = _run(n, L, B, mask, seed=600 + n, fusion="gate_by_gate")
    e_ref, loss_ref, g_ref = oracle.train_step(x, th, y, mask)
    e, loss, g = out["train"]
    assert_e_close(e, e_ref, n)
    assert_grad_close(g, g_ref)


@pytest.mark.parametrize("storage,ckpt", [("fp32", 2), ("bf16", 0)])
def test_zstring_checkpoint_and_bf16(storage, ckpt):
    n, L, B, mask = 16, 5, 2, (1 << 14) | (1 << 6) | 0b11
    say(f"[gpu] Z-string {storage} ckpt={ckpt}")
    (x, th, y), out = _run(n, L, B, mask, seed=700, storage=storage, ckpt_block=ckpt)
    e_ref, loss_ref, g_ref = oracle.train_step(x, th, y, mask)
    e, loss, g = out["train"]
    if storage == "fp32":
        assert_e_close(e, e_ref, n)
        assert_grad_close(g, g_ref)
    else:
        assert np.max(np.abs(e - e_ref)) <= 2e-2
        assert_grad_close(g, g_ref, atol=2e-2)
