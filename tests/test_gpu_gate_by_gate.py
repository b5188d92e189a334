"""Gate-by-gate comparator (no fusion) vs the CPU oracle and vs the fused path.

The comparator applies every gate as its own kernel and runs the adjoint method
gate by gate, un-computing psi in place; it must give the same E, loss and
gradient as the oracle (same tolerances as the fused path: <Z_0> within 1e-5
relative to max(|E|, 2^(-n/2)), gradients within 1e-4 absolute).
"""

import numpy as np
import pytest

import hqml_inputs
import oracle
from gpu_util import assert_e_close, assert_grad_close, golden_sample, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _ctx(n, L, B, **kw):
    import qml_gradients_amd as hq
    return hq.Context(n, L, B, fusion="gate_by_gate", **kw)


@pytest.mark.parametrize("n,L,B", [(1, 1, 3), (2, 2, 2), (4, 2, 8), (5, 3, 2), (13, 2, 2), (14, 2, 2),
                                   (17, 3, 2), (22, 2, 2)])
def test_gate_by_gate_train_step(n, L, B):
    x, th, y = hqml_inputs.make_inputs(n, L, B, seed=300 + n + L)
    say(f"[gpu] gate-by-gate train_step n={n} L={L} B={B}")
    ctx = _ctx(n, L, B)
    e, loss, g = ctx.train_step(*(torch.from_numpy(a) for a in (x, th, y)))
    e, loss, g = e.cpu().numpy(), float(loss.cpu()[0]), g.cpu().numpy()
    ctx.close()
    e_ref, loss_ref, g_ref = oracle.train_step(x, th, y)
    assert_e_close(e, e_ref, n, L)
    assert abs(loss - loss_ref) <= 1e-5 * max(1.0, loss_ref)
    assert_grad_close(g, g_ref)


def test_gate_by_gate_backward_consumes_the_saved_state():
    import qml_gradients_amd as hq
    n, L, B = 6, 2, 3
    x, th, y = hqml_inputs.make_inputs(n, L, B, seed=7)
    ctx = _ctx(n, L, B)
    X, TH = torch.from_numpy(x), torch.from_numpy(th)
    e = ctx.forward(X, TH).cpu().numpy()
    dl = torch.from_numpy(np.array([0.5, -1.0, 2.0], dtype=np.float32))
    g = ctx.backward(dl).cpu().numpy()
    with pytest.raises(hq.HqmlError) as err:
        ctx.backward(dl)
    assert err.value.status == hq.HQML_ERR_STATE
    ctx.close()
    e_ref = oracle.forward(x, th)
    g_ref, _ = oracle.backward(x, th, dl.numpy().astype(np.float64))
    assert_e_close(e, e_ref, n, L)
    assert_grad_close(g, g_ref)


def test_gate_by_gate_headline_matches_fused_and_oracle():
    """hea20q100l, batch 32: the comparator's train step agrees with the fused path,
    and samples 0 and 31 with the stored oracle values."""
    import qml_gradients_amd as hq
    name = "hea20q100l"
    w = hqml_inputs.WORKLOADS[name]
    x, th, y = hqml_inputs.workload_inputs(name)
    B, n, L = w.batch, w.n_qubits, w.n_layers
    X, TH, Y = (torch.from_numpy(a) for a in (x, th, y))
    say(f"[gpu] {name} gate-by-gate vs fused")
    fused = hq.Context(n, L, B)
    e_f, loss_f, g_f = (t.cpu().numpy() for t in fused.train_step(X, TH, Y))
    fused.close()
    ctx = _ctx(n, L, B)
    e, loss, g = (t.cpu().numpy() for t in ctx.train_step(X, TH, Y))
    # two fp32 results, each within the parity bound of the exact one: their
    # difference is within twice the bound
    assert_e_close(e.astype(np.float64), e_f.astype(np.float64), n, L, scale=2.0)
    assert abs(float(loss[0]) - float(loss_f[0])) <= 1e-5
    assert_grad_close(g, g_f.astype(np.float64), atol=2e-4)
    for b in (0, 31):
        ref = golden_sample(name, b)
        if ref is None:
            pytest.skip("golden values not generated (python tests/golden/make_golden.py full)")
        eb = ctx.forward(X, TH).cpu().numpy().astype(np.float64)
        assert_e_close(eb[b:b + 1], ref[0], n, L)
        oh = np.zeros(B, dtype=np.float32)
        oh[b] = 1.0
        gb = ctx.backward(torch.from_numpy(oh)).cpu().numpy()
        assert_grad_close(gb, ref[1])
    ctx.close()
