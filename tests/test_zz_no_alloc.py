"""The allocation-free training step (hqml_train_step_noalloc) against the context's
hqml_train_step on the same inputs: two calls in a row, the second with a smaller
batch, each bitwise equal to the context's results (same kernels, same order) and
within the parity bounds of the oracle; then the host-side refusals."""
import numpy as np
import pytest

import hqml_inputs
import oracle
from gpu_util import assert_e_close, assert_grad_close, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _noalloc(hq, cfg, x, th, y):
    dev = torch.device("cuda", 0)
    X, TH, Y = (torch.from_numpy(a).to(dev) for a in (x, th, y))
    B = x.shape[0]
    e = torch.empty(B, device=dev)
    loss = torch.empty(1, device=dev)
    g = torch.empty(th.shape, device=dev)
    hq.hqml_train_step_noalloc(cfg, B, X.data_ptr(), TH.data_ptr(), Y.data_ptr(), e.data_ptr(), loss.data_ptr(),
                               g.data_ptr())
    torch.cuda.synchronize()
    return e.cpu().numpy(), loss.cpu().numpy(), g.cpu().numpy()


@pytest.mark.parametrize("entangler", ["cz", "cnot"])
def test_noalloc_matches_train_step_twice(entangler):
    import qml_gradients_amd as hq
    w = hqml_inputs.WORKLOADS["hea12q20l"]
    n, L, B = w.n_qubits, w.n_layers, w.batch
    x, th, y = hqml_inputs.workload_inputs("hea12q20l")
    cfg = hq.make_config(n, L, B, entangler=entangler)
    ctx = hq.Context(n, L, B, entangler=entangler)
    ent = 1 if entangler == "cnot" else 0
    for Bc in (B, 13):   # the second call has a smaller batch
        say(f"[gpu] noalloc train step, {entangler}, batch {Bc}")
        xs, ys = x[:Bc], y[:Bc]
        got = _noalloc(hq, cfg, xs, th, ys)
        ref = [t.cpu().numpy() for t in ctx.train_step(*(torch.from_numpy(a) for a in (xs, th, ys)))]
        for a, b in zip(got, ref):
            assert np.array_equal(a, b)
        e_ref, loss_ref, g_ref = oracle.train_step(xs, th, ys, entangler=ent)
        assert_e_close(got[0], e_ref, n, L)
        assert abs(float(got[1][0]) - loss_ref) <= 1e-5 * max(1.0, loss_ref)
        assert_grad_close(got[2], g_ref)
    ctx.close()


def test_noalloc_refusals():
    import qml_gradients_amd as hq
    dev = torch.device("cuda", 0)
    buf = torch.zeros(1 << 16, device=dev)
    p = buf.data_ptr()
    say("[gpu] noalloc refusals")
    # a batch whose per-sample statistics exceed the scratch buffer
    with pytest.raises(hq.HqmlError) as e:
        hq.hqml_train_step_noalloc(hq.make_config(12, 1000, 200), 200, p, p, p, p, p, p)
    assert e.value.status == hq.HQML_ERR_ARG and "HQML_NOALLOC_SCRATCH_BYTES" in str(e.value)
    # tile-path sizes and the gate-by-gate comparator are not covered
    with pytest.raises(hq.HqmlError) as e:
        hq.hqml_train_step_noalloc(hq.make_config(14, 2, 1), 1, p, p, p, p, p, p)
    assert e.value.status == hq.HQML_ERR_UNSUPPORTED
    with pytest.raises(hq.HqmlError) as e:
        hq.hqml_train_step_noalloc(hq.make_config(6, 2, 1, fusion="gate_by_gate"), 1, p, p, p, p, p, p)
    assert e.value.status == hq.HQML_ERR_UNSUPPORTED
    # batch outside 1..max_batch, a NULL array, pageable host memory
    with pytest.raises(hq.HqmlError) as e:
        hq.hqml_train_step_noalloc(hq.make_config(6, 2, 4), 5, p, p, p, p, p, p)
    assert e.value.status == hq.HQML_ERR_ARG
    with pytest.raises(hq.HqmlError) as e:
        hq.hqml_train_step_noalloc(hq.make_config(6, 2, 4), 4, p, p, 0, p, p, p)
    assert e.value.status == hq.HQML_ERR_ARG
    host = np.zeros(64, dtype=np.float32)
    with pytest.raises(hq.HqmlError) as e:
        hq.hqml_train_step_noalloc(hq.make_config(6, 2, 4), 4, host.ctypes.data, p, p, p, p, p)
    assert e.value.status == hq.HQML_ERR_ARG
    # the entry point still works after the refusals
    x, th, y = hqml_inputs.make_inputs(6, 2, 4, seed=77)
    got = _noalloc(hq, hq.make_config(6, 2, 4), x, th, y)
    e_ref, _, g_ref = oracle.train_step(x, th, y)
    assert_e_close(got[0], e_ref, 6, 2)
    assert_grad_close(got[2], g_ref)
