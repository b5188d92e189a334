"""GPU parity at the full workload sizes, checkpointing, bf16 storage, 29 qubits.

Full-size references are single samples computed by the CPU oracle and stored
under tests/golden/ by ``tests/golden/make_golden.py full`` (it calls only the
oracle).  The GPU runs the whole batch in the configuration the benchmark times;
per-sample gradients are read back with a one-hot dL/dE, which the backward
pass accepts for any upstream derivative.
"""
import os

import numpy as np
import pytest

import hqml_inputs
import oracle
from gpu_util import assert_e_close, assert_grad_close, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    path = os.path.join(GOLDEN, name)
    if not os.path.exists(path):
        pytest.skip(f"{name} not generated (python tests/golden/make_golden.py full)")
    return np.load(path)


def _ctx(n, L, B, **kw):
    import qml_gradients_amd as hq
    return hq.Context(n, L, B, **kw)


def _one_hot(B, b):
    w = np.zeros(B, dtype=np.float32)
    w[b] = 1.0
    return torch.from_numpy(w)


def test_headline_workload_sampled_parity():
    """hea20q100l, batch 32, every pass output kept: samples 0 and 31 vs the oracle;
    train_step's gradient vs forward + backward with dL/dE = 2 (E - y) / B."""
    name = "hea20q100l"
    w = hqml_inputs.WORKLOADS[name]
    x, th, y = hqml_inputs.workload_inputs(name)
    B, n, L = w.batch, w.n_qubits, w.n_layers
    say(f"[gpu] {name} sampled parity")
    ctx = _ctx(n, L, B)
    X, TH, Y = (torch.from_numpy(a) for a in (x, th, y))
    e = ctx.forward(X, TH).cpu().numpy().astype(np.float64)
    for b in (0, 31):
        ref = _golden(f"{name}_b0_s{b}.npz")
        assert_e_close(e[b:b + 1], ref["expz"], n, L)
        g = ctx.backward(_one_hot(B, b)).cpu().numpy()
        assert_grad_close(g, ref["grad"])
    e2, loss, g_ts = ctx.train_step(X, TH, Y)
    e2 = e2.cpu().numpy().astype(np.float64)
    assert np.max(np.abs(e2 - e)) <= 1e-6
    dl = (2.0 * (e2 - y) / B).astype(np.float32)
    ctx.forward(X, TH)
    g_fb = ctx.backward(torch.from_numpy(dl)).cpu().numpy()
    assert np.max(np.abs(g_ts.cpu().numpy() - g_fb)) <= 1e-6
    assert abs(float(loss.cpu()[0]) - np.mean((e2 - y) ** 2)) <= 1e-6
    ctx.close()


def test_deep_checkpointed_workload_sampled_parity():
    """hea20q1000l, batch 60, checkpoint every 20 layers: sample 0 of the first batch."""
    name = "hea20q1000l"
    w = hqml_inputs.WORKLOADS[name]
    x, th, _ = hqml_inputs.workload_inputs(name)
    ref = _golden(f"{name}_b0_s0.npz")
    say(f"[gpu] {name} checkpointed sampled parity")
    ctx = _ctx(w.n_qubits, w.n_layers, w.batch, ckpt_block=w.ckpt_block)
    e = ctx.forward(torch.from_numpy(x), torch.from_numpy(th)).cpu().numpy().astype(np.float64)
    assert_e_close(e[:1], ref["expz"], w.n_qubits, w.n_layers)
    g = ctx.backward(_one_hot(w.batch, 0)).cpu().numpy()
    assert_grad_close(g, ref["grad"])
    ctx.close()


@pytest.mark.parametrize("storage", ["fp32", "bf16"])
def test_checkpointing_is_bitwise_identical(storage):
    """Recomputing blocks from checkpoints reproduces the kept-state run bit for bit."""
    n, L, B = 16, 12, 3
    x, th, y = hqml_inputs.make_inputs(n, L, B, seed=61)
    X, TH, Y = (torch.from_numpy(a) for a in (x, th, y))
    outs = []
    for ck in (0, 1, 3, 5, 11, 40):
        say(f"[gpu] checkpoint block {ck} storage {storage}")
        ctx = _ctx(n, L, B, storage=storage, ckpt_block=ck)
        e, loss, g = ctx.train_step(X, TH, Y)
        outs.append((e.cpu().numpy(), loss.cpu().numpy(), g.cpu().numpy()))
        ctx.close()
    for o in outs[1:]:
        for a, b in zip(outs[0], o):
            assert np.array_equal(a, b)


def test_bf16_storage_parity_small():
    n, L, B = 16, 6, 3
    x, th, y = hqml_inputs.make_inputs(n, L, B, seed=71)
    say("[gpu] bf16 storage n=16")
    ctx = _ctx(n, L, B, storage="bf16")
    e, loss, g = ctx.train_step(*(torch.from_numpy(a) for a in (x, th, y)))
    e_ref, loss_ref, g_ref = oracle.train_step(x, th, y)
    assert np.max(np.abs(e.cpu().numpy() - e_ref)) <= 2e-2
    assert_grad_close(g.cpu().numpy(), g_ref, atol=2e-2)
    ctx.close()


def test_bf16_deep_workload_sampled_parity():
    """hea20q1000l in bf16 storage (batch 85, checkpoint every 20 layers): sample 0."""
    name = "hea20q1000l_bf16"
    w = hqml_inputs.WORKLOADS[name]
    x, th, _ = hqml_inputs.workload_inputs(name)
    ref = _golden("hea20q1000l_b0_s0.npz")      # same circuit and first sample
    say(f"[gpu] {name} sampled parity")
    ctx = _ctx(w.n_qubits, w.n_layers, w.batch, storage="bf16", ckpt_block=w.ckpt_block)
    e = ctx.forward(torch.from_numpy(x), torch.from_numpy(th)).cpu().numpy().astype(np.float64)
    assert abs(e[0] - ref["expz"][0]) <= 2e-2
    g = ctx.backward(_one_hot(w.batch, 0)).cpu().numpy()
    assert_grad_close(g, ref["grad"], atol=2e-2)
    ctx.close()


@pytest.mark.parametrize("storage", ["fp32", "bf16"])
def test_wide_29_qubits_light_cone(storage):
    """hea29q4l (one sample, 4 GiB fp32 state, per-layer checkpoints).  With 4 layers
    <Z_0> only sees qubits 0..3, so E and the gradient equal those of the 4-qubit
    circuit on the same angles, and every other derivative is 0."""
    name = "hea29q4l"
    w = hqml_inputs.WORKLOADS[name]
    x, th, y = hqml_inputs.workload_inputs(name)
    n, L = w.n_qubits, w.n_layers
    e_ref, loss_ref, g4 = oracle.train_step(x[:, :L], th[:, :L, :], y)
    g_ref = np.zeros((L, n, 3))
    g_ref[:, :L, :] = g4
    say(f"[gpu] {name} {storage}")
    ctx = _ctx(n, L, w.batch, storage=storage, ckpt_block=w.ckpt_block)
    e, loss, g = ctx.train_step(*(torch.from_numpy(a) for a in (x, th, y)))
    e, g = e.cpu().numpy(), g.cpu().numpy()
    if storage == "fp32":
        assert_e_close(e, e_ref, n, L)
        assert_grad_close(g, g_ref)
    else:
        assert np.max(np.abs(e - e_ref)) <= 2e-2
        assert_grad_close(g, g_ref, atol=2e-2)
    ctx.close()


def test_forward_without_save_then_backward_is_an_error():
    import qml_gradients_amd as hq
    n, L, B = 14, 2, 2
    x, th, _ = hqml_inputs.make_inputs(n, L, B, seed=3)
    ctx = _ctx(n, L, B)
    ctx.forward(torch.from_numpy(x), torch.from_numpy(th), save_for_backward=False)
    with pytest.raises(hq.HqmlError) as e:
        ctx.backward(torch.ones(B))
    assert e.value.status == hq.HQML_ERR_STATE
    ctx.close()


@pytest.mark.parametrize("storage,ckpt", [("fp32", 0), ("fp32", 3), ("bf16", 2)])
def test_chunked_overlap_is_bitwise_identical(storage, ckpt):
    """Pipelining the batch in chunks over two streams gives the same bits."""
    n, L, B = 15, 7, 7
    x, th, y = hqml_inputs.make_inputs(n, L, B, seed=91)
    X, TH, Y = (torch.from_numpy(a) for a in (x, th, y))
    ctx = _ctx(n, L, B, storage=storage, ckpt_block=ckpt)
    outs = []
    for chunks in (1, 2, 3, 4, 7):
        say(f"[gpu] overlap chunks={chunks} storage={storage} ckpt={ckpt}")
        ctx.set_overlap(chunks)
        e, loss, g = ctx.train_step(X, TH, Y)
        torch.cuda.synchronize()
        outs.append((e.cpu().numpy(), loss.cpu().numpy(), g.cpu().numpy()))
    for o in outs[1:]:
        for a, b in zip(outs[0], o):
            assert np.array_equal(a, b)
    e_ref, loss_ref, g_ref = oracle.train_step(x, th, y)
    if storage == "fp32":
        assert_e_close(outs[0][0], e_ref, n, L)
        assert_grad_close(outs[0][2], g_ref)
    ctx.close()


@pytest.mark.parametrize("ckpt", [0, 2])
def test_ragged_batches_on_one_context(ckpt):
    """A context sized for 7 samples trains on batches of 7, 5 and 2 (the last batch
    of an epoch is smaller); each step matches the oracle on exactly its samples."""
    n, L, maxB = 16, 5, 7
    x, th, y = hqml_inputs.make_inputs(n, L, maxB, seed=123)
    ctx = _ctx(n, L, maxB, ckpt_block=ckpt)
    for B in (7, 5, 2):
        say(f"[gpu] ragged batch B={B} of {maxB} ckpt={ckpt}")
        out = ctx.train_step(torch.from_numpy(x[:B]), torch.from_numpy(th), torch.from_numpy(y[:B]))
        e, loss, g = (t.cpu().numpy() for t in out)
        e_ref, loss_ref, g_ref = oracle.train_step(x[:B], th, y[:B])
        assert_e_close(e, e_ref, n, L)
        assert abs(float(loss[0]) - loss_ref) <= 1e-5 * max(1.0, loss_ref)
        assert_grad_close(g, g_ref)
    ctx.close()


def test_wide_29_qubits_fp64_light_cone():
    """hea29q4l in full fp64 (8 GiB states, per-layer checkpoints): E and every
    derivative equal the 4-qubit oracle's within 1e-10."""
    name = "hea29q4l"
    w = hqml_inputs.WORKLOADS[name]
    x, th, y = hqml_inputs.workload_inputs(name)
    n, L = w.n_qubits, w.n_layers
    e_ref, loss_ref, g4 = oracle.train_step(x[:, :L], th[:, :L, :], y)
    g_ref = np.zeros((L, n, 3))
    g_ref[:, :L, :] = g4
    say(f"[gpu] {name} fp64")
    ctx = _ctx(n, L, w.batch, storage="fp64", compute="fp64", ckpt_block=w.ckpt_block)
    e, loss, g = (t.cpu().numpy() for t in ctx.train_step(*(torch.from_numpy(a.astype(np.float64))
                                                            for a in (x, th, y))))
    assert np.max(np.abs(e - e_ref)) <= 1e-10
    assert np.max(np.abs(g - g_ref)) <= 1e-10
    ctx.close()
