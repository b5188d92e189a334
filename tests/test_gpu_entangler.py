"""CNOT-chain entangler on the GPU vs the oracle (entangler=1).

Every layer ends with CNOT(q, q+1), control q, for q = 0..n-2 in that order.  The
whole-circuit kernel (n <= 13) applies the chain as a gather of the amplitude indices in
local memory (round 0 of each step); the tile path (n >= 14) runs one pass per view and layer, the
first reading its input through the chain's index map and its adjoint writing lambda
back through it; the gate-by-gate comparator runs one kernel per CNOT at any width.
Tolerances as for the CZ chain: <O> within 1e-5 relative to max(|E|, 2^(-n/2)),
gradients within 1e-4 absolute (fp32), 2e-2 (bf16 storage), 1e-10 (fp64).
"""
import numpy as np
import pytest

import hqml_inputs
import oracle
from gpu_util import assert_e_close, assert_grad_close, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

# (n, L, B, z mask, x mask); (0, 0) = Z_0
SMALL = [
    (1, 2, 3, 0, 0),
    (2, 1, 3, 0, 0),
    (2, 3, 2, 0b10, 0b01),
    (3, 2, 4, 0b100, 0),
    (4, 3, 3, 0, 0b0011),
    (5, 2, 3, 0b10010, 0b00101),
    (8, 3, 2, 0, 0),
    (9, 2, 2, 1 << 8, 1 << 3),
    (12, 3, 2, 0, 0),
    (13, 2, 2, (1 << 12) | 1, 0),
    (13, 2, 2, 0b1, (1 << 11) | (1 << 6)),
]


def _masks(zm, xm):
    return (1, 0) if (zm | xm) == 0 else (zm, xm)


def _ctx(n, L, B, zm, xm, **kw):
    import qml_gradients_amd as hq
    return hq.Context(n, L, B, obs_mask=zm, obs_x_mask=xm, entangler="cnot", **kw)


@pytest.mark.parametrize("n,L,B,zm,xm", SMALL)
def test_cnot_whole_circuit(n, L, B, zm, xm):
    say(f"[gpu] CNOT whole circuit n={n} L={L} B={B} z={zm:#x} x={xm:#x}")
    x, th, y = hqml_inputs.make_inputs(n, L, B, seed=1600 + 7 * n + L)
    X, TH, Y = (torch.from_numpy(a) for a in (x, th, y))
    ctx = _ctx(n, L, B, zm, xm)
    e, loss, g = (t.cpu().numpy() for t in ctx.train_step(X, TH, Y))
    e2 = ctx.forward(X, TH).cpu().numpy()
    w = np.linspace(-1.0, 1.0, B).astype(np.float32)
    g2 = ctx.backward(torch.from_numpy(w)).cpu().numpy()
    ctx.close()
    oz, ox = _masks(zm, xm)
    e_ref, loss_ref, g_ref = oracle.train_step(x, th, y, oz, ox, entangler=1)
    assert_e_close(e, e_ref, n, L)
    assert abs(float(loss[0]) - loss_ref) <= 1e-5 * max(1.0, loss_ref)
    assert_grad_close(g, g_ref)
    g2_ref, _ = oracle.backward(x, th, w.astype(np.float64), oz, ox, entangler=1)
    assert_e_close(e2, e_ref, n, L)
    assert_grad_close(g2, g2_ref)


def test_cnot_differs_from_cz():
    """The entangler is really switched: the same inputs give different results."""
    import qml_gradients_amd as hq
    n, L, B = 6, 3, 2
    x, th, y = hqml_inputs.make_inputs(n, L, B, seed=1700)
    X, TH = torch.from_numpy(x), torch.from_numpy(th)
    outs = []
    for ent in ("cz", "cnot"):
        ctx = hq.Context(n, L, B, obs_mask=0b100, entangler=ent)
        outs.append(ctx.forward(X, TH).cpu().numpy())
        ctx.close()
    assert_e_close(outs[0], oracle.forward(x, th, 0b100), n, L)
    assert_e_close(outs[1], oracle.forward(x, th, 0b100, entangler=1), n, L)
    assert np.max(np.abs(outs[0] - outs[1])) > 1e-3


def test_cnot_whole_circuit_fp64():
    n, L, B, zm, xm = 7, 3, 2, 0b0100001, 0b0000110
    say(f"[gpu] CNOT whole circuit fp64 n={n}")
    x, th, y = hqml_inputs.make_inputs(n, L, B, seed=1800)
    ctx = _ctx(n, L, B, zm, xm, compute="fp64", storage="fp64")
    e, loss, g = (t.cpu().numpy() for t in ctx.train_step(*(torch.from_numpy(a).double() for a in (x, th, y))))
    ctx.close()
    e_ref, loss_ref, g_ref = oracle.train_step(x, th, y, zm, xm, entangler=1)
    assert np.max(np.abs(e - e_ref)) < 1e-12
    assert abs(float(loss[0]) - loss_ref) < 1e-12
    assert np.max(np.abs(g - g_ref)) < 1e-10


def test_cnot_hea12q20l_full():
    """The 12-qubit, 20-layer, batch-64 shape with the CNOT chain, every sample."""
    w = hqml_inputs.WORKLOADS["hea12q20l"]
    x, th, y = hqml_inputs.workload_inputs("hea12q20l")
    say("[gpu] CNOT hea12q20l")
    ctx = _ctx(w.n_qubits, w.n_layers, x.shape[0], 0, 0)
    e, loss, g = (t.cpu().numpy() for t in ctx.train_step(*(torch.from_numpy(a) for a in (x, th, y))))
    ctx.close()
    e_ref, loss_ref, g_ref = oracle.train_step(x, th, y, entangler=1)
    assert_e_close(e, e_ref, w.n_qubits, w.n_layers)
    assert abs(float(loss[0]) - loss_ref) <= 1e-5 * max(1.0, loss_ref)
    assert_grad_close(g, g_ref)



@pytest.mark.parametrize("L", [1, 4])
@pytest.mark.parametrize("n", list(range(1, 14)))
def test_cnot_whole_circuit_every_width(n, L):
    """Every width 1..13: the gather of round 0 covers qubits 0..min(n, 4)-1 and its
    high part the rest (none for n <= 4; two groups per thread at n = 13); ragged batch
    on one context; an X/Y string on odd widths."""
    zm, xm = (1, 0) if n % 2 == 0 or n == 1 else ((1 << (n - 1)) | 1, (1 << (n - 1)) | (1 << (n // 2)))
    maxB = 3
    x, th, y = hqml_inputs.make_inputs(n, L, maxB, seed=3500 + 13 * n + L)
    say(f"[gpu] CNOT whole circuit every width n={n} L={L}")
    ctx = _ctx(n, L, maxB, zm, xm)
    for B in (maxB, 2):
        X, TH, Y = (torch.from_numpy(a) for a in (x[:B], th, y[:B]))
        e, loss, g = (t.cpu().numpy() for t in ctx.train_step(X, TH, Y))
        e_ref, loss_ref, g_ref = oracle.train_step(x[:B], th, y[:B], zm, xm, entangler=1)
        assert_e_close(e, e_ref, n, L)
        assert abs(float(loss[0]) - loss_ref) <= 1e-5 * max(1.0, loss_ref)
        assert_grad_close(g, g_ref)
    ctx.close()

@pytest.mark.parametrize("n,L,B,zm,xm", [(2, 2, 3, 0, 0), (5, 2, 2, 0b10010, 0b00101), (13, 2, 2, 0, 0),
                                         (14, 2, 2, 0, 0), (17, 2, 2, 1 << 16, 1 << 2)])
def test_cnot_gate_by_gate(n, L, B, zm, xm):
    say(f"[gpu] CNOT gate-by-gate n={n} L={L}")
    x, th, y = hqml_inputs.make_inputs(n, L, B, seed=1900 + n)
    ctx = _ctx(n, L, B, zm, xm, fusion="gate_by_gate")
    e, loss, g = (t.cpu().numpy() for t in ctx.train_step(*(torch.from_numpy(a) for a in (x, th, y))))
    ctx.close()
    oz, ox = _masks(zm, xm)
    e_ref, loss_ref, g_ref = oracle.train_step(x, th, y, oz, ox, entangler=1)
    assert_e_close(e, e_ref, n, L)
    assert abs(float(loss[0]) - loss_ref) <= 1e-5 * max(1.0, loss_ref)
    assert_grad_close(g, g_ref)


TILE = [
    (14, 1, 2, 0),
    (14, 2, 2, 0),
    (14, 3, 3, 0b10000000000100),
    (15, 4, 2, 0),
    (16, 3, 2, (1 << 15) | (1 << 6)),
    (17, 2, 2, 0),
    (21, 2, 1, (1 << 20) | 1),
]


def _tile_run(n, L, B, zm, seed, **kw):
    x, th, y = hqml_inputs.make_inputs(n, L, B, seed=seed)
    X, TH, Y = (torch.from_numpy(a) for a in (x, th, y))
    ctx = _ctx(n, L, B, zm, 0, **kw)
    e, loss, g = (t.cpu().numpy() for t in ctx.train_step(X, TH, Y))
    e2 = ctx.forward(X, TH).cpu().numpy()
    w = np.linspace(-1.0, 1.0, B).astype(np.float32)
    g2 = ctx.backward(torch.from_numpy(w)).cpu().numpy()
    ctx.close()
    return (x, th, y, w), (e, float(loss[0]), g, e2, g2)


@pytest.mark.parametrize("n,L,B,zm", TILE)
def test_cnot_tile_path(n, L, B, zm):
    say(f"[gpu] CNOT tile path n={n} L={L} B={B} z={zm:#x}")
    (x, th, y, w), (e, loss, g, e2, g2) = _tile_run(n, L, B, zm, seed=2000 + 3 * n + L)
    oz = zm or 1
    e_ref, loss_ref, g_ref = oracle.train_step(x, th, y, oz, entangler=1)
    assert_e_close(e, e_ref, n, L)
    assert abs(loss - loss_ref) <= 1e-5 * max(1.0, loss_ref)
    assert_grad_close(g, g_ref)
    g2_ref, _ = oracle.backward(x, th, w.astype(np.float64), oz, entangler=1)
    assert_e_close(e2, e_ref, n, L)
    assert_grad_close(g2, g2_ref)


# Pauli strings with X / Y factors on the tile path: the passes measure the string
# conjugated by the last chain (X on q -> X on q and q+1), with its sign
TILE_PAULI = [
    (14, 1, 2, 0b1, 0b110),
    (14, 2, 2, 0b1, 0b10),
    (15, 3, 2, 1 << 5, (1 << 5) | 1),
    (16, 2, 2, 1 << 15, (1 << 15) | (1 << 3)),
    (17, 3, 1, 0, (1 << 12) | (1 << 2)),
    (16, 3, 2, 0b11, 0b11),
]


@pytest.mark.parametrize("n,L,B,zm,xm", TILE_PAULI)
def test_cnot_tile_pauli_strings(n, L, B, zm, xm):
    say(f"[gpu] CNOT tile Pauli n={n} L={L} z={zm:#x} x={xm:#x}")
    x, th, y = hqml_inputs.make_inputs(n, L, B, seed=2050 + n + L)
    X, TH, Y = (torch.from_numpy(a) for a in (x, th, y))
    ctx = _ctx(n, L, B, zm, xm)
    e, loss, g = (t.cpu().numpy() for t in ctx.train_step(X, TH, Y))
    e2 = ctx.forward(X, TH).cpu().numpy()
    w = np.linspace(-1.0, 1.0, B).astype(np.float32)
    g2 = ctx.backward(torch.from_numpy(w)).cpu().numpy()
    ctx.close()
    e_ref, loss_ref, g_ref = oracle.train_step(x, th, y, zm, xm, entangler=1)
    assert_e_close(e, e_ref, n, L)
    assert abs(float(loss[0]) - loss_ref) <= 1e-5 * max(1.0, loss_ref)
    assert_grad_close(g, g_ref)
    g2_ref, _ = oracle.backward(x, th, w.astype(np.float64), zm, xm, entangler=1)
    assert_e_close(e2, e_ref, n, L)
    assert_grad_close(g2, g2_ref)


def test_cnot_tile_checkpoints_and_chunks_are_bitwise_identical():
    """Checkpoint blocks (recomputed passes, including the chain reads) and batch chunks
    change nothing in the CNOT plan's results."""
    import qml_gradients_amd as hq
    n, L, B = 15, 5, 4
    x, th, y = hqml_inputs.make_inputs(n, L, B, seed=2100)
    X, TH, Y = (torch.from_numpy(a) for a in (x, th, y))
    outs = []
    for ckpt, chunks in ((0, 1), (1, 1), (2, 1), (0, 3)):
        say(f"[gpu] CNOT tile ckpt={ckpt} chunks={chunks}")
        ctx = hq.Context(n, L, B, ckpt_block=ckpt, entangler="cnot")
        ctx.set_overlap(chunks)
        outs.append([t.cpu().numpy() for t in ctx.train_step(X, TH, Y)])
        ctx.close()
    for o in outs[1:]:
        for a, b in zip(outs[0], o):
            assert np.array_equal(a, b)
    e_ref, _, g_ref = oracle.train_step(x, th, y, entangler=1)
    assert_e_close(outs[0][0], e_ref, n, L)
    assert_grad_close(outs[0][2], g_ref)


def test_cnot_tile_pauli_checkpoints_and_ragged_batch():
    """X/Y observable with checkpoint blocks, and a smaller batch on the same context:
    bitwise equal to the stored-output run, and equal to the oracle."""
    import qml_gradients_amd as hq
    n, L, maxB, zm, xm = 15, 4, 4, 0b1, (1 << 9) | 0b10
    x, th, y = hqml_inputs.make_inputs(n, L, maxB, seed=2150)
    outs = []
    for ckpt in (0, 1):
        say(f"[gpu] CNOT tile Pauli ckpt={ckpt}")
        ctx = hq.Context(n, L, maxB, ckpt_block=ckpt, obs_mask=zm, obs_x_mask=xm, entangler="cnot")
        full = [t.cpu().numpy() for t in ctx.train_step(*(torch.from_numpy(a) for a in (x, th, y)))]
        part = [t.cpu().numpy() for t in ctx.train_step(*(torch.from_numpy(a) for a in (x[:3], th, y[:3])))]
        ctx.close()
        outs.append((full, part))
    for a, b in zip(outs[0][0] + outs[0][1], outs[1][0] + outs[1][1]):
        assert np.array_equal(a, b)
    e_ref, _, g_ref = oracle.train_step(x[:3], th, y[:3], zm, xm, entangler=1)
    assert_e_close(outs[0][1][0], e_ref, n, L)
    assert_grad_close(outs[0][1][2], g_ref)


def test_cnot_tile_pauli_batch_chunks_20_qubits():
    """X/Y observable, checkpoint every layer and two batch chunks (the default with
    checkpoints at 20 qubits, batch 4): every chunk's adjoint sweep must start from the
    lambda buffer its observable pass wrote, although the previous chunk's sweep swapped
    the two buffers an odd number of times (L = 2).  Bitwise equal to one chunk, and
    equal to the oracle."""
    import qml_gradients_amd as hq
    n, L, B, zm, xm = 20, 2, 4, 0b1, (1 << 9) | 0b10
    x, th, y = hqml_inputs.make_inputs(n, L, B, seed=2160)
    ctx = hq.Context(n, L, B, ckpt_block=1, obs_mask=zm, obs_x_mask=xm, entangler="cnot")
    outs = []
    for chunks in (2, 1):
        say(f"[gpu] CNOT tile Pauli 20 qubits, {chunks} chunk(s)")
        ctx.set_overlap(chunks)
        outs.append([t.cpu().numpy() for t in ctx.train_step(*(torch.from_numpy(a) for a in (x, th, y)))])
    ctx.close()
    for other in outs[1:]:
        for a, b in zip(outs[0], other):
            assert np.array_equal(a, b)
    e_ref, loss_ref, g_ref = oracle.train_step(x, th, y, zm, xm, entangler=1)
    assert_e_close(outs[0][0], e_ref, n, L)
    assert abs(float(outs[0][1][0]) - loss_ref) <= 1e-5 * max(1.0, loss_ref)
    assert_grad_close(outs[0][2], g_ref)


def test_cnot_tile_bf16_storage():
    n, L, B = 16, 4, 2
    say("[gpu] CNOT tile bf16")
    (x, th, y, w), (e, loss, g, e2, g2) = _tile_run(n, L, B, 0, seed=2200, storage="bf16")
    e_ref, _, g_ref = oracle.train_step(x, th, y, entangler=1)
    assert np.max(np.abs(e - e_ref)) < 2e-2
    assert_grad_close(g, g_ref, atol=2e-2)


def test_cnot_tile_fp64():
    import qml_gradients_amd as hq
    n, L, B = 14, 3, 2
    say("[gpu] CNOT tile fp64")
    x, th, y = hqml_inputs.make_inputs(n, L, B, seed=2300)
    ctx = hq.Context(n, L, B, obs_mask=0b100, compute="fp64", storage="fp64", entangler="cnot")
    e, loss, g = (t.cpu().numpy() for t in ctx.train_step(*(torch.from_numpy(a).double() for a in (x, th, y))))
    ctx.close()
    e_ref, loss_ref, g_ref = oracle.train_step(x, th, y, 0b100, entangler=1)
    assert np.max(np.abs(e - e_ref)) < 1e-12
    assert np.max(np.abs(g - g_ref)) < 1e-10


def test_cnot_tile_20_qubits_sampled():
    """20 qubits, 12 layers, batch 4: samples 0 and 3 against the oracle one by one."""
    import qml_gradients_amd as hq
    n, L, B = 20, 12, 4
    x, th, y = hqml_inputs.make_inputs(n, L, B, seed=2400)
    X, TH = torch.from_numpy(x), torch.from_numpy(th)
    say("[gpu] CNOT tile 20 qubits")
    ctx = hq.Context(n, L, B, entangler="cnot")
    e = ctx.forward(X, TH).cpu().numpy()
    for b in (0, 3):
        oh = np.zeros(B, dtype=np.float32)
        oh[b] = 1.0
        g = ctx.backward(torch.from_numpy(oh)).cpu().numpy()
        g_ref, e_ref = oracle.backward(x[b:b + 1], th, np.ones(1), entangler=1)
        assert_e_close(e[b:b + 1], e_ref, n, L)
        assert_grad_close(g, g_ref)
    ctx.close()


def test_cnot_tile_29_qubits_light_cone():
    """hea29q4l with the CNOT chain (four views, 13 passes, per-layer checkpoints, 4 GiB
    state): Z_0 passes each chain unchanged and an X on q widens to q, q+1 per earlier
    chain, so with 4 layers E and the gradient equal those of the 4-qubit circuit on the
    same angles, and every other derivative is 0."""
    import qml_gradients_amd as hq
    name = "hea29q4l"
    w = hqml_inputs.WORKLOADS[name]
    x, th, y = hqml_inputs.workload_inputs(name)
    n, L = w.n_qubits, w.n_layers
    e_ref, loss_ref, g4 = oracle.train_step(x[:, :L], th[:, :L, :], y, entangler=1)
    g_ref = np.zeros((L, n, 3))
    g_ref[:, :L, :] = g4
    say(f"[gpu] {name} CNOT")
    ctx = hq.Context(n, L, w.batch, ckpt_block=w.ckpt_block, entangler="cnot")
    assert ctx.plan_info()["fwd_passes"] == 1 + (L - 1) * 4
    e, loss, g = (t.cpu().numpy() for t in ctx.train_step(*(torch.from_numpy(a) for a in (x, th, y))))
    ctx.close()
    assert_e_close(e, e_ref, n, L)
    assert_grad_close(g, g_ref)
