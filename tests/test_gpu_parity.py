"""GPU path vs the CPU oracle, element by element, through the C ABI.

Tolerances (fp32 state storage): <Z_0> within 1e-5 relative to
max(|E_ref|, 2^(-n/2)); every dL/dtheta within 1e-4 absolute.  bf16 state
storage: 2e-2 absolute on both.  Inputs come from ``hqml_inputs`` (seeded).
"""
import numpy as np
import pytest

import hqml_inputs
import oracle
from gpu_util import assert_e_close, assert_grad_close, assert_grad_rel, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _ctx(n, L, B, **kw):
    import qml_gradients_amd as hq
    return hq.Context(n, L, B, **kw)


def _run_train(n, L, B, seed, **kw):
    x, th, y = hqml_inputs.make_inputs(n, L, B, seed)
    say(f"[gpu] train_step n={n} L={L} B={B} seed={seed} {kw}")
    ctx = _ctx(n, L, B, **kw)
    e, loss, g = ctx.train_step(torch.from_numpy(x), torch.from_numpy(th), torch.from_numpy(y))
    torch.cuda.synchronize()
    out = (e.cpu().numpy(), float(loss.cpu()[0]), g.cpu().numpy())
    ctx.close()
    return (x, th, y), out


@pytest.mark.parametrize("n,L,B", [(1, 1, 3), (2, 1, 2), (4, 2, 8), (5, 3, 5), (7, 2, 3), (13, 2, 2)])
def test_small_path_train_step(n, L, B):
    (x, th, y), (e, loss, g) = _run_train(n, L, B, seed=10 + n)
    e_ref, loss_ref, g_ref = oracle.train_step(x, th, y)
    assert_e_close(e, e_ref, n, L)
    assert abs(loss - loss_ref) <= 1e-5 * max(1.0, loss_ref)
    assert_grad_close(g, g_ref)


@pytest.mark.parametrize("n,L,B", [(14, 1, 2), (14, 2, 2), (14, 3, 3), (15, 4, 2), (16, 3, 2), (17, 5, 2)])
def test_tile_path_train_step(n, L, B):
    (x, th, y), (e, loss, g) = _run_train(n, L, B, seed=20 + n + L)
    e_ref, loss_ref, g_ref = oracle.train_step(x, th, y)
    assert_e_close(e, e_ref, n, L)
    assert abs(loss - loss_ref) <= 1e-5 * max(1.0, loss_ref)
    assert_grad_close(g, g_ref)


def test_tile_path_three_views():
    n, L, B = 21, 3, 1
    (x, th, y), (e, loss, g) = _run_train(n, L, B, seed=5)
    e_ref, loss_ref, g_ref = oracle.train_step(x, th, y)
    assert_e_close(e, e_ref, n, L)
    assert_grad_close(g, g_ref)


@pytest.mark.parametrize("ckpt", [0, 1])
def test_two_stage_reductions(ckpt):
    """n = 22: 512 tiles per sample, so the per-tile <Z_0> and statistics partials are
    first summed in 256-tile chunks.  Batch 3 in two pipelined chunks (the second one
    starting at sample 1) and a forward/backward split."""
    n, L, B = 22, 3, 3
    x, th, y = hqml_inputs.make_inputs(n, L, B, seed=42)
    say(f"[gpu] two-stage reductions n={n} ckpt={ckpt}, two chunks")
    ctx = _ctx(n, L, B, ckpt_block=ckpt)
    ctx.set_overlap(2)
    e, loss, g = (t.cpu().numpy() for t in ctx.train_step(*(torch.from_numpy(a) for a in (x, th, y))))
    loss = float(loss[0])
    ctx.close()
    e_ref, loss_ref, g_ref = oracle.train_step(x, th, y)
    assert_e_close(e, e_ref, n, L)
    assert abs(loss - loss_ref) <= 1e-5 * max(1.0, loss_ref)
    assert_grad_close(g, g_ref)
    ctx = _ctx(n, L, B, ckpt_block=ckpt)
    e2 = ctx.forward(torch.from_numpy(x), torch.from_numpy(th)).cpu().numpy()
    g2 = ctx.backward(torch.from_numpy((2.0 * (e2 - y) / B).astype(np.float32))).cpu().numpy()
    ctx.close()
    assert_e_close(e2, e_ref, n, L)
    assert_grad_close(g2, g_ref)


@pytest.mark.parametrize("n,L,B", [(4, 2, 8), (12, 3, 4), (14, 3, 3), (16, 2, 2)])
def test_forward_backward_split(n, L, B):
    x, th, _ = hqml_inputs.make_inputs(n, L, B, seed=33)
    w = np.linspace(-0.7, 1.3, B).astype(np.float32)
    say(f"[gpu] forward+backward n={n} L={L} B={B}")
    ctx = _ctx(n, L, B)
    e = ctx.forward(torch.from_numpy(x), torch.from_numpy(th), save_for_backward=True)
    g = ctx.backward(torch.from_numpy(w))
    torch.cuda.synchronize()
    g_ref, e_ref = oracle.backward(x, th, w)
    assert_e_close(e.cpu().numpy(), e_ref, n, L)
    assert_grad_close(g.cpu().numpy(), g_ref)
    ctx.close()


@pytest.mark.parametrize("name", ["hea4q2l", "hea12q20l"])
def test_named_workload_full(name):
    w = hqml_inputs.WORKLOADS[name]
    x, th, y = hqml_inputs.workload_inputs(name)
    say(f"[gpu] workload {name}")
    ctx = _ctx(w.n_qubits, w.n_layers, w.batch)
    e, loss, g = ctx.train_step(torch.from_numpy(x), torch.from_numpy(th), torch.from_numpy(y))
    torch.cuda.synchronize()
    e_ref, loss_ref, g_ref = oracle.train_step(x, th, y)
    assert_e_close(e.cpu().numpy(), e_ref, w.n_qubits, w.n_layers)
    assert abs(float(loss.cpu()[0]) - loss_ref) <= 1e-5 * max(1.0, loss_ref)
    assert_grad_close(g.cpu().numpy(), g_ref)
    # the bound that binds where gradients are small: relative to the largest entry (measured
    # 3.5e-7 at 4 qubits / 2 layers and 2.1e-6 at 12 qubits / 20 layers)
    r = assert_grad_rel(g.cpu().numpy(), g_ref, 1e-4, f"{name} batch gradient")
    say(f"[gpu] {name}: max|dg| / max|g_ref| = {r:.2e}")
    ctx.close()


def test_deterministic_and_batch_additive():
    n, L, B = 15, 3, 4
    x, th, _ = hqml_inputs.make_inputs(n, L, B, seed=44)
    w = np.array([0.3, -1.0, 0.5, 2.0], dtype=np.float32)
    say("[gpu] determinism / additivity")
    ctx = _ctx(n, L, B)
    X, TH = torch.from_numpy(x), torch.from_numpy(th)
    ctx.forward(X, TH)
    g1 = ctx.backward(torch.from_numpy(w)).cpu().numpy()
    ctx.forward(X, TH)
    g2 = ctx.backward(torch.from_numpy(w)).cpu().numpy()
    assert np.array_equal(g1, g2)
    parts = np.zeros_like(g1, dtype=np.float64)
    for b in range(B):
        ctx.forward(X[b:b + 1], TH)
        parts += ctx.backward(torch.from_numpy(w[b:b + 1])).cpu().numpy()
    assert np.max(np.abs(parts - g1)) < 1e-5
    ctx.close()


def test_error_paths():
    import qml_gradients_amd as hq
    say("[gpu] error paths")
    ctx = _ctx(14, 2, 2)
    g = torch.empty((2, 14, 3), device="cuda")
    with pytest.raises(hq.HqmlError) as e:
        hq.hqml_backward(ctx.handle, g.data_ptr(), g.data_ptr())
    assert e.value.status == hq.HQML_ERR_STATE
    with pytest.raises(hq.HqmlError) as e:
        ctx.forward(torch.zeros((3, 14)), torch.zeros((2, 14, 3)))
    assert e.value.status == hq.HQML_ERR_ARG
    # empty batch: forward does nothing, backward gives a zero gradient
    hq.hqml_forward(ctx.handle, 0, 0, 0, 0, 1)
    hq.hqml_backward(ctx.handle, 0, g.data_ptr())
    torch.cuda.synchronize()
    assert float(g[:2].abs().max()) == 0.0
    ctx.close()


@pytest.mark.parametrize("n", [20, 29])
def test_one_layer_closed_form_full_width(n):
    """L = 1 at full width: E = cos x0 cos a cos b - sin x0 sin b, with (a, b) the Rx and Ry
    angles of qubit 0; dE/da, dE/db in closed form; every other derivative is 0 (the CZ
    chain and the Rz gates commute with Z_0)."""
    import qml_gradients_amd as hq
    B = 2 if n == 20 else 1
    x, th, _ = hqml_inputs.make_inputs(n, 1, B, seed=77)
    say(f"[gpu] one-layer closed form n={n}")
    ctx = _ctx(n, 1, B, ckpt_block=1 if n == 29 else 0)
    w = np.linspace(0.5, 1.5, B).astype(np.float32)
    e = ctx.forward(torch.from_numpy(x), torch.from_numpy(th)).cpu().numpy().astype(np.float64)
    g = ctx.backward(torch.from_numpy(w)).cpu().numpy().astype(np.float64)
    ctx.close()
    x0 = x[:, 0].astype(np.float64)
    a, b = float(th[0, 0, 0]), float(th[0, 0, 1])
    e_ref = np.cos(x0) * np.cos(a) * np.cos(b) - np.sin(x0) * np.sin(b)
    assert_e_close(e, e_ref, n, 1)
    g_ref = np.zeros((1, n, 3))
    g_ref[0, 0, 0] = np.sum(w * (-np.cos(x0) * np.sin(a) * np.cos(b)))
    g_ref[0, 0, 1] = np.sum(w * (-np.cos(x0) * np.cos(a) * np.sin(b) - np.sin(x0) * np.cos(b)))
    assert_grad_close(g, g_ref)


def test_nan_inputs_propagate_and_oom_precheck():
    """A NaN angle gives NaN results without a fault; a workspace larger than the free
    device memory is refused before any allocation."""
    import qml_gradients_amd as hq
    n, L, B = 15, 2, 2
    x, th, y = hqml_inputs.make_inputs(n, L, B, seed=9)
    th[1, 3, 1] = np.nan
    for storage in ("fp32", "bf16"):
        say(f"[gpu] NaN inputs, {storage} storage")
        ctx = _ctx(n, L, B, storage=storage)
        e, loss, g = (t.cpu().numpy() for t in ctx.train_step(*(torch.from_numpy(a) for a in (x, th, y))))
        ctx.close()
        # the NaN angle reaches every amplitude of both samples (it is in layer 1 of 2):
        # every output is NaN, none has turned into an infinity or a number
        assert np.isnan(loss[0]) and np.isnan(e).all(), (storage, e, loss)
        assert np.isnan(g).any() and not np.isinf(g).any(), storage
    say("[gpu] OOM pre-check")
    with pytest.raises(hq.HqmlError) as err:
        _ctx(29, 200, 8)        # ~200 saved 32 GiB states
    assert err.value.status == hq.HQML_ERR_OOM
    ok = _ctx(14, 1, 1)        # the device is still usable afterwards
    ok.close()


def test_null_pointer_arguments():
    import qml_gradients_amd as hq
    ctx = _ctx(14, 2, 2)
    buf = torch.zeros(1024, device="cuda")
    p = buf.data_ptr()
    for args in ((2, 0, p, p, p, p, p), (2, p, 0, p, p, p, p), (2, p, p, 0, p, p, p), (2, p, p, p, p, p, 0)):
        with pytest.raises(hq.HqmlError) as e:
            hq.hqml_train_step(ctx.handle, *args)
        assert e.value.status == hq.HQML_ERR_ARG
    with pytest.raises(hq.HqmlError) as e:
        hq.hqml_train_step(ctx.handle, 3, p, p, p, p, p, p)      # B > max_batch
    assert e.value.status == hq.HQML_ERR_ARG
    ctx.close()


def test_unusable_array_arguments():
    """Arrays the kernels could not use are refused on the host with HQML_ERR_ARG:
    pageable host memory, and an array running past the end of its allocation.  Each
    case is a backward call before any forward, so a check that let the array through
    would still queue nothing (the call then fails with HQML_ERR_STATE instead)."""
    import ctypes
    import qml_gradients_amd as hq
    say("[gpu] unusable array arguments")
    ctx = _ctx(14, 2, 2)
    g = torch.zeros((2, 14, 3), device="cuda")
    host = np.zeros((2, 14, 3), dtype=np.float32)
    with pytest.raises(hq.HqmlError) as e:
        hq.hqml_backward(ctx.handle, g.data_ptr(), host.ctypes.data)
    assert e.value.status == hq.HQML_ERR_ARG and "pageable" in str(e.value)
    # the last 8 bytes of an allocation cannot hold the 336-byte gradient
    hip = ctypes.CDLL("libamdhip64.so.7")
    hip.hipMemGetAddressRange.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.POINTER(ctypes.c_size_t),
                                          ctypes.c_void_p]
    blk = torch.empty(1 << 21, dtype=torch.uint8, device="cuda")
    base, size = ctypes.c_void_p(), ctypes.c_size_t()
    assert hip.hipMemGetAddressRange(ctypes.byref(base), ctypes.byref(size), ctypes.c_void_p(blk.data_ptr())) == 0
    with pytest.raises(hq.HqmlError) as e:
        hq.hqml_backward(ctx.handle, g.data_ptr(), base.value + size.value - 8)
    assert e.value.status == hq.HQML_ERR_ARG and "needs 336 bytes" in str(e.value)
    # pinned host memory passes the check (the call then stops at the missing forward)
    pinned = torch.zeros((2, 14, 3)).pin_memory()
    with pytest.raises(hq.HqmlError) as e:
        hq.hqml_backward(ctx.handle, g.data_ptr(), pinned.data_ptr())
    assert e.value.status == hq.HQML_ERR_STATE
    # the context is still usable, with no error left behind by the refused calls
    x, th, y = hqml_inputs.make_inputs(14, 2, 2, seed=5)
    e_, loss, grad = (t.cpu().numpy() for t in ctx.train_step(*(torch.from_numpy(a) for a in (x, th, y))))
    assert np.isfinite(loss).all() and np.isfinite(grad).all()
    ctx.close()


def _whole_circuit_obs(n):
    """A Pauli string for width n: Z_0 alone on even widths, else Z_0 Y_(n-1) with an X
    on qubit n // 2 (X/Y factors read partner amplitudes across the swizzled slots)."""
    if n % 2 == 0 or n == 1:
        return 1, 0
    top, mid = 1 << (n - 1), 1 << (n // 2)
    return 1 | top, top | mid


@pytest.mark.parametrize("L", [1, 4])
@pytest.mark.parametrize("n", list(range(1, 14)))
def test_whole_circuit_every_width(n, L):
    """Whole-circuit kernels at every width 1..13 (n = 12: the register-resident kernel):
    the register rounds cover qubits 0..2, 3..5, 6..8, 9..11, 12 and so leave remainders of
    1..2 qubits; the diagonal's CZ between qubits 3 and 4 exists only for n > 4; small n leaves
    most threads idle.
    Train step and forward/backward split, a smaller batch on the same context."""
    import qml_gradients_amd as hq
    zm, xm = _whole_circuit_obs(n)
    maxB = 3
    x, th, y = hqml_inputs.make_inputs(n, L, maxB, seed=3100 + 17 * n + L)
    say(f"[gpu] whole circuit n={n} L={L} z={zm:#x} x={xm:#x}")
    ctx = hq.Context(n, L, maxB, obs_mask=zm, obs_x_mask=xm)
    for B in (maxB, 2):
        X, TH, Y = (torch.from_numpy(a) for a in (x[:B], th, y[:B]))
        e, loss, g = (t.cpu().numpy() for t in ctx.train_step(X, TH, Y))
        e_ref, loss_ref, g_ref = oracle.train_step(x[:B], th, y[:B], zm, xm)
        assert_e_close(e, e_ref, n, L)
        assert abs(float(loss[0]) - loss_ref) <= 1e-5 * max(1.0, loss_ref)
        assert_grad_close(g, g_ref)
    w = np.linspace(-0.5, 1.5, 2).astype(np.float32)
    e2 = ctx.forward(torch.from_numpy(x[:2]), torch.from_numpy(th)).cpu().numpy()
    g2 = ctx.backward(torch.from_numpy(w)).cpu().numpy()
    g2_ref, e2_ref = oracle.backward(x[:2], th, w.astype(np.float64), zm, xm)
    assert_e_close(e2, e2_ref, n, L)
    assert_grad_close(g2, g2_ref)
    ctx.close()


# Pauli strings (z mask, x mask) for the 12-qubit register kernel: factors on qubits held
# in registers and at lane bits of either layout, Y factors (both masks), and a string over
# all twelve qubits.
_S12_STRINGS = [(0x001, 0x000), (0x800, 0x001), (0x018, 0x018), (0x0c3, 0x30c), (0x000, 0x900), (0xfff, 0xa5a)]


@pytest.mark.parametrize("L", [1, 2, 5])
@pytest.mark.parametrize("zm,xm", _S12_STRINGS)
def test_whole_circuit_12_qubits(zm, xm, L):
    """12 qubits with the CZ chain run on the register-resident whole-circuit kernel (two
    layouts, one LDS transpose per layer and state; layers alternate between starting in
    either layout, so odd and even L end the forward pass in different layouts).  Train
    step with a ragged second batch on the same context, then a forward / backward split."""
    import qml_gradients_amd as hq
    n, maxB = 12, 3
    x, th, y = hqml_inputs.make_inputs(n, L, maxB, seed=3900 + 7 * L + zm % 97 + xm % 89)
    say(f"[gpu] 12-qubit register kernel L={L} z={zm:#x} x={xm:#x}")
    ctx = hq.Context(n, L, maxB, obs_mask=zm, obs_x_mask=xm)
    for B in (maxB, 1):
        X, TH, Y = (torch.from_numpy(a) for a in (x[:B], th, y[:B]))
        e, loss, g = (t.cpu().numpy() for t in ctx.train_step(X, TH, Y))
        e_ref, loss_ref, g_ref = oracle.train_step(x[:B], th, y[:B], zm, xm)
        assert_e_close(e, e_ref, n, L)
        assert abs(float(loss[0]) - loss_ref) <= 1e-5 * max(1.0, loss_ref)
        assert_grad_close(g, g_ref)
    w = np.linspace(-0.5, 1.5, maxB).astype(np.float32)
    e2 = ctx.forward(torch.from_numpy(x), torch.from_numpy(th)).cpu().numpy()
    g2 = ctx.backward(torch.from_numpy(w)).cpu().numpy()
    g2_ref, e2_ref = oracle.backward(x, th, w.astype(np.float64), zm, xm)
    assert_e_close(e2, e2_ref, n, L)
    assert_grad_close(g2, g2_ref)
    ctx.close()


def test_whole_circuit_12_qubits_deep():
    """300 layers on the 12-qubit register kernel: the rotation scales carried through both
    layouts and folded into each layer's diagonal must not drift."""
    import qml_gradients_amd as hq
    n, L, B = 12, 300, 2
    x, th, y = hqml_inputs.make_inputs(n, L, B, seed=3990)
    say(f"[gpu] 12-qubit register kernel deep L={L}")
    ctx = hq.Context(n, L, B)
    e, loss, g = (t.cpu().numpy() for t in ctx.train_step(*(torch.from_numpy(a) for a in (x, th, y))))
    ctx.close()
    e_ref, loss_ref, g_ref = oracle.train_step(x, th, y)
    assert_e_close(e, e_ref, n, L)
    assert_grad_close(g, g_ref)


def test_whole_circuit_12_qubits_split_is_bitwise():
    """At small batches the 12-qubit kernel runs a sample on 4 (batch <= CUs / 4) or 2
    (batch <= CUs / 2) workgroups that split the statistics by qubit, else on one.  Per-sample
    E and per-sample gradients (a one-hot dL/dE makes the batch sum that sample's term alone)
    must be bitwise the same in all three regimes, and match the oracle."""
    import qml_gradients_amd as hq
    n, L = 12, 4
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    batches = sorted({1, cus // 2, cus + 3})   # 4, 2 and 1 workgroups per sample
    x, th, _ = hqml_inputs.make_inputs(n, L, max(batches), seed=3995)
    ref = None
    for B in batches:
        say(f"[gpu] 12-qubit split regimes: batch {B} of {batches}")
        ctx = hq.Context(n, L, B, obs_mask=0x801, obs_x_mask=0x090)
        e = ctx.forward(torch.from_numpy(x[:B]), torch.from_numpy(th)).cpu().numpy()
        w = np.zeros(B, dtype=np.float32)
        w[0] = 1.0
        g = ctx.backward(torch.from_numpy(w)).cpu().numpy()
        ctx.close()
        if ref is None:
            ref = (e[0], g)
            g_ref, e_ref = oracle.backward(x[:1], th, np.ones(1), 0x801, 0x090)
            assert_e_close(e[:1], e_ref, n, L)
            assert_grad_close(g, g_ref)
        else:
            assert e[0] == ref[0] and np.array_equal(g, ref[1]), f"batch {B} differs from batch {batches[0]}"


@pytest.mark.parametrize("entangler", ["cz", "cnot"])
def test_whole_circuit_deep(entangler):
    """600 layers on the whole-circuit kernel (n = 9: a 4-qubit remainder round plus a
    1-qubit one): the rotation scales carried from round to round and folded into each
    layer's diagonal must not drift; the bounds grow with depth as derived for <O>."""
    import qml_gradients_amd as hq
    n, L, B = 9, 600, 2
    ent = 1 if entangler == "cnot" else 0
    x, th, y = hqml_inputs.make_inputs(n, L, B, seed=3700 + ent)
    say(f"[gpu] whole circuit deep n={n} L={L} {entangler}")
    ctx = hq.Context(n, L, B, entangler=entangler)
    e, loss, g = (t.cpu().numpy() for t in ctx.train_step(*(torch.from_numpy(a) for a in (x, th, y))))
    ctx.close()
    e_ref, loss_ref, g_ref = oracle.train_step(x, th, y, entangler=ent)
    assert_e_close(e, e_ref, n, L)
    assert_grad_close(g, g_ref)
