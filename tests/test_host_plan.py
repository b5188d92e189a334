"""Host-side checks of the C-ABI library (no GPU needed).

* the library loads and exports every function include/hqml.h declares;
* argument validation and workspace sizing work without touching a device;
* the fused-pass schedule the library plans is complete and consistent;
* a NumPy model of the kernels' algebra on that schedule matches the oracle;
* the tile layouts used by the kernels are bijective and bank-conflict free.
"""
import json
import os
import re

import numpy as np
import pytest

import hqml_inputs
import oracle
import qml_gradients_amd as hq
from tile_model import Model

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _lib():
    if not os.path.exists(hq.LIB_PATH):
        from qml_gradients_amd import build
        build.build()
    return hq.load()


def test_exports_every_declared_function():
    lib = _lib()
    header = open(os.path.join(ROOT, "include", "hqml.h")).read()
    declared = set(re.findall(r"\b(hqml_[a-z_0-9]+)\s*\(", header))
    assert declared == set(hq.EXPORTED)
    for name in declared:
        assert hasattr(lib, name), name


def test_workspace_and_validation_host_only():
    _lib()
    assert hq.hqml_workspace_bytes(hq.make_config(20, 100, 32)) > 100 * 32 * (1 << 20) * 8
    for bad in (hq.make_config(0, 1, 1), hq.make_config(30, 1, 1), hq.make_config(4, 0, 1),
                hq.make_config(4, 1, 0), hq.make_config(4, 1, 1, storage=7),
                hq.make_config(4, 1, 1, ckpt_block=-1), hq.make_config(4, 1, 1, obs_mask=16),
                hq.make_config(4, 1, 1, obs_mask=-1)):
        assert hq.hqml_workspace_bytes(bad) == 0
        with pytest.raises(hq.HqmlError) as e:
            hq.hqml_create(bad)
        assert e.value.status == hq.HQML_ERR_ARG
    assert hq.load().hqml_status_str(hq.HQML_ERR_STATE) == b"call out of order"
    assert hq.hqml_workspace_bytes(hq.make_config(4, 1, 1, obs_mask=15)) > 0


def test_gate_by_gate_config_host_only():
    _lib()
    cfg = hq.make_config(20, 100, 32, fusion="gate_by_gate")
    d = json.loads(hq.hqml_describe_plan(cfg))
    assert d == {"n": 20, "L": 100, "gate_by_gate": True, "blocks": (1 << 19) // 4096}
    # psi + lambda, fp64 block sums per parameter, sample and block, and small tables
    N, B, P, nblk = 1 << 20, 32, 6000, 128
    ws = hq.hqml_workspace_bytes(cfg)
    assert 2 * B * N * 8 + P * B * nblk * 8 <= ws < 2 * B * N * 8 + P * B * nblk * 8 + (1 << 20)
    assert json.loads(hq.hqml_describe_plan(hq.make_config(3, 2, 1, fusion="gate_by_gate")))["blocks"] == 1
    for bad in (hq.make_config(4, 1, 1, storage="bf16", fusion="gate_by_gate"),
                hq.make_config(4, 1, 1, ckpt_block=2, fusion="gate_by_gate")):
        assert hq.hqml_workspace_bytes(bad) == 0
        with pytest.raises(hq.HqmlError) as e:
            hq.hqml_create(bad)
        assert e.value.status == hq.HQML_ERR_UNSUPPORTED
    for bad in (hq.make_config(4, 1, 1, fusion=2), hq.make_config(4, 1, 70000, fusion="gate_by_gate")):
        assert hq.hqml_workspace_bytes(bad) == 0


def test_fp64_config_host_only():
    _lib()
    ws32 = hq.hqml_workspace_bytes(hq.make_config(20, 10, 4))
    ws64c = hq.hqml_workspace_bytes(hq.make_config(20, 10, 4, compute="fp64"))
    ws64 = hq.hqml_workspace_bytes(hq.make_config(20, 10, 4, storage="fp64", compute="fp64"))
    st = 4 * (1 << 20) * 8
    # fp64 compute doubles lambda; fp64 storage doubles the 10 saved states
    assert ws64c - ws32 >= st
    assert ws64 - ws64c >= 10 * st
    assert hq.hqml_workspace_bytes(hq.make_config(12, 3, 2, storage="fp64", compute="fp64")) > 0
    for bad in (hq.make_config(16, 2, 1, storage="fp64"), hq.make_config(16, 2, 1, storage="bf16", compute="fp64"),
                hq.make_config(13, 2, 1, compute="fp64"),
                hq.make_config(16, 2, 1, compute="fp64", fusion="gate_by_gate")):
        assert hq.hqml_workspace_bytes(bad) == 0
        with pytest.raises(hq.HqmlError) as e:
            hq.hqml_create(bad)
        assert e.value.status == hq.HQML_ERR_UNSUPPORTED
    assert hq.hqml_workspace_bytes(hq.make_config(16, 2, 1, compute=2)) == 0


def test_pauli_observable_config_host_only():
    _lib()
    ok = hq.make_config(20, 3, 2, obs_mask=0, obs_x_mask=sum(1 << q for q in range(11, 20)))   # 9 high X
    assert hq.hqml_workspace_bytes(ok) > 0
    too_many = hq.make_config(20, 3, 2, obs_x_mask=sum(1 << q for q in range(10, 20)))         # 10 high X
    assert hq.hqml_workspace_bytes(too_many) == 0
    with pytest.raises(hq.HqmlError) as e:
        hq.hqml_create(too_many)
    assert e.value.status == hq.HQML_ERR_UNSUPPORTED
    # the whole-circuit path and the gate-by-gate comparator take any Pauli string
    assert hq.hqml_workspace_bytes(hq.make_config(13, 3, 2, obs_x_mask=(1 << 13) - 1)) > 0
    assert hq.hqml_workspace_bytes(hq.make_config(20, 3, 2, obs_x_mask=(1 << 20) - 1, fusion="gate_by_gate")) > 0
    for bad in (hq.make_config(4, 1, 1, obs_x_mask=16), hq.make_config(4, 1, 1, obs_x_mask=-2)):
        assert hq.hqml_workspace_bytes(bad) == 0


def test_entangler_config_host_only():
    _lib()
    assert hq.hqml_workspace_bytes(hq.make_config(12, 3, 2, entangler="cnot")) > 0
    assert hq.hqml_workspace_bytes(hq.make_config(13, 3, 2, entangler="cnot", obs_x_mask=0b101)) > 0
    assert hq.hqml_workspace_bytes(hq.make_config(20, 3, 2, entangler="cnot", fusion="gate_by_gate")) > 0
    # tile path: one pass per view and layer, Z-string observables only, a second lambda buffer
    cz = hq.hqml_workspace_bytes(hq.make_config(20, 10, 4))
    cn = hq.hqml_workspace_bytes(hq.make_config(20, 10, 4, entangler="cnot"))
    st = 4 * (1 << 20) * 8
    # 19 saved pass outputs instead of 10, plus lambda; the statistics partials differ by
    # less than half a state (the CZ plan's general passes write two rows per tile)
    assert cn - cz >= 9.5 * st
    # X/Y factors: the chain-conjugated string has X on q and q+1 for each X/Y on q; it
    # must fit the observable view (at most 9 such qubits above qubit 3)
    assert hq.hqml_workspace_bytes(hq.make_config(20, 3, 2, entangler="cnot", obs_x_mask=0b1010 << 4)) > 0
    wide = hq.make_config(20, 3, 2, entangler="cnot", obs_x_mask=0b1010101010 << 4)   # 10 qubits after
    assert hq.hqml_workspace_bytes(wide) == 0
    assert hq.hqml_workspace_bytes(hq.make_config(20, 3, 2, obs_x_mask=0b1010101010 << 4)) > 0   # CZ: 5
    with pytest.raises(hq.HqmlError) as e:
        hq.hqml_create(wide)
    assert e.value.status == hq.HQML_ERR_UNSUPPORTED
    for bad in (hq.make_config(4, 1, 1, entangler=2), hq.make_config(4, 1, 1, entangler=-1)):
        assert hq.hqml_workspace_bytes(bad) == 0
        with pytest.raises(hq.HqmlError) as e:
            hq.hqml_create(bad)
        assert e.value.status == hq.HQML_ERR_ARG


def test_workspace_scaling_checkpoint_and_bf16():
    _lib()
    full = hq.hqml_workspace_bytes(hq.make_config(20, 1000, 60))
    ck20 = hq.hqml_workspace_bytes(hq.make_config(20, 1000, 60, ckpt_block=20))
    ck20b = hq.hqml_workspace_bytes(hq.make_config(20, 1000, 60, storage="bf16", ckpt_block=20))
    st = 60 * (1 << 20) * 8
    # store-all keeps ~1000 states; b=20 keeps 20 block states + 49 checkpoints + lambda
    assert full > 990 * st
    assert 60 * st < ck20 < 80 * st
    assert ck20b < ck20


def _plan(n, L, ckpt=0):
    _lib()
    return json.loads(hq.hqml_describe_plan(hq.make_config(n, L, 1, ckpt_block=ckpt)))


@pytest.mark.parametrize("n", list(range(1, 30)))
def test_plan_invariants(n):
    for L in (1, 2, 3, 5):
        p = _plan(n, L)
        assert len(p["statmap"]) == L * n
        if n <= 13:
            assert p["small"]
            continue
        V = p["V"]
        assert V == max(2, (n - 4 + 7) // 8)
        assert p["T"] == 1 << (n - 13)
        assert len(p["passes"]) == 1 + (L - 1) * (V - 1)
        seen = set()
        owner = {}
        for vi, v in enumerate(p["views"]):
            perm = v["perm"]
            assert sorted(perm[:4]) == [0, 1, 2, 3]
            assert len(set(perm)) == 13 and sorted(perm + v["tile_q"]) == list(range(n))
            assert v["group_mask"] & ~0x0FF3 == 0          # only rotatable positions
            for pos in range(13):
                if (v["group_mask"] >> pos) & 1:
                    assert perm[pos] not in owner
                    owner[perm[pos]] = vi
            # qubit 3 at an L2 low register position => qubit 4 not at L2 positions 9..11
            if perm.index(3) in (0, 1) and 4 in perm:
                assert perm.index(4) not in (9, 10, 11)
        assert sorted(owner) == list(range(n))
        for k, s in p["statmap"]:
            assert (k, s) not in seen
            seen.add((k, s))
            assert 0 <= k < len(p["passes"]) + len(p["stats_only"])
        # each pass rotates only its own view's group and the layers appear in order
        last_layer = {}
        for ps in p["passes"]:
            for key in ("rotA", "rotB"):
                if ps[key] >= 0:
                    assert ps[key] >= last_layer.get(ps["view"], 0)
                    last_layer[ps["view"]] = ps[key]


@pytest.mark.parametrize("merged", [True, False], ids=["merged", "uncompute"])
@pytest.mark.parametrize("n,L,B", [(14, 1, 2), (14, 3, 2), (15, 4, 2), (17, 2, 1), (16, 5, 1)])
def test_model_of_kernel_algebra_matches_oracle(n, L, B, merged):
    """The kernels' algebra on the library's schedule: with the merged statistics (both
    layers of a pass from its output, the saved state never un-rotated) and with the
    plain un-computation of psi to the earlier layer's point."""
    x, th, _ = hqml_inputs.make_inputs(n, L, B, seed=100 + n + L)
    m = Model(hq.hqml_describe_plan(hq.make_config(n, L, B)), x, th, merged=merged)
    w = np.linspace(0.5, -1.0, B)
    e, g = m.backward(w)
    g_ref, e_ref = oracle.backward(x, th, w)
    assert np.max(np.abs(e - e_ref)) < 1e-10
    assert np.max(np.abs(g - g_ref)) < 1e-10


@pytest.mark.parametrize("n", list(range(14, 30)))
def test_views_keep_chain_neighbours_apart(n):
    """What the merged statistics rely on: no two qubits a view rotates are chain
    neighbours, and no qubit at a register position of a layout neighbours a rotated
    qubit at a register position of the same layout (L1: positions 4..8; L2: 0, 1,
    9..11), so Z_{q-1} Z_{q+1} is constant over each thread's registers."""
    p = _plan(n, 3)
    for v in p["views"]:
        perm, gm = v["perm"], v["group_mask"]
        rot = {perm[i] for i in range(13) if (gm >> i) & 1}
        assert not any(q + 1 in rot for q in rot)
        for regs in ((4, 5, 6, 7, 8), (0, 1, 9, 10, 11)):
            for a in regs:
                if (gm >> a) & 1:
                    assert all(abs(perm[a] - perm[b]) != 1 for b in regs if b != a)


@pytest.mark.parametrize("n", list(range(14, 30)))
def test_half_views_match_full_views(n):
    """Half-tile views (the fp32 adjoint's general passes): each rotates exactly the group
    of the full view with the same index, holds qubits 0..3 at positions 0..3 with the
    rotated low qubits at 0, 1, keeps the chain neighbours of a rotated qubit off the
    register positions of the layout where its statistics are taken (H1: positions 0, 1,
    4..7 against registers 4..7; H2: 8..11 against 8..11), positions 8, 9 apart from 10, 11
    and 4, 5 from 6, 7 (the diagonal's factor tables), and sends each rotated qubit's
    statistics to its full-view slot."""
    p = _plan(n, 3)
    assert p["half"] and len(p["hviews"]) == len(p["views"])
    for v, h in zip(p["views"], p["hviews"]):
        perm, gm, hperm, hg = v["perm"], v["group_mask"], h["perm"], h["group_mask"]
        rot = {perm[i] for i in range(13) if (gm >> i) & 1}
        hrot = {hperm[i] for i in range(12) if (hg >> i) & 1}
        assert hrot == rot
        assert sorted(hperm[:4]) == [0, 1, 2, 3] and hg & 0b1100 == 0 and hg >> 12 == 0
        assert sorted(hperm + h["tile_q"]) == list(range(n))
        for a in range(12):
            if not (hg >> a) & 1:
                assert h["slot_pos"][a] == 12
                continue
            assert perm[h["slot_pos"][a]] == hperm[a]
            regs = (4, 5, 6, 7) if a in (0, 1, 4, 5, 6, 7) else (8, 9, 10, 11)
            assert all(abs(hperm[a] - hperm[b]) != 1 for b in regs if b != a)
        assert all(abs(hperm[a] - hperm[b]) != 1 for a in (8, 9) for b in (10, 11))
        assert all(abs(hperm[a] - hperm[b]) != 1 for a in (4, 5) for b in (6, 7))


@pytest.mark.parametrize("n", [14, 16, 21, 29])
def test_cnot_plan_invariants(n):
    """CNOT plan: pass 0 forms the product state and diag(p_0); then per layer one pass
    per view in view order, the first reading through the chain (diag(r_l) row L + l),
    the last applying diag(p_l) (row l); every (layer, qubit) has one statistics slot."""
    _lib()
    for L in (1, 2, 4):
        p = json.loads(hq.hqml_describe_plan(hq.make_config(n, L, 1, entangler="cnot")))
        V = p["V"]
        assert p["cnot"] and len(p["passes"]) == 1 + (L - 1) * V
        assert p["passes"][0] == {"view": 0, "init": True, "rotA": -1, "diag": 0, "rotB": -1, "gather": False}
        for l in range(1, L):
            for v in range(V):
                ps = p["passes"][1 + (l - 1) * V + v]
                assert ps["view"] == v and ps["gather"] == (v == 0) and not ps["init"]
                assert (ps["rotA"], ps["rotB"]) == ((-1, l) if v == 0 else (l, -1))
                assert ps["diag"] == (L + l if v == 0 else l if v == V - 1 else -1)
        assert len({tuple(sm) for sm in p["statmap"]}) == L * n


@pytest.mark.parametrize("n,L,B", [(14, 1, 2), (14, 3, 2), (15, 4, 1), (17, 3, 1)])
def test_model_of_cnot_plan_matches_oracle(n, L, B):
    x, th, _ = hqml_inputs.make_inputs(n, L, B, seed=200 + n + L)
    m = Model(hq.hqml_describe_plan(hq.make_config(n, L, B, entangler="cnot")), x, th)
    w = np.linspace(0.5, -1.0, B)
    e, g = m.backward(w)
    g_ref, e_ref = oracle.backward(x, th, w, entangler=1)
    assert np.max(np.abs(e - e_ref)) < 1e-10
    assert np.max(np.abs(g - g_ref)) < 1e-10


@pytest.mark.slow
def test_model_three_views_matches_oracle():
    n, L, B = 21, 3, 1
    x, th, _ = hqml_inputs.make_inputs(n, L, B, seed=7)
    m = Model(hq.hqml_describe_plan(hq.make_config(n, L, B)), x, th)
    assert m.plan["V"] == 3
    e, g = m.backward(np.ones(B))
    g_ref, e_ref = oracle.backward(x, th, np.ones(B))
    assert np.max(np.abs(e - e_ref)) < 1e-10
    assert np.max(np.abs(g - g_ref)) < 1e-10


# ---- tile layouts (restated from the kernel source's layout comments) ----

def swz(l):
    return l ^ ((l >> 4) & 3) ^ ((((l >> 6) ^ (l >> 9)) & 1) << 4)


def l1(lane, w, j):
    return (lane & 15) | ((lane >> 4) << 9) | (w << 11) | (j << 4)


def l2(lane, w, j):
    return (lane << 2) | ((w & 1) << 8) | ((w >> 1) << 12) | (j & 3) | ((j >> 2) << 9)


def test_tile_layouts_bijective_and_conflict_free():
    a1 = {l1(la, w, j) for la in range(64) for w in range(4) for j in range(32)}
    a2 = {l2(la, w, j) for la in range(64) for w in range(4) for j in range(32)}
    assert a1 == a2 == set(range(8192))
    assert {swz(i) for i in range(8192)} == set(range(8192))
    for f in (l1, l2):
        for w in range(4):
            for j in range(32):
                for half in range(2):        # 64 banks x 4 B: 32 lanes x 8 B per cycle
                    slots = {swz(f(la, w, j)) & 31 for la in range(32 * half, 32 * half + 32)}
                    assert len(slots) == 32
                for quarter in range(4):     # 32 banks x 4 B: 16 lanes x 8 B per cycle
                    slots = {swz(f(la, w, j)) & 15 for la in range(16 * quarter, 16 * quarter + 16)}
                    assert len(slots) == 16
    # linearity used to split addresses into thread and register parts
    for t in range(0, 8192, 97):
        for j in range(32):
            assert swz(l1(t & 63, t >> 6 & 3, 0) ^ (j << 4)) == swz(l1(t & 63, t >> 6 & 3, 0)) ^ swz(j << 4)


def chain_pair_slot(blk, G, T2):
    """Grid slot of workgroup blk in the passes that move a state through the CNOT chain's
    index map (hqml_kernels.hip, chain_pair_slot), restated."""
    if (G & 15) or T2 < 2:
        return blk
    p = ((blk >> 4) << 3) | (blk & 7)
    h = (blk >> 3) & 1
    half = T2 >> 1
    rel, t = divmod(p, half)
    return rel * T2 + (T2 - 1 - t if h else t)


@pytest.mark.parametrize("T2", [2, 4, 8, 64, 256, 4096])
@pytest.mark.parametrize("samples", [1, 2, 3, 5, 32])
def test_chain_pair_slot_pairs_complementary_tiles(T2, samples):
    """A bijection of the grid; where 16 divides it, workgroups b and b + 8 (one XCD, b % 8
    equal) take tiles t and T2 - 1 - t of the same sample: the two tiles whose amplitudes
    share each 128-byte line of a state moved through the chain's index map."""
    G = samples * T2
    slots = [chain_pair_slot(b, G, T2) for b in range(G)]
    assert sorted(slots) == list(range(G))
    if G % 16:
        assert slots == list(range(G))
        return
    for b in range(G):
        if (b >> 3) & 1:
            continue
        s0, s1 = slots[b], slots[b + 8]
        assert s0 // T2 == s1 // T2 and (s0 % T2) ^ (s1 % T2) == T2 - 1


@pytest.mark.parametrize("n", [14, 17, 20])
def test_chain_line_halves_come_from_complementary_tiles(n):
    """The reason for the pairing: for a line of 16 consecutive indices a (bits 4.. fixed),
    the indices j = P(a) of its amplitudes (P: bit k = parity of bits 0..k) split into two
    halves of 8 whose bits 4.. differ in every position."""
    def chain(i):
        out, par = 0, 0
        for k in range(n):
            par ^= (i >> k) & 1
            out |= par << k
        return out
    hi_mask = ((1 << n) - 1) & ~15
    for line in (0, 1, 0x2a, (1 << (n - 4)) - 1):
        js = [chain((line << 4) | a) for a in range(16)]
        highs = sorted({j & hi_mask for j in js})
        assert len(highs) == 2 and highs[0] ^ highs[1] == hi_mask
        assert sum((j & hi_mask) == highs[0] for j in js) == 8
