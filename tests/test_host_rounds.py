"""Host checks of the index algebra of the whole-circuit kernel (n <= 13).

The kernel keeps a sample's state in LDS at slot sslot(i) = i ^ ((i >> 3) & 31) and
works in rounds of up to three qubits: a round on qubits s .. s+G-1 gives thread g
(consecutive lanes = consecutive g) the amplitudes base(g) | (j << s).  With the CNOT chain, round 0 of a
forward step reads amplitude J from P^-1(J) and round 0 of an adjoint step reads
amplitude i from P(i) (bit k of P(i) = parity of bits 0..k of i), with the source index
assembled from a per-group high part and a per-j low part.  These tests restate those
formulas in Python and check them exhaustively against their definitions: the slot map
is a bijection with no LDS bank conflicts in any round shape, and the assembled sources
are exactly P^-1(J) and P(i).
"""
import numpy as np
import pytest


ROUND_BITS = 3


def sslot(i):
    return i ^ ((i >> 3) & 31)


def rounds(n):
    out, s = [], 0
    while s < n:
        G = min(ROUND_BITS, n - s)
        out.append((s, G))
        s += G
    return out


def base(g, s, G):
    return ((g >> s) << (s + G)) | (g & ((1 << s) - 1))


def chain(i, n):
    """P(i): bit k = parity of bits 0..k of i."""
    out, par = 0, 0
    for k in range(n):
        par ^= (i >> k) & 1
        out |= par << k
    return out


def chain_inv(j, n):
    return (j ^ (j << 1)) & ((1 << n) - 1)


@pytest.mark.parametrize("n", range(1, 14))
def test_slot_map_is_a_bijection(n):
    N = 1 << n
    slots = sslot(np.arange(N))
    assert slots.max() < N
    assert len(np.unique(slots)) == N


@pytest.mark.parametrize("n", [9, 12, 13])
def test_rounds_cover_every_amplitude_once(n):
    N = 1 << n
    for s, G in rounds(n):
        seen = np.zeros(N, dtype=int)
        for g in range(N >> G):
            for j in range(1 << G):
                seen[base(g, s, G) | (j << s)] += 1
        assert (seen == 1).all()


@pytest.mark.parametrize("n", range(1, 14))
def test_rounds_are_bank_conflict_free(n):
    """For every round, amplitude j and block of 32 consecutive threads, the 8-byte slots
    read or written are distinct modulo 32 slots (256 bytes = the 64 four-byte banks)."""
    for s, G in rounds(n):
        groups = (1 << n) >> G
        for j in range(1 << G):
            for start in range(0, groups, 32):
                gs = range(start, min(start + 32, groups))
                banks = {sslot(base(g, s, G) | (j << s)) % 32 for g in gs}
                assert len(banks) == len(gs), (n, s, G, j, start)


@pytest.mark.parametrize("n", range(1, 14))
def test_cnot_forward_gather_source_is_the_inverse_chain(n):
    G = min(ROUND_BITS, n)
    hmask, lmask = (1 << (n - G)) - 1, (1 << G) - 1
    for g in range(1 << (n - G)):
        ih0 = (g ^ (g << 1)) & hmask
        ih1 = ih0 ^ (hmask & 1)
        for j in range(1 << G):
            hi = ih1 if (j >> (G - 1)) & 1 else ih0
            src = (hi << G) | ((j ^ (j << 1)) & lmask)
            assert src == chain_inv((g << G) | j, n)


@pytest.mark.parametrize("n", range(1, 14))
def test_cnot_adjoint_gather_source_is_the_chain(n):
    G = min(ROUND_BITS, n)
    hmask, lmask = (1 << (n - G)) - 1, (1 << G) - 1
    for g in range(1 << (n - G)):
        pb0 = chain(g, n - G)
        pb1 = pb0 ^ hmask
        for j in range(1 << G):
            hi = pb1 if bin(j).count("1") & 1 else pb0
            src = (hi << G) | chain(j, G)
            assert src == chain((g << G) | j, n)
            assert chain_inv(src, n) == (g << G) | j


# ---- the register-resident 12-qubit kernel (k_small12) ----
#
# 256 threads (lane 0..63, wave 0..3) x 16 registers j; amplitude index of (lane, wave, j):
#   layout A: lanes 0..3 -> qubits 0..3, lanes 4, 5 -> 8, 9, waves -> 10, 11, j -> 4..7
#   layout B: lanes 0, 1 -> 2, 3, lanes 2, 3 -> 0, 1, lanes 4, 5 -> 4, 5, waves -> 6, 7, j -> 8..11
# LDS slot of index i: hswz(i) = i ^ (bit 8 of i) << 4.


def s12_index(la, lane, w, j):
    if la:
        return (lane & 15) | ((lane >> 4) << 8) | (w << 10) | (j << 4)
    return ((lane >> 2) & 3) | ((lane & 3) << 2) | (((lane >> 4) & 3) << 4) | (w << 6) | (j << 8)


def hswz(i):
    return i ^ (((i >> 8) & 1) << 4)


@pytest.mark.parametrize("la", [True, False])
def test_s12_layouts_are_bijections(la):
    idx = {s12_index(la, lane, w, j) for lane in range(64) for w in range(4) for j in range(16)}
    assert idx == set(range(1 << 12))
    assert {hswz(i) for i in range(1 << 12)} == set(range(1 << 12))


def test_s12_layouts_rotate_every_qubit():
    """A layout rotates the qubits of its register bits and of lane bits 0, 1 (DPP quad
    permutations): A covers 0, 1, 4..7, B covers 2, 3, 8..11; together all twelve, once."""
    def qubit_of(la, what):
        base = s12_index(la, 0, 0, 0)
        assert base == 0
        i = s12_index(la, *what)
        assert bin(i).count("1") == 1
        return i.bit_length() - 1
    rot = {}
    for la in (True, False):
        qs = [qubit_of(la, (1 << b, 0, 0)) for b in (0, 1)] + [qubit_of(la, (0, 0, 1 << m)) for m in range(4)]
        rot[la] = qs
    assert rot[True] == [0, 1, 4, 5, 6, 7] and rot[False] == [2, 3, 8, 9, 10, 11]


@pytest.mark.parametrize("la", [True, False])
def test_s12_transposes_are_bank_conflict_free(la):
    """For every register and half-wave, the 32 lanes' 8-byte slots are distinct modulo 32
    (256 bytes = the 64 four-byte banks)."""
    for w in range(4):
        for j in range(16):
            for h in (0, 32):
                banks = {hswz(s12_index(la, lane, w, j)) % 32 for lane in range(h, h + 32)}
                assert len(banks) == 32, (la, w, j, h)


@pytest.mark.parametrize("la", [True, False])
def test_s12_rows_store_whole_lines(la):
    """Lanes 0..15 of a register hold 16 consecutive amplitudes (128 bytes of a saved
    state) in both layouts."""
    for w in range(4):
        for j in range(16):
            for r in range(4):
                idx = sorted(s12_index(la, lane, w, j) for lane in range(16 * r, 16 * r + 16))
                assert idx == list(range(idx[0], idx[0] + 16)) and idx[0] % 16 == 0
