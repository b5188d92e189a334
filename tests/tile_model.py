"""NumPy model of the GPU path's algebra and schedule (host-logic test aid).

This is not the oracle.  It re-states, on whole state vectors, what the
library's kernels do -- the SU(2) factorisation of each layer into
diag(p) Ry(beta) diag(r), the merged diagonal D_l, the fused-pass schedule and
the places where gradient statistics are taken -- using the schedule the
library itself reports (``hqml_describe_plan``).  Comparing it with the oracle
on the CPU checks the algebra and the planner before any GPU run; the GPU
kernels are then compared with the oracle directly.
"""
from __future__ import annotations

import json

import numpy as np


def _rx(t):
    c, s = np.cos(t / 2), np.sin(t / 2)
    return np.array([[c, -1j * s], [-1j * s, c]])


def _ry(t):
    c, s = np.cos(t / 2), np.sin(t / 2)
    return np.array([[c, -s], [s, c]], dtype=complex)


def _rz(t):
    return np.diag([np.exp(-0.5j * t), np.exp(0.5j * t)])


X = np.array([[0, 1], [1, 0]], dtype=complex)
Y = np.array([[0, -1j], [1j, 0]])
Z = np.diag([1.0 + 0j, -1.0])


def factorise(theta):
    """Per (l, q): cos(beta/2), sin(beta/2), p, r with U = diag(p, p*) Ry(beta) diag(r, r*)."""
    L, n, _ = theta.shape
    cb = np.zeros((L, n))
    sb = np.zeros((L, n))
    p = np.zeros((L, n), dtype=complex)
    r = np.zeros((L, n), dtype=complex)
    H = np.zeros((L, n, 3, 3))
    for l in range(L):
        for q in range(n):
            a, b, g = (float(v) for v in theta[l, q])
            U = _rz(g) @ _ry(b) @ _rx(a)
            x, y = U[0, 0], U[1, 0]
            ax, ay = abs(x), abs(y)
            xh = x / ax if ax > 1e-300 else 1.0
            yh = y / ay if ay > 1e-300 else 1.0
            rr = np.exp(0.5j * np.angle(xh * yh))
            pp = xh * np.conj(rr)
            cb[l, q], sb[l, q], p[l, q], r[l, q] = ax, ay, pp, rr
            Lp = np.diag([pp, np.conj(pp)])
            G = [(_rz(g) @ _ry(b)) @ X @ (_rz(g) @ _ry(b)).conj().T, _rz(g) @ Y @ _rz(g).conj().T, Z]
            for k in range(3):
                S = Lp.conj().T @ G[k] @ Lp
                H[l, q, k] = [S[0, 1].real, -S[0, 1].imag, S[0, 0].real]
    return cb, sb, p, r, H


def pauli_frame(cb, sb, p, r, H):
    """Rewrite every Ry(beta) with beta > pi/2 (layers >= 1) as Ry(beta - pi) X Z and
    move the X's to the start of the circuit (see the kernels' frame comment).
    Returns (c, s) of the simulated rotations, the diagonal factors f0/f1 of D_l,
    the frame G and the adjusted gradient map."""
    L, n = cb.shape
    x = np.zeros((L, n), dtype=bool)
    x[1:] = sb[1:] > cb[1:]
    G = np.zeros((L, n), dtype=bool)
    for l in range(L - 2, -1, -1):
        G[l] = G[l + 1] ^ x[l + 1]
    c = np.where(x, sb, cb)
    s = np.where(x, -cb, sb)
    s = np.where(G, -s, s)
    f0 = np.ones((L, n), dtype=complex)
    f1 = np.ones((L, n), dtype=complex)
    for l in range(L - 1):
        w = p[l] * r[l + 1]
        a, b = w, np.conj(w)
        f0[l] = np.where(G[l], b, a)
        f1[l] = np.where(G[l], a, b)
        flip = x[l + 1].copy()
        flip[1:] ^= G[l][:-1]
        flip[:-1] ^= G[l][1:]
        f1[l] = np.where(flip, -f1[l], f1[l])
    H2 = H.copy()
    H2[..., 1] = np.where(G[..., None], -H[..., 1], H[..., 1])
    H2[..., 2] = np.where(G[..., None], -H[..., 2], H[..., 2])
    return c, s, f0, f1, G, H2


def cnot_frame(cb, sb, p, r, H):
    """The same rewrite with the CNOT chain P (|i> -> |P(i)>, bit k of P(i) = parity of
    bits 0..k).  Moving X^g left through P gives X^(P^-1 g), P^-1 g = g ^ (g << 1): no Z
    appears.  Per layer the simulated sequence is diag(r_l), Ry(beta'_l), diag(p_l), P;
    the rewrite's Z merges into diag(r_l).  Returns (c, s), the diagonal rows
    (dP[l], dR[l]) as (f0, f1) pairs, G at the statistics points and the adjusted map."""
    L, n = cb.shape
    x = np.zeros((L, n), dtype=bool)
    x[1:] = sb[1:] > cb[1:]
    G = np.zeros((L, n), dtype=bool)
    g = 0
    full = (1 << n) - 1
    for l in range(L - 1, -1, -1):
        G[l] = [(g >> q) & 1 for q in range(n)]
        if l == 0:
            break
        gb = g ^ sum(1 << q for q in range(n) if x[l, q])
        g = (gb ^ (gb << 1)) & full
    c = np.where(x, sb, cb)
    s = np.where(x, -cb, sb)
    s = np.where(G, -s, s)
    dP0 = np.where(G, np.conj(p), p)
    dP1 = np.where(G, p, np.conj(p))
    r0, r1 = r.copy(), np.where(x, -np.conj(r), np.conj(r))
    sw = G ^ x
    dR0 = np.where(sw, r1, r0)
    dR1 = np.where(sw, r0, r1)
    H2 = H.copy()
    H2[..., 1] = np.where(G[..., None], -H[..., 1], H[..., 1])
    H2[..., 2] = np.where(G[..., None], -H[..., 2], H[..., 2])
    return c, s, (dP0, dP1), (dR0, dR1), G, H2


class Model:
    def __init__(self, plan_json: str, x, theta, merged: bool = True):
        self.plan = json.loads(plan_json)
        self.merged = merged
        self.x = np.asarray(x, dtype=np.float64)
        self.theta = np.asarray(theta, dtype=np.float64)
        self.L, self.n = self.theta.shape[0], self.theta.shape[1]
        self.cb, self.sb, self.p, self.r, H0 = factorise(self.theta)
        self.cnot = bool(self.plan.get("cnot", False))
        if self.cnot:
            self.c, self.s, dP, dR, self.G, self.H = cnot_frame(self.cb, self.sb, self.p, self.r, H0)
            # table rows: l = diag(p_l), L + l = diag(r_l)
            self.f0 = np.concatenate([dP[0], dR[0]])
            self.f1 = np.concatenate([dP[1], dR[1]])
        else:
            self.c, self.s, self.f0, self.f1, self.G, self.H = pauli_frame(self.cb, self.sb, self.p, self.r, H0)
        n = self.n
        self.idx = np.arange(1 << n, dtype=np.int64)
        self.bits = [((self.idx >> q) & 1).astype(bool) for q in range(n)]
        self.cz = np.where(np.bitwise_count(self.idx & (self.idx >> 1) & ((1 << (n - 1)) - 1)) & 1, -1.0, 1.0)
        self.groups = []
        for v in self.plan["views"]:
            perm, gm = v["perm"], v["group_mask"]
            self.groups.append([perm[pos] for pos in range(13) if (gm >> pos) & 1])

    # --- circuit pieces -------------------------------------------------
    def init_state(self, b):
        n = self.n
        psi = np.ones(1, dtype=complex)
        for q in range(n - 1, -1, -1):
            c, s = np.cos(self.x[b, q] / 2), np.sin(self.x[b, q] / 2)
            v = np.array([self.r[0, q] * c, np.conj(self.r[0, q]) * s])
            u = np.array([[self.cb[0, q], -self.sb[0, q]], [self.sb[0, q], self.cb[0, q]]]) @ v
            if self.G[0, q]:
                u = u[::-1]
            psi = np.kron(psi, u)
        return psi

    def rot(self, psi, l, qubits, inverse=False):
        psi = psi.copy()
        for q in qubits:
            c, s = self.c[l, q], self.s[l, q] * (-1 if inverse else 1)
            v = psi.reshape(-1, 2, 1 << q)
            a, bb = v[:, 0, :].copy(), v[:, 1, :].copy()
            v[:, 0, :] = c * a - s * bb
            v[:, 1, :] = s * a + c * bb
        return psi

    def diag(self, l):
        d = np.ones(1 << self.n, dtype=complex) if self.cnot else self.cz.astype(complex)
        for q in range(self.n):
            d = d * np.where(self.bits[q], self.f1[l, q], self.f0[l, q])
        return d

    def stats(self, psi, lam, q, weight=None):
        """Im<lam|s_q|psi> for s = X, Y, Z; with `weight` (a +-1 per amplitude that does
        not depend on bit q), Im<lam|W s_q|psi> for the diagonal W."""
        b = self.bits[q]
        i0 = self.idx[~b]
        i1 = i0 | (1 << q)
        li, lj, pi, pj = lam[i0], lam[i1], psi[i0], psi[i1]
        wt = 1.0 if weight is None else weight[i0]
        sx = np.sum(wt * (np.imag(np.conj(li) * pj) + np.imag(np.conj(lj) * pi)))
        sy = np.sum(wt * (np.real(np.conj(lj) * pi) - np.real(np.conj(li) * pj)))
        sz = np.sum(wt * (np.imag(np.conj(li) * pi) - np.imag(np.conj(lj) * pj)))
        return np.array([sx, sy, sz])

    def neighbour_sign(self, q):
        """The eigenvalue of Z_{q-1} Z_{q+1} (chain neighbours of q) on every basis state."""
        s = np.ones(1 << self.n)
        for r in (q - 1, q + 1):
            if 0 <= r < self.n:
                s = s * np.where(self.bits[r], -1.0, 1.0)
        return s

    def merged_stats(self, psi, lam, q, la, lb):
        """Both layers' statistics of qubit q from one point: the output of a pass
        [.., D_la, Ry-layer lb on q's group] (or any point after it that only other,
        non-neighbouring group qubits' rotations separate from it).  Layer lb's are the
        plain sums; layer la's follow from the sums weighted by Z_{q-1} Z_{q+1}:
        D X_q D^dag = Z_{q-1} Z_{q+1} (Re rho X_q - Im rho Y_q), D Y_q D^dag =
        Z_{q-1} Z_{q+1} (Im rho X_q + Re rho Y_q), rho = f0 conj(f1) of qubit q in D_la,
        and Ry(b) X Ry(b)^dag = cos b X - sin b Z, Ry(b) Z Ry(b)^dag = cos b Z + sin b X."""
        X, Y, Zs = self.stats(psi, lam, q)
        sX, sY, sZ = self.stats(psi, lam, q, self.neighbour_sign(q))
        rho = self.f0[la, q] * np.conj(self.f1[la, q])
        c, s = self.c[lb, q], self.s[lb, q]
        cb, sb = c * c - s * s, 2.0 * c * s
        t = cb * sX - sb * sZ
        early = np.array([rho.real * t - rho.imag * sY, rho.imag * t + rho.real * sY, cb * Zs + sb * X])
        return np.array([X, Y, Zs]), early

    # --- fused passes -------------------------------------------------
    def chain(self, i):
        """P(i): bit k = parity of bits 0..k of i."""
        for sh in (1, 2, 4, 8, 16):
            i = i ^ (i << sh)
        return i & ((1 << self.n) - 1)

    def chain_inv(self, j):
        return (j ^ (j << 1)) & ((1 << self.n) - 1)

    def forward_pass(self, k, psi, b):
        ps = self.plan["passes"][k]
        g = self.groups[ps["view"]]
        if ps.get("gather"):
            psi = psi[self.chain_inv(self.idx)]
        if ps["init"]:
            psi = self.init_state(b)
        if ps["rotA"] >= 0:
            psi = self.rot(psi, ps["rotA"], g)
        if ps["diag"] >= 0:
            psi = psi * self.diag(ps["diag"])
        if ps["rotB"] >= 0:
            psi = self.rot(psi, ps["rotB"], g)
        return psi

    def run_sample(self, b):
        if self.cnot:
            return self.run_sample_cnot(b)
        P = len(self.plan["passes"])
        outs = []
        psi = None
        for k in range(P):
            psi = self.forward_pass(k, psi, b)
            outs.append(psi)
        e = float(np.sum(np.where(self.bits[0], -1.0, 1.0) * np.abs(psi) ** 2))
        lam = np.where(self.bits[0], -1.0, 1.0) * psi
        part = {}
        for k in range(P - 1, -1, -1):
            ps = self.plan["passes"][k]
            g = self.groups[ps["view"]]
            v = self.plan["views"][ps["view"]]
            inv = {q: pos for pos, q in enumerate(v["perm"])}
            psi = outs[k]
            if ps["rotB"] >= 0 and self.merged:
                # the adjoint kernel's form: both layers from the pass output, psi never
                # un-rotated (the view's group has no two chain neighbours)
                for q in g:
                    late, early = self.merged_stats(psi, lam, q, ps["diag"], ps["rotB"])
                    part[(k, (13 + inv[q]) * 3)] = late
                    part[(k, inv[q] * 3)] = early
                lam = self.rot(lam, ps["rotB"], g, inverse=True) * np.conj(self.diag(ps["diag"]))
                if not ps["init"]:
                    lam = self.rot(lam, ps["rotA"], g, inverse=True)
            elif ps["rotB"] >= 0:
                for q in g:
                    part[(k, (13 + inv[q]) * 3)] = self.stats(psi, lam, q)
                psi = self.rot(psi, ps["rotB"], g, inverse=True)
                lam = self.rot(lam, ps["rotB"], g, inverse=True)
                d = np.conj(self.diag(ps["diag"]))
                psi, lam = psi * d, lam * d
                for q in g:
                    part[(k, inv[q] * 3)] = self.stats(psi, lam, q)
                if not ps["init"]:
                    lam = self.rot(lam, ps["rotA"], g, inverse=True)
            elif ps["rotA"] >= 0:
                for q in g:
                    part[(k, inv[q] * 3)] = self.stats(psi, lam, q)
                lam = self.rot(lam, ps["rotA"], g, inverse=True)
            else:
                for q in g:
                    part[(k, inv[q] * 3)] = self.stats(psi, lam, q)
        psi0 = self.init_state(b)
        for i, vi in enumerate(self.plan["stats_only"]):
            v = self.plan["views"][vi]
            inv = {q: pos for pos, q in enumerate(v["perm"])}
            for q in self.groups[vi]:
                part[(P + i, inv[q] * 3)] = self.stats(psi0, lam, q)
        S = np.zeros((self.L, self.n, 3))
        for l in range(self.L):
            for q in range(self.n):
                pk, slot = self.plan["statmap"][l * self.n + q]
                S[l, q] = part[(pk, slot)]
        return e, S

    def run_sample_cnot(self, b, zmask=1):
        P = len(self.plan["passes"])
        outs = []
        psi = None
        for k in range(P):
            psi = self.forward_pass(k, psi, b)
            outs.append(psi)
        # the passes stop before the last chain: measure P^dag Z_S P = Z_S'
        zs = zmask
        for sh in (1, 2, 4, 8, 16):
            zs ^= zs >> sh
        sign = np.where(np.bitwise_count(self.idx & zs) & 1, -1.0, 1.0)
        e = float(np.sum(sign * np.abs(psi) ** 2))
        lam = sign * psi
        part = {}
        psi0 = self.init_state(b)

        def inv_of(vi):
            return {q: pos for pos, q in enumerate(self.plan["views"][vi]["perm"])}

        for k in range(P - 1, -1, -1):
            ps = self.plan["passes"][k]
            g = self.groups[ps["view"]]
            inv = inv_of(ps["view"])
            psi = outs[k]
            if ps["init"]:
                l0 = lam * np.conj(self.diag(ps["diag"]))
                for q in g:
                    part[(k, inv[q] * 3)] = self.stats(psi0, l0, q)
            elif ps["rotB"] >= 0:          # [diag(r_l), rot] read through P^-1
                for q in g:
                    part[(k, (13 + inv[q]) * 3)] = self.stats(psi, lam, q)
                lam = self.rot(lam, ps["rotB"], g, inverse=True)
                lam = lam * np.conj(self.diag(ps["diag"]))
                lam = lam[self.chain(self.idx)]
            else:                           # [rot] or [rot, diag(p_l)]
                if ps["diag"] >= 0:
                    d = np.conj(self.diag(ps["diag"]))
                    psi, lam = psi * d, lam * d
                for q in g:
                    part[(k, inv[q] * 3)] = self.stats(psi, lam, q)
                lam = self.rot(lam, ps["rotA"], g, inverse=True)
        l0 = lam * np.conj(self.diag(0))
        for i, vi in enumerate(self.plan["stats_only"]):
            inv = inv_of(vi)
            for q in self.groups[vi]:
                part[(P + i, inv[q] * 3)] = self.stats(psi0, l0, q)
        S = np.zeros((self.L, self.n, 3))
        for l in range(self.L):
            for q in range(self.n):
                pk, slot = self.plan["statmap"][l * self.n + q]
                S[l, q] = part[(pk, slot)]
        return e, S

    def backward(self, dlde):
        B = self.x.shape[0]
        E = np.zeros(B)
        grad = np.zeros((self.L, self.n, 3))
        for b in range(B):
            E[b], S = self.run_sample(b)
            grad += dlde[b] * np.einsum("lqas,lqs->lqa", self.H, S)
        return E, grad
