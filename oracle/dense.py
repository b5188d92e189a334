"""Dense-matrix checker for tiny circuits -- TEST INFRASTRUCTURE ONLY.

A structurally different second oracle for n <= 4 qubits: every gate is
expanded to its full 2^n x 2^n matrix with Kronecker products, the circuit
unitary is the ordinary matrix product of those, and the gradient is the
derivative of that product taken term by term (the product rule), with no
adjoint state at all.  Used to check the gate-by-gate oracle in
``hqml_oracle.c``; it shares no code with it.

Conventions are the same readings as the gate-by-gate oracle: qubit q is bit q
of the amplitude index, so in a Kronecker product the factor for qubit 0 is the
rightmost one; R_s(t) = exp(-i t s/2); encoding Ry(x_q) on |0...0>; each layer
applies Rx, Ry, Rz to every qubit, then CZ(q, q+1) for q = 0..n-2 (entangler 0)
or CNOT(q, q+1), control q, for q = 0, 1, ..., n-2 in that order (entangler 1),
each CNOT built as the sum of two Kronecker products; O = the
Kronecker product of one Pauli matrix per qubit: Z where only the z mask has the
qubit, X where only the x mask has it, Y where both do, I elsewhere (default Z_0).
"""
from __future__ import annotations

import numpy as np
import scipy.linalg

PAULI = {
    "X": np.array([[0, 1], [1, 0]], dtype=np.complex128),
    "Y": np.array([[0, -1j], [1j, 0]], dtype=np.complex128),
    "Z": np.array([[1, 0], [0, -1]], dtype=np.complex128),
}
AXES = ("X", "Y", "Z")


def rot(axis: str, t: float) -> np.ndarray:
    """exp(-i t s/2), taken with the matrix exponential (not the closed form)."""
    return scipy.linalg.expm(-0.5j * float(t) * PAULI[axis])


def rot_deriv(axis: str, t: float) -> np.ndarray:
    """d/dt exp(-i t s/2) = (-i/2) s exp(-i t s/2)."""
    return -0.5j * PAULI[axis] @ rot(axis, t)


def embed(op2: np.ndarray, q: int, n: int) -> np.ndarray:
    """Full matrix of a single-qubit operator on qubit q (qubit 0 rightmost)."""
    out = np.array([[1.0 + 0j]])
    for k in range(n - 1, -1, -1):
        out = np.kron(out, op2 if k == q else np.eye(2))
    return out


def cz(q: int, n: int) -> np.ndarray:
    """Full diagonal matrix of CZ on qubits q and q+1."""
    d = np.ones(1 << n, dtype=np.complex128)
    for i in range(1 << n):
        if (i >> q) & 1 and (i >> (q + 1)) & 1:
            d[i] = -1.0
    return np.diag(d)


def cnot(c: int, t: int, n: int) -> np.ndarray:
    """Full matrix of CNOT(c, t) = |0><0|_c (x) I + |1><1|_c (x) X_t."""
    p0 = np.array([[1, 0], [0, 0]], dtype=np.complex128)
    p1 = np.array([[0, 0], [0, 1]], dtype=np.complex128)

    def kron_all(factors):
        out = np.array([[1.0 + 0j]])
        for k in range(n - 1, -1, -1):
            out = np.kron(out, factors.get(k, np.eye(2)))
        return out

    return kron_all({c: p0}) + kron_all({c: p1, t: PAULI["X"]})


def gate_list(x, theta, n, entangler: int = 0):
    """The circuit as a list of (matrix, parameter index or None, derivative)."""
    theta = np.asarray(theta, dtype=np.float64).reshape(-1, n, 3)
    gates = []
    for q in range(n):
        gates.append((embed(rot("Y", x[q]), q, n), None, None))
    for l in range(theta.shape[0]):
        for q in range(n):
            for a, ax in enumerate(AXES):
                t = theta[l, q, a]
                gates.append((embed(rot(ax, t), q, n), (l, q, a), embed(rot_deriv(ax, t), q, n)))
        for q in range(n - 1):
            gates.append((cnot(q, q + 1, n) if entangler else cz(q, n), None, None))
    return gates


def state(x, theta, entangler: int = 0) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64).ravel()
    n = x.size
    psi0 = np.zeros(1 << n, dtype=np.complex128)
    psi0[0] = 1.0
    U = np.eye(1 << n, dtype=np.complex128)
    for g, _, _ in gate_list(x, theta, n, entangler):
        U = g @ U
    return U @ psi0


def observable(n: int, zmask: int = 1, xmask: int = 0) -> np.ndarray:
    """Full matrix of the Pauli string given by the two masks."""
    out = np.array([[1.0 + 0j]])
    for k in range(n - 1, -1, -1):
        z, xb = (zmask >> k) & 1, (xmask >> k) & 1
        f = PAULI["Y"] if (z and xb) else PAULI["Z"] if z else PAULI["X"] if xb else np.eye(2)
        out = np.kron(out, f)
    return out


def expz(x, theta, zmask: int = 1, xmask: int = 0, entangler: int = 0) -> float:
    x = np.asarray(x, dtype=np.float64).ravel()
    n = x.size
    psi = state(x, theta, entangler)
    O = observable(n, zmask, xmask)
    return float(np.real(np.vdot(psi, O @ psi)))


def grad_expz(x, theta, zmask: int = 1, xmask: int = 0, entangler: int = 0) -> np.ndarray:
    """dE/dtheta [L][n][3] by the product rule on the dense circuit unitary."""
    x = np.asarray(x, dtype=np.float64).ravel()
    n = x.size
    theta = np.asarray(theta, dtype=np.float64).reshape(-1, n, 3)
    gates = gate_list(x, theta, n, entangler)
    psi0 = np.zeros(1 << n, dtype=np.complex128)
    psi0[0] = 1.0
    O = observable(n, zmask, xmask)
    # prefix[k] = G_{k-1} ... G_0 psi0 ; suffix[k] = G_{m-1} ... G_{k+1}
    prefix = [psi0]
    for g, _, _ in gates:
        prefix.append(g @ prefix[-1])
    psi = prefix[-1]
    grad = np.zeros_like(theta)
    suffix = np.eye(1 << n, dtype=np.complex128)
    for k in range(len(gates) - 1, -1, -1):
        g, idx, dg = gates[k]
        if idx is not None:
            dpsi = suffix @ (dg @ prefix[k])
            grad[idx] = 2.0 * np.real(np.vdot(psi, O @ dpsi))
        suffix = suffix @ g
    return grad
