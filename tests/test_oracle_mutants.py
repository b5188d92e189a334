"""Planted mistakes in the oracle are caught by its pins.

Each case copies ``oracle/hqml_oracle.c``, makes one plausible mistake in the
copy (a wrong sign, a dropped term, a wrong index, a swapped order), compiles
it into a temporary directory and runs every pin on it.  At least one pin must
fail, otherwise the pins would not be able to tell the oracle from that
mistake.  Nothing here touches the real oracle build or the GPU.
"""
import os

import pytest

import oracle
import oracle_pins

# (name, exact text in the oracle source, replacement, occurrence to change: 0-based)
MUTANTS = [
    ("rx_sign", "g.m[0] = c; g.m[1] = -I * s; g.m[2] = -I * s; g.m[3] = c;",
     "g.m[0] = c; g.m[1] = I * s; g.m[2] = I * s; g.m[3] = c;", 0),
    ("ry_transposed", "g.m[0] = c; g.m[1] = -s; g.m[2] = s; g.m[3] = c;",
     "g.m[0] = c; g.m[1] = s; g.m[2] = -s; g.m[3] = c;", 0),
    ("rz_sign", "g.m[0] = c - I * s; g.m[1] = 0; g.m[2] = 0; g.m[3] = c + I * s;",
     "g.m[0] = c + I * s; g.m[1] = 0; g.m[2] = 0; g.m[3] = c - I * s;", 0),
    ("full_angle", "const double c = cos(0.5 * t), s = sin(0.5 * t);",
     "const double c = cos(t), s = sin(t);", 0),
    ("entangler_chain_short", "for (int q = 0; q + 1 < n; ++q) {\n        if (ent == ENT_CNOT)",
     "for (int q = 0; q + 2 < n; ++q) {\n        if (ent == ENT_CNOT)", 0),
    ("cz_wrong_pair", "const int64_t both = ((int64_t)1 << q) | ((int64_t)1 << (q + 1));",
     "const int64_t both = ((int64_t)1 << q) | ((int64_t)1 << ((q + 2) % n));", 0),
    ("gate_order_zyx", "for (int a = 0; a < 3; ++a)\n                apply_1q(psi, n, q, rotation(a,",
     "for (int a = 2; a >= 0; --a)\n                apply_1q(psi, n, q, rotation(a,", 0),
    ("encode_rx", "apply_1q(psi, n, q, rotation(AX_Y, x[q]), par);",
     "apply_1q(psi, n, q, rotation(AX_X, x[q]), par);", 0),
    ("observable_shifted_qubit", "return (__builtin_popcountll((uint64_t)i & zmask) & 1) ? -1.0 : 1.0;",
     "return (__builtin_popcountll(((uint64_t)i << 1) & zmask) & 1) ? -1.0 : 1.0;", 0),
    ("observable_ignores_z_mask", "out[i] = ph * zs_sign(j, zmask) * psi[j];", "out[i] = ph * zs_sign(j, 1u) * psi[j];", 0),
    ("observable_sign_before_flip", "out[i] = ph * zs_sign(j, zmask) * psi[j];",
     "out[i] = ph * zs_sign(i, zmask) * psi[j];", 0),
    ("observable_no_flip", "const int64_t j = i ^ (int64_t)xmask;", "const int64_t j = i;", 0),
    ("observable_y_phase_dropped", "const cplx ph = ipow[__builtin_popcount(zmask & xmask) & 3];",
     "const cplx ph = 1.0;", 0),
    ("expectation_conjugate_dropped", "acc += creal(conj(psi[i]) * scratch[i]);",
     "acc += creal(psi[i] * scratch[i]);", 0),
    ("seed_no_factor2", "for (int64_t i = 0; i < dim; ++i) lam[i] *= 2.0 * g;",
     "for (int64_t i = 0; i < dim; ++i) lam[i] *= g;", 0),
    ("no_uncompute", "apply_1q(psi, n, q, dagger(u), par);", "(void)u;", 0),
    ("lambda_not_propagated", "apply_1q(lam, n, q, dagger(u), par);", "(void)u;", 0),
    ("ry_derivative_sign", "g.m[0] = -0.5 * s; g.m[1] = -0.5 * c; g.m[2] = 0.5 * c;",
     "g.m[0] = -0.5 * s; g.m[1] = 0.5 * c; g.m[2] = -0.5 * c;", 0),
    ("braket_conjugate_dropped", "acc += creal(conj(lam[i]) * di) + creal(conj(lam[j]) * dj);",
     "acc += creal(lam[i] * di) + creal(lam[j] * dj);", 0),
    ("mse_no_mean", "const double g = 2.0 * (expz[b] - y[b]) / (double)B;",
     "const double g = 2.0 * (expz[b] - y[b]);", 0),
    ("cnot_control_target_swapped", "apply_cnot(psi, n, q, q + 1, par);",
     "apply_cnot(psi, n, q + 1, q, par);", 0),
    ("cnot_chain_reversed", "apply_cnot(psi, n, q, q + 1, par);",
     "apply_cnot(psi, n, n - 2 - q, n - 1 - q, par);", 0),
    ("cnot_undo_in_circuit_order", "for (int q = n - 2; q >= 0; --q) {\n        if (ent == ENT_CNOT)",
     "for (int q = 0; q + 1 < n; ++q) {\n        if (ent == ENT_CNOT)", 0),
    ("cnot_swaps_every_pair", "if (!(i & cb) || (i & tb)) continue;", "if (i & tb) continue;", 0),
    ("theta_index_transposed", "rotation(a, theta[((size_t)l * n + q) * 3 + a]), par);",
     "rotation(a, theta[((size_t)q * (L > 0 ? L : 1) + (l % (n > 0 ? n : 1))) * 3 + a]), par);", 0),
]


def _mutate(src: str, old: str, new: str, k: int) -> str:
    pos = -1
    for _ in range(k + 1):
        pos = src.index(old, pos + 1)
    return src[:pos] + new + src[pos + len(old):]


@pytest.mark.parametrize("name,old,new,k", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, old, new, k, tmp_path):
    src = open(oracle.SOURCE).read()
    assert old in src, f"mutation anchor for {name} no longer in the oracle source"
    mutated = _mutate(src, old, new, k)
    c = os.path.join(tmp_path, f"{name}.c")
    with open(c, "w") as f:
        f.write(mutated)
    so = oracle.compile_source(c, os.path.join(tmp_path, f"lib{name}.so"))
    o = oracle.Oracle(so)
    failed = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(o)
        except AssertionError:
            failed.append(pin.__name__)
        except ValueError:
            failed.append(pin.__name__ + " (rejected)")
    assert failed, f"no pin catches the planted mistake {name}"
