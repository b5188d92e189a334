/*
 * hqml oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, gate-by-gate fp64 state-vector simulation of the
 * hardware-efficient ansatz (HEA) training step, with the adjoint-method
 * gradient.  Only the tests, the smoke check and the benchmark's CPU-baseline
 * leg may load it; the product path never does.  It shares no code with the
 * GPU path (no headers, tables or helpers).
 *
 * What it computes follows Kawase, "Fast and memory-efficient classical
 * simulation of quantum machine learning via forward and backward gate
 * fusion" (arXiv:2603.02804), as summarised on the hugo-pages page
 * "深度解析：正向与反向门融合驱动的高效量子机器学习仿真":
 *   section 1.2: the state is a vector in C^(2^n); a parameterised circuit is
 *     a sequence of rotation gates U_j(theta_j); E(theta) = <psi_M|O|psi_M>;
 *     the adjoint gradient is dL/dtheta_j = Re<lambda_j| dU_j/dtheta_j |psi_{j-1}>
 *     with lambda_{j-1} = U_j^dagger lambda_j;
 *   section 2.1: the HEA uses single-qubit Rx, Ry, Rz rotations and CZ gates;
 *   section 3.2: CZ is a sign flip when both qubit bits are set; CNOT gates are
 *     fused by recomputing amplitude indices (a CNOT permutes basis states).
 * Circuit details the pages leave open are fixed as follows (each is a reading,
 * listed with its reason in the design notes):
 *   - qubit q is bit q of the amplitude index (qubit 0 = least significant);
 *   - R_s(t) = exp(-i t s / 2) for s in {X, Y, Z};
 *   - encoding: Ry(x_q)|0> on every qubit, once;
 *   - layer l: on every qubit q apply Rx(theta[l][q][0]), then Ry(theta[l][q][1]),
 *     then Rz(theta[l][q][2]); then the entangler: CZ(q, q+1) for q = 0..n-2 (open
 *     chain, the default), or, as the second entangler, CNOT(q, q+1) (control q,
 *     target q+1) for q = 0, 1, ..., n-2 in that order;
 *   - observable O = a Pauli string, the general O of section 1.2 restricted to
 *     tensor products of I, X, Y, Z: two bit masks (bit q = qubit q) give qubit
 *     q the factor I (in neither), Z (z only), X (x only) or Y (both); the default
 *     is z = {0}, x = {} (Z on qubit 0); loss = mean over the batch of (E_b - y_b)^2;
 *   - the factor 2 of d<psi|O|psi> is carried by the adjoint seed:
 *     lambda_M = 2 (dL/dE) O psi_M, so the section-1.2 gradient formula holds
 *     literally.
 *
 * Numbers are fp64 throughout; fp32 inputs are promoted by the caller.
 * Samples are independent; OpenMP runs them in parallel (or, for a batch too
 * small to fill the threads, runs the amplitude loops in parallel).  Every sum
 * over amplitudes has one fixed order that depends only on the number of
 * amplitudes (sum_blocks below), whether its blocks run on one thread or many,
 * and per-sample results are summed over the batch in sample order, so results
 * do not depend on the thread count.
 */
#include <complex.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

typedef double _Complex cplx;

/* A 2x2 complex matrix, row major: m[0]=U00, m[1]=U01, m[2]=U10, m[3]=U11. */
typedef struct { cplx m[4]; } gate2;

enum { AX_X = 0, AX_Y = 1, AX_Z = 2 };

/* R_s(t) = exp(-i t s/2) = cos(t/2) I - i sin(t/2) s. */
static gate2 rotation(int axis, double t)
{
    const double c = cos(0.5 * t), s = sin(0.5 * t);
    gate2 g;
    switch (axis) {
    case AX_X: /* [[c, -i s], [-i s, c]] */
        g.m[0] = c; g.m[1] = -I * s; g.m[2] = -I * s; g.m[3] = c;
        break;
    case AX_Y: /* [[c, -s], [s, c]] */
        g.m[0] = c; g.m[1] = -s; g.m[2] = s; g.m[3] = c;
        break;
    default:   /* diag(e^{-i t/2}, e^{+i t/2}) */
        g.m[0] = c - I * s; g.m[1] = 0; g.m[2] = 0; g.m[3] = c + I * s;
        break;
    }
    return g;
}

/* d/dt R_s(t) = -(i/2) s R_s(t), written out element by element. */
static gate2 rotation_derivative(int axis, double t)
{
    const double c = cos(0.5 * t), s = sin(0.5 * t);
    gate2 g;
    switch (axis) {
    case AX_X: /* d/dt [[c, -i s], [-i s, c]] */
        g.m[0] = -0.5 * s; g.m[1] = -0.5 * I * c; g.m[2] = -0.5 * I * c; g.m[3] = -0.5 * s;
        break;
    case AX_Y: /* d/dt [[c, -s], [s, c]] */
        g.m[0] = -0.5 * s; g.m[1] = -0.5 * c; g.m[2] = 0.5 * c; g.m[3] = -0.5 * s;
        break;
    default:   /* d/dt diag(c - i s, c + i s) */
        g.m[0] = -0.5 * s - 0.5 * I * c; g.m[1] = 0; g.m[2] = 0; g.m[3] = -0.5 * s + 0.5 * I * c;
        break;
    }
    return g;
}

static gate2 dagger(gate2 g)
{
    gate2 d;
    d.m[0] = conj(g.m[0]); d.m[1] = conj(g.m[2]);
    d.m[2] = conj(g.m[1]); d.m[3] = conj(g.m[3]);
    return d;
}

/* Apply a single-qubit gate to qubit q: for every index i with bit q clear and
 * j = i | 2^q, (psi_i, psi_j) <- (U00 psi_i + U01 psi_j, U10 psi_i + U11 psi_j). */
static void apply_1q(cplx *psi, int n, int q, gate2 g, int par)
{
    const int64_t dim = (int64_t)1 << n;
    const int64_t bit = (int64_t)1 << q;
    (void)par;
#pragma omp parallel for if (par) schedule(static)
    for (int64_t i = 0; i < dim; ++i) {
        if (i & bit) continue;
        const int64_t j = i | bit;
        const cplx a = psi[i], b = psi[j];
        psi[i] = g.m[0] * a + g.m[1] * b;
        psi[j] = g.m[2] * a + g.m[3] * b;
    }
}

/* CZ(q, q+1): negate every amplitude whose bits q and q+1 are both set. */
static void apply_cz(cplx *psi, int n, int q, int par)
{
    const int64_t dim = (int64_t)1 << n;
    const int64_t both = ((int64_t)1 << q) | ((int64_t)1 << (q + 1));
    (void)par;
#pragma omp parallel for if (par) schedule(static)
    for (int64_t i = 0; i < dim; ++i)
        if ((i & both) == both) psi[i] = -psi[i];
}

/* CNOT(c, t): swap the amplitudes of i and i ^ 2^t wherever bit c of i is set. */
static void apply_cnot(cplx *psi, int n, int c, int t, int par)
{
    const int64_t dim = (int64_t)1 << n;
    const int64_t cb = (int64_t)1 << c, tb = (int64_t)1 << t;
    (void)par;
#pragma omp parallel for if (par) schedule(static)
    for (int64_t i = 0; i < dim; ++i) {
        if (!(i & cb) || (i & tb)) continue;
        const cplx a = psi[i];
        psi[i] = psi[i | tb];
        psi[i | tb] = a;
    }
}

enum { ENT_CZ = 0, ENT_CNOT = 1 };

/* The entangling block that ends every layer, in circuit order. */
static void apply_entangler(cplx *psi, int n, int ent, int par)
{
    for (int q = 0; q + 1 < n; ++q) {
        if (ent == ENT_CNOT)
            apply_cnot(psi, n, q, q + 1, par);
        else
            apply_cz(psi, n, q, par);
    }
}

/* Its inverse: the same self-inverse gates in reverse order. */
static void undo_entangler(cplx *psi, int n, int ent, int par)
{
    for (int q = n - 2; q >= 0; --q) {
        if (ent == ENT_CNOT)
            apply_cnot(psi, n, q, q + 1, par);
        else
            apply_cz(psi, n, q, par);
    }
}

/* Summation order of every sum over the 2^n amplitude indices: the range is cut
 * into SUM_BLOCKS equal blocks of consecutive indices (one block below 2^12
 * indices), each block is summed in index order, and the block sums are added
 * in block order.  The order depends on n only; 'par' only lets the blocks run
 * on several threads. */
enum { SUM_BLOCKS = 64 };

static int64_t sum_blocks(int64_t dim) { return dim >= 4096 ? SUM_BLOCKS : 1; }

static double add_blocks(const double *part, int64_t nb)
{
    double acc = 0.0;
    for (int64_t c = 0; c < nb; ++c) acc += part[c];
    return acc;
}

/* Re<lam| D_q |phi>, D a 2x2 matrix on qubit q (fixed order, see sum_blocks). */
static double re_braket_1q(const cplx *lam, const cplx *phi, int n, int q, gate2 d, int par)
{
    const int64_t dim = (int64_t)1 << n;
    const int64_t bit = (int64_t)1 << q;
    const int64_t nb = sum_blocks(dim), len = dim / nb;
    double part[SUM_BLOCKS];
    (void)par;
#pragma omp parallel for if (par) schedule(static)
    for (int64_t c = 0; c < nb; ++c) {
        double acc = 0.0;
        for (int64_t i = c * len; i < (c + 1) * len; ++i) {
            if (i & bit) continue;
            const int64_t j = i | bit;
            const cplx di = d.m[0] * phi[i] + d.m[1] * phi[j];
            const cplx dj = d.m[2] * phi[i] + d.m[3] * phi[j];
            acc += creal(conj(lam[i]) * di) + creal(conj(lam[j]) * dj);
        }
        part[c] = acc;
    }
    return add_blocks(part, nb);
}

/* (-1)^(number of qubits of S set in basis state i): the eigenvalue of prod_{q in S} Z_q. */
static double zs_sign(int64_t i, uint32_t zmask)
{
    return (__builtin_popcountll((uint64_t)i & zmask) & 1) ? -1.0 : 1.0;
}

/* out = O psi for the Pauli string (zmask, xmask).  Each Y is i X Z on its qubit, so
 * O = i^(#Y) X^xmask Z^zmask, and
 *   (O psi)_i = i^(#Y) (-1)^|(i ^ xmask) & zmask| psi_(i ^ xmask). */
static void apply_observable(const cplx *psi, cplx *out, int n, uint32_t zmask, uint32_t xmask, int par)
{
    const int64_t dim = (int64_t)1 << n;
    static const double _Complex ipow[4] = {1.0, I, -1.0, -I};
    const cplx ph = ipow[__builtin_popcount(zmask & xmask) & 3];
    (void)par;
#pragma omp parallel for if (par) schedule(static)
    for (int64_t i = 0; i < dim; ++i) {
        const int64_t j = i ^ (int64_t)xmask;
        out[i] = ph * zs_sign(j, zmask) * psi[j];
    }
}

/* <psi|O|psi> (real: O is Hermitian).  scratch holds 2^n amplitudes. */
static double expect_obs(const cplx *psi, cplx *scratch, int n, uint32_t zmask, uint32_t xmask, int par)
{
    const int64_t dim = (int64_t)1 << n;
    const int64_t nb = sum_blocks(dim), len = dim / nb;
    double part[SUM_BLOCKS];
    apply_observable(psi, scratch, n, zmask, xmask, par);
#pragma omp parallel for if (par) schedule(static)
    for (int64_t c = 0; c < nb; ++c) {
        double acc = 0.0;
        for (int64_t i = c * len; i < (c + 1) * len; ++i) acc += creal(conj(psi[i]) * scratch[i]);
        part[c] = acc;
    }
    return add_blocks(part, nb);
}

/* psi <- encoding followed by all L layers; |psi| must hold 2^n amplitudes. */
static void run_circuit(cplx *psi, int n, int L, const double *x, const double *theta, int ent, int par)
{
    const int64_t dim = (int64_t)1 << n;
    memset(psi, 0, sizeof(cplx) * (size_t)dim);
    psi[0] = 1.0;
    for (int q = 0; q < n; ++q) apply_1q(psi, n, q, rotation(AX_Y, x[q]), par);
    for (int l = 0; l < L; ++l) {
        for (int q = 0; q < n; ++q)
            for (int a = 0; a < 3; ++a)
                apply_1q(psi, n, q, rotation(a, theta[((size_t)l * n + q) * 3 + a]), par);
        apply_entangler(psi, n, ent, par);
    }
}

/* Adjoint sweep for one sample.  psi holds psi_M on entry (it is uncomputed
 * gate by gate), lam is scratch.  grad[(l*n+q)*3+a] receives dL/dtheta for
 * upstream derivative g = dL/dE. */
static void adjoint_sample(cplx *psi, cplx *lam, int n, int L, const double *theta, uint32_t zmask,
                           uint32_t xmask, int ent, double g, double *grad, int par)
{
    const int64_t dim = (int64_t)1 << n;
    /* lambda_M = 2 g O psi_M */
    apply_observable(psi, lam, n, zmask, xmask, par);
    for (int64_t i = 0; i < dim; ++i) lam[i] *= 2.0 * g;
    for (int l = L - 1; l >= 0; --l) {
        /* the entangler, gate by gate in reverse order, on both states */
        undo_entangler(psi, n, ent, par);
        undo_entangler(lam, n, ent, par);
        for (int q = n - 1; q >= 0; --q) {
            for (int a = 2; a >= 0; --a) {
                const double t = theta[((size_t)l * n + q) * 3 + a];
                const gate2 u = rotation(a, t);
                /* psi_{j-1} = U_j^dagger psi_j */
                apply_1q(psi, n, q, dagger(u), par);
                /* dL/dtheta_j = Re<lambda_j| dU_j/dtheta_j |psi_{j-1}> */
                grad[((size_t)l * n + q) * 3 + a] =
                    re_braket_1q(lam, psi, n, q, rotation_derivative(a, t), par);
                /* lambda_{j-1} = U_j^dagger lambda_j */
                apply_1q(lam, n, q, dagger(u), par);
            }
        }
    }
}

static int choose_par(int n, int B)
{
#ifdef _OPENMP
    return (B < omp_get_max_threads() && n >= 14) ? 1 : 0;
#else
    (void)n; (void)B;
    return 0;
#endif
}

void oracle_set_num_threads(int t)
{
#ifdef _OPENMP
    if (t > 0) omp_set_num_threads(t);
#else
    (void)t;
#endif
}

int oracle_get_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Final state of one sample after encoding and all L layers (psi: 2^n
 * interleaved (re, im) doubles).  Returns 0, or -1 on bad arguments / memory. */
int oracle_state(int n, int L, int ent, const double *x, const double *theta, double *psi_out)
{
    if (n < 1 || n > 30 || L < 0 || (ent != ENT_CZ && ent != ENT_CNOT) || !x || (L > 0 && !theta) || !psi_out)
        return -1;
    run_circuit((cplx *)psi_out, n, L, x, theta, ent, n >= 14);
    return 0;
}

/* Largest |1 - ||psi||^2| after any single gate of the circuit (unitarity check). */
double oracle_max_norm_drift(int n, int L, int ent, const double *x, const double *theta)
{
    if (n < 1 || n > 24 || L < 0 || (ent != ENT_CZ && ent != ENT_CNOT)) return -1.0;
    const int64_t dim = (int64_t)1 << n;
    cplx *psi = (cplx *)calloc((size_t)dim, sizeof(cplx));
    if (!psi) return -1.0;
    double worst = 0.0;
#define HQML_ORACLE_TRACK()                                                        \
    do {                                                                           \
        double nn = 0.0;                                                           \
        for (int64_t i_ = 0; i_ < dim; ++i_)                                       \
            nn += creal(psi[i_]) * creal(psi[i_]) + cimag(psi[i_]) * cimag(psi[i_]); \
        if (fabs(1.0 - nn) > worst) worst = fabs(1.0 - nn);                        \
    } while (0)
    psi[0] = 1.0;
    for (int q = 0; q < n; ++q) { apply_1q(psi, n, q, rotation(AX_Y, x[q]), 0); HQML_ORACLE_TRACK(); }
    for (int l = 0; l < L; ++l) {
        for (int q = 0; q < n; ++q)
            for (int a = 0; a < 3; ++a) {
                apply_1q(psi, n, q, rotation(a, theta[((size_t)l * n + q) * 3 + a]), 0);
                HQML_ORACLE_TRACK();
            }
        for (int q = 0; q + 1 < n; ++q) {
            if (ent == ENT_CNOT)
                apply_cnot(psi, n, q, q + 1, 0);
            else
                apply_cz(psi, n, q, 0);
            HQML_ORACLE_TRACK();
        }
    }
#undef HQML_ORACLE_TRACK
    free(psi);
    return worst;
}

/* Observable masks must name qubits of the circuit; the identity string is rejected. */
static int bad_mask(int n, uint32_t zmask, uint32_t xmask)
{
    return (zmask | xmask) == 0 || (n < 32 && ((zmask | xmask) >> n) != 0);
}

static int bad_ent(int ent) { return ent != ENT_CZ && ent != ENT_CNOT; }

/* E_b = <psi_M|O|psi_M> for every sample.  x: [B][n], theta: [L][n][3]. */
int oracle_forward(int n, int L, int B, uint32_t zmask, uint32_t xmask, int ent, const double *x,
                   const double *theta, double *expz)
{
    if (n < 1 || n > 30 || L < 0 || B < 0 || (B > 0 && (!x || !expz)) || (L > 0 && !theta) ||
        bad_mask(n, zmask, xmask) || bad_ent(ent))
        return -1;
    const int par = choose_par(n, B);
    const int64_t dim = (int64_t)1 << n;
    int err = 0;
#pragma omp parallel for if (!par) schedule(dynamic, 1) reduction(| : err)
    for (int b = 0; b < B; ++b) {
        cplx *psi = (cplx *)malloc(sizeof(cplx) * (size_t)dim);
        cplx *tmp = (cplx *)malloc(sizeof(cplx) * (size_t)dim);
        if (!psi || !tmp) { free(psi); free(tmp); err |= 1; continue; }
        run_circuit(psi, n, L, x + (size_t)b * n, theta, ent, par);
        expz[b] = expect_obs(psi, tmp, n, zmask, xmask, par);
        free(psi);
        free(tmp);
    }
    return err ? -1 : 0;
}

/* Adjoint gradient for an arbitrary upstream derivative dLdE[b]:
 * grad[(l*n+q)*3+a] = sum_b (per-sample adjoint gradient), summed in sample
 * order.  expz (optional) receives E_b. */
int oracle_backward(int n, int L, int B, uint32_t zmask, uint32_t xmask, int ent, const double *x,
                    const double *theta, const double *dLdE, double *grad, double *expz)
{
    if (n < 1 || n > 30 || L < 0 || B < 0 || (B > 0 && (!x || !dLdE)) || (L > 0 && (!theta || !grad)) ||
        bad_mask(n, zmask, xmask) || bad_ent(ent))
        return -1;
    const size_t P = (size_t)L * n * 3;
    const int par = choose_par(n, B);
    const int64_t dim = (int64_t)1 << n;
    double *per = (double *)calloc((size_t)(B > 0 ? B : 1) * (P ? P : 1), sizeof(double));
    if (!per) return -1;
    int err = 0;
#pragma omp parallel for if (!par) schedule(dynamic, 1) reduction(| : err)
    for (int b = 0; b < B; ++b) {
        cplx *psi = (cplx *)malloc(sizeof(cplx) * (size_t)dim);
        cplx *lam = (cplx *)malloc(sizeof(cplx) * (size_t)dim);
        if (!psi || !lam) { free(psi); free(lam); err |= 1; continue; }
        run_circuit(psi, n, L, x + (size_t)b * n, theta, ent, par);
        if (expz) expz[b] = expect_obs(psi, lam, n, zmask, xmask, par);
        adjoint_sample(psi, lam, n, L, theta, zmask, xmask, ent, dLdE[b], per + (size_t)b * P, par);
        free(psi);
        free(lam);
    }
    if (!err) {
        for (size_t p = 0; p < P; ++p) grad[p] = 0.0;
        for (int b = 0; b < B; ++b)
            for (size_t p = 0; p < P; ++p) grad[p] += per[(size_t)b * P + p];
    }
    free(per);
    return err ? -1 : 0;
}

/* One training step with the mean-squared-error loss on <O>:
 * loss = (1/B) sum_b (E_b - y_b)^2, dL/dE_b = 2 (E_b - y_b) / B.
 * Each sample is simulated once: forward, E_b, then its adjoint sweep. */
int oracle_train_step(int n, int L, int B, uint32_t zmask, uint32_t xmask, int ent, const double *x,
                      const double *theta, const double *y, double *expz, double *loss, double *grad)
{
    if (n < 1 || n > 30 || L < 0 || B < 1 || !x || !y || !expz || !loss || (L > 0 && (!theta || !grad)) ||
        bad_mask(n, zmask, xmask) || bad_ent(ent))
        return -1;
    const size_t P = (size_t)L * n * 3;
    const int par = choose_par(n, B);
    const int64_t dim = (int64_t)1 << n;
    double *per = (double *)calloc((size_t)B * (P ? P : 1), sizeof(double));
    if (!per) return -1;
    int err = 0;
#pragma omp parallel for if (!par) schedule(dynamic, 1) reduction(| : err)
    for (int b = 0; b < B; ++b) {
        cplx *psi = (cplx *)malloc(sizeof(cplx) * (size_t)dim);
        cplx *lam = (cplx *)malloc(sizeof(cplx) * (size_t)dim);
        if (!psi || !lam) { free(psi); free(lam); err |= 1; continue; }
        run_circuit(psi, n, L, x + (size_t)b * n, theta, ent, par);
        expz[b] = expect_obs(psi, lam, n, zmask, xmask, par);
        const double g = 2.0 * (expz[b] - y[b]) / (double)B;
        adjoint_sample(psi, lam, n, L, theta, zmask, xmask, ent, g, per + (size_t)b * P, par);
        free(psi);
        free(lam);
    }
    if (!err) {
        double acc = 0.0;
        for (int b = 0; b < B; ++b) {
            const double d = expz[b] - y[b];
            acc += d * d;
        }
        *loss = acc / (double)B;
        for (size_t p = 0; p < P; ++p) grad[p] = 0.0;
        for (int b = 0; b < B; ++b)
            for (size_t p = 0; p < P; ++p) grad[p] += per[(size_t)b * P + p];
    }
    free(per);
    return err ? -1 : 0;
}
