// gfx950 kernel of the whole training step for n <= 13: one workgroup holds one sample's
// state in LDS and runs the forward pass, <O>, the adjoint sweep and the gradient
// statistics (k_small; instance <R, 0> with the CZ chain, <R, 1> with the CNOT chain).
//
// Method: Kawase, arXiv:2603.02804 (hugo-pages summary "深度解析：正向与反向门融合
// 驱动的高效量子机器学习仿真", sections 1.2-1.4 and 3.2).  The layer algebra is described
// in hqml_internal.hpp.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hqml_device.hpp"
#include "hqml_host.hpp"
#include "hqml_internal.hpp"

namespace hqml {

// ------------------------------------------------------------------ small circuits (n <= 13)

constexpr int kSmallThreads = 512;               // eight waves: two per SIMD hide each other's latency
constexpr int kRoundBits = 3;                    // qubits per register round
constexpr int kSmallRows = kSmallThreads / 16;   // DPP row partials per workgroup

// D_l of amplitude i: CZ-chain sign times the per-qubit factors f0 / f1.
template <typename R>
__device__ __forceinline__ V2<R> small_diag(const V4<R> *wl, int n, uint32_t i)
{
    V2<R> f = mk2((R)1, (R)0);
    for (int q = 0; q < n; ++q) {
        const V4<R> g = uniform_v4<R>(wl + q);
        f = cmul(f, ((i >> q) & 1u) ? mk2(g.z, g.w) : mk2(g.x, g.y));
    }
    if (__builtin_popcount(i & (i >> 1)) & 1) {
        f.x = -f.x;
        f.y = -f.y;
    }
    return f;
}

// LDS slot of amplitude i: bits 0..4 XOR bits 3..7 (a bijection: bits 5 and up are
// unchanged, which then fix bits 4, 3 and 0..2 in turn).  With it every round shape
// (qubits 0..2, 3..5, 6..8, 9..11, 12 in registers) gives each 32 consecutive lanes
// distinct 8-byte slots modulo 256 bytes, so the LDS accesses are free of bank conflicts.
__device__ __forceinline__ uint32_t sslot(uint32_t i) { return i ^ ((i >> 3) & 31u); }

// (O phi)_i for the Pauli string (zm, xm), phi = D_trail psi the true final state held
// at slots sslot(i) (wl: the trailing diagonal's factors; applied only when xm != 0,
// since D_trail commutes with Z):  i^(#Y) (-1)^|(i ^ xm) & zm| phi_(i ^ xm).
template <typename R>
__device__ __forceinline__ V2<R> small_obs(const V2<R> *psi, uint32_t i, uint32_t zm, uint32_t xm, const V4<R> *wl,
                                           int n)
{
    const uint32_t j = i ^ xm;
    V2<R> w = psi[sslot(j)];
    if (xm) w = cmul(w, small_diag<R>(wl, n, j));
    R re = (__builtin_popcount(j & zm) & 1) ? -w.x : w.x;
    R im = (__builtin_popcount(j & zm) & 1) ? -w.y : w.y;
    mul_ipow(re, im, __builtin_popcount(zm & xm) & 3);
    return mk2(re, im);
}

// ---- CNOT entangler (whole state in local memory)
//
// The chain CNOT(0,1), CNOT(1,2), ..., CNOT(n-2,n-1), applied in that order, sends basis
// state |i> to |P(i)> where bit k of P(i) is the parity of bits 0..k of i; its inverse
// is P^-1(j) = j ^ (j << 1).  The chain is applied by moving amplitudes to their new
// indices (the hugo-pages summary, section 3.2, fuses CNOTs by recomputing indices).
__device__ __forceinline__ uint32_t cnot_chain(uint32_t i, uint32_t mask)
{
    i ^= i << 1;
    i ^= i << 2;
    i ^= i << 4;
    i ^= i << 8;   // parities of up to 16 low bits; n <= 13 here
    return i & mask;
}

__device__ __forceinline__ uint32_t cnot_chain_inv(uint32_t j, uint32_t mask) { return (j ^ (j << 1)) & mask; }

// Factor of amplitude i in prod_q diag(f_q, conj f_q); f_q = (x, y) of wl[q] (SECOND =
// false) or (z, w) (SECOND = true).
template <bool SECOND, typename R>
__device__ __forceinline__ V2<R> small_phase(const V4<R> *wl, int n, uint32_t i)
{
    V2<R> f = mk2((R)1, (R)0);
    for (int q = 0; q < n; ++q) {
        const V4<R> g = uniform_v4<R>(wl + q);
        V2<R> h = SECOND ? mk2(g.z, g.w) : mk2(g.x, g.y);
        if ((i >> q) & 1u) h.y = -h.y;
        f = cmul(f, h);
    }
    return f;
}

// ---- whole circuit per workgroup with the CZ chain: register rounds
//
// The state of one sample lives in LDS.  A "round" on qubits s .. s+G-1 (G <= 3) hands
// every thread whole groups of 2^G amplitudes {base + (j << s)}, gathers a group into
// registers, applies the round's work there and writes it back, so each LDS round trip
// covers three qubits (eight amplitudes per thread and 512 threads keep two waves on
// each SIMD; four-qubit rounds with one wave per SIMD, and two-qubit rounds with four,
// were slower).  Round 0 (qubits 0 .. G0-1) also applies the merged diagonal D_l,
// factored as T[j] (qubits below G0 and the CZ signs among them: uniform, built once per
// layer) times a per-group factor over the other qubits (with their CZ signs and the
// CZ between qubits G0-1 and G0).  Rotations use the scaled tangent form of rot_bit;
// the uniform scale is carried along and folded into the next diagonal.

template <typename R>
__device__ __forceinline__ R lane_bcast(R v, int lane);

template <>
__device__ __forceinline__ float lane_bcast<float>(float v, int lane)
{
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

template <>
__device__ __forceinline__ double lane_bcast<double>(double v, int lane)
{
    const long long b = __double_as_longlong(v);
    const int lo = __builtin_amdgcn_readlane((int)(b & 0xffffffffll), lane);
    const int hi = __builtin_amdgcn_readlane((int)(b >> 32), lane);
    return __longlong_as_double(((long long)hi << 32) | (unsigned int)lo);
}

// Factor of the low qubits: prod_{q < G0} f_q(bit q of j) for j = lane & 15, with the CZ
// signs among those qubits if cz.  f_q = (x, y) for bit value 0, (z, w) for 1.
template <typename R>
__device__ __forceinline__ V2<R> low_factor(const V4<R> *f, int G0, bool cz, int lane)
{
    const uint32_t j = (uint32_t)lane & 15u;
    V2<R> t = mk2((R)1, (R)0);
    for (int q = 0; q < G0; ++q) {
        const V4<R> g = uniform_v4<R>(f + q);
        t = cmul(t, ((j >> q) & 1u) ? mk2(g.z, g.w) : mk2(g.x, g.y));
    }
    if (cz && (__builtin_popcount(j & (j >> 1) & ((1u << G0) - 1u)) & 1)) t = mk2(-t.x, -t.y);
    return t;
}

// Factor of the high qubits of group g of round 0: prod_{q >= G0} f_q(bit q - G0 of g),
// with the CZ signs among them if cz.
template <int G0, typename R>
__device__ __forceinline__ V2<R> high_factor(const V4<R> *f, int n, uint32_t g, bool cz)
{
    V2<R> h = mk2((R)1, (R)0);
    for (int q = G0; q < n; ++q) {
        const V4<R> w = uniform_v4<R>(f + q);
        h = cmul(h, ((g >> (q - G0)) & 1u) ? mk2(w.z, w.w) : mk2(w.x, w.y));
    }
    if (cz && (__builtin_popcount(g & (g >> 1)) & 1)) h = mk2(-h.x, -h.y);
    return h;
}

template <int G, typename R>
struct SmallGroup {
    R re[1 << G], im[1 << G];
};

template <int G, typename R>
__device__ __forceinline__ void sg_load(SmallGroup<G, R> &v, const V2<R> *st, uint32_t base, int s)
{
#pragma unroll
    for (int j = 0; j < (1 << G); ++j) {
        const V2<R> a = st[sslot(base | ((uint32_t)j << s))];
        v.re[j] = a.x;
        v.im[j] = a.y;
    }
}

template <int G, typename R>
__device__ __forceinline__ void sg_store(const SmallGroup<G, R> &v, V2<R> *st, uint32_t base, int s)
{
#pragma unroll
    for (int j = 0; j < (1 << G); ++j) st[sslot(base | ((uint32_t)j << s))] = mk2(v.re[j], v.im[j]);
}

// Tangent-form rotation of register bit m of a group (INV: the inverse); see rot_bit.
template <int G, bool INV, typename R>
__device__ __forceinline__ void sg_rot(SmallGroup<G, R> &v, int m, R k)
{
    const R kk = INV ? -k : k;
#pragma unroll
    for (int j = 0; j < (1 << G); ++j) {
        if ((j >> m) & 1) continue;
        const int o = j | (1 << m);
        const R ar = v.re[j], ai = v.im[j], br = v.re[o], bi = v.im[o];
        v.re[j] = fmar(-kk, br, ar);
        v.im[j] = fmar(-kk, bi, ai);
        v.re[o] = fmar(kk, ar, br);
        v.im[o] = fmar(kk, ai, bi);
    }
}

// The entries T[j] of the low-qubit factor, held by lanes j = lane & 15, as uniform
// values.  Called with every lane of the wave active (readlane reads a lane whether or
// not it is active, so the entries must be computed outside divergent code).
template <int G, typename R>
__device__ __forceinline__ void bcast_low(V2<R> (&t)[1 << G], V2<R> tl)
{
#pragma unroll
    for (int j = 0; j < (1 << G); ++j) t[j] = mk2(lane_bcast<R>(tl.x, j), lane_bcast<R>(tl.y, j));
}

// Multiply a round-0 group by its diagonal D_j = T[j] * (h or hx).  SEL = 0: hx for j with
// bit G-1 set (the CZ chain's CZ between qubits G-1 and G, or, through the CNOT chain's
// inverse map, bit G of the source index); SEL = 1: hx for j of odd parity (every bit of
// the CNOT chain's image above G flips with it).  CONJ: by conj(D).
template <int G, bool CONJ, int SEL = 0, typename R>
__device__ __forceinline__ void sg_diag(SmallGroup<G, R> &v, const V2<R> (&t)[1 << G], V2<R> h, V2<R> hx)
{
#pragma unroll
    for (int j = 0; j < (1 << G); ++j) {
        const bool x = SEL == 0 ? ((j >> (G - 1)) & 1) != 0 : (__builtin_popcount(j) & 1) != 0;
        V2<R> d = cmul(t[j], x ? hx : h);
        if (CONJ) d.y = -d.y;
        const R re = v.re[j] * d.x - v.im[j] * d.y;
        const R im = v.re[j] * d.y + v.im[j] * d.x;
        v.re[j] = re;
        v.im[j] = im;
    }
}

// Rotation Ry on register bit m of a group in (sin, cos) form (INV: its inverse).
template <int G, bool INV, typename R>
__device__ __forceinline__ void sg_rot_cs(SmallGroup<G, R> &v, int m, R sn, R cs)
{
    const R ss = INV ? -sn : sn;
#pragma unroll
    for (int j = 0; j < (1 << G); ++j) {
        if ((j >> m) & 1) continue;
        const int o = j | (1 << m);
        const R ar = v.re[j], ai = v.im[j], br = v.re[o], bi = v.im[o];
        v.re[j] = fmar(cs, ar, -ss * br);
        v.im[j] = fmar(cs, ai, -ss * bi);
        v.re[o] = fmar(ss, ar, cs * br);
        v.im[o] = fmar(ss, ai, cs * bi);
    }
}

// X, Y, Z statistics of register bit m of a group pair (psi p, lambda l), added to
// sx, sy, sz (the same sums as xy_stats and the Z fold of stats_visit).
template <int G, typename R>
__device__ __forceinline__ void sg_stats(const SmallGroup<G, R> &p, const SmallGroup<G, R> &l, int m, R &sx, R &sy,
                                         R &sz)
{
    R xp = 0, xn = 0, yp = 0, yn = 0, zp = 0, zn = 0;
#pragma unroll
    for (int j = 0; j < (1 << G); ++j) {
        if ((j >> m) & 1) continue;
        const int o = j | (1 << m);
        xp = fmar(l.re[j], p.im[o], xp);
        xp = fmar(l.re[o], p.im[j], xp);
        xn = fmar(l.im[j], p.re[o], xn);
        xn = fmar(l.im[o], p.re[j], xn);
        yp = fmar(l.re[o], p.re[j], yp);
        yp = fmar(l.im[o], p.im[j], yp);
        yn = fmar(l.re[j], p.re[o], yn);
        yn = fmar(l.im[j], p.im[o], yn);
        zp = fmar(l.re[j], p.im[j], zp);
        zp = fmar(l.im[o], p.re[o], zp);
        zn = fmar(l.im[j], p.re[j], zn);
        zn = fmar(l.re[o], p.im[o], zn);
    }
    sx += xp - xn;
    sy += yp - yn;
    sz += zp - zn;
}

// Row partials (16 per workgroup) of the statistics of qubits s .. s+G-1 into red.
template <int G, typename R>
__device__ __forceinline__ void round_stats_out(const R (&sx)[G], const R (&sy)[G], const R (&sz)[G], R corr, int s,
                                                R *red)
{
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
    for (int m = 0; m < G; ++m) {
        R x = sx[m] * corr, y = sy[m] * corr, z = sz[m] * corr;
        row_sum16x3(x, y, z);
        if ((lane & 15) == 15) {
            const int r = w * 4 + (lane >> 4), q = s + m;
            red[(q * 3 + 0) * kSmallRows + r] = x;
            red[(q * 3 + 1) * kSmallRows + r] = y;
            red[(q * 3 + 2) * kSmallRows + r] = z;
        }
    }
}

struct SmallRound {
    int s, G;          // qubits s .. s+G-1
    uint32_t groups;   // 2^(n - G)
};

__device__ __forceinline__ uint32_t sg_base(uint32_t g, int s, int G)
{
    return ((g >> s) << (s + G)) | (g & ((1u << s) - 1u));
}

// Forward round: [round 0: init from the product-state factors (INIT) or multiply by
// scale * D], rotations of the round's qubits with layer lr's coefficients (lr < 0:
// none; CS: (sin, cos) form, else tangent form), [LAST: multiply by fin times this
// round's own scale].  Returns the product of the scales of its tangent-form rotations
// (1 in the (sin, cos) form), so the caller needs no second read of the table.
template <int G, typename R, bool CS>
__device__ __forceinline__ R small_fwd_round(V2<R> *psi, const SmallArgs &a, SmallRound rd, int lr, bool init,
                                                bool diag, const V4<R> *f, V2<R> tl, R scale, bool last, R fin)
{
    const V2<R> *rtf = reinterpret_cast<const V2<R> *>(a.rot_tf);
    R k[G], c[G];
#pragma unroll
    for (int m = 0; m < G; ++m) {
        const V2<R> kf = lr >= 0 ? ldu2(reinterpret_cast<const R *>(rtf + (size_t)lr * a.n + rd.s + m)) : mk2((R)0, (R)1);
        k[m] = kf.x;
        c[m] = kf.y;
    }
    R own = 1;
#pragma unroll
    for (int m = 0; m < G; ++m) own *= (CS || lr < 0) ? (R)1 : c[m];
    fin *= own;
    V2<R> t[1 << G];
    bcast_low<G, R>(t, tl);
    for (uint32_t g = threadIdx.x; g < rd.groups; g += kSmallThreads) {
        const uint32_t base = sg_base(g, rd.s, G);
        SmallGroup<G, R> v;
        if (init || diag) {
            V2<R> h = high_factor<G, R>(f, a.n, g, !init);
            h = mk2(h.x * scale, h.y * scale);
            const V2<R> hx = (!init && G < a.n && (g & 1u)) ? mk2(-h.x, -h.y) : h;
            if (init) {   // the product state: T[j] * h
#pragma unroll
                for (int j = 0; j < (1 << G); ++j) {
                    v.re[j] = (R)1;
                    v.im[j] = (R)0;
                }
            } else {
                sg_load<G>(v, psi, base, rd.s);
            }
            sg_diag<G, false>(v, t, h, hx);
        } else {
            sg_load<G>(v, psi, base, rd.s);
        }
        if (lr >= 0) {
#pragma unroll
            for (int m = 0; m < G; ++m) {
                if constexpr (CS)
                    sg_rot_cs<G, false>(v, m, k[m], c[m]);
                else
                    sg_rot<G, false>(v, m, k[m]);
            }
        }
        if (last) {
#pragma unroll
            for (int j = 0; j < (1 << G); ++j) {
                v.re[j] *= fin;
                v.im[j] *= fin;
            }
        }
        sg_store<G>(v, psi, base, rd.s);
    }
    return own;
}

// Adjoint round at layer l: [round 0 and D: multiply psi and lambda by scale * conj(D)],
// statistics of the round's qubits (scaled by corr) into red, then, if urot, the inverse
// rotations of layer l on both states; the groups are written back if anything changed.
// Returns the product of the scales of its tangent-form inverse rotations (1 if none).
template <int G, typename R, bool CS>
__device__ __forceinline__ R small_adj_round(V2<R> *psi, V2<R> *lam, const SmallArgs &a, SmallRound rd, int l,
                                                bool diag, const V4<R> *f, V2<R> tl, R scale, R corr, bool urot,
                                                R *red)
{
    const V2<R> *rtf = reinterpret_cast<const V2<R> *>(a.rot_tf);
    R k[G], c[G], sx[G], sy[G], sz[G];
#pragma unroll
    for (int m = 0; m < G; ++m) {
        const V2<R> kf = ldu2(reinterpret_cast<const R *>(rtf + (size_t)l * a.n + rd.s + m));
        k[m] = kf.x;
        c[m] = kf.y;
        sx[m] = sy[m] = sz[m] = (R)0;
    }
    V2<R> t[1 << G];
    bcast_low<G, R>(t, tl);
    for (uint32_t g = threadIdx.x; g < rd.groups; g += kSmallThreads) {
        const uint32_t base = sg_base(g, rd.s, G);
        SmallGroup<G, R> p, q;
        sg_load<G>(p, psi, base, rd.s);
        sg_load<G>(q, lam, base, rd.s);
        if (diag) {
            V2<R> h = high_factor<G, R>(f, a.n, g, true);
            h = mk2(h.x * scale, h.y * scale);
            const V2<R> hx = (G < a.n && (g & 1u)) ? mk2(-h.x, -h.y) : h;
            sg_diag<G, true>(p, t, h, hx);
            sg_diag<G, true>(q, t, h, hx);
        }
#pragma unroll
        for (int m = 0; m < G; ++m) sg_stats<G>(p, q, m, sx[m], sy[m], sz[m]);
        if (urot) {
#pragma unroll
            for (int m = 0; m < G; ++m) {
                if constexpr (CS) {
                    sg_rot_cs<G, true>(p, m, k[m], c[m]);
                    sg_rot_cs<G, true>(q, m, k[m], c[m]);
                } else {
                    sg_rot<G, true>(p, m, k[m]);
                    sg_rot<G, true>(q, m, k[m]);
                }
            }
        }
        if (urot || diag) {   // at l = 0 the later rounds still need D_0^dagger applied
            sg_store<G>(p, psi, base, rd.s);
            sg_store<G>(q, lam, base, rd.s);
        }
    }
    round_stats_out<G>(sx, sy, sz, corr, rd.s, red);
    R own = 1;
#pragma unroll
    for (int m = 0; m < G; ++m) own *= (CS || !urot) ? (R)1 : c[m];
    return own;
}

__device__ __forceinline__ SmallRound small_round(int n, int r)
{
    SmallRound rd;
    rd.s = kRoundBits * r;
    rd.G = n - rd.s < kRoundBits ? n - rd.s : kRoundBits;
    rd.groups = (1u << n) >> rd.G;
    return rd;
}

template <typename R, bool CS = false>
__device__ __forceinline__ R small_fwd_round_g(V2<R> *psi, const SmallArgs &a, SmallRound rd, int lr, bool init,
                                                  bool diag, const V4<R> *f, V2<R> tl, R scale, bool last, R fin)
{
    switch (rd.G) {
    case 1: return small_fwd_round<1, R, CS>(psi, a, rd, lr, init, diag, f, tl, scale, last, fin);
    case 2: return small_fwd_round<2, R, CS>(psi, a, rd, lr, init, diag, f, tl, scale, last, fin);
    default: return small_fwd_round<3, R, CS>(psi, a, rd, lr, init, diag, f, tl, scale, last, fin);
    }
}

template <typename R, bool CS = false>
__device__ __forceinline__ R small_adj_round_g(V2<R> *psi, V2<R> *lam, const SmallArgs &a, SmallRound rd, int l,
                                                  bool diag, const V4<R> *f, V2<R> tl, R scale, R corr, bool urot,
                                                  R *red)
{
    switch (rd.G) {
    case 1: return small_adj_round<1, R, CS>(psi, lam, a, rd, l, diag, f, tl, scale, corr, urot, red);
    case 2: return small_adj_round<2, R, CS>(psi, lam, a, rd, l, diag, f, tl, scale, corr, urot, red);
    default: return small_adj_round<3, R, CS>(psi, lam, a, rd, l, diag, f, tl, scale, corr, urot, red);
    }
}

// ---- whole circuit per workgroup with the CNOT chain: the same register rounds
//
// Per layer l the simulated sequence is diag(r_l), Ry-layer l, diag(p_l), then the chain P
// (bit k of P(i) = parity of bits 0..k of i; P^-1(j) = j ^ (j << 1)); layer 0 up to Ry is
// the product state.  The statistics are taken at P_l, just after Ry-layer l.  A forward
// step l -> l+1 gathers in round 0 amplitude J of the new state from i = P^-1(J), times
// p_l(i) r_{l+1}(J); an adjoint step back to P_l gathers amplitude i from P(i), times
// conj(r_{l+1}(P(i)) p_l(i)).  Both factors split into T[j] over qubits 0..G-1 (uniform)
// and a per-group factor with two variants: in the forward, bit G of i also depends on
// bit G-1 of j; in the adjoint, every bit of P(i) from G up flips with the parity of j.
// A gather reads all sources of a thread's groups before the workgroup barrier and writes
// after it, so it runs in place: at most two groups per thread (2^(n-4) <= 512 for n <= 13;
// fp64 compute is limited to n <= 12 by the host, so one).  The rotations
// use the (sin, cos) form: these tables carry no Pauli frame.

template <typename R>
constexpr int kGatherGroups = sizeof(R) == 4 ? 2 : 1;

// Factor diag(h, conj h) of qubit q at bit value b; h = (x, y) of f[q], or (z, w) (SECOND).
template <bool SECOND, typename R>
__device__ __forceinline__ V2<R> cphase(const V4<R> *f, int q, uint32_t b)
{
    const V4<R> g = uniform_v4<R>(f + q);
    const R im = SECOND ? g.w : g.y;
    return mk2(SECOND ? g.z : g.x, b ? -im : im);
}

// T[j] (j = lane & 15) of a forward step l -> l+1: p_l (wl) over the low bits of
// P^-1(j) times r_{l+1} (wn) over the bits of j.
template <typename R>
__device__ __forceinline__ V2<R> cnot_low_fwd(const V4<R> *wl, const V4<R> *wn, int G, int lane)
{
    const uint32_t j = (uint32_t)lane & 15u, ji = (j ^ (j << 1)) & ((1u << G) - 1u);
    V2<R> t = mk2((R)1, (R)0);
    for (int q = 0; q < G; ++q) {
        t = cmul(t, cphase<false, R>(wl, q, (ji >> q) & 1u));
        t = cmul(t, cphase<true, R>(wn, q, (j >> q) & 1u));
    }
    return t;
}

// T[j] of an adjoint step back to P_l: conj(r_{l+1} over the low bits of P(j) times p_l
// over the bits of j).
template <typename R>
__device__ __forceinline__ V2<R> cnot_low_adj(const V4<R> *wl, const V4<R> *wn, int G, int lane)
{
    const uint32_t lm = (1u << G) - 1u, j = (uint32_t)lane & lm & 15u, jp = cnot_chain(j, lm);
    V2<R> t = mk2((R)1, (R)0);
    for (int q = 0; q < G; ++q) {
        t = cmul(t, cphase<true, R>(wn, q, (jp >> q) & 1u));
        t = cmul(t, cphase<false, R>(wl, q, (j >> q) & 1u));
    }
    return mk2(t.x, -t.y);
}

// Round 0 of a forward step l -> l+1 (G = qubits of round 0): gather through P^-1 with
// the two diagonals, then Ry-layer l+1 on qubits 0..G-1.
template <int G, typename R>
__device__ __forceinline__ void cnot_fwd_gather(V2<R> *psi, const SmallArgs &a, int l, V2<R> tl)
{
    const int n = a.n;
    const uint32_t groups = (1u << n) >> G, hmask = groups - 1u, lmask = (1u << G) - 1u;
    const V4<R> *wl = reinterpret_cast<const V4<R> *>(a.dw) + (size_t)l * n, *wn = wl + n;
    const V2<R> *rcs = reinterpret_cast<const V2<R> *>(a.rot_tf) + (size_t)(l + 1) * n;
    V2<R> t[1 << G];
    bcast_low<G, R>(t, tl);
    constexpr int KG = kGatherGroups<R>;
    SmallGroup<G, R> v[KG];
    V2<R> h[KG], hx[KG];
#pragma unroll
    for (int k = 0; k < KG; ++k) {
        const uint32_t g = threadIdx.x + (uint32_t)k * kSmallThreads;
        if (g >= groups) continue;
        // high bits of the source index i = P^-1((g << G) | j): (g ^ (g << 1)), with bit 0
        // flipped when bit G-1 of j is set
        const uint32_t ih0 = (g ^ (g << 1)) & hmask, ih1 = ih0 ^ (hmask & 1u);
        V2<R> hr = mk2((R)1, (R)0), hp0 = hr, hp1 = hr;
        for (int q = G; q < n; ++q) {
            hr = cmul(hr, cphase<true, R>(wn, q, (g >> (q - G)) & 1u));
            hp0 = cmul(hp0, cphase<false, R>(wl, q, (ih0 >> (q - G)) & 1u));
            hp1 = cmul(hp1, cphase<false, R>(wl, q, (ih1 >> (q - G)) & 1u));
        }
        h[k] = cmul(hp0, hr);
        hx[k] = cmul(hp1, hr);
#pragma unroll
        for (int j = 0; j < (1 << G); ++j) {
            const uint32_t hi = ((j >> (G - 1)) & 1) ? ih1 : ih0;
            const V2<R> x = psi[sslot((hi << G) | (((uint32_t)j ^ ((uint32_t)j << 1)) & lmask))];
            v[k].re[j] = x.x;
            v[k].im[j] = x.y;
        }
    }
    __syncthreads();   // every source read before any amplitude is overwritten
    R sn[G], cs[G];
#pragma unroll
    for (int m = 0; m < G; ++m) {
        const V2<R> sc = ldu2(reinterpret_cast<const R *>(rcs + m));
        sn[m] = sc.x;
        cs[m] = sc.y;
    }
#pragma unroll
    for (int k = 0; k < KG; ++k) {
        const uint32_t g = threadIdx.x + (uint32_t)k * kSmallThreads;
        if (g >= groups) continue;
        sg_diag<G, false, 0>(v[k], t, h[k], hx[k]);
#pragma unroll
        for (int m = 0; m < G; ++m) sg_rot_cs<G, false>(v[k], m, sn[m], cs[m]);
        sg_store<G>(v[k], psi, g << G, 0);
    }
}

// Round 0 of an adjoint step back to P_l: gather psi and lambda through P with the
// conjugate diagonals, the statistics of qubits 0..G-1 at P_l, then (urot) the inverse
// rotations of Ry-layer l.
template <int G, typename R>
__device__ __forceinline__ void cnot_adj_gather(V2<R> *psi, V2<R> *lam, const SmallArgs &a, int l, V2<R> tl,
                                                bool urot, R *red)
{
    const int n = a.n;
    const uint32_t groups = (1u << n) >> G, hmask = groups - 1u, lmask = (1u << G) - 1u;
    const V4<R> *wl = reinterpret_cast<const V4<R> *>(a.dw) + (size_t)l * n, *wn = wl + n;
    const V2<R> *rcs = reinterpret_cast<const V2<R> *>(a.rot_tf) + (size_t)l * n;
    V2<R> t[1 << G];
    bcast_low<G, R>(t, tl);
    constexpr int KG = kGatherGroups<R>;
    SmallGroup<G, R> p[KG], q[KG];
    V2<R> h[KG], hx[KG];
#pragma unroll
    for (int k = 0; k < KG; ++k) {
        const uint32_t g = threadIdx.x + (uint32_t)k * kSmallThreads;
        if (g >= groups) continue;
        // high bits of P((g << G) | j): the prefix parities of g, all flipped for odd j
        const uint32_t pb0 = cnot_chain(g, hmask), pb1 = pb0 ^ hmask;
        V2<R> hp = mk2((R)1, (R)0), hr0 = hp, hr1 = hp;
        for (int qq = G; qq < n; ++qq) {
            hp = cmul(hp, cphase<false, R>(wl, qq, (g >> (qq - G)) & 1u));
            hr0 = cmul(hr0, cphase<true, R>(wn, qq, (pb0 >> (qq - G)) & 1u));
            hr1 = cmul(hr1, cphase<true, R>(wn, qq, (pb1 >> (qq - G)) & 1u));
        }
        const V2<R> d0 = cmul(hp, hr0), d1 = cmul(hp, hr1);
        h[k] = mk2(d0.x, -d0.y);
        hx[k] = mk2(d1.x, -d1.y);
#pragma unroll
        for (int j = 0; j < (1 << G); ++j) {
            const uint32_t hi = (__builtin_popcount(j) & 1) ? pb1 : pb0;
            const uint32_t src = sslot((hi << G) | cnot_chain((uint32_t)j, lmask));
            const V2<R> x = psi[src], y = lam[src];
            p[k].re[j] = x.x;
            p[k].im[j] = x.y;
            q[k].re[j] = y.x;
            q[k].im[j] = y.y;
        }
    }
    __syncthreads();   // every source read before any amplitude is overwritten
    R sn[G], cs[G], sx[G], sy[G], sz[G];
#pragma unroll
    for (int m = 0; m < G; ++m) {
        const V2<R> sc = ldu2(reinterpret_cast<const R *>(rcs + m));
        sn[m] = sc.x;
        cs[m] = sc.y;
        sx[m] = sy[m] = sz[m] = (R)0;
    }
#pragma unroll
    for (int k = 0; k < KG; ++k) {
        const uint32_t g = threadIdx.x + (uint32_t)k * kSmallThreads;
        if (g >= groups) continue;
        sg_diag<G, false, 1>(p[k], t, h[k], hx[k]);
        sg_diag<G, false, 1>(q[k], t, h[k], hx[k]);
#pragma unroll
        for (int m = 0; m < G; ++m) sg_stats<G>(p[k], q[k], m, sx[m], sy[m], sz[m]);
        if (urot) {
#pragma unroll
            for (int m = 0; m < G; ++m) {
                sg_rot_cs<G, true>(p[k], m, sn[m], cs[m]);
                sg_rot_cs<G, true>(q[k], m, sn[m], cs[m]);
            }
        }
        sg_store<G>(p[k], psi, g << G, 0);
        sg_store<G>(q[k], lam, g << G, 0);
    }
    round_stats_out<G>(sx, sy, sz, (R)1, 0, red);
}

template <typename R>
__device__ __forceinline__ void cnot_fwd_gather_g(V2<R> *psi, const SmallArgs &a, int G, int l, V2<R> tl)
{
    switch (G) {
    case 1: cnot_fwd_gather<1, R>(psi, a, l, tl); break;
    case 2: cnot_fwd_gather<2, R>(psi, a, l, tl); break;
    default: cnot_fwd_gather<3, R>(psi, a, l, tl); break;
    }
}

template <typename R>
__device__ __forceinline__ void cnot_adj_gather_g(V2<R> *psi, V2<R> *lam, const SmallArgs &a, int G, int l,
                                                  V2<R> tl, bool urot, R *red)
{
    switch (G) {
    case 1: cnot_adj_gather<1, R>(psi, lam, a, l, tl, urot, red); break;
    case 2: cnot_adj_gather<2, R>(psi, lam, a, l, tl, urot, red); break;
    default: cnot_adj_gather<3, R>(psi, lam, a, l, tl, urot, red); break;
    }
}

// Whole circuit of one sample with the CNOT entangler.  lambda at P_{L-1} is
// D^dag P^dag O P D psi with D = diag(p_{L-1}):
//   lambda_i = conj(D_i) c(P(i)) D_(i^x') psi_(i^x'),  x' = P^-1(xm),
//   c(j) = i^(#Y) (-1)^|(j ^ xm) & zm|,
// and E = Re <psi|lambda>.
template <typename R>
__device__ void small_cnot_rounds(const SmallArgs &a, V2<R> *psi, V2<R> *lam, R *red)
{
    const int n = a.n, L = a.L;
    const uint32_t N = 1u << n, mask = N - 1;
    const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const V4<R> *dw = reinterpret_cast<const V4<R> *>(a.dw);
    V2<R> *save = reinterpret_cast<V2<R> *>(a.psi_save) + (size_t)b * N;
    const int G0 = n < kRoundBits ? n : kRoundBits;
    const int nr = (n + kRoundBits - 1) / kRoundBits;
    const V2<R> one = mk2((R)1, (R)0);

    if (a.mode != 1) {
        const V4<R> *u = reinterpret_cast<const V4<R> *>(a.init_u) + (size_t)b * n;
        small_fwd_round_g<R>(psi, a, small_round(n, 0), -1, true, false, u, low_factor<R>(u, G0, false, lane), (R)1,
                             false, (R)1);
        __syncthreads();
        for (int l = 0; l + 1 < L; ++l) {
            const V4<R> *wl = dw + (size_t)l * n;
            cnot_fwd_gather_g<R>(psi, a, G0, l, cnot_low_fwd<R>(wl, wl + n, G0, lane));
            __syncthreads();
            for (int r = 1; r < nr; ++r) {
                small_fwd_round_g<R, true>(psi, a, small_round(n, r), l + 1, false, false, wl, one, (R)1, false,
                                           (R)1);
                __syncthreads();
            }
        }
    } else {
        for (uint32_t i = tid; i < N; i += kSmallThreads) psi[sslot(i)] = save[i];
        __syncthreads();
    }

    const V4<R> *wt = dw + (size_t)(L - 1) * n;
    const uint32_t zm = a.obs, xm = a.obs_x, xs = cnot_chain_inv(xm, mask);
    const int yph = __builtin_popcount(zm & xm) & 3;
    R e = 0;
    for (uint32_t i = tid; i < N; i += kSmallThreads) {
        const uint32_t j = i ^ xs;
        V2<R> v = cmul(small_phase<false, R>(wt, n, j), psi[sslot(j)]);
        if (__builtin_popcount((cnot_chain(i, mask) ^ xm) & zm) & 1) v = mk2(-v.x, -v.y);
        mul_ipow(v.x, v.y, yph);
        V2<R> d = small_phase<false, R>(wt, n, i);
        d.y = -d.y;
        const V2<R> li = cmul(d, v), pi = psi[sslot(i)];
        lam[sslot(i)] = li;
        e += pi.x * li.x + pi.y * li.y;
    }
    if (a.mode != 1) {
        e = row_sum16(e);
        if ((lane & 15) == 15) red[w * 4 + (lane >> 4)] = e;
        __syncthreads();
        if (tid == 0) {
            double s = 0.0;
            for (int k = 0; k < kSmallRows; ++k) s += (double)red[k];
            static_cast<R *>(a.e_out)[b] = (R)s;
        }
        if (a.mode == 0) {
            for (uint32_t i = tid; i < N; i += kSmallThreads) save[i] = psi[sslot(i)];
            return;
        }
    }
    __syncthreads();

    for (int l = L - 1; l >= 0; --l) {
        R *rl = red + (l & 1) * (3 * kSmallMaxQubits * kSmallRows);
        const V4<R> *wl = dw + (size_t)l * n;
        if (l + 1 < L)
            cnot_adj_gather_g<R>(psi, lam, a, G0, l, cnot_low_adj<R>(wl, wl + n, G0, lane), l > 0, rl);
        else
            small_adj_round_g<R, true>(psi, lam, a, small_round(n, 0), l, false, wl, one, (R)1, (R)1, l > 0, rl);
        __syncthreads();
        for (int r = 1; r < nr; ++r) {
            small_adj_round_g<R, true>(psi, lam, a, small_round(n, r), l, false, wl, one, (R)1, (R)1, l > 0, rl);
            __syncthreads();
        }
        if (tid < 3 * n) {
            double s = 0.0;
            for (int k = 0; k < kSmallRows; ++k) s += (double)rl[tid * kSmallRows + k];
            a.stats[(((size_t)b * L + l) * n) * 3 + tid] = s;
        }
    }
}

// ENT: the entangler (0 CZ chain, 1 CNOT chain), one instance each so that the CZ
// kernel keeps its own register budget.
template <typename R, int ENT>
__global__ __launch_bounds__(kSmallThreads) void k_small(SmallArgs a)
{
    extern __shared__ __align__(16) unsigned char smem[];
    __shared__ R red[2 * 3 * kSmallMaxQubits * kSmallRows + kSmallRows];
    const int n = a.n, L = a.L;
    const uint32_t N = 1u << n;
    V2<R> *psi = reinterpret_cast<V2<R> *>(smem);
    V2<R> *lam = psi + N;
    const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const V4<R> *dw = reinterpret_cast<const V4<R> *>(a.dw);
    V2<R> *save = reinterpret_cast<V2<R> *>(a.psi_save) + (size_t)b * N;
    if constexpr (ENT != 0) {
        small_cnot_rounds<R>(a, psi, lam, red);
        return;
    }

    const int G0 = n < kRoundBits ? n : kRoundBits;
    const int nr = (n + kRoundBits - 1) / kRoundBits;   // rounds per layer: qubits 0..2, 3..5, 6..8, 9..11, 12
    if (a.mode != 1) {
        const V4<R> *u = reinterpret_cast<const V4<R> *>(a.init_u) + (size_t)b * n;
        small_fwd_round_g<R>(psi, a, small_round(n, 0), -1, true, false, u, low_factor<R>(u, G0, false, lane), (R)1,
                             false, (R)1);
        __syncthreads();
        R c = 1;   // true state = stored state * c
        for (int l = 0; l + 1 < L; ++l) {
            // D_l (with the pending scale c), then Ry-layer l+1 round by round
            const V4<R> *wl = dw + (size_t)l * n;
            const V2<R> tl = low_factor<R>(wl, G0, true, lane);
            R cn = 1;
            for (int r = 0; r < nr; ++r) {
                const bool last = l + 2 == L && r + 1 == nr;
                cn *= small_fwd_round_g<R>(psi, a, small_round(n, r), l + 1, false, r == 0, wl, tl, c, last, cn);
                __syncthreads();
            }
            c = cn;
        }
        // <O> = sum_i Re(conj(psi_i) (O psi)_i)
        R e = 0;
        for (uint32_t i = tid; i < N; i += kSmallThreads) {
            V2<R> v = psi[sslot(i)];
            if (a.obs_x) v = cmul(v, small_diag<R>(dw + (size_t)(L - 1) * n, n, i));
            const V2<R> o = small_obs<R>(psi, i, a.obs, a.obs_x, dw + (size_t)(L - 1) * n, n);
            e += v.x * o.x + v.y * o.y;
        }
        e = row_sum16(e);
        if ((lane & 15) == 15) red[w * 4 + (lane >> 4)] = e;
        __syncthreads();
        if (tid == 0) {
            double s = 0.0;
            for (int k = 0; k < kSmallRows; ++k) s += (double)red[k];
            static_cast<R *>(a.e_out)[b] = (R)s;
        }
        if (a.mode == 0) {
            for (uint32_t i = tid; i < N; i += kSmallThreads) save[i] = psi[sslot(i)];
            return;
        }
        __syncthreads();
    } else {
        for (uint32_t i = tid; i < N; i += kSmallThreads) psi[sslot(i)] = save[i];
        __syncthreads();
    }

    // Adjoint sweep: lambda = O psi at P_{L-1}; statistics at every P_l; uncompute.
    // lambda at the last Ry layer = D_trail^dagger O D_trail psi (= O psi for a Z-string)
    for (uint32_t i = tid; i < N; i += kSmallThreads) {
        V2<R> o = small_obs<R>(psi, i, a.obs, a.obs_x, dw + (size_t)(L - 1) * n, n);
        if (a.obs_x) {
            V2<R> f = small_diag<R>(dw + (size_t)(L - 1) * n, n, i);
            f.y = -f.y;
            o = cmul(o, f);
        }
        lam[sslot(i)] = o;
    }
    __syncthreads();
    // Layer l: [D_l^dagger with the pending scale], then per round the statistics of its
    // qubits at P_l and the inverse rotations of Ry-layer l (none at l = 0).  The
    // statistics partials alternate between two halves of red, so the sums of layer l
    // are read while layer l-1 writes the other half.
    R c = 1;
    for (int l = L - 1; l >= 0; --l) {
        R *rl = red + (l & 1) * (3 * kSmallMaxQubits * kSmallRows);
        const bool diag = l + 1 < L;
        const V4<R> *wl = dw + (size_t)l * n;
        const V2<R> tl = low_factor<R>(wl, G0, true, lane);
        R cc = 1;
        for (int r = 0; r < nr; ++r) {
            cc *= small_adj_round_g<R>(psi, lam, a, small_round(n, r), l, diag && r == 0, wl, tl, c, cc * cc, l > 0, rl);
            __syncthreads();
        }
        if (tid < 3 * n) {
            double s = 0.0;
            for (int k = 0; k < kSmallRows; ++k) s += (double)rl[tid * kSmallRows + k];
            a.stats[(((size_t)b * L + l) * n) * 3 + tid] = s;
        }
        c = cc;
    }
}

}  // namespace hqml

// ------------------------------------------------------------------ launch wrappers (host)

namespace hqml {

hipError_t configure_small()
{
    constexpr int kMaxShm = 2 * (1 << kSmallMaxQubits) * (int)sizeof(float2);   // = 2 * 2^12 * sizeof(double2)
    const void *f[4] = {reinterpret_cast<const void *>(&k_small<float, 0>),
                        reinterpret_cast<const void *>(&k_small<float, 1>),
                        reinterpret_cast<const void *>(&k_small<double, 0>),
                        reinterpret_cast<const void *>(&k_small<double, 1>)};
    for (const void *k : f) {
        const hipError_t e = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, kMaxShm);
        if (e != hipSuccess) return e;
    }
    return configure_small12();
}

hipError_t launch_small(const SmallArgs &a, int B, int r64, hipStream_t s)
{
    if (!r64 && a.ent == 0 && a.n == 12) return launch_small12(a, B, s);
    const size_t shm = (size_t)2 * ((size_t)1 << a.n) * (r64 ? sizeof(double2) : sizeof(float2));
    if (r64) {
        if (a.ent)
            k_small<double, 1><<<B, kSmallThreads, shm, s>>>(a);
        else
            k_small<double, 0><<<B, kSmallThreads, shm, s>>>(a);
    } else {
        if (a.ent)
            k_small<float, 1><<<B, kSmallThreads, shm, s>>>(a);
        else
            k_small<float, 0><<<B, kSmallThreads, shm, s>>>(a);
    }
    return hipGetLastError();
}

}  // namespace hqml
