// gfx950 kernels of the fused forward / fused adjoint training step.
//
// Method: Kawase, arXiv:2603.02804 (hugo-pages summary "深度解析：正向与反向门融合
// 驱动的高效量子机器学习仿真", sections 1.2-1.4 and 3.2).  The layer algebra (each
// layer = one real rotation layer plus one merged diagonal) is described in
// hqml_internal.hpp.
//
// Kernels:
//   k_prep_zyz      theta -> per (layer, qubit) factorisation U = diag(p) Ry(beta) diag(r)
//   k_prep_frame    Pauli frame that keeps every simulated rotation in tan form
//   k_prep_tables   -> rot_tf (tan form of each rotation), dw (diagonal factors), H (gradient map)
//   k_prep_init     x -> layer-0 product-state factors u_q per sample
//   k_prep_fused    the four steps above in one workgroup, for small tables
//   k_tile_fwd      fused forward pass over one 2^13-amplitude tile (forward gate fusion)
//   k_tile_bwd      fused adjoint pass over one tile (backward gate fusion): re-derives the
//                   earlier state with U^dagger on chip, forms the gradient statistics and
//                   propagates lambda <- U^dagger lambda
//   (k_small, the whole circuit of one sample per workgroup for n <= 13, is in hqml_small.hip)
//   k_ez_reduce     per-tile <O> partials -> E_b, loss, dL/dE_b (fixed-order fp64)
//   k_stats_reduce  per-tile statistics -> per-sample statistics (fixed-order fp64)
//   k_grad_reduce   per-sample statistics x dL/dE x H -> dL/dtheta (fixed-order fp64)
// No floating-point atomics anywhere: every reduction has a fixed order.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "hqml_device.hpp"
#include "hqml_half.hpp"
#include "hqml_internal.hpp"

// 1: the compilation unit of the fp32 adjoint launches (see the launch wrappers below).
#ifndef HQML_BWD32_UNIT
#define HQML_BWD32_UNIT 0
#endif

namespace hqml {

// Element access of a stored state.  Every state read is a streaming read (each pass
// reads its input once), so loads carry the non-temporal hint: measured on the fused
// forward pass it cuts the pass from 0.132 to 0.110 ms at 20 qubits, batch 32.
template <int ST>
struct StateIO;

template <>
struct StateIO<0> {
    using elem = float2;
    template <typename R>
    __device__ static __forceinline__ void load(const elem *p, R &re, R &im)
    {
        const unsigned long long u = __builtin_nontemporal_load(reinterpret_cast<const unsigned long long *>(p));
        re = (R)__uint_as_float((uint32_t)u);
        im = (R)__uint_as_float((uint32_t)(u >> 32));
    }
    template <typename R>
    __device__ static __forceinline__ void store(elem *p, R re, R im)
    {
        *p = make_float2((float)re, (float)im);
    }
    template <typename R>
    __device__ static __forceinline__ void load_temporal(const elem *p, R &re, R &im)
    {
        const float2 v = *p;
        re = (R)v.x;
        im = (R)v.y;
    }
    template <typename R>
    __device__ static __forceinline__ void store_nt(elem *p, R re, R im)
    {
        const unsigned long long u =
            (unsigned long long)__float_as_uint((float)re) | ((unsigned long long)__float_as_uint((float)im) << 32);
        __builtin_nontemporal_store(u, reinterpret_cast<unsigned long long *>(p));
    }
};

template <>
struct StateIO<1> {
    using elem = uint32_t;
    template <typename R>
    __device__ static __forceinline__ void load(const elem *p, R &re, R &im)
    {
        const uint32_t v = __builtin_nontemporal_load(p);
        re = (R)bf16_to_f32(v & 0xFFFFu);
        im = (R)bf16_to_f32(v >> 16);
    }
    template <typename R>
    __device__ static __forceinline__ void store(elem *p, R re, R im)
    {
        *p = f32x2_to_bf16x2((float)re, (float)im);
    }
};

template <>
struct StateIO<2> {
    using elem = double2;
    template <typename R>
    __device__ static __forceinline__ void load(const elem *p, R &re, R &im)
    {
        typedef double d2 __attribute__((ext_vector_type(2)));
        const d2 v = __builtin_nontemporal_load(reinterpret_cast<const d2 *>(p));
        re = (R)v.x;
        im = (R)v.y;
    }
    template <typename R>
    __device__ static __forceinline__ void store(elem *p, R re, R im)
    {
        *p = make_double2((double)re, (double)im);
    }
};

// Storage element type of the adjoint state lambda: the compute type.
template <typename R>
constexpr int kLamIO = sizeof(R) == 4 ? 0 : 2;

// A copy of a per-thread value that the compiler cannot identify with earlier uses: values derived
// from it (addresses of the stores of a tile, offsets inside a loop) are recomputed where
// they are used instead of being kept live in registers.  (An empty asm: no instruction.)
__device__ __forceinline__ uint32_t opaque_u32(uint32_t v)
{
    asm volatile("" : "+v"(v));
    return v;
}

// ------------------------------------------------------------------ tile layouts

// LDS bank swizzle on the 8-byte amplitude index.  Linear over GF(2), so
// swz(a ^ b) = swz(a) ^ swz(b).  Chosen so that both L1 and L2 accesses of a
// half-wave touch 32 distinct 8-byte slots (no bank conflicts with 64 x 4-byte banks).
__host__ __device__ constexpr uint32_t swz(uint32_t l)
{
    return l ^ ((l >> 4) & 3u) ^ ((((l >> 6) ^ (l >> 9)) & 1u) << 4);
}

// Local index of register j in each layout (register part only).
__host__ __device__ constexpr uint32_t l1_reg(int j) { return (uint32_t)j << 4; }
__host__ __device__ constexpr uint32_t l2_reg(int j) { return ((uint32_t)j & 3u) | (((uint32_t)j >> 2) << 9); }

template <typename R>
struct Tile {
    R re[kRegs];
    R im[kRegs];
};

__device__ __forceinline__ uint32_t l1_thread_local(int lane, int w)
{
    return (uint32_t)(lane & 15) | ((uint32_t)(lane >> 4) << 9) | ((uint32_t)w << 11);
}

__device__ __forceinline__ uint32_t l2_thread_local(int lane, int w)
{
    return ((uint32_t)lane << 2) | ((uint32_t)(w & 1) << 8) | ((uint32_t)(w >> 1) << 12);
}

// Move a tile between layouts through LDS (2^13 amplitudes).  'from_l1' selects direction.
template <typename R>
__device__ __forceinline__ void transpose(Tile<R> &t, V2<R> *lds, uint32_t a1, uint32_t a2, bool from_l1)
{
    __syncthreads();
    if (from_l1) {
#pragma unroll
        for (int j = 0; j < kRegs; ++j) lds[a1 ^ swz(l1_reg(j))] = mk2(t.re[j], t.im[j]);
    } else {
#pragma unroll
        for (int j = 0; j < kRegs; ++j) lds[a2 ^ swz(l2_reg(j))] = mk2(t.re[j], t.im[j]);
    }
    __syncthreads();
    if (from_l1) {
#pragma unroll
        for (int j = 0; j < kRegs; ++j) {
            const V2<R> v = lds[a2 ^ swz(l2_reg(j))];
            t.re[j] = v.x;
            t.im[j] = v.y;
        }
    } else {
#pragma unroll
        for (int j = 0; j < kRegs; ++j) {
            const V2<R> v = lds[a1 ^ swz(l1_reg(j))];
            t.re[j] = v.x;
            t.im[j] = v.y;
        }
    }
}

// The same move through a 32 KB buffer.  Local position 12 is wave bit 1 in both
// layouts, so waves 0-1 and waves 2-3 hold disjoint halves of the tile in both and
// never exchange data; the two halves take turns in the buffer.  (swz keeps bit 12.)
template <typename R>
__device__ __forceinline__ void transpose_half(Tile<R> &t, V2<R> *lds, uint32_t a1, uint32_t a2, bool from_l1,
                                               int w)
{
    constexpr uint32_t kHalf = (1u << (kTileBits - 1)) - 1u;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        __syncthreads();
        if ((w >> 1) == h) {
            if (from_l1) {
#pragma unroll
                for (int j = 0; j < kRegs; ++j) lds[(a1 ^ swz(l1_reg(j))) & kHalf] = mk2(t.re[j], t.im[j]);
            } else {
#pragma unroll
                for (int j = 0; j < kRegs; ++j) lds[(a2 ^ swz(l2_reg(j))) & kHalf] = mk2(t.re[j], t.im[j]);
            }
        }
        __syncthreads();
        if ((w >> 1) == h) {
            if (from_l1) {
#pragma unroll
                for (int j = 0; j < kRegs; ++j) {
                    const V2<R> v = lds[(a2 ^ swz(l2_reg(j))) & kHalf];
                    t.re[j] = v.x;
                    t.im[j] = v.y;
                }
            } else {
#pragma unroll
                for (int j = 0; j < kRegs; ++j) {
                    const V2<R> v = lds[(a1 ^ swz(l1_reg(j))) & kHalf];
                    t.re[j] = v.x;
                    t.im[j] = v.y;
                }
            }
        }
    }
}

// Real rotation Ry(beta) on register bit M in scaled form, one FMA per real output:
//   Ry(beta) = f * [[1, -k], [k, 1]],  k = tan(beta/2) in [-1, 1],  f = cos(beta/2).
// INV applies Ry^dagger.  The scale f (>= 1/sqrt 2) is not applied here: callers track
// it as a uniform scalar and fold it into the next diagonal, a statistics correction
// or the final store.  k = 0 is the identity (used for register bits a view does not
// rotate), so the code has no data-dependent branches.
template <int M, bool INV, typename R>
__device__ __forceinline__ void rot_bit(Tile<R> &t, R k)
{
    const R kk = INV ? -k : k;
#pragma unroll
    for (int j = 0; j < kRegs; ++j) {
        if (j & (1 << M)) continue;
        const int o = j | (1 << M);
        const R ar = t.re[j], ai = t.im[j], br = t.re[o], bi = t.im[o];
        t.re[j] = fmar(-kk, br, ar);
        t.im[j] = fmar(-kk, bi, ai);
        t.re[o] = fmar(kk, ar, br);
        t.im[o] = fmar(kk, ai, bi);
    }
}

// Rotation coefficients of the register bits for one layer.
template <typename R>
struct RotCoef {
    R k[5];
    R F;         // product of the scale factors of the rotated bits
};

// rot_tf[l][q] = (k, f).  Bits outside regmask get k = 0, f = 1 (identity).  The table is
// read for every bit (any qubit's entry is valid) and the mask selects, so the uniform
// values stay in scalar registers without branches.
template <typename R>
__device__ __forceinline__ RotCoef<R> load_coef(const R *rot_tf, int n, int layer, const int *qpos_to_q,
                                                uint32_t regmask)
{
    RotCoef<R> rc;
    rc.F = (R)1;
#pragma unroll
    for (int m = 0; m < 5; ++m) {
        const V2<R> kf = ldu2(rot_tf + ((size_t)layer * n + qpos_to_q[m]) * 2);
        const bool on = (regmask >> m) & 1u;
        rc.k[m] = on ? kf.x : (R)0;
        rc.F *= on ? kf.y : (R)1;
    }
    return rc;
}

template <bool INV, typename R>
__device__ __forceinline__ void rot_layer(Tile<R> &t, const RotCoef<R> &rc)
{
    rot_bit<0, INV>(t, rc.k[0]);
    rot_bit<1, INV>(t, rc.k[1]);
    rot_bit<2, INV>(t, rc.k[2]);
    rot_bit<3, INV>(t, rc.k[3]);
    rot_bit<4, INV>(t, rc.k[4]);
}

template <bool INV, typename R>
__device__ __forceinline__ void rot_layer2(Tile<R> &a, Tile<R> &b, const RotCoef<R> &rc)
{
    rot_layer<INV>(a, rc);
    rot_layer<INV>(b, rc);
}

template <typename R>
__device__ __forceinline__ void scale_tile(Tile<R> &t, R s)
{
#pragma unroll
    for (int j = 0; j < kRegs; ++j) {
        t.re[j] *= s;
        t.im[j] *= s;
    }
}

// X / Y statistics of register bit M (pairs j, o = j | 2^M):
//   Im<lam|X_q|psi> = sum Im(conj(l_j) p_o) + Im(conj(l_o) p_j)
//   Im<lam|Y_q|psi> = sum Re(conj(l_o) p_j) - Re(conj(l_j) p_o)
// written as chains of plain FMAs into separate positive / negative accumulators
// (no negated operand copies).
template <int M, typename R>
__device__ __forceinline__ void xy_stats(const Tile<R> &p, const Tile<R> &l, R &sx, R &sy)
{
    R xp = 0, xn = 0, yp = 0, yn = 0;
#pragma unroll
    for (int j = 0; j < kRegs; ++j) {
        if (j & (1 << M)) continue;
        const int o = j | (1 << M);
        xp = fmar(l.re[j], p.im[o], xp);
        xp = fmar(l.re[o], p.im[j], xp);
        xn = fmar(l.im[j], p.re[o], xn);
        xn = fmar(l.im[o], p.re[j], xn);
        yp = fmar(l.re[o], p.re[j], yp);
        yp = fmar(l.im[o], p.im[j], yp);
        yn = fmar(l.re[j], p.re[o], yn);
        yn = fmar(l.im[j], p.im[o], yn);
    }
    sx = xp - xn;
    sy = yp - yn;
}

// Reduce the three statistics of one qubit over the workgroup into the LDS stat
// area (16 row partials per slot, slots base .. base+2).
template <typename R>
__device__ __forceinline__ void stat_out3(R x, R y, R z, R *lds_stat, int base, int lane, int w)
{
    row_sum16x3(x, y, z);
    if ((lane & 15) == 15) {
        const int r = w * 4 + (lane >> 4);
        lds_stat[(base + 0) * 16 + r] = x;
        lds_stat[(base + 1) * 16 + r] = y;
        lds_stat[(base + 2) * 16 + r] = z;
    }
}

// Local position of register bit m in layout L1 / L2.
__host__ __device__ constexpr int l1_pos(int m) { return 4 + m; }
__host__ __device__ constexpr int l2_pos(int m) { return m < 2 ? m : 7 + m; }

// Z statistics of the register bits: d_m = sum_j (-1)^{bit m of j} w_j with
// w_j = Im(conj(l_j) p_j).  zsum<K, LO> returns the sum of w over registers LO..LO+2^K-1
// and adds the differences of its two halves to d_{K-1} (and recursively below), depth
// first, so at most one pending half-sum per level is live (5 values, not 16).
template <int J, typename R>
__device__ __forceinline__ R zw(const Tile<R> &p, const Tile<R> &l)
{
    return fmar(l.re[J], p.im[J], -l.im[J] * p.re[J]);
}

template <int K, int LO, typename R>
__device__ __forceinline__ R zsum(const Tile<R> &p, const Tile<R> &l, R *dz)
{
    if constexpr (K == 0) {
        return zw<LO>(p, l);
    } else {
        const R a = zsum<K - 1, LO>(p, l, dz);
        const R b = zsum<K - 1, LO + (1 << (K - 1))>(p, l, dz);
        if constexpr (LO == 0)
            dz[K - 1] = a - b;
        else
            dz[K - 1] += a - b;
        return a + b;
    }
}

// Statistics of the 5 register bits: slots ((sel*13 + pos)*3 + {X,Y,Z}).  Bits a
// view does not rotate land in slots nobody reads.  'corr' is the uniform factor
// (product of the tracked scales of psi and lambda) that turns the stored-state
// statistics into those of the true states.
template <bool L2, typename R>
__device__ __forceinline__ void stats_visit(const Tile<R> &p, const Tile<R> &l, int sel, R *lds_stat, int lane,
                                            int w, R corr)
{
    R dz[5];
    (void)zsum<5, 0>(p, l, dz);
    R sx, sy;
#define HQML_STAT_BIT(M)                                                        \
    {                                                                           \
        xy_stats<M>(p, l, sx, sy);                                              \
        const int base = (sel * 13 + (L2 ? l2_pos(M) : l1_pos(M))) * 3;         \
        stat_out3(sx * corr, sy * corr, dz[M] * corr, lds_stat, base, lane, w);  \
    }
    HQML_STAT_BIT(0)
    HQML_STAT_BIT(1)
    HQML_STAT_BIT(2)
    HQML_STAT_BIT(3)
    HQML_STAT_BIT(4)
#undef HQML_STAT_BIT
}

// Sign of Z_{q-1} Z_{q+1} for the qubit q[m] of each register bit m (bit m set: -1), on
// this thread's amplitudes.  'fixed' holds the thread's lane, wave and tile qubit values;
// the view keeps the chain neighbours of a rotated qubit off the register bits of its
// layout, so for those qubits the sign is the same on all 32 registers of the thread.
__device__ __forceinline__ uint32_t nb_sign_mask(uint32_t fixed, const int *q, int n)
{
    uint32_t m = 0;
#pragma unroll
    for (int r = 0; r < 5; ++r) {
        const int qq = q[r];
        uint32_t nb = qq + 1 < n ? 1u << (qq + 1) : 0u;
        if (qq > 0) nb |= 1u << (qq - 1);
        m |= (uint32_t)(__builtin_popcount(fixed & nb) & 1) << r;
    }
    return m;
}

// Merged statistics of the 5 register bits: one set of sums gives both rotation layers
// of a pass [Ry-layer la, D_la, Ry-layer lb].  Taken where qubit q of the group is at the
// point after Ry_q(lb) (the pass output, with at most other group qubits un-rotated on
// both states), for register bit m (qubit q):
//   slots (13 + pos)*3 + {X,Y,Z}: S_s = Im<lam|s_q|psi>, layer lb's statistics as they are;
//   slots pos*3 + {X,Y,Z}: T_s = Im<lam|Z_{q-1} Z_{q+1} s_q|psi>, from which flush_merged
//     forms layer la's statistics (the neighbours' Z is a per-thread sign, nb bit m).
// Layer la's statistics at its own point need no un-rotated psi: the group holds no
// two chain neighbours, so only D_la and Ry_q(lb) separate that point from this one, and
//   D X_q D^dag = Z_{q-1} Z_{q+1} (Re rho X_q - Im rho Y_q),
//   D Y_q D^dag = Z_{q-1} Z_{q+1} (Im rho X_q + Re rho Y_q),  D Z_q D^dag = Z_q,
// rho = f0 conj(f1) of qubit q in D_la, then Ry X Ry^dag = cos b X - sin b Z and
// Ry Z Ry^dag = cos b Z + sin b X.
template <bool L2, typename R>
__device__ __forceinline__ void stats_visit_merged(const Tile<R> &p, const Tile<R> &l, R *lds_stat, int lane, int w,
                                                   R corr, uint32_t nb)
{
    R dz[5];
    (void)zsum<5, 0>(p, l, dz);
    R sx, sy;
#define HQML_STAT_BIT(M)                                                                           \
    {                                                                                              \
        xy_stats<M>(p, l, sx, sy);                                                                 \
        const int pos = L2 ? l2_pos(M) : l1_pos(M);                                                \
        const R sg = ((nb >> (M)) & 1u) ? -corr : corr;                                            \
        stat_out3(sx * corr, sy * corr, dz[M] * corr, lds_stat, (13 + pos) * 3, lane, w);          \
        stat_out3(sx * sg, sy * sg, dz[M] * sg, lds_stat, pos * 3, lane, w);                       \
    }
    HQML_STAT_BIT(0)
    HQML_STAT_BIT(1)
    HQML_STAT_BIT(2)
    HQML_STAT_BIT(3)
    HQML_STAT_BIT(4)
#undef HQML_STAT_BIT
}

// Factor of qubit q in D_l for bit value 1 (sel) or 0, read as uniform values into scalar
// registers before the per-lane choice (otherwise the compiler turns the choice into a
// per-lane address and a vector load per qubit).
__device__ __forceinline__ float rfl(float x)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, x)));
}

__device__ __forceinline__ double rfl(double x)
{
    const uint64_t u = __builtin_bit_cast(uint64_t, x);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)u);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(u >> 32));
    return __builtin_bit_cast(double, (uint64_t)lo | ((uint64_t)hi << 32));
}

template <typename R>
__device__ __forceinline__ V2<R> hfactor(const V4<R> *wl, int q, bool sel)
{
    const V4<R> f = ldu4(reinterpret_cast<const R *>(wl + __builtin_amdgcn_readfirstlane(q)));
    const R x = rfl(f.x), y = rfl(f.y), z = rfl(f.z), w = rfl(f.w);
    return sel ? mk2(z, w) : mk2(x, y);
}

// Per-thread factor tables of the diagonal D_l in layout L2:
// D(i) = Plo[j & 3] * Phi[j >> 2] for register j of this thread.  dw[l][q] holds the
// factor (f0, f1) of qubit q for bit value 0 / 1; CZ signs between register and
// fixed qubits are folded into the register factors, signs between two register
// qubits of the same table into its entries (the planner keeps the two tables'
// qubits non-adjacent).
template <typename R>
struct DiagTables {
    V2<R> lo[4];
    V2<R> hi[8];
};

// cz = false (CNOT-chain plan): a plain product of single-qubit factors, no CZ signs.
// The thread constant is a product over the lane and wave qubits of L2 (positions 2..8 and
// 12, per lane) and the tile's qubits (uniform), every factor read as a uniform value before
// the per-lane choice.
struct TileCtx;
template <typename R>
__device__ __forceinline__ DiagTables<R> diag_tables(const R *dw, int n, int layer, const TileCtx &c, const ViewDev &v,
                                                     bool cz = true);
template <typename R>
__device__ __forceinline__ void scale_lo(DiagTables<R> &d, R s)
{
#pragma unroll
    for (int a = 0; a < 4; ++a) {
        d.lo[a].x *= s;
        d.lo[a].y *= s;
    }
}

// Apply s * D in layout L2 (s folded into the thread's factor table).
template <typename R>
__device__ __forceinline__ void apply_diag(Tile<R> &t, DiagTables<R> d, R s)
{
    scale_lo(d, s);
#pragma unroll
    for (int j = 0; j < kRegs; ++j) {
        const V2<R> f = cmul(d.lo[j & 3], d.hi[j >> 2]);
        const R r = t.re[j], i = t.im[j];
        t.re[j] = r * f.x - i * f.y;
        t.im[j] = r * f.y + i * f.x;
    }
}

// Apply s * D^dagger to two tiles in layout L2.
template <typename R>
__device__ __forceinline__ void apply_diag2(Tile<R> &a, Tile<R> &b, DiagTables<R> d, R s)
{
    scale_lo(d, s);
#pragma unroll
    for (int j = 0; j < kRegs; ++j) {
        V2<R> f = cmul(d.lo[j & 3], d.hi[j >> 2]);
        f.y = -f.y;
        R r = a.re[j], i = a.im[j];
        a.re[j] = r * f.x - i * f.y;
        a.im[j] = r * f.y + i * f.x;
        r = b.re[j];
        i = b.im[j];
        b.re[j] = r * f.x - i * f.y;
        b.im[j] = r * f.y + i * f.x;
    }
}

// Apply s * D^dagger to one tile in layout L2.
template <typename R>
__device__ __forceinline__ void apply_diag_dag(Tile<R> &t, DiagTables<R> d, R s)
{
    scale_lo(d, s);
#pragma unroll
    for (int j = 0; j < kRegs; ++j) {
        V2<R> f = cmul(d.lo[j & 3], d.hi[j >> 2]);
        f.y = -f.y;
        const R r = t.re[j], i = t.im[j];
        t.re[j] = r * f.x - i * f.y;
        t.im[j] = r * f.y + i * f.x;
    }
}

// Per-tile geometry shared by the forward and backward tile kernels.
struct TileCtx {
    int lane, w, sample, tile;
    uint64_t tile_off;        // global amplitude offset of the tile's fixed (tile-index) bits
    uint32_t tile_bits;       // the same as a qubit bitmask (bit q = value of qubit q)
    uint32_t t1;              // L1: thread's amplitude offset within the tile
    uint32_t a1, a2;          // LDS base addresses (swizzled) of the thread in L1 / L2
    uint32_t fixed1, fixed2;  // qubit bitmask of this thread's fixed bits (incl. tile) in L1 / L2
    uint32_t fx1t, fx2t;      // the thread (lane and wave) part of fixed1 / fixed2
    uint32_t rs[5];           // L1: amplitude stride of each register bit (uniform)
    int q1[5], q2[5];         // global qubits of the register bits in L1 / L2
    uint32_t gm1, gm2;        // register masks of the rotated group in L1 / L2
};

// Point the context at tile 'blk' (= (sample - sample0) * T + tile index).
__device__ __forceinline__ void tile_retarget(TileCtx &c, const ViewDev &v, int T, int blk, int sample0)
{
    const int rel = blk / T;
    c.tile = blk - rel * T;
    c.sample = sample0 + rel;
    uint64_t toff = 0;
    uint32_t tb = 0;
    const int nt = ldu(&v.n_tile);
    for (int k = 0; k < nt; ++k) {
        if ((c.tile >> k) & 1) {
            const int q = ldu(&v.tile_q[k]);
            toff |= 1ull << q;
            tb |= 1u << q;
        }
    }
    c.tile_off = toff;
    c.tile_bits = tb;
    c.fixed1 = c.fx1t | tb;
    c.fixed2 = c.fx2t | tb;
}

// Grid slot of workgroup blk renumbered so that each XCD works on one contiguous range of
// the grid's (sample, tile) pairs: the dispatcher places workgroup blk on XCD blk % 8, so
// slot (blk % 8) * (G / 8) + blk / 8 keeps each sample on one XCD from pass to pass.  The
// passes below run faster so although their HBM byte counts do not change (the gain is in
// access latency, not traffic).  A bijection of 0..G-1 when 8 divides G; otherwise the
// plain order.  Used by the fp32 forward pass
// and by the adjoint shapes of the CZ-chain plan (there with lambda loaded and stored
// through L2); the CNOT-chain adjoint shapes and the fp64 forward run slower with it and
// keep the plain order, except the passes that move a state through the chain's index map
// (chain_pair_slot).
__device__ __forceinline__ int xcd_slot(int blk, int G)
{
    return (G & 7) ? blk : (blk & 7) * (G >> 3) + (blk >> 3);
}

// Grid slot of workgroup blk for a pass that reads its input, or writes lambda back, through
// the CNOT chain's index map P^-1.  The 16 amplitudes of one 128-byte line (consecutive
// indices a) belong to tile indices j = P(a), whose bits 4.. all flip with the parity of a's
// bits 0..3: half of the line belongs to tile t, the other half to tile T2 - 1 - t of the same
// sample.  Workgroups blk and blk + 8 (one XCD, dispatched together) take such a pair, so both
// halves meet in that XCD's L2 (written back as whole lines: the [diag, rotB] adjoint pass
// 0.210 -> 0.151 ms at 20 qubits; read once from memory: the forward passes 3 % faster on average).
// A bijection of 0..G-1 when 16 divides G (G = samples x T2, T2 a power of two); otherwise
// the plain order.
__device__ __forceinline__ int chain_pair_slot(int blk, int G, int T2)
{
    if ((G & 15) || T2 < 2) return blk;
    const int p = ((blk >> 4) << 3) | (blk & 7);   // pair index: (sample, tile < T2 / 2)
    const int h = (blk >> 3) & 1;
    const int half = T2 >> 1;
    const int rel = p / half, t = p - rel * half;
    return rel * T2 + (h ? T2 - 1 - t : t);
}

__device__ __forceinline__ void tile_ctx(TileCtx &c, const ViewDev &v, int T, int blk, int sample0)
{
    const int tid = threadIdx.x;
    c.lane = tid & 63;
    c.w = tid >> 6;
    const int lane = c.lane, w = c.w;
    // L1 thread bits: lane 0..3 -> pos 0..3, lane 4,5 -> pos 9,10, wave 0,1 -> pos 11,12
    const int l1p[8] = {0, 1, 2, 3, 9, 10, 11, 12};
    const uint32_t l1v = (uint32_t)(lane & 15) | ((uint32_t)(lane >> 4) << 4) | ((uint32_t)w << 6);
    uint32_t t1 = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k)
        if ((l1v >> k) & 1u) t1 |= 1u << ldu(&v.perm[l1p[k]]);
    c.t1 = t1;
    c.fx1t = t1;
    // L2 thread bits: lane 0..5 -> pos 2..7, wave 0 -> pos 8, wave 1 -> pos 12
    const int l2p[8] = {2, 3, 4, 5, 6, 7, 8, 12};
    const uint32_t l2v = (uint32_t)lane | ((uint32_t)w << 6);
    uint32_t f2 = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k)
        if ((l2v >> k) & 1u) f2 |= 1u << ldu(&v.perm[l2p[k]]);
    c.fx2t = f2;
    c.a1 = swz(l1_thread_local(lane, w));
    c.a2 = swz(l2_thread_local(lane, w));
#pragma unroll
    for (int m = 0; m < 5; ++m) {
        c.q1[m] = ldu(&v.perm[4 + m]);
        c.q2[m] = ldu(&v.perm[m < 2 ? m : 7 + m]);
        c.rs[m] = 1u << c.q1[m];
    }
    const uint32_t gm = (uint32_t)ldu(&v.group_mask);
    c.gm1 = (gm >> 4) & 31u;
    c.gm2 = (gm & 3u) | (((gm >> 9) & 7u) << 2);
    tile_retarget(c, v, T, blk, sample0);
}

template <typename R>
__device__ __forceinline__ DiagTables<R> diag_tables(const R *dw, int n, int layer, const TileCtx &c, const ViewDev &v,
                                                     bool cz)
{
    const V4<R> *wl = reinterpret_cast<const V4<R> *>(dw) + (size_t)layer * n;
    const uint32_t fixed_bits = c.fixed2;
    const int *rq = c.q2;
    const int l2p[8] = {2, 3, 4, 5, 6, 7, 8, 12};
    const uint32_t tv = (uint32_t)c.lane | ((uint32_t)c.w << 6);
    V2<R> ct = mk2((R)1, (R)0);
#pragma unroll 1
    for (int k = 0; k < 8; ++k) ct = cmul(ct, hfactor<R>(wl, ldu(&v.perm[l2p[k]]), (tv >> k) & 1u));
    V2<R> cu = mk2((R)1, (R)0);
    const int nt = ldu(&v.n_tile);
    for (int k = 0; k < nt; ++k) cu = cmul(cu, hfactor<R>(wl, ldu(&v.tile_q[k]), (c.tile >> k) & 1));
    V2<R> cc = cmul(ct, cu);
    if (cz && (__builtin_popcount(fixed_bits & (fixed_bits >> 1)) & 1)) {
        cc.x = -cc.x;
        cc.y = -cc.y;
    }
    V2<R> g0[5], g1[5];
#pragma unroll
    for (int m = 0; m < 5; ++m) {
        const int q = rq[m];
        g0[m] = hfactor<R>(wl, q, false);
        g1[m] = hfactor<R>(wl, q, true);
        uint32_t nb = (fixed_bits >> (q + 1)) & 1u;
        if (q > 0) nb += (fixed_bits >> (q - 1)) & 1u;
        if (cz && (nb & 1u)) {
            g1[m].x = -g1[m].x;
            g1[m].y = -g1[m].y;
        }
    }
    auto adj = [&](int a, int b) { const int d = rq[a] - rq[b]; return cz && (d == 1 || d == -1); };
    DiagTables<R> t;
#pragma unroll
    for (int a = 0; a < 4; ++a) {
        V2<R> x = cmul(cc, cmul((a & 1) ? g1[0] : g0[0], (a & 2) ? g1[1] : g0[1]));
        if (a == 3 && adj(0, 1)) { x.x = -x.x; x.y = -x.y; }
        t.lo[a] = x;
    }
#pragma unroll
    for (int h = 0; h < 8; ++h) {
        V2<R> x = cmul(cmul((h & 1) ? g1[2] : g0[2], (h & 2) ? g1[3] : g0[3]), (h & 4) ? g1[4] : g0[4]);
        int flips = 0;
        if ((h & 3) == 3 && adj(2, 3)) ++flips;
        if ((h & 6) == 6 && adj(3, 4)) ++flips;
        if ((h & 5) == 5 && adj(2, 4)) ++flips;
        if (flips & 1) { x.x = -x.x; x.y = -x.y; }
        t.hi[h] = x;
    }
    return t;
}

// Amplitude offset of register j in layout L1 (sum of the strides of its set bits).
__device__ __forceinline__ uint32_t roff(const TileCtx &c, int j)
{
    uint32_t o = 0;
#pragma unroll
    for (int m = 0; m < 5; ++m)
        if (j & (1 << m)) o += c.rs[m];
    return o;
}

// Global-memory access of a tile in layout L1: a workgroup-uniform 64-bit tile
// origin plus a byte offset (thread part + register part).  The amplitude offset
// within a sample is below 2^29 (n <= 29), so for elements of at most 8 bytes the
// byte offset fits 32 bits and maps onto the scalar-base + vector-offset addressing
// form; 16-byte (fp64) elements need a 64-bit offset.
template <uint32_t ESZ>
using TileOff = typename std::conditional<(ESZ <= 8), uint32_t, uint64_t>::type;

// NT = false: ordinary loads (fp32 only), used for lambda in the XCD-contiguous order,
// where they measured faster than non-temporal loads.
template <int ST, typename R, bool NT = true>
__device__ __forceinline__ void load_l1(Tile<R> &t, const void *state, const TileCtx &c, uint64_t nelem)
{
    using IO = StateIO<ST>;
    constexpr uint32_t esz = sizeof(typename IO::elem);
    using Off = TileOff<esz>;
    const char *base = reinterpret_cast<const char *>(state) + ((uint64_t)c.sample * nelem + c.tile_off) * esz;
    const Off tb = (Off)c.t1 * esz;
#pragma unroll
    for (int j = 0; j < kRegs; ++j) {
        const Off off = tb + (Off)roff(c, j) * esz;
        if constexpr (NT)
            IO::load(reinterpret_cast<const typename IO::elem *>(base + off), t.re[j], t.im[j]);
        else
            IO::load_temporal(reinterpret_cast<const typename IO::elem *>(base + off), t.re[j], t.im[j]);
    }
}

// NT: non-temporal stores (fp32 lambda of the CNOT-chain adjoint shapes; the forward pass
// outputs, read by the very next pass, are slower with them).
template <int ST, typename R, bool NT = false>
__device__ __forceinline__ void store_l1(const Tile<R> &t, void *state, const TileCtx &c, uint64_t nelem)
{
    using IO = StateIO<ST>;
    constexpr uint32_t esz = sizeof(typename IO::elem);
    using Off = TileOff<esz>;
    char *base = reinterpret_cast<char *>(state) + ((uint64_t)c.sample * nelem + c.tile_off) * esz;
    const Off tb = (Off)opaque_u32(c.t1) * esz;
#pragma unroll
    for (int j = 0; j < kRegs; ++j) {
        const Off off = tb + (Off)roff(c, j) * esz;
        if constexpr (NT)
            IO::store_nt(reinterpret_cast<typename IO::elem *>(base + off), t.re[j], t.im[j]);
        else
            IO::store(reinterpret_cast<typename IO::elem *>(base + off), t.re[j], t.im[j]);
    }
}

// The CNOT chain CNOT(0,1), ..., CNOT(n-2,n-1) sends basis state i to P(i), bit k of
// P(i) = parity of bits 0..k of i; P^-1(j) = j ^ (j << 1), linear over XOR.  A pass that
// follows a chain reads its tile (amplitude indices j) from P^-1(j) of the previous
// output, and its adjoint writes lambda back to P^-1(j).  The tile's index bits (tile,
// thread, register parts) are disjoint, so P^-1 of the index is the XOR of P^-1 of the
// parts: one per-thread value and one uniform value per register.
__device__ __forceinline__ uint32_t chain_inv(uint32_t i, uint32_t mask) { return (i ^ (i << 1)) & mask; }

// fp32 states are read through L2 here: the partner tile of chain_pair_slot reads the other
// half of each line.
template <int ST, typename R>
__device__ __forceinline__ void load_l1_chain(Tile<R> &t, const void *state, const TileCtx &c, uint64_t nelem)
{
    using IO = StateIO<ST>;
    constexpr uint32_t esz = sizeof(typename IO::elem);
    using Off = TileOff<esz>;
    const uint32_t mask = (uint32_t)(nelem - 1);
    const char *base = reinterpret_cast<const char *>(state) + (uint64_t)c.sample * nelem * esz;
    const uint32_t pt = chain_inv((uint32_t)c.tile_off | c.t1, mask);
#pragma unroll
    for (int j = 0; j < kRegs; ++j) {
        const Off off = (Off)(pt ^ chain_inv(roff(c, j), mask)) * esz;
        if constexpr (ST == 0)
            IO::load_temporal(reinterpret_cast<const typename IO::elem *>(base + off), t.re[j], t.im[j]);
        else
            IO::load(reinterpret_cast<const typename IO::elem *>(base + off), t.re[j], t.im[j]);
    }
}

template <int ST, typename R>
__device__ __forceinline__ void store_l1_chain(const Tile<R> &t, void *state, const TileCtx &c, uint64_t nelem)
{
    using IO = StateIO<ST>;
    constexpr uint32_t esz = sizeof(typename IO::elem);
    using Off = TileOff<esz>;
    const uint32_t mask = (uint32_t)(nelem - 1);
    char *base = reinterpret_cast<char *>(state) + (uint64_t)c.sample * nelem * esz;
    const uint32_t pt = chain_inv((uint32_t)c.tile_off | c.t1, mask);
#pragma unroll
    for (int j = 0; j < kRegs; ++j) {
        const Off off = (Off)(pt ^ chain_inv(roff(c, j), mask)) * esz;
        IO::store(reinterpret_cast<typename IO::elem *>(base + off), t.re[j], t.im[j]);
    }
}

// Layer-0 product state in layout L1: psi(i) = prod_q u_q[bit_q(i)].
template <typename R>
__device__ __forceinline__ void init_l1(Tile<R> &t, const R *init_u, const TileCtx &c, int n)
{
    const V4<R> *u = reinterpret_cast<const V4<R> *>(init_u) + (size_t)c.sample * n;
    uint32_t regq = 0;
#pragma unroll
    for (int m = 0; m < 5; ++m) regq |= 1u << c.q1[m];
    V2<R> cst = mk2((R)1, (R)0);
    for (int q = 0; q < n; ++q) {
        if (regq & (1u << q)) continue;
        cst = cmul(cst, hfactor<R>(u, q, (c.fixed1 >> q) & 1u));
    }
    t.re[0] = cst.x;
    t.im[0] = cst.y;
#pragma unroll
    for (int m = 0; m < 5; ++m) {
        const V4<R> f = ldu4(reinterpret_cast<const R *>(u + c.q1[m]));
        const V2<R> g0 = mk2(f.x, f.y), g1 = mk2(f.z, f.w);
        const int half = 1 << m;
#pragma unroll
        for (int k = 0; k < half; ++k) {
            const V2<R> v = mk2(t.re[k], t.im[k]);
            const V2<R> a = cmul(v, g0), b = cmul(v, g1);
            t.re[k] = a.x;
            t.im[k] = a.y;
            t.re[k + half] = b.x;
            t.im[k + half] = b.y;
        }
    }
}

// Sign pattern of the observable O = prod_{q in S} Z_q over the 32 registers of this
// thread: bit j is set when O has eigenvalue -1 on register j's amplitude, i.e. when
// an odd number of the qubits of S are 1 there.  'fixed' holds the thread's non-register
// qubit values (lane, wave and tile bits); register bit m holds qubit q[m].
__device__ __forceinline__ uint32_t obs_sign_mask(uint32_t fixed, const int *q, uint32_t S)
{
    constexpr uint32_t kRegBit[5] = {0xAAAAAAAAu, 0xCCCCCCCCu, 0xF0F0F0F0u, 0xFF00FF00u, 0xFFFF0000u};
    uint32_t m = (__builtin_popcount(fixed & S) & 1) ? 0xFFFFFFFFu : 0u;
#pragma unroll
    for (int r = 0; r < 5; ++r)
        if ((S >> q[r]) & 1u) m ^= kRegBit[r];
    return m;
}

__device__ __forceinline__ uint32_t obs_mask_l1(const TileCtx &c, uint32_t S)
{
    return obs_sign_mask(c.fixed1, c.q1, S);
}

__device__ __forceinline__ uint32_t obs_mask_l2(const TileCtx &c, uint32_t S)
{
    return obs_sign_mask(c.fixed2, c.q2, S);
}

// Workgroup sum of the per-thread <O> partial -> e_part[sample][tile].
template <typename R>
__device__ __forceinline__ void emit_e(R e, R *lds_stat, R *e_part, const TileCtx &c, int T)
{
    e = row_sum16(e);
    __syncthreads();
    if ((c.lane & 15) == 15) lds_stat[kSlots * 16 + c.w * 4 + (c.lane >> 4)] = e;
    __syncthreads();
    if (threadIdx.x == 0) {
        R s = 0;
        for (int k = 0; k < 16; ++k) s += lds_stat[kSlots * 16 + k];
        e_part[(size_t)c.sample * T + c.tile] = s;
    }
}

template <typename R>
__device__ __forceinline__ R z0_partial(const Tile<R> &t, uint32_t zmask)
{
    R e = 0;
#pragma unroll
    for (int j = 0; j < kRegs; ++j) {
        const R p = t.re[j] * t.re[j] + t.im[j] * t.im[j];
        e += ((zmask >> j) & 1u) ? -p : p;
    }
    return e;
}

template <typename R>
__device__ __forceinline__ void seed_lambda(Tile<R> &l, const Tile<R> &p, uint32_t zmask)
{
#pragma unroll
    for (int j = 0; j < kRegs; ++j) {
        const bool neg = (zmask >> j) & 1u;
        l.re[j] = neg ? -p.re[j] : p.re[j];
        l.im[j] = neg ? -p.im[j] : p.im[j];
    }
}

// ------------------------------------------------------------------ forward tile pass

// Forward ops of one pass on a tile held in layout L1; stores the pass output.
template <int ST, typename R>
__device__ __forceinline__ void fwd_ops(Tile<R> &t, const TilePassArgs &a, const TileCtx &c, V2<R> *lds,
                                        R *lds_stat, uint64_t nelem)
{
    const R *rot_tf = static_cast<const R *>(a.rot_tf);
    // true state = stored tile * sigma (uniform), see rot_bit
    R sigma = 1;
    const bool need_l2 = (a.rotA >= 0) || (a.diag >= 0) || (a.rotB >= 0);
    if (a.rotA >= 0) {
        const RotCoef<R> r = load_coef(rot_tf, a.n, a.rotA, c.q1, c.gm1);
        rot_layer<false>(t, r);
        sigma *= r.F;
    }
    if (need_l2) {
        transpose_half(t, lds, c.a1, c.a2, true, c.w);
        if (a.rotA >= 0) {
            const RotCoef<R> r = load_coef(rot_tf, a.n, a.rotA, c.q2, c.gm2);
            rot_layer<false>(t, r);
            sigma *= r.F;
        }
        RotCoef<R> rb1, rb2;
        if (a.rotB >= 0) {
            rb1 = load_coef(rot_tf, a.n, a.rotB, c.q1, c.gm1);
            rb2 = load_coef(rot_tf, a.n, a.rotB, c.q2, c.gm2);
        }
        if (a.diag >= 0) {
            // fold the pending scale and the scale of the rotations that follow into D
            const R fb = a.rotB >= 0 ? rb1.F * rb2.F : (R)1;
            apply_diag(t, diag_tables(static_cast<const R *>(a.dw), a.n, a.diag, c, *a.view, !(a.flags & PF_CNOT)),
                       sigma * fb);
            sigma = (R)1 / fb;
        }
        if (a.rotB >= 0) {
            rot_layer<false>(t, rb2);
            sigma *= rb2.F;
        }
        transpose_half(t, lds, c.a1, c.a2, false, c.w);
        if (a.rotB >= 0) {
            rot_layer<false>(t, rb1);
            sigma *= rb1.F;
        }
    }
    if (a.diag < 0 && (a.rotA >= 0 || a.rotB >= 0)) scale_tile(t, sigma);
    if (a.flags & PF_EMIT_E)
        emit_e(z0_partial(t, obs_mask_l1(c, a.obs)), lds_stat, static_cast<R *>(a.e_part), c, a.T);
    if (a.flags & PF_STORE) store_l1<ST>(t, a.psi_out, c, nelem);
}

// 37 KB of LDS and 128 VGPRs: four workgroups (16 waves) per compute unit, so one
// workgroup's loads overlap another's rotations.
template <int ST, typename R>
__global__ __launch_bounds__(kThreads, sizeof(R) == 4 ? 4 : 2) void k_tile_fwd(TilePassArgs a)
{
    __shared__ V2<R> lds[1 << (kTileBits - 1)];
    __shared__ R lds_stat[kSlots * 16 + 16];
    const ViewDev &v = *a.view;
    TileCtx c;
    // fp64 compute (twice the bytes per sample) streams faster in the plain order; a pass that
    // reads through the CNOT chain's index map takes complementary tiles in pairs (each 128-byte
    // line it reads is split between tiles t and T - 1 - t)
    const int blk = (int)blockIdx.x, G = (int)gridDim.x;
    tile_ctx(c, v, a.T, (a.flags & PF_GATHER) ? chain_pair_slot(blk, G, a.T) : sizeof(R) == 4 ? xcd_slot(blk, G) : blk,
             a.sample0);
    const uint64_t nelem = 1ull << a.n;
    Tile<R> t;
    if (a.flags & PF_INIT)
        init_l1(t, static_cast<const R *>(a.init_u), c, a.n);
    else if (a.flags & PF_GATHER)
        load_l1_chain<ST>(t, a.psi_in, c, nelem);
    else
        load_l1<ST>(t, a.psi_in, c, nelem);
    fwd_ops<ST>(t, a, c, lds, lds_stat, nelem);
}

// ------------------------------------------------------------------ observable pass

// Pauli-string observable with X or Y factors, O = i^(#Y) X^xm Z^zm (Y = iXZ), on the
// final state: (O psi)_i = i^(#Y) (-1)^|(i ^ xm) & zm| psi_(i ^ xm).  The pass's view
// keeps every qubit of xm on chip, so the partner amplitude i ^ xm is in the same
// tile: the tile goes to LDS and each thread reads its partners.  Emits the per-tile
// <O> partials (PF_EMIT_E) and/or writes lambda = O psi (PF_SEED).
template <int ST, typename R>
__global__ __launch_bounds__(kThreads, sizeof(R) == 4 ? 2 : 1) void k_tile_obs(TilePassArgs a)
{
    __shared__ V2<R> lds[1 << kTileBits];
    __shared__ R lds_stat[kSlots * 16 + 16];
    const ViewDev &v = *a.view;
    TileCtx c;
    tile_ctx(c, v, a.T, blockIdx.x, a.sample0);
    const uint64_t nelem = 1ull << a.n;
    Tile<R> p;
    load_l1<ST>(p, a.psi_in, c, nelem);
    // phi = D_trail psi, D_trail(i) = CZ-chain sign x prod_q f_q(bit q of i) (layer L-1's
    // left factors): the true final state.  D_trail commutes with Z but not with X or Y.
    // The CNOT-chain plan has applied diag(p_(L-1)) in its last pass (PF_CNOT: no D_trail;
    // the string is the chain-conjugated one, possibly with a sign, PF_OBS_NEG).
    const bool trail = !(a.flags & PF_CNOT);
    const V4<R> *wl = reinterpret_cast<const V4<R> *>(a.dw) + (size_t)(a.L - 1) * a.n;
    uint32_t regq = 0;
#pragma unroll
    for (int m = 0; m < 5; ++m) regq |= 1u << c.q1[m];
    V2<R> cst = mk2((R)1, (R)0);
    for (int q = 0; trail && q < a.n; ++q) {
        if ((regq >> q) & 1u) continue;
        const V4<R> f = ldu4(reinterpret_cast<const R *>(wl + q));
        cst = cmul(cst, ((c.fixed1 >> q) & 1u) ? mk2(f.z, f.w) : mk2(f.x, f.y));
    }
    V2<R> dj[kRegs];
#pragma unroll
    for (int j = 0; j < kRegs; ++j) {
        if (!trail) {
            dj[j] = mk2((R)1, (R)0);
            continue;
        }
        uint32_t g = c.fixed1;
        V2<R> f = cst;
#pragma unroll
        for (int m = 0; m < 5; ++m) {
            const V4<R> w = ldu4(reinterpret_cast<const R *>(wl + c.q1[m]));
            if ((j >> m) & 1) {
                g |= 1u << c.q1[m];
                f = cmul(f, mk2(w.z, w.w));
            } else {
                f = cmul(f, mk2(w.x, w.y));
            }
        }
        if (__builtin_popcount(g & (g >> 1)) & 1) f = mk2(-f.x, -f.y);
        dj[j] = f;
        const R r = p.re[j], i = p.im[j];
        p.re[j] = r * f.x - i * f.y;
        p.im[j] = r * f.y + i * f.x;
    }
    uint32_t xl = 0;   // local positions of the X part
    for (int q = 0; q < a.n; ++q)
        if ((a.obs_x >> q) & 1u) xl |= 1u << ldu(&v.inv[q]);
    const uint32_t sx = swz(xl);
#pragma unroll
    for (int j = 0; j < kRegs; ++j) lds[c.a1 ^ swz(l1_reg(j))] = mk2(p.re[j], p.im[j]);
    __syncthreads();
    // sign of Z^zm at the partner: parity((i ^ xm) & zm) = parity(i & zm) ^ parity(xm & zm)
    uint32_t neg = obs_mask_l1(c, a.obs);
    if (__builtin_popcount(a.obs & a.obs_x) & 1) neg = ~neg;
    const int ph = (__builtin_popcount(a.obs & a.obs_x) + ((a.flags & PF_OBS_NEG) ? 2 : 0)) & 3;
    Tile<R> o;
    R e = 0;
#pragma unroll
    for (int j = 0; j < kRegs; ++j) {
        const V2<R> w = lds[(c.a1 ^ swz(l1_reg(j))) ^ sx];
        R re = ((neg >> j) & 1u) ? -w.x : w.x;
        R im = ((neg >> j) & 1u) ? -w.y : w.y;
        mul_ipow(re, im, ph);
        o.re[j] = re;
        o.im[j] = im;
        e = fmar(p.re[j], re, fmar(p.im[j], im, e));
    }
    if (a.flags & PF_EMIT_E) emit_e(e, lds_stat, static_cast<R *>(a.e_part), c, a.T);
    if (a.flags & PF_SEED) {
        // lambda at the last Ry layer = D_trail^dagger O phi
#pragma unroll
        for (int j = 0; j < kRegs; ++j) {
            const R r = o.re[j], i = o.im[j];
            o.re[j] = r * dj[j].x + i * dj[j].y;
            o.im[j] = i * dj[j].x - r * dj[j].y;
        }
        store_l1<kLamIO<R>>(o, a.lam, c, nelem);
    }
}

// ------------------------------------------------------------------ backward tile pass

template <typename R>
__device__ __forceinline__ void zero_stats(R *lds_stat)
{
    for (int i = threadIdx.x; i < kSlots * 16 + 16; i += kThreads) lds_stat[i] = 0;
}

// Where a full tile's statistics partials go: row (sample * T + tile) * stat_mul of the
// pass's partials; with stat_mul = 2 (the context's general passes run on half tiles, two
// rows per full tile) the row after it is written with zeros.
template <typename R>
__device__ __forceinline__ R *stat_row(const TilePassArgs &a, const TileCtx &c)
{
    return static_cast<R *>(a.stat_part) + ((size_t)c.sample * a.T + c.tile) * (size_t)a.stat_mul * kSlots;
}

template <typename R>
__device__ __forceinline__ void flush_stats(const R *lds_stat, R *dst, bool zero_next)
{
    __syncthreads();
    if (threadIdx.x < kSlots) {
        R s = 0;
#pragma unroll
        for (int k = 0; k < 16; ++k) s += lds_stat[threadIdx.x * 16 + k];
        dst[threadIdx.x] = s;
        if (zero_next) dst[kSlots + threadIdx.x] = 0;
    }
}

// flush_stats for a pass whose statistics were taken by stats_visit_merged: the sums of
// the slots of each group position are combined into layer la's statistics (see
// stats_visit_merged) with rho = f0 conj(f1) of qubit q in D_la (dw row la) and
// cos b, sin b of Ry_q(lb) from its tan form k = tan(b/2) (rot_tf row lb).  lds_stat row 0
// of every slot receives the slot's workgroup sum first.
template <typename R>
__device__ __forceinline__ void flush_merged(R *lds_stat, R *dst, bool zero_next, const ViewDev &v, const R *rot_tf,
                                             const R *dw, int n, int la, int lb)
{
    __syncthreads();
    const int t = threadIdx.x;
    R sum = 0;
    if (t < kSlots) {
#pragma unroll
        for (int k = 0; k < 16; ++k) sum += lds_stat[t * 16 + k];
    }
    __syncthreads();
    if (t < kSlots) lds_stat[t * 16] = sum;
    __syncthreads();
    if (t < kSlots) {
        R out = sum;
        const int pos = (t / 3) % 13, sel = t / 39, sig = t % 3;
        if (t < 78 && sel == 0 && ((ldu(&v.group_mask) >> pos) & 1)) {
            const int q = ldu(&v.perm[pos]);
            const V4<R> f = ldu4(dw + ((size_t)la * n + q) * 4);
            const R rr = f.x * f.z + f.y * f.w, ri = f.y * f.z - f.x * f.w;   // rho = f0 conj(f1)
            const R k = ldu(rot_tf + ((size_t)lb * n + q) * 2);
            const R inv = (R)1 / ((R)1 + k * k);
            const R cb = ((R)1 - k * k) * inv, sb = (R)2 * k * inv;
            const R tx = lds_stat[(pos * 3 + 0) * 16], ty = lds_stat[(pos * 3 + 1) * 16];
            const R tz = lds_stat[(pos * 3 + 2) * 16];
            const R sxl = lds_stat[((13 + pos) * 3 + 0) * 16], szl = lds_stat[((13 + pos) * 3 + 2) * 16];
            const R u = cb * tx - sb * tz;
            out = sig == 0 ? rr * u - ri * ty : sig == 1 ? ri * u + rr * ty : cb * szl + sb * sxl;
        }
        dst[t] = out;
        if (zero_next) dst[kSlots + t] = 0;
    }
}

// Backward pass shapes (one kernel instance each, to keep register use per shape low).
enum BwdShape : int {
    BW_GENERAL = 0,      // [rotA(la), D_la, rotB(la+1)]
    BW_INIT_GENERAL = 5, // [init, D_0, rotB(1)]
    BW_ROTA = 1,         // [rotA(la)]
    BW_L0 = 2,           // layer-0 statistics only (one-layer circuit, or stats-only view)
    BW_FUSED_LAST = 3,   // forward [rotA(la)] + E + seed + its backward
    BW_FUSED_INIT = 4,   // one-layer circuit: product state + E + seed + layer-0 statistics
    // CNOT-chain plan (no merged diagonals; see the plan builder):
    BW_DROTB = 6,        // [diag(r_l), rotB(l)] read through the chain; lambda written back through it
    BW_ROTAD = 7,        // [rotA(l), diag(p_l)]
    BW_L0D = 8,          // layer-0 statistics, lambda taken back through diag(p_0)
    BW_L0D_SEED = 9      // one-layer circuit: seed, layer-0 statistics of view 0, diag(p_0) lambda stored
};

template <int ST, int SHAPE, typename R>
__global__ __launch_bounds__(kThreads, sizeof(R) == 4 ? 2 : 1) void k_tile_bwd(TilePassArgs a)
{
    __shared__ V2<R> lds[1 << kTileBits];
    __shared__ R lds_stat[kSlots * 16 + 16];
    const R *rot_tf = static_cast<const R *>(a.rot_tf);
    const R *init_u = static_cast<const R *>(a.init_u);
    R *e_part = static_cast<R *>(a.e_part);
    constexpr int LIO = kLamIO<R>;
    const ViewDev &v = *a.view;
    // CZ-chain plan shapes: XCD-contiguous tiles, fp32 lambda read and written through L2
    constexpr bool kXcd = SHAPE == BW_GENERAL || SHAPE == BW_INIT_GENERAL || SHAPE == BW_FUSED_LAST ||
                          SHAPE == BW_FUSED_INIT || SHAPE == BW_L0;
    constexpr bool kLamNT = LIO == 0 && !kXcd;
    TileCtx c;
    tile_ctx(c, v, a.T, kXcd ? xcd_slot((int)blockIdx.x, (int)gridDim.x) : (int)blockIdx.x, a.sample0);
    zero_stats(lds_stat);
    __syncthreads();
    const uint64_t nelem = 1ull << a.n;
    const bool init = (a.flags & PF_INIT) != 0;
    const int la = init ? 0 : a.rotA;   // layer of the A-side statistics
    Tile<R> p, l;
    // Scales: true psi = stored psi * sp, true lambda = stored lambda * sl (uniform).
    R sl = 1;

    if constexpr (SHAPE == BW_FUSED_INIT) {
        init_l1(p, init_u, c, a.n);
        const uint32_t zm = obs_mask_l1(c, a.obs);
        emit_e(z0_partial(p, zm), lds_stat, e_part, c, a.T);
        seed_lambda(l, p, zm);
        stats_visit<false>(p, l, 0, lds_stat, c.lane, c.w, (R)1);
        transpose(p, lds, c.a1, c.a2, true);
        transpose(l, lds, c.a1, c.a2, true);
        stats_visit<true>(p, l, 0, lds_stat, c.lane, c.w, (R)1);
        transpose(l, lds, c.a1, c.a2, false);
    } else if constexpr (SHAPE == BW_FUSED_LAST) {
        load_l1<ST>(p, a.psi_in, c, nelem);
        const RotCoef<R> r1 = load_coef(rot_tf, a.n, la, c.q1, c.gm1);
        const RotCoef<R> r2 = load_coef(rot_tf, a.n, la, c.q2, c.gm2);
        rot_layer<false>(p, r1);
        transpose(p, lds, c.a1, c.a2, true);
        rot_layer<false>(p, r2);
        const R fa = r1.F * r2.F;              // psi (and the seeded lambda) carry scale fa
        const uint32_t zm = obs_mask_l2(c, a.obs);
        emit_e(z0_partial(p, zm) * (fa * fa), lds_stat, e_part, c, a.T);
        seed_lambda(l, p, zm);
        stats_visit<true>(p, l, 0, lds_stat, c.lane, c.w, fa * fa);
        rot_layer2<true>(p, l, r2);
        transpose(p, lds, c.a1, c.a2, false);
        transpose(l, lds, c.a1, c.a2, false);
        const R s2 = fa * r2.F;
        stats_visit<false>(p, l, 0, lds_stat, c.lane, c.w, s2 * s2);
        rot_layer<true>(l, r1);
        sl = s2 * r1.F;
    } else {
        if (a.flags & PF_STATS_ONLY)
            init_l1(p, init_u, c, a.n);
        else
            load_l1<ST>(p, a.psi_in, c, nelem);
        if (a.flags & PF_SEED)
            seed_lambda(l, p, obs_mask_l1(c, a.obs));
        else
            load_l1<LIO, R, kLamNT || LIO != 0>(l, a.lam, c, nelem);
        if constexpr (SHAPE == BW_GENERAL || SHAPE == BW_INIT_GENERAL) {
            // Backward gate fusion with merged statistics: both layers of the pass from one
            // set of sums per layout (stats_visit_merged), so psi is only brought into L2
            // (its L1 group qubits un-rotated alongside lambda to keep the two states at one
            // point) and never through D_la; lambda goes back through the whole pass.
            const uint32_t nb1 = nb_sign_mask(c.fixed1, c.q1, a.n);
            const uint32_t nb2 = nb_sign_mask(c.fixed2, c.q2, a.n);
            const RotCoef<R> b1 = load_coef(rot_tf, a.n, a.rotB, c.q1, c.gm1);
            stats_visit_merged<false>(p, l, lds_stat, c.lane, c.w, (R)1, nb1);
            rot_layer2<true>(p, l, b1);
            const R fb1 = b1.F;
            transpose(p, lds, c.a1, c.a2, true);
            transpose(l, lds, c.a1, c.a2, true);
            stats_visit_merged<true>(p, l, lds_stat, c.lane, c.w, fb1 * fb1, nb2);
            const RotCoef<R> b2 = load_coef(rot_tf, a.n, a.rotB, c.q2, c.gm2);
            rot_layer<true>(l, b2);
            // lambda carries scale fb1 * b2.F; D^dagger removes it
            apply_diag_dag(l, diag_tables(static_cast<const R *>(a.dw), a.n, a.diag, c, *a.view), fb1 * b2.F);
            if constexpr (SHAPE == BW_GENERAL) {
                const RotCoef<R> a2 = load_coef(rot_tf, a.n, la, c.q2, c.gm2);
                rot_layer<true>(l, a2);
                transpose(l, lds, c.a1, c.a2, false);
                const RotCoef<R> a1 = load_coef(rot_tf, a.n, la, c.q1, c.gm1);
                rot_layer<true>(l, a1);
                sl = a2.F * a1.F;
            } else {
                transpose(l, lds, c.a1, c.a2, false);
            }
            if (sl != (R)1) scale_tile(l, sl);
            store_l1<LIO, R, kLamNT>(l, a.lam, c, nelem);
            flush_merged(lds_stat, stat_row<R>(a, c), a.stat_mul == 2, v, rot_tf, static_cast<const R *>(a.dw), a.n,
                         a.diag, a.rotB);
            return;
        } else if constexpr (SHAPE == BW_DROTB) {
            const RotCoef<R> b1 = load_coef(rot_tf, a.n, a.rotB, c.q1, c.gm1);
            stats_visit<false>(p, l, 1, lds_stat, c.lane, c.w, (R)1);
            rot_layer2<true>(p, l, b1);
            const R fb1 = b1.F;
            transpose(p, lds, c.a1, c.a2, true);
            transpose(l, lds, c.a1, c.a2, true);
            stats_visit<true>(p, l, 1, lds_stat, c.lane, c.w, fb1 * fb1);
            const RotCoef<R> b2 = load_coef(rot_tf, a.n, a.rotB, c.q2, c.gm2);
            rot_layer<true>(l, b2);
            // lambda carries scale fb1 * b2.F; diag(r_l)^dagger removes it
            apply_diag_dag(l, diag_tables(static_cast<const R *>(a.dw), a.n, a.diag, c, *a.view, false),
                           fb1 * b2.F);
            transpose(l, lds, c.a1, c.a2, false);
        } else if constexpr (SHAPE == BW_ROTAD) {
            transpose(p, lds, c.a1, c.a2, true);
            transpose(l, lds, c.a1, c.a2, true);
            apply_diag2(p, l, diag_tables(static_cast<const R *>(a.dw), a.n, a.diag, c, *a.view, false), (R)1);
            stats_visit<true>(p, l, 0, lds_stat, c.lane, c.w, (R)1);
            const RotCoef<R> a2 = load_coef(rot_tf, a.n, la, c.q2, c.gm2);
            rot_layer2<true>(p, l, a2);
            const R fa2 = a2.F;
            transpose(p, lds, c.a1, c.a2, false);
            transpose(l, lds, c.a1, c.a2, false);
            stats_visit<false>(p, l, 0, lds_stat, c.lane, c.w, fa2 * fa2);
            const RotCoef<R> a1 = load_coef(rot_tf, a.n, la, c.q1, c.gm1);
            rot_layer<true>(l, a1);
            sl = fa2 * a1.F;
        } else if constexpr (SHAPE == BW_L0D) {
            // psi = the layer-0 product state; lambda (at the output of the product-state
            // pass, after diag(p_0)) is taken back through diag(p_0).
            transpose(p, lds, c.a1, c.a2, true);
            transpose(l, lds, c.a1, c.a2, true);
            apply_diag_dag(l, diag_tables(static_cast<const R *>(a.dw), a.n, a.diag, c, *a.view, false), (R)1);
            stats_visit<true>(p, l, 0, lds_stat, c.lane, c.w, (R)1);
            transpose(p, lds, c.a1, c.a2, false);
            transpose(l, lds, c.a1, c.a2, false);
            stats_visit<false>(p, l, 0, lds_stat, c.lane, c.w, (R)1);
            flush_stats(lds_stat, stat_row<R>(a, c), a.stat_mul == 2);
            return;
        } else if constexpr (SHAPE == BW_L0D_SEED) {
            // One-layer circuit: the seeded lambda = O psi is already at the statistics point
            // (O is diagonal and commutes with diag(p_0)).  The other views' passes read
            // lambda at the pass output, so diag(p_0) lambda is stored for them.
            stats_visit<false>(p, l, 0, lds_stat, c.lane, c.w, (R)1);
            transpose(p, lds, c.a1, c.a2, true);
            transpose(l, lds, c.a1, c.a2, true);
            stats_visit<true>(p, l, 0, lds_stat, c.lane, c.w, (R)1);
            apply_diag(l, diag_tables(static_cast<const R *>(a.dw), a.n, a.diag, c, *a.view, false), (R)1);
            transpose(l, lds, c.a1, c.a2, false);
            store_l1<LIO>(l, a.lam, c, nelem);
            flush_stats(lds_stat, stat_row<R>(a, c), a.stat_mul == 2);
            return;
        } else if constexpr (SHAPE == BW_ROTA) {
            // statistics of both layouts at the pass output; psi is not un-rotated
            stats_visit<false>(p, l, 0, lds_stat, c.lane, c.w, (R)1);
            transpose(p, lds, c.a1, c.a2, true);
            transpose(l, lds, c.a1, c.a2, true);
            stats_visit<true>(p, l, 0, lds_stat, c.lane, c.w, (R)1);
            const RotCoef<R> a2 = load_coef(rot_tf, a.n, la, c.q2, c.gm2);
            rot_layer<true>(l, a2);
            transpose(l, lds, c.a1, c.a2, false);
            const RotCoef<R> a1 = load_coef(rot_tf, a.n, la, c.q1, c.gm1);
            rot_layer<true>(l, a1);
            sl = a1.F * a2.F;
        } else {   // BW_L0
            stats_visit<false>(p, l, 0, lds_stat, c.lane, c.w, (R)1);
            transpose(p, lds, c.a1, c.a2, true);
            transpose(l, lds, c.a1, c.a2, true);
            stats_visit<true>(p, l, 0, lds_stat, c.lane, c.w, (R)1);
            if (a.flags & PF_STATS_ONLY) {
                flush_stats(lds_stat, stat_row<R>(a, c), a.stat_mul == 2);
                return;
            }
            transpose(l, lds, c.a1, c.a2, false);
        }
    }
    if (sl != (R)1) scale_tile(l, sl);
    if constexpr (SHAPE == BW_DROTB)
        store_l1_chain<LIO>(l, a.psi_out, c, nelem);   // the second lambda buffer (others read a.lam)
    else
        store_l1<LIO, R, kLamNT>(l, a.lam, c, nelem);
    flush_stats(lds_stat, stat_row<R>(a, c), a.stat_mul == 2);
}

// ------------------------------------------------------------------ half-tile adjoint pass
//
// The general adjoint shape [Ry-layer la on the group, D_la, Ry-layer lb on the group] on
// half tiles: 2^12 amplitudes in 256 threads x 16 registers (layouts H1 / H2,
// hqml_internal.hpp).  With half the registers of the full tile for the two states, four
// workgroups share a compute unit instead of two, so the loads of some overlap the
// arithmetic of others.  The arithmetic is that of the full-tile general shape (merged
// statistics into the same slots), in this order: load psi and lambda (H1); merged
// statistics of positions 0, 1 (lane bits: the partner lane's psi through a DPP quad
// permutation) and 4..7 (register bits); transpose both states; merged statistics of
// 8..11.  All of them are taken at the pass output (a qubit's statistics do not change
// under the rotations of the other group qubits, which are not its chain neighbours), so
// psi is never rotated and is dead here.  On lambda: un-rotate layer lb at 8..11 and 0, 1;
// transpose; un-rotate lb at 4..7, apply D_la^dagger, un-rotate layer la at 4..7 and 0, 1;
// transpose; un-rotate la at 8..11; store from H2, whose lane bits 0..3 are positions 0..3
// as in H1, so the stores stay 128-byte runs.  Written once for the compute type R: in fp64
// (complex128 lambda) the two states take 128 VGPRs and two workgroups share a compute unit.

struct HCtx {
    int lane, w, sample, tile;
    uint64_t tile_off;        // global amplitude offset of the tile's fixed (tile-index) bits
    uint32_t t1, t2;          // H1 / H2: thread's amplitude offset within the tile
    uint32_t a1, a2;          // swizzled LDS bases of the thread in H1 / H2
    uint32_t fixed1, fixed2;  // qubit bitmask of the thread's fixed bits (with the tile's) in H1 / H2
    uint32_t rs[4];           // H1: amplitude stride of register bit m (uniform)
    int q0[2], q1[4], q2[4];  // qubits at positions 0, 1 / 4..7 / 8..11
    uint32_t gm0, gm1, gm2;   // rotated-group masks of those positions
};

__device__ __forceinline__ void hctx(HCtx &c, const ViewDevH &v, int T2, int blk, int sample0)
{
    const int tid = threadIdx.x;
    c.lane = tid & 63;
    c.w = tid >> 6;
    const int lane = c.lane, w = c.w;
    // thread bits (lane 0..5, wave 0..1): H1 -> positions 0,1,2,3,8,9,10,11; H2 -> 0..7
    const int h1p[8] = {0, 1, 2, 3, 8, 9, 10, 11};
    const uint32_t tv = (uint32_t)lane | ((uint32_t)w << 6);
    uint32_t t1 = 0, t2 = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k)
        if ((tv >> k) & 1u) {
            t1 |= 1u << ldu(&v.perm[h1p[k]]);
            t2 |= 1u << ldu(&v.perm[k]);
        }
    c.t1 = t1;
    c.t2 = t2;
    c.a1 = hswz((uint32_t)(lane & 15) | ((uint32_t)(lane >> 4) << 8) | ((uint32_t)w << 10));
    c.a2 = hswz(tv);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        c.q1[m] = ldu(&v.perm[4 + m]);
        c.q2[m] = ldu(&v.perm[8 + m]);
        c.rs[m] = 1u << c.q1[m];
    }
    c.q0[0] = ldu(&v.perm[0]);
    c.q0[1] = ldu(&v.perm[1]);
    const uint32_t gm = (uint32_t)ldu(&v.group_mask);
    c.gm0 = gm & 3u;
    c.gm1 = (gm >> 4) & 15u;
    c.gm2 = (gm >> 8) & 15u;
    const int rel = blk / T2;
    c.tile = blk - rel * T2;
    c.sample = sample0 + rel;
    uint64_t toff = 0;
    uint32_t tb = 0;
    const int nt = ldu(&v.n_tile);
    for (int k = 0; k < nt; ++k)
        if ((c.tile >> k) & 1) {
            const int q = ldu(&v.tile_q[k]);
            toff |= 1ull << q;
            tb |= 1u << q;
        }
    c.tile_off = toff;
    c.fixed1 = t1 | tb;
    c.fixed2 = t2 | tb;
}

__device__ __forceinline__ uint32_t hroff(const HCtx &c, int j)
{
    uint32_t o = 0;
#pragma unroll
    for (int m = 0; m < 4; ++m)
        if (j & (1 << m)) o += c.rs[m];
    return o;
}

// Global-memory access of a half tile in layout H1 (NT: non-temporal loads).
template <int ST, bool NT, typename R>
__device__ __forceinline__ void hload(HTile<R> &t, const void *state, const HCtx &c, uint64_t nelem)
{
    using IO = StateIO<ST>;
    constexpr uint32_t esz = sizeof(typename IO::elem);
    using Off = TileOff<esz>;
    const char *base = reinterpret_cast<const char *>(state) + ((uint64_t)c.sample * nelem + c.tile_off) * esz;
    const Off tb = (Off)c.t1 * esz;
#pragma unroll
    for (int j = 0; j < kHalfRegs; ++j) {
        const Off off = tb + (Off)hroff(c, j) * esz;
        if constexpr (NT)
            IO::load(reinterpret_cast<const typename IO::elem *>(base + off), t.re[j], t.im[j]);
        else
            IO::load_temporal(reinterpret_cast<const typename IO::elem *>(base + off), t.re[j], t.im[j]);
    }
}

// Store lambda in layout H2 (positions 0..3 are lane bits 0..3 here as in H1, so a 16-lane
// row writes 16 consecutive amplitudes).
template <typename R>
__device__ __forceinline__ void hstore2(const HTile<R> &t, void *state, const HCtx &c, uint64_t nelem)
{
    using IO = StateIO<kLamIO<R>>;
    constexpr uint32_t esz = sizeof(typename IO::elem);
    using Off = TileOff<esz>;
    char *base = reinterpret_cast<char *>(state) + ((uint64_t)c.sample * nelem + c.tile_off) * esz;
    const Off tb = (Off)opaque_u32(c.t2) * esz;
#pragma unroll
    for (int j = 0; j < kHalfRegs; ++j) {
        uint32_t o = 0;
#pragma unroll
        for (int m = 0; m < 4; ++m)
            if (j & (1 << m)) o += 1u << c.q2[m];
        IO::store(reinterpret_cast<typename IO::elem *>(base + tb + (Off)o * esz), t.re[j], t.im[j]);
    }
}

// Store lambda in layout H1: at its own amplitudes, or (CHAIN) at P^-1 of them, P the CNOT
// chain's index map (P^-1 is linear over XOR, so the tile, thread and register parts of the
// index map separately); non-temporal (the CNOT-chain passes keep the plain tile order).
template <bool CHAIN, typename R>
__device__ __forceinline__ void hstore1(const HTile<R> &t, void *state, const HCtx &c, uint64_t nelem)
{
    using IO = StateIO<kLamIO<R>>;
    constexpr uint32_t esz = sizeof(typename IO::elem);
    using Off = TileOff<esz>;
    if constexpr (CHAIN) {
        const uint32_t mask = (uint32_t)(nelem - 1);
        char *base = reinterpret_cast<char *>(state) + (uint64_t)c.sample * nelem * esz;
        const uint32_t pt = chain_inv((uint32_t)c.tile_off | opaque_u32(c.t1), mask);
#pragma unroll
        for (int j = 0; j < kHalfRegs; ++j) {
            const Off off = (Off)(pt ^ chain_inv(hroff(c, j), mask)) * esz;
            IO::store(reinterpret_cast<typename IO::elem *>(base + off), t.re[j], t.im[j]);
        }
    } else {
        char *base = reinterpret_cast<char *>(state) + ((uint64_t)c.sample * nelem + c.tile_off) * esz;
        const Off tb = (Off)opaque_u32(c.t1) * esz;
#pragma unroll
        for (int j = 0; j < kHalfRegs; ++j) {
            const Off off = tb + (Off)hroff(c, j) * esz;
            if constexpr (sizeof(R) == 4)
                IO::store_nt(reinterpret_cast<typename IO::elem *>(base + off), t.re[j], t.im[j]);
            else
                IO::store(reinterpret_cast<typename IO::elem *>(base + off), t.re[j], t.im[j]);
        }
    }
}

// Move a half tile between H1 and H2 through the LDS buffer (32 KB in fp32, 64 KB in fp64).
template <typename R>
__device__ __forceinline__ void htranspose(HTile<R> &t, V2<R> *lds, uint32_t a1, uint32_t a2, bool from_h1)
{
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kHalfRegs; ++j) {
        const uint32_t i = from_h1 ? (a1 ^ ((uint32_t)j << 4)) : (a2 ^ hswz((uint32_t)j << 8));
        lds[i] = mk2(t.re[j], t.im[j]);
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kHalfRegs; ++j) {
        const uint32_t i = from_h1 ? (a2 ^ hswz((uint32_t)j << 8)) : (a1 ^ ((uint32_t)j << 4));
        const V2<R> v = lds[i];
        t.re[j] = v.x;
        t.im[j] = v.y;
    }
}

template <typename R>
struct HCoef {
    R k[4];
    R F;      // product of the scale factors of the rotated bits
};

// Tan-form coefficients of NB positions (qubits q[m]); positions outside mask: identity.
template <int NB, typename R>
__device__ __forceinline__ HCoef<R> hcoef(const R *rot_tf, int n, int layer, const int *q, uint32_t mask)
{
    HCoef<R> rc;
    rc.F = (R)1;
#pragma unroll
    for (int m = 0; m < NB; ++m) {
        const V2<R> kf = ldu2(rot_tf + ((size_t)layer * n + q[m]) * 2);
        const bool on = (mask >> m) & 1u;
        rc.k[m] = on ? kf.x : (R)0;
        rc.F *= on ? kf.y : (R)1;
    }
    return rc;
}

template <typename R>
__device__ __forceinline__ void hunrot_regs(HTile<R> &t, const HCoef<R> &rc)
{
    hrot_bit<0>(t, -rc.k[0]);
    hrot_bit<1>(t, -rc.k[1]);
    hrot_bit<2>(t, -rc.k[2]);
    hrot_bit<3>(t, -rc.k[3]);
}

// Parity of this thread's chain neighbours of qubit q (1: Z_{q-1} Z_{q+1} = -1).
__device__ __forceinline__ bool nb_odd(uint32_t fixed, int q, int n)
{
    uint32_t nb = q + 1 < n ? 1u << (q + 1) : 0u;
    if (q > 0) nb |= 1u << (q - 1);
    return __builtin_popcount(fixed & nb) & 1;
}

// Plain (layer lb) and neighbour-signed (layer la, see stats_visit_merged) sums of one
// position's statistics into its slots.  A DPP row is lane bits 0..3, i.e. positions 0..3,
// which hold qubits 0..3: for a qubit q >= 5 neither chain neighbour is there, the
// neighbours' sign is the same on the whole row, and the row leader forms the signed sums
// from the plain ones (one reduction instead of two).  q is uniform, so is the branch.
template <typename R>
__device__ __forceinline__ void hstat_out(R sx, R sy, R sz, R corr, bool odd, int q, int sp, R *lds_stat, int lane,
                                          int w)
{
    if (q >= 5) {
        row_sum16x3(sx, sy, sz);
        if ((lane & 15) == 15) {
            const int r = w * 4 + (lane >> 4);
            const R sg = odd ? -corr : corr;
            lds_stat[((13 + sp) * 3 + 0) * 16 + r] = sx * corr;
            lds_stat[((13 + sp) * 3 + 1) * 16 + r] = sy * corr;
            lds_stat[((13 + sp) * 3 + 2) * 16 + r] = sz * corr;
            lds_stat[(sp * 3 + 0) * 16 + r] = sx * sg;
            lds_stat[(sp * 3 + 1) * 16 + r] = sy * sg;
            lds_stat[(sp * 3 + 2) * 16 + r] = sz * sg;
        }
    } else {
        const R sg = odd ? -corr : corr;
        stat_out3(sx * corr, sy * corr, sz * corr, lds_stat, (13 + sp) * 3, lane, w);
        stat_out3(sx * sg, sy * sg, sz * sg, lds_stat, sp * 3, lane, w);
    }
}

// Statistics of one position into its slots (sel*13 + pos)*3 (one rotation layer per pass).
template <typename R>
__device__ __forceinline__ void hstat_plain(R sx, R sy, R sz, int sel, int sp, R *lds_stat, int lane, int w)
{
    stat_out3(sx, sy, sz, lds_stat, (sel * 13 + sp) * 3, lane, w);
}

// Factor tables of D_l in layout H2: D(i) = lo[j & 3] * hi[j >> 2] for register j
// (positions 8, 9 and 10, 11), thread constant and CZ signs with fixed qubits folded in
// as in diag_tables; the half view keeps positions 8, 9 apart from 10, 11 in the chain.
template <typename R>
struct HDiag {
    V2<R> lo[4];
    V2<R> hi[4];
};

// Factor tables of D_l in layout H1 (H1 = true: registers at positions 4..7, lo = 4, 5 and
// hi = 6, 7) or H2 (registers at 8..11, lo = 8, 9 and hi = 10, 11).  tv: the thread's lane
// and wave bits, at H1 positions 0,1,2,3,8,9,10,11 or H2 positions 0..7.
template <bool H1, typename R>
__device__ __forceinline__ HDiag<R> hdiag_tables(const R *dw, int n, int layer, const HCtx &c, const ViewDevH &v,
                                                 uint32_t tv, bool cz = true)
{
    const V4<R> *wl = reinterpret_cast<const V4<R> *>(dw) + (size_t)layer * n;
    const uint32_t fixed_bits = H1 ? c.fixed1 : c.fixed2;
    // thread constant: lane and wave qubits (per lane), then the tile's qubits (uniform)
    V2<R> ct = mk2((R)1, (R)0);
#pragma unroll 1
    for (int k = 0; k < 8; ++k) {
        const int pos = H1 ? (k < 4 ? k : k + 4) : k;
        ct = cmul(ct, hfactor<R>(wl, ldu(&v.perm[pos]), (tv >> k) & 1u));
    }
    const int nt = ldu(&v.n_tile);
    V2<R> cu = mk2((R)1, (R)0);
    for (int k = 0; k < nt; ++k) {
        const int q = ldu(&v.tile_q[k]);
        cu = cmul(cu, hfactor<R>(wl, q, (c.tile >> k) & 1));
    }
    V2<R> cc = cmul(ct, cu);
    if (cz && (__builtin_popcount(fixed_bits & (fixed_bits >> 1)) & 1)) {   // CZ signs among fixed qubits
        cc.x = -cc.x;
        cc.y = -cc.y;
    }
    const int *rq = H1 ? c.q1 : c.q2;
    V2<R> g0[4], g1[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const int q = rq[m];
        g0[m] = hfactor<R>(wl, q, false);
        g1[m] = hfactor<R>(wl, q, true);
        if (cz && nb_odd(fixed_bits, q, n)) {   // CZ with a fixed neighbour at 1
            g1[m].x = -g1[m].x;
            g1[m].y = -g1[m].y;
        }
    }
    auto adj = [&](int a, int b) { const int d = rq[a] - rq[b]; return cz && (d == 1 || d == -1); };
    HDiag<R> t;
#pragma unroll
    for (int a = 0; a < 4; ++a) {
        V2<R> x = cmul(cc, cmul((a & 1) ? g1[0] : g0[0], (a & 2) ? g1[1] : g0[1]));
        if (a == 3 && adj(0, 1)) {
            x.x = -x.x;
            x.y = -x.y;
        }
        t.lo[a] = x;
        V2<R> h = cmul((a & 1) ? g1[2] : g0[2], (a & 2) ? g1[3] : g0[3]);
        if (a == 3 && adj(2, 3)) {
            h.x = -h.x;
            h.y = -h.y;
        }
        t.hi[a] = h;
    }
    return t;
}

// s * D^dagger on a half tile (the tables of its layout).
template <typename R>
__device__ __forceinline__ void hdiag_dag(HTile<R> &t, HDiag<R> d, R s)
{
#pragma unroll
    for (int a = 0; a < 4; ++a) {
        d.lo[a].x *= s;
        d.lo[a].y *= s;
    }
#pragma unroll
    for (int j = 0; j < kHalfRegs; ++j) {
        V2<R> f = cmul(d.lo[j & 3], d.hi[j >> 2]);
        f.y = -f.y;
        const R r = t.re[j], i = t.im[j];
        t.re[j] = r * f.x - i * f.y;
        t.im[j] = r * f.y + i * f.x;
    }
}

// Shapes of the half-tile adjoint pass.
enum HalfShape : int {
    HB_GENERAL = 0,   // CZ-chain plan: [rotA(la), D_la, rotB(lb)], merged statistics
    HB_ROTAD = 1,     // CNOT-chain plan: [rotA(l), diag(p_l)]
    HB_DROTB = 2      // CNOT-chain plan: [diag(r_l), rotB(l)], lambda written back through P^-1
};

template <int ST, int HS, typename R>
__global__ __launch_bounds__(kThreads, sizeof(R) == 4 ? 4 : 2) void k_tile_bwdh(TilePassArgs a)
{
    __shared__ V2<R> lds[1 << kHalfBits];
    __shared__ R lds_stat[kSlots * 16 + 16];
    const R *rot_tf = static_cast<const R *>(a.rot_tf);
    const R *dw = static_cast<const R *>(a.dw);
    const ViewDevH &v = *a.hview;
    const int T2 = a.T * 2, n = a.n, la = a.rotA, lb = a.rotB;
    const uint32_t tv = (uint32_t)threadIdx.x;
    // the CZ plan's general passes go in the XCD-contiguous order with lambda through L2; the
    // CNOT chain's [rotA, diag] passes in the plain order, its [diag, rotB] passes (lambda
    // written through the chain's index map) with complementary tiles paired
    constexpr bool kXcd = HS == HB_GENERAL;
    HCtx c;
    const int blk = (int)blockIdx.x, G = (int)gridDim.x;
    hctx(c, v, T2, kXcd ? xcd_slot(blk, G) : HS == HB_DROTB ? chain_pair_slot(blk, G, T2) : blk, a.sample0);
    zero_stats(lds_stat);
    __syncthreads();
    const uint64_t nelem = 1ull << n;
    HTile<R> p, l;
    hload<ST, true>(p, a.psi_in, c, nelem);
    if constexpr (sizeof(R) == 4 && kXcd)
        hload<0, false>(l, a.lam, c, nelem);   // through L2 (the XCD-contiguous order keeps it there)
    else
        hload<kLamIO<R>, true>(l, a.lam, c, nelem);
    if constexpr (HS == HB_ROTAD) {   // diag(p_l)^dagger on both states: to the point after rotA
        const HDiag<R> d = hdiag_tables<true>(dw, n, a.diag, c, v, tv, false);
        hdiag_dag(p, d, (R)1);
        hdiag_dag(l, d, (R)1);
    }
    // statistics of every position at one point (the pass output, or after diag(p_l)^dagger)
    // the CZ plan's merged statistics; a CNOT-chain pass's single rotation layer: slot group sel
    constexpr int sel = HS == HB_DROTB ? 1 : 0;
    {   // positions 0, 1 and 4..7 (H1)
        R dz[4];
        const R W = hzsum<4, 0>(p, l, dz);
        R sx, sy;
        hxy_lane<0>(p, l, c.lane, sx, sy);
        if constexpr (HS == HB_GENERAL)
            hstat_out(sx, sy, (c.lane & 1) ? -W : W, (R)1, nb_odd(c.fixed1, c.q0[0], n), c.q0[0], ldu(&v.slot_pos[0]),
                      lds_stat, c.lane, c.w);
        else
            hstat_plain(sx, sy, (c.lane & 1) ? -W : W, sel, ldu(&v.slot_pos[0]), lds_stat, c.lane, c.w);
        hxy_lane<1>(p, l, c.lane, sx, sy);
        if constexpr (HS == HB_GENERAL)
            hstat_out(sx, sy, (c.lane & 2) ? -W : W, (R)1, nb_odd(c.fixed1, c.q0[1], n), c.q0[1], ldu(&v.slot_pos[1]),
                      lds_stat, c.lane, c.w);
        else
            hstat_plain(sx, sy, (c.lane & 2) ? -W : W, sel, ldu(&v.slot_pos[1]), lds_stat, c.lane, c.w);
#define HQML_HSTAT1(M)                                                                                         \
    hxy_reg<M>(p, l, sx, sy);                                                                                  \
    if constexpr (HS == HB_GENERAL)                                                                            \
        hstat_out(sx, sy, dz[M], (R)1, nb_odd(c.fixed1, c.q1[M], n), c.q1[M], ldu(&v.slot_pos[4 + M]), lds_stat, \
                  c.lane, c.w);                                                                                \
    else                                                                                                       \
        hstat_plain(sx, sy, dz[M], sel, ldu(&v.slot_pos[4 + M]), lds_stat, c.lane, c.w);
        HQML_HSTAT1(0)
        HQML_HSTAT1(1)
        HQML_HSTAT1(2)
        HQML_HSTAT1(3)
#undef HQML_HSTAT1
    }
    htranspose(p, lds, c.a1, c.a2, true);
    htranspose(l, lds, c.a1, c.a2, true);
    {   // positions 8..11 (H2), at the same point
        R dz[4];
        (void)hzsum<4, 0>(p, l, dz);
        R sx, sy;
#define HQML_HSTAT2(M)                                                                                         \
    hxy_reg<M>(p, l, sx, sy);                                                                                  \
    if constexpr (HS == HB_GENERAL)                                                                            \
        hstat_out(sx, sy, dz[M], (R)1, nb_odd(c.fixed2, c.q2[M], n), c.q2[M], ldu(&v.slot_pos[8 + M]), lds_stat, \
                  c.lane, c.w);                                                                                \
    else                                                                                                       \
        hstat_plain(sx, sy, dz[M], sel, ldu(&v.slot_pos[8 + M]), lds_stat, c.lane, c.w);
        HQML_HSTAT2(0)
        HQML_HSTAT2(1)
        HQML_HSTAT2(2)
        HQML_HSTAT2(3)
#undef HQML_HSTAT2
    }
    R *dst = static_cast<R *>(a.stat_part) + ((size_t)c.sample * T2 + c.tile) * kSlots;
    if constexpr (HS == HB_GENERAL) {
        // lambda: layer lb at 8..11 and 0, 1 (H2), at 4..7 (H1); D_la^dagger (H1), which removes
        // the scales so far; layer la at 4..7 and 0, 1 (H1), at 8..11 (H2); store from H2
        const HCoef<R> b2 = hcoef<4>(rot_tf, n, lb, c.q2, c.gm2);
        hunrot_regs(l, b2);
        const HCoef<R> b0 = hcoef<2>(rot_tf, n, lb, c.q0, c.gm0);
        hunrot_lane<0>(l, b0.k[0], c.lane);
        hunrot_lane<1>(l, b0.k[1], c.lane);
        htranspose(l, lds, c.a1, c.a2, false);
        const HCoef<R> b1 = hcoef<4>(rot_tf, n, lb, c.q1, c.gm1);
        hunrot_regs(l, b1);
        hdiag_dag(l, hdiag_tables<true>(dw, n, a.diag, c, v, tv), b1.F * b2.F * b0.F);
        const HCoef<R> a1 = hcoef<4>(rot_tf, n, la, c.q1, c.gm1);
        hunrot_regs(l, a1);
        const HCoef<R> a0 = hcoef<2>(rot_tf, n, la, c.q0, c.gm0);
        hunrot_lane<0>(l, a0.k[0], c.lane);
        hunrot_lane<1>(l, a0.k[1], c.lane);
        htranspose(l, lds, c.a1, c.a2, true);
        const HCoef<R> a2 = hcoef<4>(rot_tf, n, la, c.q2, c.gm2);
        hunrot_regs(l, a2);
        const R sl = a2.F * a0.F * a1.F;
        if (sl != (R)1) {
#pragma unroll
            for (int j = 0; j < kHalfRegs; ++j) {
                l.re[j] *= sl;
                l.im[j] *= sl;
            }
        }
        hstore2(l, a.lam, c, nelem);
        flush_merged(lds_stat, dst, false, *a.view, rot_tf, dw, n, a.diag, lb);
    } else {
        // the pass's rotation layer lr at 8..11 and 0, 1 (H2) and at 4..7 (H1); DROTB then takes
        // lambda back through diag(r_l) (removing the scales) and writes it through P^-1
        const int lr = HS == HB_DROTB ? lb : la;
        const HCoef<R> r2 = hcoef<4>(rot_tf, n, lr, c.q2, c.gm2);
        hunrot_regs(l, r2);
        const HCoef<R> r0 = hcoef<2>(rot_tf, n, lr, c.q0, c.gm0);
        hunrot_lane<0>(l, r0.k[0], c.lane);
        hunrot_lane<1>(l, r0.k[1], c.lane);
        htranspose(l, lds, c.a1, c.a2, false);
        const HCoef<R> r1 = hcoef<4>(rot_tf, n, lr, c.q1, c.gm1);
        hunrot_regs(l, r1);
        const R sl = r2.F * r0.F * r1.F;
        if constexpr (HS == HB_DROTB) {
            hdiag_dag(l, hdiag_tables<true>(dw, n, a.diag, c, v, tv, false), sl);
            hstore1<true>(l, a.psi_out, c, nelem);   // the second lambda buffer (other tiles read a.lam)
        } else {
            if (sl != (R)1) {
#pragma unroll
                for (int j = 0; j < kHalfRegs; ++j) {
                    l.re[j] *= sl;
                    l.im[j] *= sl;
                }
            }
            hstore1<false>(l, a.lam, c, nelem);
        }
        flush_stats(lds_stat, dst, false);
    }
}

// ------------------------------------------------------------------ table preparation (fp64)

struct cd {
    double re, im;
};
__device__ __forceinline__ cd cmk(double r, double i) { return cd{r, i}; }
__device__ __forceinline__ cd operator*(cd a, cd b) { return cd{a.re * b.re - a.im * b.im, a.re * b.im + a.im * b.re}; }
__device__ __forceinline__ cd operator+(cd a, cd b) { return cd{a.re + b.re, a.im + b.im}; }
__device__ __forceinline__ cd cconj(cd a) { return cd{a.re, -a.im}; }

struct m2 {
    cd m[4];
};
__device__ __forceinline__ m2 mmul(const m2 &a, const m2 &b)
{
    m2 r;
    r.m[0] = a.m[0] * b.m[0] + a.m[1] * b.m[2];
    r.m[1] = a.m[0] * b.m[1] + a.m[1] * b.m[3];
    r.m[2] = a.m[2] * b.m[0] + a.m[3] * b.m[2];
    r.m[3] = a.m[2] * b.m[1] + a.m[3] * b.m[3];
    return r;
}
__device__ __forceinline__ m2 mdag(const m2 &a)
{
    m2 r;
    r.m[0] = cconj(a.m[0]);
    r.m[1] = cconj(a.m[2]);
    r.m[2] = cconj(a.m[1]);
    r.m[3] = cconj(a.m[3]);
    return r;
}
__device__ __forceinline__ m2 m_rx(double t)
{
    double s, c;
    sincos(0.5 * t, &s, &c);
    return m2{{cmk(c, 0), cmk(0, -s), cmk(0, -s), cmk(c, 0)}};
}
__device__ __forceinline__ m2 m_ry(double t)
{
    double s, c;
    sincos(0.5 * t, &s, &c);
    return m2{{cmk(c, 0), cmk(-s, 0), cmk(s, 0), cmk(c, 0)}};
}
__device__ __forceinline__ m2 m_rz(double t)
{
    double s, c;
    sincos(0.5 * t, &s, &c);
    return m2{{cmk(c, -s), cmk(0, 0), cmk(0, 0), cmk(c, s)}};
}

// zyz[(l*n+q)*6]: cos(beta/2), sin(beta/2), p.re, p.im, r.re, r.im
constexpr int kPrepThreads = 512;   // workgroup of the fused preparation kernel

template <typename TI>
__device__ __forceinline__ void prep_zyz_at(const TI *theta, int L, int n, double *zyz, int idx)
{
    if (idx >= L * n) return;
    const double ax = theta[idx * 3 + 0], ay = theta[idx * 3 + 1], az = theta[idx * 3 + 2];
    const m2 U = mmul(m_rz(az), mmul(m_ry(ay), m_rx(ax)));
    const cd x = U.m[0], y = U.m[2];
    const double ax_ = sqrt(x.re * x.re + x.im * x.im), ay_ = sqrt(y.re * y.re + y.im * y.im);
    const double nrm = sqrt(ax_ * ax_ + ay_ * ay_);
    const double cb = ax_ / nrm, sb = ay_ / nrm;
    const cd xh = ax_ > 1e-300 ? cmk(x.re / ax_, x.im / ax_) : cmk(1, 0);
    const cd yh = ay_ > 1e-300 ? cmk(y.re / ay_, y.im / ay_) : cmk(1, 0);
    // r = principal sqrt of xh*yh (a unit complex number); p = xh * conj(r)
    const cd z = xh * yh;
    const double ang = atan2(z.im, z.re) * 0.5;
    double sr, cr;
    sincos(ang, &sr, &cr);
    const cd r = cmk(cr, sr);
    const cd p = xh * cconj(r);
    double *o = zyz + (size_t)idx * 6;
    o[0] = cb;
    o[1] = sb;
    o[2] = p.re;
    o[3] = p.im;
    o[4] = r.re;
    o[5] = r.im;
}

template <typename TI>
__global__ void k_prep_zyz(const TI *theta, int L, int n, double *zyz)
{
    prep_zyz_at(theta, L, n, zyz, blockIdx.x * blockDim.x + threadIdx.x);
}

// Pauli frame.  Where beta_{l,q} > pi/2 (sin > cos, l >= 1) the real rotation is
// rewritten exactly as Ry(beta) = Ry(beta - pi) X Z, so every rotation the tile
// kernels apply has |tan(beta'/2)| <= 1.  Each X is moved to the start of the
// circuit: it flips the sign of every earlier Ry angle of that qubit, swaps the
// qubit's factors in every earlier diagonal (and turns CZ(q, q +- 1) into CZ times a
// Z on the neighbour), and swaps the qubit's layer-0 product factors.  Each Z merges
// into the preceding diagonal.  Global phases are dropped (they cancel in E and in
// every gradient statistic).  G[l][q] = parity of the X's from layers after l; the
// simulated state at P_l is X^G times the original one, so the Y and Z statistics
// of such qubits change sign, which the gradient map H absorbs.
// ent = 1 (CNOT chain, whole-circuit kernel): no frame, G = 0.  ent = 2 (CNOT chain,
// tile passes): the same rewrite, but an X^g moved left through the chain P becomes
// X^(P^-1 g), P^-1 g = g ^ (g << 1) (no Z appears), so the frame is a qubit mask carried
// from layer to layer by one thread.
// Rewrite flags (sin > cos, layers l >= 1) of qubit q for the 32 layers lhi, lhi - 1, ...:
// bit k for layer lhi - k.  The 64 loads are issued before any is used (the scan below
// stores between its reads, and a byte store may alias the table, so reading layer by
// layer would wait a memory round trip per layer).
__device__ __forceinline__ uint32_t prep_rewrite_flags(const double *zyz, int n, int q, int lhi)
{
    double s[32], c[32];
#pragma unroll
    for (int k = 0; k < 32; ++k) {
        const int l = lhi - k;
        const double *z = zyz + ((size_t)(l >= 1 ? l : 1) * n + q) * 6;
        c[k] = z[0];
        s[k] = z[1];
    }
    uint32_t f = 0;
#pragma unroll
    for (int k = 0; k < 32; ++k)
        if (lhi - k >= 1 && s[k] > c[k]) f |= 1u << k;
    return f;
}

__device__ __forceinline__ void prep_frame_at(const double *zyz, int L, int n, int ent, unsigned char *G, int q)
{
    if (ent == 2) {
        // one wave, lane q = qubit q (n <= 29 < 64); the mask g is the same in every lane
        const uint32_t full = (uint32_t)((1ull << n) - 1ull);
        uint32_t g = 0;
        for (int lhi = L - 1; lhi >= 0; lhi -= 32) {
            const uint32_t f = (q < n && L > 1) ? prep_rewrite_flags(zyz, n, q, lhi) : 0u;
            for (int k = 0; k < 32 && lhi - k >= 0; ++k) {
                const int l = lhi - k;
                if (q < n) G[(size_t)l * n + q] = (unsigned char)((g >> q) & 1u);
                if (l == 0) break;
                // qubits rewritten at layer l: their X enters before Ry, after diag(r_l)
                const uint32_t rw = (uint32_t)__ballot((f >> k) & 1u) & full;
                const uint32_t gb = g ^ rw;
                g = (gb ^ (gb << 1)) & full;
            }
        }
        return;
    }
    if (q >= n) return;
    unsigned char g = 0;
    for (int lhi = L - 1; lhi >= 0; lhi -= 32) {
        const uint32_t f = (ent == 0 && L > 1) ? prep_rewrite_flags(zyz, n, q, lhi) : 0u;
        for (int k = 0; k < 32 && lhi - k >= 0; ++k) {
            const int l = lhi - k;
            G[(size_t)l * n + q] = g;
            if ((f >> k) & 1u) g ^= 1;
        }
    }
}

#if HQML_BWD32_UNIT == 0   // a non-template kernel: defined in one compilation unit only
__global__ void __launch_bounds__(64) k_prep_frame(const double *zyz, int L, int n, int ent, unsigned char *G)
{
    prep_frame_at(zyz, L, n, ent, G, blockIdx.x * blockDim.x + threadIdx.x);
}
#endif

// rot_tf[l][q] = (k, f): the simulated rotation is Ry(beta') = f [[1, -k], [k, 1]],
//   f = cos(beta'/2) >= 1/sqrt 2, k = tan(beta'/2) in [-1, 1] (frame sign included);
// dw[l][q] = (f0, f1): D_l's factor of qubit q for bit value 0 / 1 (l < L-1),
//   from w = p_{l,q} r_{l+1,q} (f0 = w, f1 = conj w) in the frame described above;
// H[l][q][a][s]: Pauli coefficients of diag(p)^dag G_a diag(p), G_a the generator of
//   theta[l][q][a] moved to just after U_{l,q} (G_z = Z, G_y = Rz Y Rz^dag,
//   G_x = Rz Ry X Ry^dag Rz^dag), with the Y and Z coefficients negated where G[l][q].
// With the CNOT entangler the diagonals cannot merge across the chain (a permutation).
// ent = 1 (whole-circuit kernel, no frame): rot_tf[l][q] = (sin(beta/2), cos(beta/2)) and
// dw[l][q] = (p, r), the factors of diag(p, conj p) after and diag(r, conj r) before
// Ry(beta).  ent = 2 (tile passes): rot_tf in the tan form with the frame, dw row l =
// (f0, f1) of diag(p_l) and row L + l of diag(r_l) (times the rewrite's Z), the two
// factors swapped where an X of the frame passes them.
template <typename TI, typename R>
__device__ __forceinline__ void prep_tables_at(const TI *theta, const double *zyz, const unsigned char *G, int L, int n,
                                               int ent, R *rot_tf, R *dw, double *H, int idx)
{
    if (idx >= L * n) return;
    const int l = idx / n, q = idx - l * n;
    const double *z = zyz + (size_t)idx * 6;
    const bool gq = G[idx] != 0;
    if (ent == 1) {
        rot_tf[idx * 2 + 0] = (R)z[1];
        rot_tf[idx * 2 + 1] = (R)z[0];
        for (int k = 0; k < 4; ++k) dw[(size_t)idx * 4 + k] = (R)z[2 + k];
    } else if (ent == 2) {
        const bool x_here = l >= 1 && z[1] > z[0];
        double k = x_here ? -z[0] / z[1] : z[1] / z[0];
        if (gq) k = -k;
        rot_tf[idx * 2 + 0] = (R)k;
        rot_tf[idx * 2 + 1] = (R)(x_here ? z[1] : z[0]);
        const cd p = cmk(z[2], z[3]), r = cmk(z[4], z[5]);
        const cd p0 = gq ? cconj(p) : p, p1 = gq ? p : cconj(p);
        R *dp = dw + (size_t)idx * 4;
        dp[0] = (R)p0.re;
        dp[1] = (R)p0.im;
        dp[2] = (R)p1.re;
        dp[3] = (R)p1.im;
        cd r1 = cconj(r);
        if (x_here) r1 = cmk(-r1.re, -r1.im);   // the rewrite's Z, applied after diag(r_l)
        const bool sw = gq != x_here;           // the X's at the point before Ry(beta')
        const cd f0 = sw ? r1 : r, f1 = sw ? r : r1;
        R *dr = dw + ((size_t)L * n + idx) * 4;
        dr[0] = (R)f0.re;
        dr[1] = (R)f0.im;
        dr[2] = (R)f1.re;
        dr[3] = (R)f1.im;
    } else {
        const bool x_here = l >= 1 && z[1] > z[0];
        double k = x_here ? -z[0] / z[1] : z[1] / z[0];
        const double f = x_here ? z[1] : z[0];
        if (gq) k = -k;
        rot_tf[idx * 2 + 0] = (R)k;
        rot_tf[idx * 2 + 1] = (R)f;
        R *d = dw + (size_t)idx * 4;
        if (l + 1 < L) {
            const double *zn = zyz + (size_t)(idx + n) * 6;
            const cd w = cmk(z[2], z[3]) * cmk(zn[4], zn[5]);
            cd f0 = w, f1 = cconj(w);
            if (gq) {
                const cd t = f0;
                f0 = f1;
                f1 = t;
            }
            int sflip = (zn[1] > zn[0]) ? 1 : 0;            // Z from the next layer's rewrite
            if (q > 0) sflip ^= G[idx - 1];                 // CZ(q-1, q) conjugated by X on q-1
            if (q + 1 < n) sflip ^= G[idx + 1];             // CZ(q, q+1) conjugated by X on q+1
            if (sflip) f1 = cmk(-f1.re, -f1.im);
            d[0] = (R)f0.re;
            d[1] = (R)f0.im;
            d[2] = (R)f1.re;
            d[3] = (R)f1.im;
        } else {
            // the trailing diagonal (layer L-1's left factors; with the CZ chain it follows the
            // last Ry layer): never applied by the passes, which drop it since it commutes
            // with a Z-string observable; Pauli strings with X/Y factors apply it.  No frame
            // bit reaches past the last layer.
            d[0] = (R)z[2];
            d[1] = (R)z[3];
            d[2] = (R)z[2];
            d[3] = (R)-z[3];
        }
    }
    const double ay = theta[idx * 3 + 1], az = theta[idx * 3 + 2];
    const m2 X = m2{{cmk(0, 0), cmk(1, 0), cmk(1, 0), cmk(0, 0)}};
    const m2 Y = m2{{cmk(0, 0), cmk(0, -1), cmk(0, 1), cmk(0, 0)}};
    const m2 Z = m2{{cmk(1, 0), cmk(0, 0), cmk(0, 0), cmk(-1, 0)}};
    const m2 Rz = m_rz(az), RzRy = mmul(m_rz(az), m_ry(ay));
    const cd p = cmk(z[2], z[3]);
    const m2 Lp = m2{{p, cmk(0, 0), cmk(0, 0), cconj(p)}};
    m2 Gen[3];
    Gen[0] = mmul(RzRy, mmul(X, mdag(RzRy)));
    Gen[1] = mmul(Rz, mmul(Y, mdag(Rz)));
    Gen[2] = Z;
    for (int a = 0; a < 3; ++a) {
        const m2 S = mmul(mdag(Lp), mmul(Gen[a], Lp));
        double *h = H + ((size_t)idx * 3 + a) * 3;
        h[0] = S.m[1].re;                        // X coefficient
        h[1] = gq ? S.m[1].im : -S.m[1].im;      // Y coefficient
        h[2] = gq ? -S.m[0].re : S.m[0].re;      // Z coefficient
    }
}

template <typename TI, typename R>
__global__ void k_prep_tables(const TI *theta, const double *zyz, const unsigned char *G, int L, int n, int ent,
                              R *rot_tf, R *dw, double *H)
{
    prep_tables_at(theta, zyz, G, L, n, ent, rot_tf, dw, H, blockIdx.x * blockDim.x + threadIdx.x);
}

// u[b][q] = Ry(beta_{0,q}) diag(r, conj r) (cos x/2, sin x/2): the layer-0 product
// factor, with its two components swapped where the frame has an X on qubit q.
template <typename TI, typename R>
__device__ __forceinline__ void prep_init_at(const TI *x, const double *zyz, const unsigned char *G, int B, int n, R *init_u,
                                             int idx)
{
    if (idx >= B * n) return;
    const int q = idx % n;
    const double *z = zyz + (size_t)q * 6;
    double s, c;
    sincos(0.5 * (double)x[idx], &s, &c);
    const cd r = cmk(z[4], z[5]);
    const cd a0 = cmk(r.re * c, r.im * c);        // r cos
    const cd a1 = cmk(r.re * s, -r.im * s);       // conj(r) sin
    const double cb = z[0], sb = z[1];
    const cd u0 = cmk(cb * a0.re - sb * a1.re, cb * a0.im - sb * a1.im);
    const cd u1 = cmk(sb * a0.re + cb * a1.re, sb * a0.im + cb * a1.im);
    const bool sw = G[q] != 0;
    R *o = init_u + (size_t)idx * 4;
    o[0] = (R)(sw ? u1.re : u0.re);
    o[1] = (R)(sw ? u1.im : u0.im);
    o[2] = (R)(sw ? u0.re : u1.re);
    o[3] = (R)(sw ? u0.im : u1.im);
}

template <typename TI, typename R>
__global__ void k_prep_init(const TI *x, const double *zyz, const unsigned char *G, int B, int n, R *init_u)
{
    prep_init_at(x, zyz, G, B, n, init_u, blockIdx.x * blockDim.x + threadIdx.x);
}

// All four preparation steps in one workgroup, for small tables (one launch instead of
// four: at 12 qubits / 20 layers the separate launches cost 19 us of a 0.27 ms step).
template <typename TI, typename R>
__global__ void __launch_bounds__(kPrepThreads) k_prep_fused(const TI *theta, const TI *x, int L, int n, int B, int ent,
                                                              double *zyz, unsigned char *G, R *rot_tf, R *dw,
                                                              double *H, R *init_u)
{
    // the factorisation and the frame stay in LDS (no later kernel reads them), so the steps
    // after each barrier read them without a memory round trip
    (void)zyz;
    (void)G;
    __shared__ double zs[kPrepThreads * 6];
    __shared__ unsigned char gs[kPrepThreads];
    const int t = threadIdx.x;
    for (int i = t; i < L * n; i += kPrepThreads) prep_zyz_at(theta, L, n, zs, i);
    __syncthreads();
    if (t < 64) prep_frame_at(zs, L, n, ent, gs, t);   // wave 0: the frame is a scan over layers
    __syncthreads();
    for (int i = t; i < L * n; i += kPrepThreads) prep_tables_at(theta, zs, gs, L, n, ent, rot_tf, dw, H, i);
    for (int i = t; i < B * n; i += kPrepThreads) prep_init_at(x, zs, gs, B, n, init_u, i);
}

// ------------------------------------------------------------------ reductions (fixed order)

// E_b = sum over tiles (fp64); with y: loss = mean (E - y)^2 and dLdE = 2 (E - y) / B.
// First stage for samples with many tiles: out[b][ch] = sum of the <O> partials of
// tiles ch*kTileChunk .. (ch+1)*kTileChunk-1 of sample b, by a fixed-order tree.
// Grid (T / kTileChunk, B), kTileChunk threads.
template <typename P>
__global__ void __launch_bounds__(kTileChunk) k_ez_chunks(const P *e_part, int T, double *out)
{
    __shared__ double red[kTileChunk];
    const int nch = gridDim.x, ch = blockIdx.x, b = blockIdx.y, i = threadIdx.x;
    red[i] = (double)e_part[(size_t)b * T + (size_t)ch * kTileChunk + i];
    __syncthreads();
    for (int h = kTileChunk / 2; h > 0; h >>= 1) {
        if (i < h) red[i] += red[i + h];
        __syncthreads();
    }
    if (i == 0) out[(size_t)b * nch + ch] = red[0];
}

// E_b = sum over the T per-tile (or per-chunk) partials of sample b in order; with
// labels y also the MSE loss and dL/dE_b = 2 (E_b - y_b) / B.  IO is the caller's
// array type (float or double).  One workgroup of kEzThreads threads.
constexpr int kEzThreads = 256;
// The loss: thread t adds the squared errors of samples t, t + 256, ... in order, then
// thread 0 adds the 256 partials in order (a fixed order; the partials stay on chip).
template <typename P, typename IO>
__global__ void __launch_bounds__(kEzThreads) k_ez_reduce(const P *e_part, int B, int T, const IO *y, IO *e_out,
                                                         IO *loss, double *dlde, double *e_work)
{
    __shared__ double part[kEzThreads];
    double acc = 0.0;
    for (int b = threadIdx.x; b < B; b += kEzThreads) {
        double s = 0.0;
        for (int t = 0; t < T; ++t) s += (double)e_part[(size_t)b * T + t];
        e_work[b] = s;
        e_out[b] = (IO)s;
        if (y) {
            const double d = s - (double)y[b];
            dlde[b] = 2.0 * d / (double)B;
            acc += d * d;
        }
    }
    part[threadIdx.x] = acc;
    __syncthreads();
    if (y && threadIdx.x == 0) {
        double sum = 0.0;
        for (int k = 0; k < kEzThreads; ++k) sum += part[k];
        *loss = (IO)(sum / (double)B);
    }
}

template <typename IO>
__global__ void k_copy_dlde(const IO *src, int B, double *dlde)
{
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b < B) dlde[b] = (double)src[b];
}

// First stage for samples with many tiles: for pass p (relative to the first pass
// of the range), sample b0+bi and chunk ch, out[p][bi][ch][slot] = sum of the slot
// over tiles ch*kStatChunk .. (ch+1)*kStatChunk-1.  Thread i owns slot i % kSlots of
// every fourth tile starting at i / kSlots (consecutive threads read consecutive
// floats); the four lanes are then added in a fixed order.
// Grid (T / kStatChunk, Bc, passes), 4 * kSlots threads.
template <typename P>
__global__ void __launch_bounds__(4 * kSlots) k_stats_chunks(const P *part, int Bs, int b0, int T, double *out)
{
    __shared__ double red[4 * kSlots];
    const int nch = gridDim.x, ch = blockIdx.x, bi = blockIdx.y, p = blockIdx.z, Bc = gridDim.y;
    const int i = threadIdx.x, slot = i % kSlots, lane = i / kSlots;
    const P *src = part + (((size_t)p * Bs + b0 + bi) * T + (size_t)ch * kStatChunk) * kSlots + slot;
    double acc = 0.0;
    for (int t = lane; t < kStatChunk; t += 4) acc += (double)src[(size_t)t * kSlots];
    red[i] = acc;
    __syncthreads();
    if (i < kSlots)
        out[(((size_t)p * Bc + bi) * nch + ch) * kSlots + i] =
            ((red[i] + red[kSlots + i]) + red[2 * kSlots + i]) + red[3 * kSlots + i];
}

// S[b][l][q][s] = sum over tiles (or first-stage chunks) of the slot that holds
// (l, q, s), for samples b0 .. b0+Bc-1.  map[l*n+q] = (pass, slot base); part is
// [pass - pass_lo][Bs][T][slots], its sample index being b - bofs.
template <typename P>
__global__ void k_stats_reduce(const P *part, const int2 *map, int Bs, int bofs, int b0, int Bc, int L, int n,
                               int T, int pass_lo, int pass_hi, double *S)
{
    const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    const size_t total = (size_t)Bc * L * n * 3;
    if (idx >= total) return;
    const int s = (int)(idx % 3);
    const size_t lq = (idx / 3) % ((size_t)L * n);
    const int b = b0 + (int)(idx / 3 / ((size_t)L * n));
    const int2 m = map[lq];
    if (m.x < pass_lo || m.x >= pass_hi) return;
    const P *pp = part + (((size_t)(m.x - pass_lo) * Bs + (b - bofs)) * T) * kSlots + m.y + s;
    double acc = 0.0;
    for (int t = 0; t < T; ++t) acc += (double)pp[(size_t)t * kSlots];
    S[((size_t)b * L * n + lq) * 3 + s] = acc;
}

// grad[l][q][a] = sum_b dLdE_b * sum_s H[l][q][a][s] * S[b][l][q][s].  One wave per
// output: lane t sums samples t, t + 64, ... in order, then the lanes combine in a fixed
// butterfly, so every run adds in the same order.
template <typename IO>
__global__ void __launch_bounds__(256) k_grad_reduce(const double *S, const double *H, const double *dlde, int B, int L,
                                                      int n, IO *grad)
{
    const int idx = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
    if (idx >= L * n * 3) return;   // whole waves leave together
    const int lq = idx / 3;
    const double *h = H + (size_t)idx * 3;
    const double h0 = h[0], h1 = h[1], h2 = h[2];
    double acc = 0.0;
    for (int b = lane; b < B; b += 64) {
        const double *sb = S + ((size_t)b * L * n + lq) * 3;
        acc += dlde[b] * (h0 * sb[0] + h1 * sb[1] + h2 * sb[2]);
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, 64);
    if (lane == 0) grad[idx] = (IO)acc;
}

// The training step's reductions on the whole-circuit path (one <O> per sample) in one
// launch: block 0 also forms E_b, the loss and dL/dE_b exactly as k_ez_reduce does with one
// partial per sample, and every wave of the gradient reduction (as k_grad_reduce) forms the
// dL/dE_b = 2 (E_b - y_b) / B it needs itself, by the same operations, so no block waits for
// another.  Grid and block as k_grad_reduce (4 outputs per 256-thread block, at least one
// block).
template <typename P, typename IO>
__global__ void __launch_bounds__(256) k_small_reduce(const P *e_part, const IO *y, int B, const double *S,
                                                       const double *H, int L, int n, IO *e_out, IO *loss,
                                                       double *dlde, IO *grad)
{
    static_assert(kEzThreads == 256, "block 0 reduces the loss as k_ez_reduce does");
    if (blockIdx.x == 0) {
        __shared__ double part[kEzThreads];
        double acc = 0.0;
        for (int b = threadIdx.x; b < B; b += kEzThreads) {
            const double s = (double)e_part[b];
            e_out[b] = (IO)s;
            const double d = s - (double)y[b];
            dlde[b] = 2.0 * d / (double)B;
            acc += d * d;
        }
        part[threadIdx.x] = acc;
        __syncthreads();
        if (threadIdx.x == 0) {
            double sum = 0.0;
            for (int k = 0; k < kEzThreads; ++k) sum += part[k];
            *loss = (IO)(sum / (double)B);
        }
    }
    const int idx = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
    if (idx >= L * n * 3) return;   // whole waves leave together
    const int lq = idx / 3;
    const double *h = H + (size_t)idx * 3;
    const double h0 = h[0], h1 = h[1], h2 = h[2];
    double acc = 0.0;
    for (int b = lane; b < B; b += 64) {
        const double *sb = S + ((size_t)b * L * n + lq) * 3;
        const double g = 2.0 * ((double)e_part[b] - (double)y[b]) / (double)B;
        acc += g * (h0 * sb[0] + h1 * sb[1] + h2 * sb[2]);
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, 64);
    if (lane == 0) grad[idx] = (IO)acc;
}

}  // namespace hqml

// ------------------------------------------------------------------ launch wrappers (host)
//
// Type codes: io64 = the caller's arrays are double (else float); r64 = compute in
// double (else float); storage 0 = float2, 1 = bf16 pair, 2 = double2 states.
//
// This file is compiled twice.  HQML_BWD32_UNIT = 1 builds only the fp32 adjoint
// launches (and so the only instances of k_tile_bwd<*, *, float>), with the backend's
// max-ilp instruction schedule: measured 4 % faster for that kernel at 20 qubits, but
// slower for the fp64 adjoint (+7 %) and the bf16 forward pass (+5 %), which the default
// build (HQML_BWD32_UNIT = 0) compiles with the default schedule.
namespace hqml {

template <int ST, typename R>
static void launch_bwd_shape(const TilePassArgs &a, dim3 grid, hipStream_t s, bool *bad);

// The fp32 adjoint launches (the other compilation unit).
void launch_tile_bwd_f32(const TilePassArgs &a, dim3 grid, int storage, hipStream_t s, bool *bad);

#if HQML_BWD32_UNIT == 0

template <typename TI, typename R>
static void prep_typed(const void *theta, const void *x, int L, int n, int B, double *zyz, unsigned char *G,
                       void *rot_tf, void *dw, double *H, void *init_u, int ent, hipStream_t s)
{
    const int ln = L * n;
    if (ln <= kPrepThreads && B * n <= 8 * kPrepThreads) {   // small tables: one launch (at 20 qubits
        // x 100 layers one workgroup takes 72 us against 43 us for the four launches)
        k_prep_fused<TI, R><<<1, kPrepThreads, 0, s>>>(static_cast<const TI *>(theta), static_cast<const TI *>(x), L, n,
                                                        B, ent, zyz, G, static_cast<R *>(rot_tf), static_cast<R *>(dw),
                                                        H, static_cast<R *>(init_u));
        return;
    }
    k_prep_zyz<TI><<<(ln + 127) / 128, 128, 0, s>>>(static_cast<const TI *>(theta), L, n, zyz);
    k_prep_frame<<<1, 64, 0, s>>>(zyz, L, n, ent, G);
    k_prep_tables<TI, R><<<(ln + 127) / 128, 128, 0, s>>>(static_cast<const TI *>(theta), zyz, G, L, n, ent,
                                                           static_cast<R *>(rot_tf), static_cast<R *>(dw), H);
    if (B > 0)
        k_prep_init<TI, R><<<(B * n + 127) / 128, 128, 0, s>>>(static_cast<const TI *>(x), zyz, G, B, n,
                                                               static_cast<R *>(init_u));
}

hipError_t launch_prep(const void *theta, const void *x, int io64, int L, int n, int B, double *zyz,
                       unsigned char *G, void *rot_tf, void *dw, double *H, void *init_u, int ent, int r64,
                       hipStream_t s)
{
    if (io64) {
        if (r64)
            prep_typed<double, double>(theta, x, L, n, B, zyz, G, rot_tf, dw, H, init_u, ent, s);
        else
            prep_typed<double, float>(theta, x, L, n, B, zyz, G, rot_tf, dw, H, init_u, ent, s);
    } else {
        if (r64)
            prep_typed<float, double>(theta, x, L, n, B, zyz, G, rot_tf, dw, H, init_u, ent, s);
        else
            prep_typed<float, float>(theta, x, L, n, B, zyz, G, rot_tf, dw, H, init_u, ent, s);
    }
    return hipGetLastError();
}

hipError_t launch_tile_obs(const TilePassArgs &a, int B, int storage, int r64, hipStream_t s)
{
    const dim3 grid((unsigned)(B * a.T));
    if (r64) {
        if (storage == 2)
            k_tile_obs<2, double><<<grid, kThreads, 0, s>>>(a);
        else
            k_tile_obs<0, double><<<grid, kThreads, 0, s>>>(a);
    } else {
        if (storage == 1)
            k_tile_obs<1, float><<<grid, kThreads, 0, s>>>(a);
        else
            k_tile_obs<0, float><<<grid, kThreads, 0, s>>>(a);
    }
    return hipGetLastError();
}

hipError_t launch_tile_fwd(const TilePassArgs &a, int B, int storage, int r64, hipStream_t s)
{
    const dim3 grid((unsigned)(B * a.T));
    if (r64) {
        if (storage == 2)
            k_tile_fwd<2, double><<<grid, kThreads, 0, s>>>(a);
        else
            k_tile_fwd<0, double><<<grid, kThreads, 0, s>>>(a);
    } else {
        if (storage == 1)
            k_tile_fwd<1, float><<<grid, kThreads, 0, s>>>(a);
        else
            k_tile_fwd<0, float><<<grid, kThreads, 0, s>>>(a);
    }
    return hipGetLastError();
}

#endif  // HQML_BWD32_UNIT == 0

template <int ST, typename R>
static void launch_bwd_shape(const TilePassArgs &a, dim3 grid, hipStream_t s, bool *bad)
{
    if (a.flags & PF_HALF) {
        // the general shape (CZ chain) and the CNOT chain's [rotA, diag] and [diag, rotB] shapes on
        // half tiles (fp32 compute with fp32 or bf16 psi, fp64 compute with fp32 or fp64 psi): two
        // per full tile
        if constexpr ((std::is_same<R, float>::value && ST != 2) || (std::is_same<R, double>::value && ST != 1)) {
            const dim3 g2(grid.x * 2);
            if (a.hview && !(a.flags & (PF_FUSED | PF_INIT | PF_SEED | PF_STATS_ONLY))) {
                if (!(a.flags & PF_CNOT) && a.rotA >= 0 && a.diag >= 0 && a.rotB >= 0) {
                    k_tile_bwdh<ST, HB_GENERAL, R><<<g2, kThreads, 0, s>>>(a);
                    return;
                }
                if ((a.flags & PF_CNOT) && a.rotA >= 0 && a.diag >= 0 && a.rotB < 0) {
                    k_tile_bwdh<ST, HB_ROTAD, R><<<g2, kThreads, 0, s>>>(a);
                    return;
                }
                if ((a.flags & PF_CNOT) && (a.flags & PF_GATHER) && a.rotA < 0 && a.diag >= 0 && a.rotB >= 0) {
                    k_tile_bwdh<ST, HB_DROTB, R><<<g2, kThreads, 0, s>>>(a);
                    return;
                }
            }
        }
        *bad = true;
        return;
    }
    if (a.flags & PF_CNOT) {
        if ((a.flags & PF_STATS_ONLY) && (a.flags & PF_SEED))
            k_tile_bwd<ST, BW_L0D_SEED, R><<<grid, kThreads, 0, s>>>(a);
        else if (a.flags & PF_STATS_ONLY)
            k_tile_bwd<ST, BW_L0D, R><<<grid, kThreads, 0, s>>>(a);
        else if (a.rotA < 0)
            k_tile_bwd<ST, BW_DROTB, R><<<grid, kThreads, 0, s>>>(a);
        else if (a.diag >= 0)
            k_tile_bwd<ST, BW_ROTAD, R><<<grid, kThreads, 0, s>>>(a);
        else
            k_tile_bwd<ST, BW_ROTA, R><<<grid, kThreads, 0, s>>>(a);
        return;
    }
    if (a.flags & PF_FUSED) {
        if (a.flags & PF_INIT)
            k_tile_bwd<ST, BW_FUSED_INIT, R><<<grid, kThreads, 0, s>>>(a);
        else
            k_tile_bwd<ST, BW_FUSED_LAST, R><<<grid, kThreads, 0, s>>>(a);
    } else if (a.rotB >= 0) {
        // the plans end every sweep with a pass without rotB, so the general shapes are
        // never seeded and never statistics-only (their kernels do not handle either)
        if (a.flags & (PF_SEED | PF_STATS_ONLY)) {
            *bad = true;
            return;
        }
        if (a.flags & PF_INIT) {
            k_tile_bwd<ST, BW_INIT_GENERAL, R><<<grid, kThreads, 0, s>>>(a);
        } else {
            k_tile_bwd<ST, BW_GENERAL, R><<<grid, kThreads, 0, s>>>(a);
        }
    } else if (a.rotA >= 0 && !(a.flags & (PF_INIT | PF_STATS_ONLY))) {
        k_tile_bwd<ST, BW_ROTA, R><<<grid, kThreads, 0, s>>>(a);
    } else {
        k_tile_bwd<ST, BW_L0, R><<<grid, kThreads, 0, s>>>(a);
    }
}

#if HQML_BWD32_UNIT == 1
void launch_tile_bwd_f32(const TilePassArgs &a, dim3 grid, int storage, hipStream_t s, bool *bad)
{
    if (storage == 1)
        launch_bwd_shape<1, float>(a, grid, s, bad);
    else
        launch_bwd_shape<0, float>(a, grid, s, bad);
}
#else
hipError_t launch_tile_bwd(const TilePassArgs &a, int B, int storage, int r64, hipStream_t s)
{
    const dim3 grid((unsigned)(B * a.T));
    bool bad = false;
    if (r64) {
        if (storage == 2)
            launch_bwd_shape<2, double>(a, grid, s, &bad);
        else
            launch_bwd_shape<0, double>(a, grid, s, &bad);
    } else {
        launch_tile_bwd_f32(a, grid, storage, s, &bad);
    }
    if (bad) return hipErrorInvalidValue;   // a pass the kernels have no shape for (nothing queued)
    return hipGetLastError();
}

template <typename P, typename IO>
static void ez_typed(const void *e_part, int B, int T, const void *y, void *e_out, void *loss, double *dlde,
                     double *e_work, double *chunks, hipStream_t s)
{
    const IO *yy = static_cast<const IO *>(y);
    IO *eo = static_cast<IO *>(e_out), *lo = static_cast<IO *>(loss);
    if (T > kTileChunk) {
        const int nch = T / kTileChunk;
        k_ez_chunks<P><<<dim3((unsigned)nch, (unsigned)B), kTileChunk, 0, s>>>(static_cast<const P *>(e_part), T,
                                                                               chunks);
        k_ez_reduce<double, IO><<<1, kEzThreads, 0, s>>>(chunks, B, nch, yy, eo, lo, dlde, e_work);
    } else {
        k_ez_reduce<P, IO><<<1, kEzThreads, 0, s>>>(static_cast<const P *>(e_part), B, T, yy, eo, lo, dlde, e_work);
    }
}

hipError_t launch_ez_reduce(const void *e_part, int r64, int B, int T, const void *y, void *e_out, void *loss,
                            int io64, double *dlde, double *e_work, double *chunks, hipStream_t s)
{
    if (r64) {
        if (io64)
            ez_typed<double, double>(e_part, B, T, y, e_out, loss, dlde, e_work, chunks, s);
        else
            ez_typed<double, float>(e_part, B, T, y, e_out, loss, dlde, e_work, chunks, s);
    } else {
        if (io64)
            ez_typed<float, double>(e_part, B, T, y, e_out, loss, dlde, e_work, chunks, s);
        else
            ez_typed<float, float>(e_part, B, T, y, e_out, loss, dlde, e_work, chunks, s);
    }
    return hipGetLastError();
}

hipError_t launch_copy_dlde(const void *src, int io64, int B, double *dlde, hipStream_t s)
{
    if (io64)
        k_copy_dlde<double><<<(B + 255) / 256, 256, 0, s>>>(static_cast<const double *>(src), B, dlde);
    else
        k_copy_dlde<float><<<(B + 255) / 256, 256, 0, s>>>(static_cast<const float *>(src), B, dlde);
    return hipGetLastError();
}

template <typename P>
static void stats_typed(const void *part, const int2 *map, int Bs, int b0, int Bc, int L, int n, int T,
                        int pass_lo, int pass_hi, double *S, double *chunks, hipStream_t s)
{
    const size_t total = (size_t)Bc * L * n * 3;
    const unsigned grid = (unsigned)((total + 255) / 256);
    if (T > kStatChunk) {
        const int nch = T / kStatChunk;
        k_stats_chunks<P><<<dim3((unsigned)nch, (unsigned)Bc, (unsigned)(pass_hi - pass_lo)), 4 * kSlots, 0, s>>>(
            static_cast<const P *>(part), Bs, b0, T, chunks);
        k_stats_reduce<double><<<grid, 256, 0, s>>>(chunks, map, Bc, b0, b0, Bc, L, n, nch, pass_lo, pass_hi, S);
    } else {
        k_stats_reduce<P><<<grid, 256, 0, s>>>(static_cast<const P *>(part), map, Bs, 0, b0, Bc, L, n, T, pass_lo,
                                               pass_hi, S);
    }
}

hipError_t launch_stats_reduce(const void *part, int r64, const int2 *map, int Bs, int b0, int Bc, int L, int n,
                               int T, int pass_lo, int pass_hi, double *S, double *chunks, hipStream_t s)
{
    if (r64)
        stats_typed<double>(part, map, Bs, b0, Bc, L, n, T, pass_lo, pass_hi, S, chunks, s);
    else
        stats_typed<float>(part, map, Bs, b0, Bc, L, n, T, pass_lo, pass_hi, S, chunks, s);
    return hipGetLastError();
}

hipError_t launch_grad_reduce(const double *S, const double *H, const double *dlde, int B, int L, int n,
                              void *grad, int io64, hipStream_t s)
{
    const int total = L * n * 3, blocks = (total + 3) / 4;   // four outputs (waves) per block
    if (io64)
        k_grad_reduce<double><<<blocks, 256, 0, s>>>(S, H, dlde, B, L, n, static_cast<double *>(grad));
    else
        k_grad_reduce<float><<<blocks, 256, 0, s>>>(S, H, dlde, B, L, n, static_cast<float *>(grad));
    return hipGetLastError();
}

hipError_t launch_small_reduce(const void *e_part, int r64, int B, const void *y, void *e_out, void *loss, int io64,
                               double *dlde, const double *S, const double *H, int L, int n, void *grad,
                               hipStream_t s)
{
    const unsigned blocks = (unsigned)std::max(1, (L * n * 3 + 3) / 4);
#define HQML_SMALL_REDUCE(P, IO)                                                                               \
    k_small_reduce<P, IO><<<blocks, 256, 0, s>>>(static_cast<const P *>(e_part), static_cast<const IO *>(y), B, S, H, \
                                                 L, n, static_cast<IO *>(e_out), static_cast<IO *>(loss), dlde,     \
                                                 static_cast<IO *>(grad))
    if (r64) {
        if (io64)
            HQML_SMALL_REDUCE(double, double);
        else
            HQML_SMALL_REDUCE(double, float);
    } else {
        if (io64)
            HQML_SMALL_REDUCE(float, double);
        else
            HQML_SMALL_REDUCE(float, float);
    }
#undef HQML_SMALL_REDUCE
    return hipGetLastError();
}
#endif  // HQML_BWD32_UNIT

}  // namespace hqml
