// gfx950 kernel of the whole training step at 12 qubits with the CZ chain, fp32 compute
// (k_small12): one workgroup per sample, as k_small, but the sample's state stays in
// registers.  Method: Kawase, arXiv:2603.02804 (hugo-pages summary "深度解析：正向与反向门
// 融合驱动的高效量子机器学习仿真", sections 1.2-1.4): the forward pass keeps the state on chip
// for the whole circuit, and the adjoint sweep re-derives each earlier state on chip with
// U^dagger while it forms the gradient statistics and propagates lambda.  The layer algebra
// (tan-form rotations, merged diagonals D_l, statistics at the points P_l) is described in
// hqml_internal.hpp.
//
// 2^12 amplitudes are exactly one register-resident half tile (hqml_half.hpp): 256 threads x
// 16 registers, in two layouts
//   A: registers <- qubits 4..7, lanes <- qubits 0, 1, 2, 3, 8, 9, waves <- 10, 11
//   B: registers <- qubits 8..11, lanes <- qubits 2, 3, 0, 1, 4, 5, waves <- 6, 7
// A rotates qubits 4..7 in registers and 0, 1 at lane bits 0, 1 (DPP quad permutations),
// B rotates 8..11 in registers and 2, 3 at lane bits 0, 1, so one LDS transpose per layer
// and state covers all twelve qubits (k_small's register rounds take four LDS round trips
// per layer and state).  Layers alternate between starting in A and in B.  LDS slots use the
// half tile's swizzle, which keeps both layouts free of bank conflicts (lanes 0..15 of a
// register cover qubits 0..3 in both; lanes 16..31 differ from them in qubit 8 in A, in
// qubit 4 in B).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hqml_device.hpp"
#include "hqml_half.hpp"
#include "hqml_host.hpp"
#include "hqml_internal.hpp"

namespace hqml {

constexpr int kS12Qubits = 12;
constexpr int kS12Threads = 256;
constexpr int kS12Rows = kS12Threads / 16;        // DPP rows: statistics partials per value
constexpr int kS12Stats = 3 * kS12Qubits;          // statistics per layer

// Amplitude index of register 0 of this thread in layout A / B (register j adds j << 4 in A,
// j << 8 in B).  Its lane and wave bits are the values of the thread's fixed qubits (those
// not at register bits, which are zero here).
__device__ __forceinline__ uint32_t s12_base(bool la, int lane, int w)
{
    const uint32_t l = (uint32_t)lane, ww = (uint32_t)w;
    return la ? (l & 15u) | ((l >> 4) << 8) | (ww << 10)
              : ((l >> 2) & 3u) | ((l & 3u) << 2) | (((l >> 4) & 3u) << 4) | (ww << 6);
}

template <bool LA>
__device__ __forceinline__ uint32_t s12_reg(int j)
{
    return (uint32_t)j << (LA ? 4 : 8);
}

// Factor tables of a diagonal prod_q f_q(bit q) (times the CZ chain's signs if CZ, times
// scale) for the 16 registers of a thread in layout LA: factor of register j =
// lo[j & 3] * hi[j >> 2], negated when CZ and bits 1 and 2 of j are set (the CZ between the
// middle two register qubits).  f[q] = (f0.re, f0.im, f1.re, f1.im) for bit value 0 / 1.
// Each lane reads the factors of its eight fixed qubits at their bit values itself (eight
// vector loads issued together, one wait); the register qubits' factors are uniform.
struct S12Diag {
    float2 lo[4];
    float2 hi[4];
};

template <bool LA, bool CZ>
__device__ __forceinline__ S12Diag s12_tables(const float4 *f, uint32_t fix, float scale)
{
    constexpr int q0 = LA ? 4 : 8;   // first register qubit
    float2 fv[8];
#pragma unroll
    for (int q = 0, k = 0; q < kS12Qubits; ++q) {
        if (q >= q0 && q < q0 + 4) continue;
        fv[k++] = reinterpret_cast<const float2 *>(f + q)[(fix >> q) & 1u];
    }
    float4 gr[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) gr[m] = ldu4(reinterpret_cast<const float *>(f + q0 + m));
    // thread constant: the eight fixed qubits (lanes and waves)
    float2 ct = mk2(scale, 0.0f);
#pragma unroll
    for (int k = 0; k < 8; ++k) ct = cmul(ct, fv[k]);
    if (CZ && (__builtin_popcount(fix & (fix >> 1)) & 1)) ct = mk2(-ct.x, -ct.y);   // CZ among fixed qubits
    float2 g0[4], g1[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const int q = q0 + m;
        g0[m] = mk2(gr[m].x, gr[m].y);
        g1[m] = mk2(gr[m].z, gr[m].w);
        // CZ with a fixed chain neighbour holding 1 (the other register qubits are 0 in fix)
        if (CZ && (__builtin_popcount(fix & ((1u << (q + 1)) | (1u << (q - 1)))) & 1)) g1[m] = mk2(-g1[m].x, -g1[m].y);
    }
    S12Diag t;
#pragma unroll
    for (int a = 0; a < 4; ++a) {
        float2 x = cmul(ct, cmul((a & 1) ? g1[0] : g0[0], (a & 2) ? g1[1] : g0[1]));
        float2 h = cmul((a & 1) ? g1[2] : g0[2], (a & 2) ? g1[3] : g0[3]);
        if (CZ && a == 3) {   // CZ between register qubits 0, 1 and between 2, 3
            x = mk2(-x.x, -x.y);
            h = mk2(-h.x, -h.y);
        }
        t.lo[a] = x;
        t.hi[a] = h;
    }
    return t;
}

template <bool CZ>
__device__ __forceinline__ float2 s12_factor(const S12Diag &d, int j)
{
    float2 f = cmul(d.lo[j & 3], d.hi[j >> 2]);
    if (CZ && (j & 2) && (j & 4)) f = mk2(-f.x, -f.y);
    return f;
}

__device__ __forceinline__ void s12_mul(HTile<float> &t, int j, float2 f)
{
    const float r = t.re[j], i = t.im[j];
    t.re[j] = r * f.x - i * f.y;
    t.im[j] = r * f.y + i * f.x;
}

// Tan-form coefficients of layer l for the six qubits layout LA rotates: k[0], k[1] the
// qubits at lane bits 0, 1; k[2..5] those at register bits 0..3; F the product of scales.
struct S12Coef {
    float k[6];
    float F;
};

template <bool LA>
__device__ __forceinline__ S12Coef s12_coef(const float *rot_tf, int l)
{
    constexpr int qs[6] = {LA ? 0 : 2, LA ? 1 : 3, LA ? 4 : 8, LA ? 5 : 9, LA ? 6 : 10, LA ? 7 : 11};
    S12Coef c;
    c.F = 1.0f;
#pragma unroll
    for (int m = 0; m < 6; ++m) {
        const float2 kf = ldu2(rot_tf + ((size_t)l * kS12Qubits + qs[m]) * 2);
        c.k[m] = kf.x;
        c.F *= kf.y;
    }
    return c;
}

// Ry of the six qubits of layout LA (INV: Ry^dagger), scales left out.  At a lane bit the
// thread holding bit value 0 computes a - k b (a + k b for the inverse) and the one holding
// 1 computes b + k a (b - k a), b / a the partner lane's amplitude.
template <bool LA, bool INV>
__device__ __forceinline__ void s12_rotate(HTile<float> &t, const S12Coef &c, int lane)
{
    const float sg = INV ? -1.0f : 1.0f;
    hrot_bit<0>(t, sg * c.k[2]);
    hrot_bit<1>(t, sg * c.k[3]);
    hrot_bit<2>(t, sg * c.k[4]);
    hrot_bit<3>(t, sg * c.k[5]);
    const float k0 = (lane & 1) ? sg * c.k[0] : -sg * c.k[0];
    dpp_self8<0>(t.re, k0);
    dpp_self8<0>(t.re + 8, k0);
    dpp_self8<0>(t.im, k0);
    dpp_self8<0>(t.im + 8, k0);
    const float k1 = (lane & 2) ? sg * c.k[1] : -sg * c.k[1];
    dpp_self8<1>(t.re, k1);
    dpp_self8<1>(t.re + 8, k1);
    dpp_self8<1>(t.im, k1);
    dpp_self8<1>(t.im + 8, k1);
}

// Statistics S_X, S_Y, S_Z of the qubits of layout LA that sel names (bit 0: those at lane
// bits 0, 1 and register bit 0; bit 1: those at register bits 1..3) from (psi p, lambda l):
// the thread sums first, then their DPP row sums interleaved (independent chains hide the
// DPP latency), then one leader branch writes them, times corr, to
// red[(q * 3 + s) * kS12Rows + row].  Every value goes through the same operations whatever
// sel is, so a split of the qubits over workgroups gives the same bits.
template <int NV>
__device__ __forceinline__ void s12_rows_out(float (&v)[NV], const int (&qv)[NV / 3], float corr, float *red, int lane,
                                             int w)
{
#pragma unroll
    for (int k = 0; k < NV; ++k) v[k] += dppf<0xB1>(v[k]);   // quad_perm [1,0,3,2]
#pragma unroll
    for (int k = 0; k < NV; ++k) v[k] += dppf<0x4E>(v[k]);   // quad_perm [2,3,0,1]
#pragma unroll
    for (int k = 0; k < NV; ++k) v[k] += dppf<0x141>(v[k]);  // row_half_mirror
#pragma unroll
    for (int k = 0; k < NV; ++k) {
        v[k] += dppf<0x140>(v[k]);                            // row_mirror
        // keep the last add out of the leader's branch (where it cannot take the DPP operand)
        asm volatile("" : "+v"(v[k]));
    }
    if ((lane & 15) == 15) {
        const int r = w * 4 + (lane >> 4);
#pragma unroll
        for (int k = 0; k < NV; ++k) red[(qv[k / 3] * 3 + k % 3) * kS12Rows + r] = v[k] * corr;
    }
}

template <bool LA>
__device__ __forceinline__ void s12_stats(const HTile<float> &p, const HTile<float> &l, float corr, float *red,
                                          int lane, int w, int sel)
{
    constexpr int qa = LA ? 0 : 2, q0 = LA ? 4 : 8;
    float dz[4];
    const float W = hzsum<4, 0>(p, l, dz);
    float v0[9], v1[9];   // (x, y, z) of lane bit 0, lane bit 1, register bit 0 / register bits 1..3
    if (sel & 1) {
        hxy_lane<0>(p, l, lane, v0[0], v0[1]);
        v0[2] = (lane & 1) ? -W : W;
        hxy_lane<1>(p, l, lane, v0[3], v0[4]);
        v0[5] = (lane & 2) ? -W : W;
        hxy_reg<0>(p, l, v0[6], v0[7]);
        v0[8] = dz[0];
    }
    if (sel & 2) {
        hxy_reg<1>(p, l, v1[0], v1[1]);
        v1[2] = dz[1];
        hxy_reg<2>(p, l, v1[3], v1[4]);
        v1[5] = dz[2];
        hxy_reg<3>(p, l, v1[6], v1[7]);
        v1[8] = dz[3];
    }
    constexpr int q0s[3] = {qa, qa + 1, q0}, q1s[3] = {q0 + 1, q0 + 2, q0 + 3};
    if (sel == 3) {   // both halves: eighteen chains in one interleaved set
        float v[18];
        constexpr int qv[6] = {qa, qa + 1, q0, q0 + 1, q0 + 2, q0 + 3};
#pragma unroll
        for (int k = 0; k < 9; ++k) {
            v[k] = v0[k];
            v[9 + k] = v1[k];
        }
        s12_rows_out<18>(v, qv, corr, red, lane, w);
    } else if (sel == 1) {
        s12_rows_out<9>(v0, q0s, corr, red, lane, w);
    } else if (sel == 2) {
        s12_rows_out<9>(v1, q1s, corr, red, lane, w);
    }
}

template <bool LA>
__device__ __forceinline__ void s12_put(const HTile<float> &t, float2 *buf, uint32_t base)
{
#pragma unroll
    for (int j = 0; j < kHalfRegs; ++j) buf[hswz(base ^ s12_reg<LA>(j))] = mk2(t.re[j], t.im[j]);
}

template <bool LA>
__device__ __forceinline__ void s12_get(HTile<float> &t, const float2 *buf, uint32_t base)
{
#pragma unroll
    for (int j = 0; j < kHalfRegs; ++j) {
        const float2 v = buf[hswz(base ^ s12_reg<LA>(j))];
        t.re[j] = v.x;
        t.im[j] = v.y;
    }
}

// Sum of the 16 row partials of each statistic of layer l, in row order, into the output
// (the statistics of the qubits in qmask: those this workgroup takes).
__device__ __forceinline__ void s12_stats_flush(const float *red, const SmallArgs &a, int b, int l, uint32_t qmask)
{
    const int tid = threadIdx.x;
    if (tid < kS12Stats && ((qmask >> (tid / 3)) & 1u)) {
        double s = 0.0;
        for (int r = 0; r < kS12Rows; ++r) s += (double)red[tid * kS12Rows + r];
        a.stats[((size_t)b * a.L + l) * kS12Stats + tid] = s;
    }
}

// LDS: four transpose buffers (psi and lambda of two consecutive steps, so a step needs one
// workgroup barrier: a buffer is written again two steps later, after every thread has
// passed the barrier of the step in between) and three sets of statistics partials (layer
// l's are summed out during step l-1 and written again by step l-3).
constexpr int kS12Buf = 1 << kS12Qubits;                              // float2 per buffer
constexpr int kS12Shm = 4 * kS12Buf * (int)sizeof(float2);            // 128 KiB
constexpr int kS12Red = kS12Stats * kS12Rows;                         // floats per partials set

// Forward step l -> l+1 starting in layout LA: D_l (times the pending scale c), Ry-layer l+1
// on LA's qubits, transpose through buffer l & 1, Ry-layer l+1 on the other layout's qubits.
// Returns the product of the rotation scales (the next pending scale).
template <bool LA>
__device__ __forceinline__ float s12_fwd_step(HTile<float> &p, const SmallArgs &a, int l, float c, float2 *bufs,
                                              int lane, int w)
{
    const uint32_t bx = s12_base(LA, lane, w), by = s12_base(!LA, lane, w);
    const float *rot = static_cast<const float *>(a.rot_tf);
    const S12Coef cx = s12_coef<LA>(rot, l + 1), cy = s12_coef<!LA>(rot, l + 1);
    const S12Diag d = s12_tables<LA, true>(reinterpret_cast<const float4 *>(a.dw) + (size_t)l * kS12Qubits, bx, c);
#pragma unroll
    for (int j = 0; j < kHalfRegs; ++j) s12_mul(p, j, s12_factor<true>(d, j));
    s12_rotate<LA, false>(p, cx, lane);
    float2 *P = bufs + (l & 1) * kS12Buf;
    s12_put<LA>(p, P, bx);
    __syncthreads();
    s12_get<!LA>(p, P, by);
    s12_rotate<!LA, false>(p, cy, lane);
    return cx.F * cy.F;
}

// Adjoint step at layer l starting in layout LA: [D_l^dagger times the pending scale c on
// both states, unless l is the last layer], statistics of LA's qubits at P_l, [Ry-layer l
// undone on LA's qubits], transpose through buffers 2 (l & 1) and 2 (l & 1) + 1, the sums of
// layer l+1's statistics, statistics of the other qubits (their values unchanged by the
// first undone rotations, which act on other qubits: only their scale enters), [Ry-layer l
// undone on those].  Statistics only of the workgroup's share of the qubits (sel, qmask; see
// s12_part).  Returns the next pending scale.
template <bool LA>
__device__ __forceinline__ float s12_adj_step(HTile<float> &p, HTile<float> &q, const SmallArgs &a, int b, int l,
                                              float c, float2 *bufs, float *red, const int (&sel)[2], uint32_t qmask,
                                              int lane, int w)
{
    const uint32_t bx = s12_base(LA, lane, w), by = s12_base(!LA, lane, w);
    const float *rot = static_cast<const float *>(a.rot_tf);
    const S12Coef cx = s12_coef<LA>(rot, l), cy = s12_coef<!LA>(rot, l);
    if (l + 1 < a.L) {
        const S12Diag d =
            s12_tables<LA, true>(reinterpret_cast<const float4 *>(a.dw) + (size_t)l * kS12Qubits, bx, c);
#pragma unroll
        for (int j = 0; j < kHalfRegs; ++j) {
            float2 f = s12_factor<true>(d, j);
            f.y = -f.y;
            s12_mul(p, j, f);
            s12_mul(q, j, f);
        }
    }
    float *rl = red + (l % 3) * kS12Red;
    const int selx = sel[LA ? 0 : 1], sely = sel[LA ? 1 : 0];
    if (selx) s12_stats<LA>(p, q, 1.0f, rl, lane, w, selx);
    float2 *P = bufs + 2 * (l & 1) * kS12Buf, *Q = P + kS12Buf;
    float fx = 1.0f, fy = 1.0f;
    if (l > 0) {
        s12_rotate<LA, true>(p, cx, lane);
        s12_put<LA>(p, P, bx);
        s12_rotate<LA, true>(q, cx, lane);
        s12_put<LA>(q, Q, bx);
        fx = cx.F;
    } else {
        s12_put<LA>(p, P, bx);
        s12_put<LA>(q, Q, bx);
    }
    __syncthreads();   // also: layer l+1's partials are complete
    s12_get<!LA>(p, P, by);
    s12_get<!LA>(q, Q, by);
    if (l + 1 < a.L) s12_stats_flush(red + ((l + 1) % 3) * kS12Red, a, b, l + 1, qmask);
    if (sely) s12_stats<!LA>(p, q, fx * fx, rl, lane, w, sely);
    if (l > 0) {
        s12_rotate<!LA, true>(p, cy, lane);
        s12_rotate<!LA, true>(q, cy, lane);
        fy = cy.F;
    }
    return fx * fy;
}

// lambda at P_{L-1} = D_t^dagger O D_t psi for the Pauli string O = i^(#Y) X^xm Z^zm (D_t
// = D_{L-1}, the trailing diagonal; it commutes with a Z string and is left out there):
// with phi = D_t psi,
//   lambda_i = conj(D_t(i)) i^(#Y) (-1)^|(i ^ xm) & zm| phi_(i ^ xm),
// and the thread's share of E = Re <psi|lambda>.  phi goes through P (index order), where
// the partners i ^ xm are read.
template <bool LA>
__device__ __forceinline__ float s12_seed(const HTile<float> &p, HTile<float> &q, const SmallArgs &a, float2 *P,
                                          int lane, int w)
{
    const uint32_t bx = s12_base(LA, lane, w), zm = a.obs, xm = a.obs_x;
    const int yph = __builtin_popcount(zm & xm) & 3;
    S12Diag dt;
    if (xm) dt = s12_tables<LA, true>(reinterpret_cast<const float4 *>(a.dw) + (size_t)(a.L - 1) * kS12Qubits, bx, 1.0f);
    __syncthreads();   // every earlier read of P is done (mode 1: none)
#pragma unroll
    for (int j = 0; j < kHalfRegs; ++j) {
        float2 v = mk2(p.re[j], p.im[j]);
        if (xm) v = cmul(v, s12_factor<true>(dt, j));
        P[hswz(bx ^ s12_reg<LA>(j))] = v;
    }
    __syncthreads();
    float e = 0.0f;
#pragma unroll
    for (int j = 0; j < kHalfRegs; ++j) {
        const uint32_t i = bx ^ s12_reg<LA>(j);
        float2 v = P[hswz(i ^ xm)];
        if (__builtin_popcount((i ^ xm) & zm) & 1) v = mk2(-v.x, -v.y);
        mul_ipow(v.x, v.y, yph);
        if (xm) {
            float2 d = s12_factor<true>(dt, j);
            d.y = -d.y;
            v = cmul(v, d);
        }
        q.re[j] = v.x;
        q.im[j] = v.y;
        e = fmaf(p.re[j], v.x, fmaf(p.im[j], v.y, e));
    }
    return e;
}

template <bool LA>
__device__ __forceinline__ void s12_save(const HTile<float> &p, float2 *save, int lane, int w)
{
    const uint32_t bx = s12_base(LA, lane, w);
#pragma unroll
    for (int j = 0; j < kHalfRegs; ++j) save[bx ^ s12_reg<LA>(j)] = mk2(p.re[j], p.im[j]);
}

// Qubits whose statistics workgroup `part` of a sample takes when `parts` workgroups share the
// sample (1, 2 or 4): sel[0] / sel[1] name them among layout A's / B's qubits as s12_stats
// does; the mask lists them.  Every part runs the whole forward pass and un-computes psi and
// lambda itself: the split costs no exchange between workgroups, and at small batches it
// puts otherwise idle compute units to work on the statistics.
__device__ __forceinline__ uint32_t s12_part(int parts, int part, int (&sel)[2])
{
    constexpr uint32_t a0 = 0x013u, a1 = 0x0e0u, b0 = 0x10cu, b1 = 0xe00u;   // {0,1,4} {5,6,7} {2,3,8} {9,10,11}
    if (parts == 4) {
        sel[0] = part == 0 ? 1 : part == 1 ? 2 : 0;
        sel[1] = part == 2 ? 1 : part == 3 ? 2 : 0;
        return part == 0 ? a0 : part == 1 ? a1 : part == 2 ? b0 : b1;
    }
    if (parts == 2) {
        sel[0] = part == 0 ? 3 : 0;
        sel[1] = part == 1 ? 3 : 0;
        return part == 0 ? a0 | a1 : b0 | b1;
    }
    sel[0] = sel[1] = 3;
    return 0xfffu;
}

// The whole step of one sample (modes as k_small: 0 forward, 1 backward from psi_save, 2
// both), on `parts` workgroups (consecutive blocks; part 0 writes <O> and the saved state).
// Statistics of layer l go to a.stats[b][l][q][s] (fp64 sums of 16 row partials in row
// order), <O> to a.e_out[b].
__global__ __launch_bounds__(kS12Threads, 1) void k_small12(SmallArgs a, int parts)
{
    extern __shared__ __align__(16) unsigned char smem[];
    __shared__ float red[3 * kS12Red + kS12Rows];
    float2 *bufs = reinterpret_cast<float2 *>(smem);
    const int b = (int)blockIdx.x / parts, part = (int)blockIdx.x - b * parts;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, L = a.L;
    int sel[2];
    const uint32_t qmask = s12_part(parts, part, sel);
    float2 *save = reinterpret_cast<float2 *>(a.psi_save) + ((size_t)b << kS12Qubits);
    HTile<float> p, q;
    bool inA = true;
    if (a.mode != 1) {
        // product state: prod_q u_q(bit q), layer 0 complete
        const S12Diag u = s12_tables<true, false>(
            reinterpret_cast<const float4 *>(a.init_u) + (size_t)b * kS12Qubits, s12_base(true, lane, w), 1.0f);
#pragma unroll
        for (int j = 0; j < kHalfRegs; ++j) {
            const float2 f = s12_factor<false>(u, j);
            p.re[j] = f.x;
            p.im[j] = f.y;
        }
        float c = 1.0f;   // true state = registers * c
        for (int l = 0; l + 1 < L; ++l) {
            c = inA ? s12_fwd_step<true>(p, a, l, c, bufs, lane, w) : s12_fwd_step<false>(p, a, l, c, bufs, lane, w);
            inA = !inA;
        }
        if (L > 1) {
#pragma unroll
            for (int j = 0; j < kHalfRegs; ++j) {
                p.re[j] *= c;
                p.im[j] *= c;
            }
        }
    } else {
        const float2 *src = save;
#pragma unroll
        for (int j = 0; j < kHalfRegs; ++j) {
            const float2 v = src[s12_base(true, lane, w) ^ s12_reg<true>(j)];
            p.re[j] = v.x;
            p.im[j] = v.y;
        }
    }
    if (a.mode == 0 && part == 0) {   // forward only: the final state for a later backward
        if (inA)
            s12_save<true>(p, save, lane, w);
        else
            s12_save<false>(p, save, lane, w);
    }
    // lambda through buffer 2, which the forward steps (buffers 0, 1) never use
    float2 *S = bufs + 2 * kS12Buf;
    float e = inA ? s12_seed<true>(p, q, a, S, lane, w) : s12_seed<false>(p, q, a, S, lane, w);
    if (a.mode != 1) {
        e = row_sum16(e);
        float *re = red + 3 * kS12Red;
        if ((lane & 15) == 15) re[w * 4 + (lane >> 4)] = e;
        __syncthreads();
        if (tid == 0 && part == 0) {
            double s = 0.0;
            for (int r = 0; r < kS12Rows; ++r) s += (double)re[r];
            static_cast<float *>(a.e_out)[b] = (float)s;
        }
        if (a.mode == 0) return;
    }
    __syncthreads();   // the seed's reads of buffer 2 are done before the adjoint steps write it
    float c = 1.0f;
    for (int l = L - 1; l >= 0; --l) {
        c = inA ? s12_adj_step<true>(p, q, a, b, l, c, bufs, red, sel, qmask, lane, w)
                : s12_adj_step<false>(p, q, a, b, l, c, bufs, red, sel, qmask, lane, w);
        inA = !inA;
    }
    __syncthreads();
    s12_stats_flush(red, a, b, 0, qmask);
}

hipError_t configure_small12()
{
    return hipFuncSetAttribute(reinterpret_cast<const void *>(&k_small12), hipFuncAttributeMaxDynamicSharedMemorySize,
                               kS12Shm);
}

// Workgroups per sample: 4 or 2 while the whole grid still fits one workgroup per compute
// unit (the kernel's LDS allows one), else 1; 1 for a forward-only launch (no statistics).
// The split changes no result bit.
hipError_t launch_small12(const SmallArgs &a, int B, hipStream_t s)
{
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    const int parts = a.mode == 0 ? 1 : 4 * (long long)B <= cus ? 4 : 2 * (long long)B <= cus ? 2 : 1;
    k_small12<<<(unsigned)B * (unsigned)parts, kS12Threads, kS12Shm, s>>>(a, parts);
    return hipGetLastError();
}

}  // namespace hqml
