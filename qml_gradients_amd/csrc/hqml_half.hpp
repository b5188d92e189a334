// Register-resident half tiles: 2^12 amplitudes held by 256 threads x 16 registers, in
// two layouts whose register bits cover different positions, moved between them through
// LDS.  Shared by the half-tile adjoint pass (hqml_kernels.hip) and the 12-qubit
// whole-circuit kernel (hqml_small12.hip): register rotations in tan form, DPP forms of
// the rotations and statistics of the qubits at lane bits 0 and 1, and the X / Y / Z
// statistics sums.
#pragma once
#include <type_traits>

#include "hqml_device.hpp"
#include "hqml_internal.hpp"

namespace hqml {

template <typename R>
struct HTile {
    R re[kHalfRegs];
    R im[kHalfRegs];
};

// LDS swizzle of the 12-bit local index: bit 4 ^= bit 8.  Linear over GF(2).  A half-wave
// then touches 32 distinct 8-byte slots in both layouts: in H1 its lanes 16..31 differ from
// lanes 0..15 in position 8, which moves them to the other half of the 32 slots; in H2
// they differ in position 4 and the flip by register bit 0 (position 8) is uniform.
__host__ __device__ constexpr uint32_t hswz(uint32_t i) { return i ^ (((i >> 8) & 1u) << 4); }

// Ry (kk = k) or Ry^dagger (kk = -k) on register bit M, scale f left out (as rot_bit in
// hqml_kernels.hip).
template <int M, typename R>
__device__ __forceinline__ void hrot_bit(HTile<R> &t, R kk)
{
#pragma unroll
    for (int j = 0; j < kHalfRegs; ++j) {
        if (j & (1 << M)) continue;
        const int o = j | (1 << M);
        const R ar = t.re[j], ai = t.im[j], br = t.re[o], bi = t.im[o];
        t.re[j] = fmar(-kk, br, ar);
        t.im[j] = fmar(-kk, bi, ai);
        t.re[o] = fmar(kk, ar, br);
        t.im[o] = fmar(kk, ai, bi);
    }
}

// DPP forms of a multiply-add with the partner lane's operand.  The compiler does not fold
// a DPP move into v_fmac_f32, so these are written as instructions: a quad permutation of
// src0 (lane index XOR 1 or XOR 2, so every lane's source is valid), no memory access.
// Each block starts with two wait states (a VALU write of a VGPR followed by a DPP read of
// it needs two on this hardware); inside a block no instruction reads through DPP a
// register that an earlier one wrote.
#define HQML_QP0 " quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf"
#define HQML_QP1 " quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf"
#define HQML_SELF8(QP)                                                                        \
    asm("s_nop 1\n\t"                                                                         \
        "v_fmac_f32_dpp %0, %0, %8" QP "\n\t"                                                 \
        "v_fmac_f32_dpp %1, %1, %8" QP "\n\t"                                                 \
        "v_fmac_f32_dpp %2, %2, %8" QP "\n\t"                                                 \
        "v_fmac_f32_dpp %3, %3, %8" QP "\n\t"                                                 \
        "v_fmac_f32_dpp %4, %4, %8" QP "\n\t"                                                 \
        "v_fmac_f32_dpp %5, %5, %8" QP "\n\t"                                                 \
        "v_fmac_f32_dpp %6, %6, %8" QP "\n\t"                                                 \
        "v_fmac_f32_dpp %7, %7, %8" QP                                                        \
        : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]), "+v"(x[4]), "+v"(x[5]), "+v"(x[6]), \
          "+v"(x[7])                                                                          \
        : "v"(k))

// x[i] += k * (x[i] of the partner lane), eight values, in place.
template <int B>
__device__ __forceinline__ void dpp_self8(float *x, float k)
{
    if constexpr (B == 0)
        HQML_SELF8(HQML_QP0);
    else
        HQML_SELF8(HQML_QP1);
}

// Statistics of two registers with the partner lane's psi:
//   xp += l.re * p.im', xn += l.im * p.re', rp += l.re * p.re', rq += l.im * p.im'
// (primes: the partner lane's value), for registers j and j + 1.
#define HQML_XY2(QP)                                                                         \
    asm("s_nop 1\n\t"                                                                        \
        "v_fmac_f32_dpp %0, %5, %4" QP "\n\t"                                                \
        "v_fmac_f32_dpp %1, %6, %7" QP "\n\t"                                                \
        "v_fmac_f32_dpp %2, %6, %4" QP "\n\t"                                                \
        "v_fmac_f32_dpp %3, %5, %7" QP "\n\t"                                                \
        "v_fmac_f32_dpp %0, %9, %8" QP "\n\t"                                                \
        "v_fmac_f32_dpp %1, %10, %11" QP "\n\t"                                              \
        "v_fmac_f32_dpp %2, %10, %8" QP "\n\t"                                               \
        "v_fmac_f32_dpp %3, %9, %11" QP                                                      \
        : "+v"(xp), "+v"(xn), "+v"(rp), "+v"(rq)                                             \
        : "v"(l.re[j]), "v"(p.im[j]), "v"(p.re[j]), "v"(l.im[j]), "v"(l.re[j + 1]),          \
          "v"(p.im[j + 1]), "v"(p.re[j + 1]), "v"(l.im[j + 1]))

// Ry^dagger on the qubit at lane bit B (position B) in tan form, scale left out: the thread
// holding bit value 0 computes a + k b, the one holding 1 computes b - k a, with the partner
// lane's amplitude (every source is read before any lane writes, so the update is in place).
template <int B, typename R>
__device__ __forceinline__ void hunrot_lane(HTile<R> &t, R k, int lane)
{
    const R ks = ((lane >> B) & 1) ? -k : k;
    if constexpr (std::is_same<R, float>::value) {
        dpp_self8<B>(t.re, ks);
        dpp_self8<B>(t.re + 8, ks);
        dpp_self8<B>(t.im, ks);
        dpp_self8<B>(t.im + 8, ks);
    } else {   // fp64: no DPP form of the 64-bit multiply-add; move the partner's value first
        constexpr int CTRL = B == 0 ? 0xB1 : 0x4E;
#pragma unroll
        for (int j = 0; j < kHalfRegs; ++j) {
            const R pr = dppf<CTRL>(t.re[j]), pi = dppf<CTRL>(t.im[j]);
            t.re[j] = fmar(ks, pr, t.re[j]);
            t.im[j] = fmar(ks, pi, t.im[j]);
        }
    }
}

// X / Y statistics of register bit M (as xy_stats in hqml_kernels.hip).
template <int M, typename R>
__device__ __forceinline__ void hxy_reg(const HTile<R> &p, const HTile<R> &l, R &sx, R &sy)
{
    R xp = 0, xn = 0, yp = 0, yn = 0;
#pragma unroll
    for (int j = 0; j < kHalfRegs; ++j) {
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

// X / Y statistics of the qubit at lane bit B: with c = conj(l_i) p_{i ^ 2^B} (the partner
// lane's psi), Im<lam|X|psi> = sum Im c and Im<lam|Y|psi> = sum (bit ? Re c : -Re c), since
// (Y psi)_i = -i psi_partner where bit B of i is 0 and +i psi_partner where it is 1.
template <int B, typename R>
__device__ __forceinline__ void hxy_lane(const HTile<R> &p, const HTile<R> &l, int lane, R &sx, R &sy)
{
    R xp = 0, xn = 0, rp = 0, rq = 0;
    if constexpr (std::is_same<R, float>::value) {
#pragma unroll
        for (int j = 0; j < kHalfRegs; j += 2) {
            if constexpr (B == 0)
                HQML_XY2(HQML_QP0);
            else
                HQML_XY2(HQML_QP1);
        }
    } else {
        constexpr int CTRL = B == 0 ? 0xB1 : 0x4E;
#pragma unroll
        for (int j = 0; j < kHalfRegs; ++j) {
            const R pr = dppf<CTRL>(p.re[j]), pi = dppf<CTRL>(p.im[j]);
            xp = fmar(l.re[j], pi, xp);
            xn = fmar(l.im[j], pr, xn);
            rp = fmar(l.re[j], pr, rp);
            rq = fmar(l.im[j], pi, rq);
        }
    }
    sx = xp - xn;
    const R r = rp + rq;
    sy = ((lane >> B) & 1) ? r : -r;
}

// Z statistics of the register bits (zsum of hqml_kernels.hip on 16 registers): returns
// the sum of w_j = Im(conj(l_j) p_j) over the registers, d_m = sum (-1)^{bit m of j} w_j.
template <int J, typename R>
__device__ __forceinline__ R hzw(const HTile<R> &p, const HTile<R> &l)
{
    return fmar(l.re[J], p.im[J], -l.im[J] * p.re[J]);
}

template <int K, int LO, typename R>
__device__ __forceinline__ R hzsum(const HTile<R> &p, const HTile<R> &l, R *dz)
{
    if constexpr (K == 0) {
        return hzw<LO>(p, l);
    } else {
        const R a = hzsum<K - 1, LO>(p, l, dz);
        const R b = hzsum<K - 1, LO + (1 << (K - 1))>(p, l, dz);
        if constexpr (LO == 0)
            dz[K - 1] = a - b;
        else
            dz[K - 1] += a - b;
        return a + b;
    }
}

}  // namespace hqml
