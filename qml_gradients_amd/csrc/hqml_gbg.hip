// Gate-by-gate comparator: the same training step with no gate fusion.
//
// Every gate of the circuit is one kernel over the whole state, and the adjoint
// backward pass visits the gates one at a time, as an unfused adjoint simulator
// does (the comparison of fused against gate-by-gate execution in the hugo-pages
// summary, sections 2.1 and 2.2):
//   forward   psi <- U psi for every encoding gate, rotation and entangling gate (CZ or
//             CNOT) in circuit order;
//   adjoint   for every gate in reverse order, with psi and lambda at the point just
//             after the gate: grad += (1/2) Im<lambda| sigma |psi> for a rotation
//             exp(-i t sigma / 2) (the gate's term Re<lambda| dU/dt |psi_prev>), then
//             psi <- U^dagger psi and lambda <- U^dagger lambda (section 1.2).
// Each adjoint gate reads and writes psi and lambda (32 bytes per amplitude); a
// forward gate reads and writes psi (16 bytes).  fp32 states, fp64 block sums.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hqml_internal.hpp"

namespace hqml {

constexpr int kGbgThreads = 256;
constexpr int kGbgPairsPerThread = kGbgPairsPerBlock / kGbgThreads;

enum GbgGate : int { GBG_RX = 0, GBG_RY = 1, GBG_RZ = 2 };

// Index of the k-th amplitude pair (bit q clear) of a state.
__device__ __forceinline__ uint32_t gbg_pair(uint32_t k, int q)
{
    return ((k >> q) << (q + 1)) | (k & ((1u << q) - 1u));
}

// 2x2 matrix of exp(-i t sigma / 2), row-major complex entries u[0..3].
template <int G>
__device__ __forceinline__ void gbg_matrix(float t, float2 *u)
{
    double sd, cd;
    sincos(0.5 * (double)t, &sd, &cd);
    const float c = (float)cd, s = (float)sd;
    if constexpr (G == GBG_RX) {
        u[0] = make_float2(c, 0.f);
        u[1] = make_float2(0.f, -s);
        u[2] = make_float2(0.f, -s);
        u[3] = make_float2(c, 0.f);
    } else if constexpr (G == GBG_RY) {
        u[0] = make_float2(c, 0.f);
        u[1] = make_float2(-s, 0.f);
        u[2] = make_float2(s, 0.f);
        u[3] = make_float2(c, 0.f);
    } else {
        u[0] = make_float2(c, -s);
        u[1] = make_float2(0.f, 0.f);
        u[2] = make_float2(0.f, 0.f);
        u[3] = make_float2(c, s);
    }
}

__device__ __forceinline__ float2 gbg_mad(float2 a, float2 x, float2 b, float2 y)
{
    // a*x + b*y (complex)
    return make_float2(a.x * x.x - a.y * x.y + b.x * y.x - b.y * y.y,
                       a.x * x.y + a.y * x.x + b.x * y.y + b.y * y.x);
}

// Fixed-order block sum in fp64 (tree over the 256 threads).
__device__ __forceinline__ double gbg_block_sum(double v, double *red)
{
    const int i = threadIdx.x;
    red[i] = v;
    __syncthreads();
    for (int h = kGbgThreads / 2; h > 0; h >>= 1) {
        if (i < h) red[i] += red[i + h];
        __syncthreads();
    }
    return red[0];
}

// psi <- |0...0> for every sample.  Grid (ceil(N / 256), B).
__global__ void __launch_bounds__(kGbgThreads) k_gbg_zero(float2 *psi, uint32_t N)
{
    const uint32_t i = blockIdx.x * kGbgThreads + threadIdx.x;
    if (i >= N) return;
    psi[(size_t)blockIdx.y * N + i] = make_float2(i == 0 ? 1.f : 0.f, 0.f);
}

// One rotation on qubit q of every sample; sample b's angle is ang[b * ang_stride].
// Grid (blocks of kGbgPairsPerBlock pairs, B).
template <int G>
__global__ void __launch_bounds__(kGbgThreads) k_gbg_rot(float2 *psi, uint32_t N, int q, const float *ang,
                                                          int ang_stride)
{
    const int b = blockIdx.y;
    float2 u[4];
    gbg_matrix<G>(ang[(size_t)b * ang_stride], u);
    float2 *s = psi + (size_t)b * N;
    const uint32_t half = N >> 1;
#pragma unroll 4
    for (int j = 0; j < kGbgPairsPerThread; ++j) {
        const uint32_t k = blockIdx.x * kGbgPairsPerBlock + j * kGbgThreads + threadIdx.x;
        if (k >= half) break;
        const uint32_t i0 = gbg_pair(k, q), i1 = i0 | (1u << q);
        const float2 a = s[i0], c = s[i1];
        s[i0] = gbg_mad(u[0], a, u[1], c);
        s[i1] = gbg_mad(u[2], a, u[3], c);
    }
}

// CZ(q, q+1): negate the amplitudes with both bits set, in psi and (if given) lambda.
// Grid (ceil((N / 4) / 256), B).
__global__ void __launch_bounds__(kGbgThreads) k_gbg_cz(float2 *psi, float2 *lam, uint32_t N, int q)
{
    const uint32_t k = blockIdx.x * kGbgThreads + threadIdx.x;
    if (k >= (N >> 2)) return;
    const uint32_t i = ((k >> q) << (q + 2)) | (3u << q) | (k & ((1u << q) - 1u));
    const size_t o = (size_t)blockIdx.y * N + i;
    float2 v = psi[o];
    psi[o] = make_float2(-v.x, -v.y);
    if (lam) {
        v = lam[o];
        lam[o] = make_float2(-v.x, -v.y);
    }
}

// CNOT(q, q+1) (control q, target q+1): swap the amplitudes whose bit q is set and whose
// bit q+1 differs, in psi and (if given) lambda.  Grid (ceil((N / 4) / 256), B).
__global__ void __launch_bounds__(kGbgThreads) k_gbg_cnot(float2 *psi, float2 *lam, uint32_t N, int q)
{
    const uint32_t k = blockIdx.x * kGbgThreads + threadIdx.x;
    if (k >= (N >> 2)) return;
    const uint32_t i = ((k >> q) << (q + 2)) | (1u << q) | (k & ((1u << q) - 1u));
    const size_t o0 = (size_t)blockIdx.y * N + i, o1 = o0 + ((size_t)1 << (q + 1));
    float2 v = psi[o0];
    psi[o0] = psi[o1];
    psi[o1] = v;
    if (lam) {
        v = lam[o0];
        lam[o0] = lam[o1];
        lam[o1] = v;
    }
}

// (O psi)_i for the Pauli string with Z part zm and X part xm (Y = iXZ):
// i^(#Y) (-1)^|(i ^ xm) & zm| psi_(i ^ xm).
__device__ __forceinline__ float2 gbg_obs(const float2 *s, uint32_t i, uint32_t zm, uint32_t xm)
{
    const uint32_t j = i ^ xm;
    float2 w = s[j];
    if (__builtin_popcount(j & zm) & 1) w = make_float2(-w.x, -w.y);
    switch (__builtin_popcount(zm & xm) & 3) {
    case 1: return make_float2(-w.y, w.x);
    case 2: return make_float2(-w.x, -w.y);
    case 3: return make_float2(w.y, -w.x);
    default: return w;
    }
}

// Per-block <O> partials: e_part[b][blk] = sum over the block's amplitudes i (two per
// pair slot) of Re(conj(psi_i) (O psi)_i).  Grid (nblk, B).
__global__ void __launch_bounds__(kGbgThreads) k_gbg_expz(const float2 *psi, uint32_t N, uint32_t obs,
                                                           uint32_t obs_x, float *e_part)
{
    __shared__ double red[kGbgThreads];
    const int b = blockIdx.y;
    const float2 *s = psi + (size_t)b * N;
    const uint32_t half = N >> 1;
    float acc = 0.f;
    for (int j = 0; j < kGbgPairsPerThread; ++j) {
        const uint32_t k = blockIdx.x * kGbgPairsPerBlock + j * kGbgThreads + threadIdx.x;
        if (k >= half) break;
        const float2 a = s[2 * k], c = s[2 * k + 1];
        const float2 oa = gbg_obs(s, 2 * k, obs, obs_x), oc = gbg_obs(s, 2 * k + 1, obs, obs_x);
        acc += (a.x * oa.x + a.y * oa.y) + (c.x * oc.x + c.y * oc.y);
    }
    const double t = gbg_block_sum((double)acc, red);
    if (threadIdx.x == 0) e_part[(size_t)b * gridDim.x + blockIdx.x] = (float)t;
}

// lambda = 2 O psi (the upstream dL/dE_b is applied in the final reduction).
// Grid (ceil(N / 256), B).
__global__ void __launch_bounds__(kGbgThreads) k_gbg_seed(const float2 *psi, float2 *lam, uint32_t N, uint32_t obs,
                                                           uint32_t obs_x)
{
    const uint32_t i = blockIdx.x * kGbgThreads + threadIdx.x;
    if (i >= N) return;
    const size_t base = (size_t)blockIdx.y * N;
    const float2 v = gbg_obs(psi + base, i, obs, obs_x);
    lam[base + i] = make_float2(2.f * v.x, 2.f * v.y);
}

// Adjoint step of one rotation exp(-i t sigma_G / 2) on qubit q, with psi and lambda
// just after the gate: gpart[b][blk] = (1/2) sum over the block's pairs of
// Im<lambda|sigma_G|psi>, then psi <- U^dagger psi, lambda <- U^dagger lambda.
// Grid (nblk, B); gpart points at this gate's [B][nblk] block sums.
template <int G>
__global__ void __launch_bounds__(kGbgThreads) k_gbg_rot_adj(float2 *psi, float2 *lam, uint32_t N, int q,
                                                              const float *ang, double *gpart)
{
    __shared__ double red[kGbgThreads];
    const int b = blockIdx.y;
    float2 u[4];
    gbg_matrix<G>(*ang, u);
    // U^dagger = conjugate transpose
    const float2 d0 = make_float2(u[0].x, -u[0].y), d1 = make_float2(u[2].x, -u[2].y);
    const float2 d2 = make_float2(u[1].x, -u[1].y), d3 = make_float2(u[3].x, -u[3].y);
    float2 *s = psi + (size_t)b * N;
    float2 *l = lam + (size_t)b * N;
    const uint32_t half = N >> 1;
    float acc = 0.f;
    for (int j = 0; j < kGbgPairsPerThread; ++j) {
        const uint32_t k = blockIdx.x * kGbgPairsPerBlock + j * kGbgThreads + threadIdx.x;
        if (k >= half) break;
        const uint32_t i0 = gbg_pair(k, q), i1 = i0 | (1u << q);
        const float2 p0 = s[i0], p1 = s[i1], l0 = l[i0], l1 = l[i1];
        // Im<lambda|sigma|psi> over the pair: conj(l) . (sigma p)
        if constexpr (G == GBG_RX) {           // sigma p = (p1, p0)
            acc += (l0.x * p1.y - l0.y * p1.x) + (l1.x * p0.y - l1.y * p0.x);
        } else if constexpr (G == GBG_RY) {    // sigma p = (-i p1, i p0)
            acc += -(l0.x * p1.x + l0.y * p1.y) + (l1.x * p0.x + l1.y * p0.y);
        } else {                               // sigma p = (p0, -p1)
            acc += (l0.x * p0.y - l0.y * p0.x) - (l1.x * p1.y - l1.y * p1.x);
        }
        s[i0] = gbg_mad(d0, p0, d1, p1);
        s[i1] = gbg_mad(d2, p0, d3, p1);
        l[i0] = gbg_mad(d0, l0, d1, l1);
        l[i1] = gbg_mad(d2, l0, d3, l1);
    }
    const double t = gbg_block_sum((double)acc, red);
    if (threadIdx.x == 0) gpart[(size_t)b * gridDim.x + blockIdx.x] = 0.5 * t;
}

// grad[p] = sum_b dlde[b] * sum_blk gpart[p][b][blk], fixed order.  One block per p.
__global__ void __launch_bounds__(kGbgThreads) k_gbg_grad(const double *gpart, const double *dlde, int B, int nblk,
                                                           float *grad)
{
    __shared__ double red[kGbgThreads];
    const int p = blockIdx.x;
    const double *g = gpart + (size_t)p * B * nblk;
    const int total = B * nblk;
    double acc = 0.0;
    for (int i = threadIdx.x; i < total; i += kGbgThreads) acc += dlde[i / nblk] * g[i];
    const double t = gbg_block_sum(acc, red);
    if (threadIdx.x == 0) grad[p] = (float)t;
}

__global__ void k_gbg_copy(const float *src, int count, float *dst)
{
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < count) dst[i] = src[i];
}

// ------------------------------------------------------------------ launchers (host)

int gbg_blocks(int n)
{
    const uint32_t half = (uint32_t)1 << (n - 1);
    return (int)((half + kGbgPairsPerBlock - 1) / kGbgPairsPerBlock);
}

hipError_t launch_gbg_zero(float2 *psi, int n, int B, hipStream_t s)
{
    const uint32_t N = 1u << n;
    k_gbg_zero<<<dim3((N + kGbgThreads - 1) / kGbgThreads, (unsigned)B), kGbgThreads, 0, s>>>(psi, N);
    return hipGetLastError();
}

hipError_t launch_gbg_rot(int gate, float2 *psi, int n, int B, int q, const float *ang, int ang_stride,
                          hipStream_t s)
{
    const dim3 grid((unsigned)gbg_blocks(n), (unsigned)B);
    const uint32_t N = 1u << n;
    if (gate == GBG_RX)
        k_gbg_rot<GBG_RX><<<grid, kGbgThreads, 0, s>>>(psi, N, q, ang, ang_stride);
    else if (gate == GBG_RY)
        k_gbg_rot<GBG_RY><<<grid, kGbgThreads, 0, s>>>(psi, N, q, ang, ang_stride);
    else
        k_gbg_rot<GBG_RZ><<<grid, kGbgThreads, 0, s>>>(psi, N, q, ang, ang_stride);
    return hipGetLastError();
}

hipError_t launch_gbg_cz(float2 *psi, float2 *lam, int n, int B, int q, hipStream_t s)
{
    const uint32_t N = 1u << n, quarter = N >> 2;
    k_gbg_cz<<<dim3((quarter + kGbgThreads - 1) / kGbgThreads, (unsigned)B), kGbgThreads, 0, s>>>(psi, lam, N, q);
    return hipGetLastError();
}

hipError_t launch_gbg_cnot(float2 *psi, float2 *lam, int n, int B, int q, hipStream_t s)
{
    const uint32_t N = 1u << n, quarter = N >> 2;
    k_gbg_cnot<<<dim3((quarter + kGbgThreads - 1) / kGbgThreads, (unsigned)B), kGbgThreads, 0, s>>>(psi, lam, N, q);
    return hipGetLastError();
}

hipError_t launch_gbg_expz(const float2 *psi, int n, int B, uint32_t obs, uint32_t obs_x, float *e_part,
                           hipStream_t s)
{
    k_gbg_expz<<<dim3((unsigned)gbg_blocks(n), (unsigned)B), kGbgThreads, 0, s>>>(psi, 1u << n, obs, obs_x, e_part);
    return hipGetLastError();
}

hipError_t launch_gbg_seed(const float2 *psi, float2 *lam, int n, int B, uint32_t obs, uint32_t obs_x,
                           hipStream_t s)
{
    const uint32_t N = 1u << n;
    k_gbg_seed<<<dim3((N + kGbgThreads - 1) / kGbgThreads, (unsigned)B), kGbgThreads, 0, s>>>(psi, lam, N, obs,
                                                                                              obs_x);
    return hipGetLastError();
}

hipError_t launch_gbg_rot_adj(int gate, float2 *psi, float2 *lam, int n, int B, int q, const float *ang,
                              double *gpart, hipStream_t s)
{
    const dim3 grid((unsigned)gbg_blocks(n), (unsigned)B);
    const uint32_t N = 1u << n;
    if (gate == GBG_RX)
        k_gbg_rot_adj<GBG_RX><<<grid, kGbgThreads, 0, s>>>(psi, lam, N, q, ang, gpart);
    else if (gate == GBG_RY)
        k_gbg_rot_adj<GBG_RY><<<grid, kGbgThreads, 0, s>>>(psi, lam, N, q, ang, gpart);
    else
        k_gbg_rot_adj<GBG_RZ><<<grid, kGbgThreads, 0, s>>>(psi, lam, N, q, ang, gpart);
    return hipGetLastError();
}

hipError_t launch_gbg_grad(const double *gpart, const double *dlde, int B, int n, int n_params, float *grad,
                           hipStream_t s)
{
    k_gbg_grad<<<(unsigned)n_params, kGbgThreads, 0, s>>>(gpart, dlde, B, gbg_blocks(n), grad);
    return hipGetLastError();
}

hipError_t launch_gbg_copy(const float *src, int count, float *dst, hipStream_t s)
{
    k_gbg_copy<<<(count + 255) / 256, 256, 0, s>>>(src, count, dst);
    return hipGetLastError();
}

}  // namespace hqml
