// Device helpers shared by the kernel sources: uniform loads, complex and vector types,
// DPP row sums, bf16 conversion.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hqml_internal.hpp"

namespace hqml {

// ------------------------------------------------------------------ helpers

// Read a value that is the same for the whole workgroup (tables, views) through the
// constant address space: a scalar load, which does not share the vector-memory
// counter with the state loads and so never waits on a prefetched tile.
__device__ __forceinline__ float ldu(const float *p)
{
    return *(const __attribute__((address_space(4))) float *)(p);
}

__device__ __forceinline__ int ldu(const int *p)
{
    return *(const __attribute__((address_space(4))) int *)(p);
}

__device__ __forceinline__ float2 ldu2(const float *p)
{
    return make_float2(ldu(p), ldu(p + 1));
}

__device__ __forceinline__ float4 ldu4(const float *p)
{
    return make_float4(ldu(p), ldu(p + 1), ldu(p + 2), ldu(p + 3));
}

__device__ __forceinline__ double ldu(const double *p)
{
    return *(const __attribute__((address_space(4))) double *)(p);
}

__device__ __forceinline__ double2 ldu2(const double *p)
{
    return make_double2(ldu(p), ldu(p + 1));
}

__device__ __forceinline__ double4 ldu4(const double *p)
{
    return make_double4(ldu(p), ldu(p + 1), ldu(p + 2), ldu(p + 3));
}

// The kernels are written once for the compute type R (float: the fp32 path; double:
// the fp64-compute path).  V2<R> / V4<R> are the matching vector types.
template <typename R>
struct Vec;
template <>
struct Vec<float> {
    using v2 = float2;
    using v4 = float4;
};
template <>
struct Vec<double> {
    using v2 = double2;
    using v4 = double4;
};
template <typename R>
using V2 = typename Vec<R>::v2;
template <typename R>
using V4 = typename Vec<R>::v4;

__device__ __forceinline__ float2 mk2(float a, float b) { return make_float2(a, b); }
__device__ __forceinline__ double2 mk2(double a, double b) { return make_double2(a, b); }
__device__ __forceinline__ float fmar(float a, float b, float c) { return fmaf(a, b, c); }
__device__ __forceinline__ double fmar(double a, double b, double c) { return fma(a, b, c); }

// Table entry (factor for bit value 0 in x, y; for 1 in z, w) as a uniform value held in
// scalar registers.  Without the pin the compiler may turn a per-lane choice between the
// two factors into a per-lane load address: one vector load, waited on, per use.
template <typename R>
__device__ __forceinline__ V4<R> uniform_v4(const V4<R> *p)
{
    V4<R> f = ldu4(reinterpret_cast<const R *>(p));
    asm volatile("" : "+s"(f.x), "+s"(f.y), "+s"(f.z), "+s"(f.w));
    return f;
}

template <int CTRL>
__device__ __forceinline__ float dppf(float v)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                                  0xF, 0xF, false));
}

// The same lane permutation on a double (its two 32-bit halves moved alike).
template <int CTRL>
__device__ __forceinline__ double dppf(double v)
{
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, CTRL, 0xF, 0xF, false);
    const int hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), CTRL, 0xF, 0xF, false);
    return __builtin_bit_cast(double, (uint64_t)(uint32_t)lo | ((uint64_t)(uint32_t)hi << 32));
}

// Sum over the 16 lanes of a DPP row; every lane of the row ends with the row sum.
template <typename R>
__device__ __forceinline__ R row_sum16(R v)
{
    v += dppf<0xB1>(v);   // quad_perm [1,0,3,2]
    v += dppf<0x4E>(v);   // quad_perm [2,3,0,1]
    v += dppf<0x141>(v);  // row_half_mirror
    v += dppf<0x140>(v);  // row_mirror
    return v;
}

// (re, im) -> packed bf16 (re in the low half), rounded to nearest even by gfx950's packed
// conversion instruction (a NaN stays a NaN).  Written as the instruction itself: through
// the compiler's bf16 vector conversion the same instruction came with a different schedule
// that spilled the forward kernel's registers (the pass took 4.3x as long); in isolation the
// instruction converts 3.6x faster than rounding on the bit pattern with integer operations.
__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float re, float im)
{
    uint32_t r;
    asm("v_cvt_pk_bf16_f32 %0, %1, %2" : "=v"(r) : "v"(re), "v"(im));
    return r;
}

__device__ __forceinline__ float bf16_to_f32(uint32_t h)
{
    return __builtin_bit_cast(float, h << 16);
}

// Storage element of a state: ST = 0 -> float2 (re, im); ST = 1 -> packed bf16 (re low,
// im high); ST = 2 -> double2.  Loads widen to, stores round from, the compute type R.
// Row sums of three independent values, interleaved so that no DPP step waits on
// the one just before it.
template <typename R>
__device__ __forceinline__ void row_sum16x3(R &a, R &b, R &c)
{
    a += dppf<0xB1>(a);
    b += dppf<0xB1>(b);
    c += dppf<0xB1>(c);
    a += dppf<0x4E>(a);
    b += dppf<0x4E>(b);
    c += dppf<0x4E>(c);
    a += dppf<0x141>(a);
    b += dppf<0x141>(b);
    c += dppf<0x141>(c);
    a += dppf<0x140>(a);
    b += dppf<0x140>(b);
    c += dppf<0x140>(c);
    // The callers use the sums in one lane of the row only; without this the compiler
    // moves the last add under that lane's branch, where it cannot take the DPP operand,
    // and emits a separate DPP move (and the move's zero fill) instead of one DPP add.
    asm volatile("" : "+v"(a), "+v"(b), "+v"(c));
}

__device__ __forceinline__ float2 cmul(float2 a, float2 b)
{
    return make_float2(a.x * b.x - a.y * b.y, a.x * b.y + a.y * b.x);
}

__device__ __forceinline__ double2 cmul(double2 a, double2 b)
{
    return make_double2(a.x * b.x - a.y * b.y, a.x * b.y + a.y * b.x);
}

// Multiply by i^ph (ph = 0..3).
template <typename R>
__device__ __forceinline__ void mul_ipow(R &re, R &im, int ph)
{
    const R a = re, b = im;
    if (ph == 1) { re = -b; im = a; }
    else if (ph == 2) { re = -a; im = -b; }
    else if (ph == 3) { re = b; im = -a; }
}

}  // namespace hqml
