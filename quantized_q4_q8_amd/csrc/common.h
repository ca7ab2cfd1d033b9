// Internal helpers shared by the libqk kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

#include <algorithm>
#include <stdint.h>

#include "qk.h"

namespace qk {

constexpr int QBLK = 32;    // values per Q4_0 / Q8_0 block
constexpr int WAVE = 64;    // CDNA wavefront width

// ---------------------------------------------------------------- fp16 bits
__device__ __forceinline__ float h2f(uint16_t h) {
    return (float)__builtin_bit_cast(_Float16, h);
}
// fp32 -> binary16, round to nearest even, subnormals kept (v_cvt_f16_f32).
__device__ __forceinline__ uint16_t f2h(float f) {
    return __builtin_bit_cast(uint16_t, (_Float16)f);
}

// ---------------------------------------------------------- wave reductions
// Lane exchanges inside a row of 16 lanes go through DPP (a few cycles);
// exchanges across rows through ds_bpermute.  DPP patterns: quad_perm
// [1,0,3,2] (xor 1), quad_perm [2,3,0,1] (xor 2), row_half_mirror (lane i of
// 8 <-> 7 - i), row_mirror (lane i of 16 <-> 15 - i).  In a full reduction
// the mirrors pair lanes from the two halves that already hold equal values,
// so every lane of a group of W adjacent lanes ends with the group's total.
constexpr int DPP_XOR1 = 0xB1, DPP_XOR2 = 0x4E, DPP_HALF_MIRROR = 0x141, DPP_MIRROR = 0x140;

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ double dpp(double v) {
    const long long b = __builtin_bit_cast(long long, v);
    const int lo = __builtin_amdgcn_update_dpp(0, (int)(b & 0xFFFFFFFF), CTRL, 0xF, 0xF, false);
    const int hi = __builtin_amdgcn_update_dpp(0, (int)(b >> 32), CTRL, 0xF, 0xF, false);
    return __builtin_bit_cast(double, ((long long)hi << 32) | (unsigned int)lo);
}
template <int CTRL>
__device__ __forceinline__ int dpp(int v) {
    return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}

template <typename T>
struct SumOp {
    __device__ static T f(T a, T b) { return a + b; }
};
template <typename T>
struct MaxOp {
    __device__ static T f(T a, T b) { return b > a ? b : a; }
};

// Reduction over groups of W adjacent lanes (W a power of two <= 64).
template <int W, typename Op, typename T>
__device__ __forceinline__ T group_reduce(T v) {
    if (W >= 2) v = Op::f(v, dpp<DPP_XOR1>(v));
    if (W >= 4) v = Op::f(v, dpp<DPP_XOR2>(v));
    if (W >= 8) v = Op::f(v, dpp<DPP_HALF_MIRROR>(v));
    if (W >= 16) v = Op::f(v, dpp<DPP_MIRROR>(v));
    if (W >= 32) v = Op::f(v, __shfl_xor(v, 16, WAVE));
    if (W >= 64) v = Op::f(v, __shfl_xor(v, 32, WAVE));
    return v;
}
template <int W, typename T>
__device__ __forceinline__ T group_sum(T v) {
    return group_reduce<W, SumOp<T>>(v);
}
template <int W, typename T>
__device__ __forceinline__ T group_max(T v) {
    return group_reduce<W, MaxOp<T>>(v);
}

// Arithmetic precision.  Activations and outputs are stored as fp32, but
// every floating-point reduction of the path (block-scaled matmul sums,
// norms, softmax and attention sums, SwiGLU, router and combine) is carried
// in fp64 and rounded to fp32 once, where the result is stored.  The Q8_0
// quantization of activations is discontinuous (a value that moves across a
// rounding boundary changes a whole code step), and over a stack of layers
// such flips compound; computing each stored value to within an fp64
// rounding of its exact value makes it equal to the correctly rounded fp32
// result except in vanishingly rare midpoint cases, so the quantization
// decisions follow the mathematical values and not the summation order.

// -------------------------------------------------------------- RoPE angles
// sin and cos of a RoPE angle x = position * theta (0 <= x < 2^22) in fp64:
// Cody-Waite reduction by pi/2 with a two-part constant (the double nearest
// pi/2 and the double nearest the remainder; fused multiply-adds keep each
// step to one rounding), the Taylor series of sin and cos on [-pi/4, pi/4]
// (truncation error below 1e-24), then the quadrant.  Within a few ulps of
// the correctly rounded values, far below what the fp32 results resolve.
__device__ __forceinline__ void rope_sincos(double x, double& sn, double& cs) {
    const double PIO2_HI = 1.5707963267948966;       // nearest double to pi/2
    const double PIO2_LO = 6.123233995736766e-17;    // nearest double to pi/2 - PIO2_HI
    const double k = rint(x * 0.6366197723675814);   // x * 2/pi
    double r = fma(-k, PIO2_HI, x);
    r = fma(-k, PIO2_LO, r);
    const double z = r * r;
    // sin r = r + r^3 (-1/3! + z/5! - z^2/7! + ... + z^9/21!)
    double p = 1.0 / 51090942171709440000.0;
    p = fma(p, z, -1.0 / 121645100408832000.0);
    p = fma(p, z, 1.0 / 355687428096000.0);
    p = fma(p, z, -1.0 / 1307674368000.0);
    p = fma(p, z, 1.0 / 6227020800.0);
    p = fma(p, z, -1.0 / 39916800.0);
    p = fma(p, z, 1.0 / 362880.0);
    p = fma(p, z, -1.0 / 5040.0);
    p = fma(p, z, 1.0 / 120.0);
    p = fma(p, z, -1.0 / 6.0);
    const double S = fma(r * z, p, r);
    // cos r = 1 + z (-1/2! + z/4! - z^2/6! + ... + z^9/20!)
    double q = 1.0 / 2432902008176640000.0;
    q = fma(q, z, -1.0 / 6402373705728000.0);
    q = fma(q, z, 1.0 / 20922789888000.0);
    q = fma(q, z, -1.0 / 87178291200.0);
    q = fma(q, z, 1.0 / 479001600.0);
    q = fma(q, z, -1.0 / 3628800.0);
    q = fma(q, z, 1.0 / 40320.0);
    q = fma(q, z, -1.0 / 720.0);
    q = fma(q, z, 1.0 / 24.0);
    q = fma(q, z, -0.5);
    const double C = fma(z, q, 1.0);
    const int n = (int)((long long)k & 3);
    sn = n == 0 ? S : (n == 1 ? C : (n == 2 ? -S : -C));
    cs = n == 0 ? C : (n == 1 ? -S : (n == 2 ? -C : S));
}

// ------------------------------------------------------------ Q8_0 helpers
// Four adjacent lanes (lane % 4 == 0..3) hold the 32 values of one block,
// eight consecutive values each.  Computes d = max|x| / 127 (IEEE division)
// and the eight codes round-half-away-from-zero(v / d) clamped to +-127,
// packed little-endian into two dwords.  Every lane of the quad gets d.
__device__ __forceinline__ void q8_quad(const float v[8], uint32_t& lo, uint32_t& hi, float& d) {
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
    amax = fmaxf(amax, dpp<DPP_XOR1>(amax));
    amax = fmaxf(amax, dpp<DPP_XOR2>(amax));
    d = amax / 127.0f;
    uint32_t b[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        int q = 0;
        if (d != 0.0f) {
            float r = roundf(v[i] / d);
            r = fminf(127.0f, fmaxf(-127.0f, r));
            q = (int)r;
        }
        b[i] = (uint32_t)(q & 0xFF);
    }
    lo = b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24);
    hi = b[4] | (b[5] << 8) | (b[6] << 16) | (b[7] << 24);
}

}  // namespace qk

// ------------------------------------------------------------- host checks
#define QK_REQUIRE(cond, code) \
    do {                       \
        if (!(cond)) return (code); \
    } while (0)

#define QK_ALIGNED(p, a) ((((uintptr_t)(p)) & ((a)-1)) == 0)

static inline int qk_launch_status() {
    return hipGetLastError() == hipSuccess ? QK_OK : QK_EHIP;
}
