// Device helpers shared by the gfx950 kernels of the fused input projection.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp {
namespace dev {

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void glb_void;

// ---------------------------------------------------------------- epilogue arithmetic
// erf by Abramowitz & Stegun, Handbook of Mathematical Functions, eq. 7.1.26
// (Hastings' rational-exponential form): erf(x) = 1 - (a1 t + ... + a5 t^5) e^{-x^2},
// t = 1/(1 + p x) for x >= 0, odd extension; |error| <= 1.5e-7.
__device__ __forceinline__ float erf_as7126(float x) {
    const float ax = fabsf(x);
    const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f, ax, 1.0f));
    float p = fmaf(1.061405429f, t, -1.453152027f);
    p = fmaf(p, t, 1.421413741f);
    p = fmaf(p, t, -0.284496736f);
    p = fmaf(p, t, 0.254829592f);
    p *= t;
    const float e = __builtin_amdgcn_exp2f(-(ax * ax) * 1.4426950408889634f);
    return copysignf(fmaf(-p, e, 1.0f), x);
}
// Exact-erf GELU: y * Phi(y) = 0.5 y (1 + erf(y / sqrt 2)).
__device__ __forceinline__ float gelu_erf(float y) {
    return 0.5f * y * (1.0f + erf_as7126(y * 0.70710678118654752440f));
}

// The same GELU with one exp2 and no reciprocal. With a = |y| and q(a) = Phi(-a) =
// erfc(a / sqrt 2) / 2, GELU(y) = max(y, 0) - |y| q(|y|); log2 q is smooth on [0, 6]
// and is taken as one degree-6 polynomial in a (near-minimax fit from
// gelu_poly_fit.py; absolute error of the whole GELU under 1e-5 in fp32, far below the
// bf16 rounding of the outputs this serves). a is clamped
// to 6 in both places it is used: past 6, |y| q(|y|) < 1e-8 and 6 q(6) stands for it.
// The clamp is one v_med3_f32 (fminf would put a canonicalizing v_max_f32 in front in
// IEEE mode). The positive part is (y + |y|) / 2, which is max(y, 0) exactly for finite y
// and, unlike v_max_f32 / v_med3_f32 (which drop a quiet NaN), keeps what the defining
// y Phi(y) gives in IEEE arithmetic: NaN for NaN, +inf for +inf, NaN for -inf (a
// NaN-keeping v_maximum3_f32 would give about 0 for -inf). 11 VALU instructions per value.
__device__ __forceinline__ float gelu_erf_poly(float y) {
    const float a = __builtin_amdgcn_fmed3f(fabsf(y), 0.0f, 6.0f);
    float p = 2.2990056e-05f;
    p = fmaf(p, a, -0.00061110023f);
    p = fmaf(p, a, 0.0071955691f);
    p = fmaf(p, a, -0.051185358f);
    p = fmaf(p, a, -0.46127188f);
    p = fmaf(p, a, -1.1501743f);
    p = fmaf(p, a, -1.0000647f);
    return fmaf(-a, __builtin_amdgcn_exp2f(p), 0.5f * (y + fabsf(y)));
}

// Its derivative with the same Phi(-a) = 2^P(a): d/dy [y Phi(y)] = Phi(y) + y phi(y), with
// Phi(y) = 1 - Phi(-|y|) for y >= 0 and Phi(-|y|) otherwise, phi(y) = e^(-y^2/2) / sqrt(2 pi).
// Absolute error under 3e-5 in fp32 (pinned on the CPU with the same coefficients).
__device__ __forceinline__ float gelu_erf_grad_poly(float y) {
    const float a = __builtin_amdgcn_fmed3f(fabsf(y), 0.0f, 6.0f);
    float p = 2.2990056e-05f;
    p = fmaf(p, a, -0.00061110023f);
    p = fmaf(p, a, 0.0071955691f);
    p = fmaf(p, a, -0.051185358f);
    p = fmaf(p, a, -0.46127188f);
    p = fmaf(p, a, -1.1501743f);
    p = fmaf(p, a, -1.0000647f);
    const float q = __builtin_amdgcn_exp2f(p);
    const float cdf = y >= 0.0f ? 1.0f - q : q;
    const float pdf = 0.39894228040143267794f * __builtin_amdgcn_exp2f(-0.72134752044448170368f * (y * y));
    return fmaf(y, pdf, cdf);
}

// tanh form of GELU (Hendrycks and Gimpel, "Gaussian Error Linear Units (GELUs)",
// 2016): 0.5 y (1 + tanh(u)), u = sqrt(2/pi) (y + 0.044715 y^3). Since
// 0.5 (1 + tanh u) = 1 / (1 + e^(-2u)), it is y / (1 + 2^(-2u log2 e)): one exp2 and
// one reciprocal, each within a few ulps in fp32. For large |u| the exp2 goes to 0 or
// +inf and the result to y or -0.
__device__ __forceinline__ float gelu_tanh(float y) {
    const float u2 = (y + 0.044715f * (y * y * y)) * (2.0f * 0.79788456080286536f * 1.4426950408889634f);
    return y * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-u2));
}
// Squared ReLU, max(y, 0)^2, with a max that keeps NaN (v_maximum3_f32), as torch's relu does.
__device__ __forceinline__ float relu_squared(float y) {
    const float r = __builtin_elementwise_maximum(y, 0.0f);
    return r * r;
}

// ---------------------------------------------------------------- activation derivatives
// (the backward pass: dy = d_ff * act'(y))
// Exact GELU: d/dy [y Phi(y)] = Phi(y) + y phi(y), phi(y) = e^(-y^2/2) / sqrt(2 pi).
__device__ __forceinline__ float gelu_erf_grad(float y) {
    const float cdf = 0.5f * (1.0f + erf_as7126(y * 0.70710678118654752440f));
    const float pdf = 0.39894228040143267794f * __builtin_amdgcn_exp2f(-0.5f * y * y * 1.4426950408889634f);
    return fmaf(y, pdf, cdf);
}
// tanh GELU: with s = 1 / (1 + e^(-2u)) = (1 + tanh u) / 2, u = sqrt(2/pi) (y + 0.044715 y^3),
// d/dy [y s] = s + y * 2 s (1 - s) * u'(y), u'(y) = sqrt(2/pi) (1 + 3 * 0.044715 y^2). For
// large |u| the exp2 goes to 0 or +inf and s to 1 or 0.
__device__ __forceinline__ float gelu_tanh_grad(float y) {
    const float k = 0.79788456080286536f;
    const float u2 = (y + 0.044715f * (y * y * y)) * (2.0f * k * 1.4426950408889634f);
    const float s = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-u2));
    const float du = k * (1.0f + 3.0f * 0.044715f * (y * y));
    return s + 2.0f * y * s * (1.0f - s) * du;
}
// Squared ReLU: 2 max(y, 0).
__device__ __forceinline__ float relu_squared_grad(float y) { return y > 0.0f ? 2.0f * y : 0.0f; }

// Tile of linear block id. Workgroups are dispatched round-robin over the 8 XCDs
// (each with its own L2): every XCD is given a contiguous range of tiles, walked in
// groups of group_m tile rows that sweep the tile columns together.
__device__ __forceinline__ void tile_coords(int bid, int tiles_m, int tiles_n, int group_m, int& tm, int& tn) {
    const int total = tiles_m * tiles_n;
    const int xcd = bid & 7, idx = bid >> 3;
    const int q = total >> 3, r = total & 7;
    const int lin = xcd * q + (xcd < r ? xcd : r) + idx;
    const int per_group = group_m * tiles_n;
    const int grp = lin / per_group;
    const int first_m = grp * group_m;
    const int gsz = (tiles_m - first_m) < group_m ? (tiles_m - first_m) : group_m;
    const int in = lin - grp * per_group;
    tm = first_m + in % gsz;
    tn = in / gsz;
}

}  // namespace dev
}  // namespace fp
