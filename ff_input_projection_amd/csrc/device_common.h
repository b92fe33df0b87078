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

// ---------------------------------------------------------------- LDS swizzles (16-byte chunks)
// The LDS has 64 four-byte banks (256 bytes per sweep); measured on gfx950 these
// layouts let every MFMA-operand read run at the full ds_read rate.
//
// K-major tile: rows of CPR chunks (the contiguous k axis). Chunk c of row r sits
// at c ^ ((r * CPR / 16) mod CPR): the 16 rows read together by one 16-lane
// phase then cover all 16 chunk slots of a bank sweep.
template <int CPR>
__device__ __forceinline__ int kmaj_chunk(int r, int c) {
    static_assert(CPR == 4 || CPR == 8 || CPR == 16, "K-major rows of 4, 8 or 16 chunks");
    return r * CPR + (c ^ ((r * CPR / 16) % CPR));
}
// M/N-major tile: rows are k, CPR chunks of the contiguous m (or n) axis. Chunk c of
// row k sits at c ^ (4 * (k mod 4)), so the 4 k rows read by one transposing load
// land in 4 different 64-byte bank groups.
template <int CPR>
__device__ __forceinline__ int mnmaj_chunk(int k, int c) {
    static_assert(CPR >= 16, "M/N-major rows need at least 16 chunks");
    return k * CPR + (c ^ ((k & 3) << 2));
}

// ---------------------------------------------------------------- MFMA operands from LDS
// 32x32x16 bf16 operand for rows rb..rb+31 (the MFMA row for A, column for B) at
// k step kk of the tile: lane l holds row rb + l%32, k = 16kk + 8(l/32) + [0..7].
template <int CPR>
__device__ __forceinline__ bf16x8 operand_kmajor(const __bf16* tile, int rb, int kk, int lane) {
    const int r = rb + (lane & 31);
    const int c = kk * 2 + (lane >> 5);
    const u32x4 v = reinterpret_cast<const u32x4*>(tile)[kmaj_chunk<CPR>(r, c)];
    return __builtin_bit_cast(bf16x8, v);
}
// Transposing variant for an M/N-major tile. ds_read_b64_tr_b16: in each 16-lane
// group, lane 4r+c names row r, columns 4c..4c+3 of a 4 x 16 block and receives
// column (lane mod 16) of the 4 rows. Two reads give the 8 k of one operand.
template <int CPR>
__device__ __forceinline__ bf16x8 operand_mnmajor(const __bf16* tile, int rb, int kk, int lane) {
    const int g = lane >> 4, q = lane & 15;
    const int m = rb + (g & 1) * 16 + (q & 3) * 4;
    const int k = kk * 16 + (g >> 1) * 8 + (q >> 2);
    const short* base = reinterpret_cast<const short*>(tile);
    const int e1 = mnmaj_chunk<CPR>(k, m >> 3) * 8 + (m & 7);
    const int e2 = mnmaj_chunk<CPR>(k + 4, m >> 3) * 8 + (m & 7);
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + e1));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + e2));
    const i16x8 v = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    return __builtin_bit_cast(bf16x8, v);
}

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

// The same GELU, rearranged for fewer instructions. With a = |y|, eq. 7.1.26 gives
// erfc(a/sqrt2) ~= P(t) exp(-a^2/2), t = 1/(1 + (p/sqrt2) a). Phi(y) = 1 - erfc/2 for
// y >= 0 and erfc/2 for y < 0, so with h = y P(t) exp(-y^2/2) / 2 (sign of y):
// GELU(y) = y - h (y >= 0), h (y < 0), i.e. max(y, 0) - |h|. The 1/2 is folded into
// the coefficients and log2(e)/2 into the exponent.
__device__ __forceinline__ float gelu_erf_fast(float y) {
    const float a = fabsf(y);
    const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f * 0.70710678118654752440f, a, 1.0f));
    float q = fmaf(0.5f * 1.061405429f, t, 0.5f * -1.453152027f);
    q = fmaf(q, t, 0.5f * 1.421413741f);
    q = fmaf(q, t, 0.5f * -0.284496736f);
    q = fmaf(q, t, 0.5f * 0.254829592f);
    q *= t;
    const float e = __builtin_amdgcn_exp2f((y * y) * -0.72134752044448170368f);  // exp(-y^2/2)
    const float h = (y * q) * e;
    return fmaxf(y, 0.0f) - fabsf(h);
}

// The same GELU with one exp2 and no reciprocal. With a = |y| and q(a) = Phi(-a) =
// erfc(a / sqrt 2) / 2, GELU(y) = max(y, 0) - |y| q(|y|); log2 q is smooth on [0, 6]
// and is taken as one degree-6 polynomial in a (near-minimax fit from
// gelu_poly_fit.py; absolute error of the whole GELU under 1e-5 in fp32, far below the
// bf16 rounding of the outputs this serves). a is clamped
// to 6 in both places it is used: past 6, |y| q(|y|) < 1e-8 and 6 q(6) stands for it.
// Both clamps go through v_med3_f32: fminf / fmaxf would each put a canonicalizing
// v_max_f32 in front (IEEE mode), 12 VALU instructions per value instead of 10. For
// finite y, med3(|y|, 0, 6) = min(|y|, 6) and med3(y, 0, FLT_MAX) = max(y, 0) exactly.
__device__ __forceinline__ float gelu_erf_poly(float y) {
    const float a = __builtin_amdgcn_fmed3f(fabsf(y), 0.0f, 6.0f);
    float p = 2.2990056e-05f;
    p = fmaf(p, a, -0.00061110023f);
    p = fmaf(p, a, 0.0071955691f);
    p = fmaf(p, a, -0.051185358f);
    p = fmaf(p, a, -0.46127188f);
    p = fmaf(p, a, -1.1501743f);
    p = fmaf(p, a, -1.0000647f);
    return fmaf(-a, __builtin_amdgcn_exp2f(p), __builtin_amdgcn_fmed3f(y, 0.0f, 3.40282347e+38f));
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
// Squared ReLU, max(y, 0)^2.
__device__ __forceinline__ float relu_squared(float y) {
    const float r = y > 0.0f ? y : 0.0f;
    return r * r;
}

__device__ __forceinline__ float bf16_to_f32(__bf16 v) { return (float)v; }

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
