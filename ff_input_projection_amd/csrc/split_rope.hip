// Standalone split + RoPE (gfx950): a q/k/v projection computed elsewhere, split into
// head-major q, k and v with rotate-half RoPE on q and k (NVIDIA/Fuser issue "Improve
// performance on RoPE (and code around it)": split_qkv, rope_one_entry), the key
// optionally transposed (memory-efficient-attention issue "Improve performance via
// batched-matmul and fused multiplies": key_needs_transpose).
//
// The op moves bytes: every input element is read once from HBM and every output
// element written once. One thread writes one 16-byte chunk of an output (8 bf16), and
// consecutive threads write consecutive chunks, so every wave stores 1 KB of contiguous
// output. The chunk's 8 input elements are 16 contiguous bytes of the token's row; the
// RoPE partners (j +- rope_dims/2 in the same head) are read again, from the caches.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <new>
#include <vector>

#include "../../include/split_rope.h"
#include "fused_proj_kernels.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

struct SplitRopeArgs {
    const __bf16* qkv;       // [b*T, Fq]
    __bf16* q;               // [b*H, T, hd]
    __bf16* k;               // [b*KVH, T, hd] or [b*KVH, hd, T]
    __bf16* v;               // [b*KVH, T, hd]
    const float* rope_cos;   // [T, rd/2]
    const float* rope_sin;
    int64_t Fq;              // (H + 2*KVH) * hd
    int64_t q_chunks;        // 16-byte chunks of q, and of k (= of v); all of them fit 31 bits
    int64_t kv_chunks;
    int32_t T, H, KVH, hd, grouped, rope, rd, k_transposed;
    // the chunk index's divisions, by multiply-high: hd/8, T, H, KVH, T/8, hd
    fp::FastDivU31 div_c8, div_t, div_h, div_kvh, div_t8, div_hd;
};

// Column of element j of head h of slice which (0 q, 1 k, 2 v) in a token's row.
__device__ __forceinline__ int64_t qkv_col(const SplitRopeArgs& p, int which, int h, int j) {
    if (!p.grouped) {
        const int64_t base = which == 0 ? 0 : which == 1 ? (int64_t)p.H * p.hd : (int64_t)(p.H + p.KVH) * p.hd;
        return base + (int64_t)h * p.hd + j;
    }
    const int qpk = p.H / p.KVH, gw = (qpk + 2) * p.hd;
    if (which == 0) return (int64_t)(h / qpk) * gw + (int64_t)(h % qpk) * p.hd + j;
    return (int64_t)h * gw + (int64_t)(qpk + which - 1) * p.hd + j;
}

// Value of element j of head h (slice which) of a token row after RoPE at table row s.
__device__ __forceinline__ float roped(const SplitRopeArgs& p, const __bf16* row, int which, int h, int j, float y,
                                       int s) {
    if (!p.rope || which == 2 || j >= p.rd) return y;
    const int half = p.rd >> 1;
    const bool first = j < half;
    const int i = first ? j : j - half;
    const float yp = (float)row[qkv_col(p, which, h, first ? j + half : j - half)];
    const float c = p.rope_cos[(int64_t)s * half + i], sn = p.rope_sin[(int64_t)s * half + i];
    return first ? y * c - yp * sn : y * c + yp * sn;
}

// Element idx (0..7, a runtime value) of an 8-element vector, by selects rather than an
// indexed register access.
__device__ __forceinline__ float pick8(const bf16x8& v, int idx) {
    float r = (float)v[0];
#pragma unroll
    for (int k = 1; k < 8; ++k) r = idx == k ? (float)v[k] : r;
    return r;
}

__global__ __launch_bounds__(256) void split_rope_kernel(SplitRopeArgs p) {
    const uint32_t c = blockIdx.x * 256u + threadIdx.x;
    const uint32_t qc = (uint32_t)p.q_chunks, kc = (uint32_t)p.kv_chunks;
    if (c >= qc + 2 * kc) return;
    const int which = c < qc ? 0 : c < qc + kc ? 1 : 2;
    const uint32_t cc = which == 0 ? c : which == 1 ? c - qc : c - qc - kc;
    const int heads = which == 0 ? p.H : p.KVH;
    const fp::FastDivU31 div_heads = which == 0 ? p.div_h : p.div_kvh;
    __bf16* const out = which == 0 ? p.q : which == 1 ? p.k : p.v;
    bf16x8 o;
    if (which == 1 && p.k_transposed) {
        // chunk (slab, j, 8 tokens): k[slab, j, s0 .. s0+7]
        const uint32_t sj = fp::fastdiv_u31(cc, p.div_t8);
        const int sc = (int)(cc - sj * (uint32_t)(p.T >> 3));
        const uint32_t slab = fp::fastdiv_u31(sj, p.div_hd);
        const int j = (int)(sj - slab * (uint32_t)p.hd);
        const uint32_t bi = fp::fastdiv_u31(slab, div_heads);
        const int g = (int)(slab - bi * (uint32_t)heads);
        const int64_t col = qkv_col(p, 1, g, j);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int s = sc * 8 + e;
            const __bf16* row = p.qkv + ((int64_t)bi * p.T + s) * p.Fq;
            o[e] = (__bf16)roped(p, row, 1, g, j, (float)row[col], s);
        }
    } else {
        // chunk (slab, token, 8 elements): out[slab, s, j0 .. j0+7]
        const uint32_t st = fp::fastdiv_u31(cc, p.div_c8);
        const int j0 = (int)(cc - st * (uint32_t)(p.hd >> 3)) * 8;
        const uint32_t slab = fp::fastdiv_u31(st, p.div_t);
        const int s = (int)(st - slab * (uint32_t)p.T);
        const uint32_t bi = fp::fastdiv_u31(slab, div_heads);
        const int h = (int)(slab - bi * (uint32_t)heads);
        const __bf16* row = p.qkv + ((int64_t)bi * p.T + s) * p.Fq;
        const bf16x8 x = *reinterpret_cast<const bf16x8*>(row + qkv_col(p, which, h, j0));
        const int half = p.rd >> 1;
        if (!p.rope || which == 2 || j0 >= p.rd) {
            o = x;   // v, and elements past the rotated width: copies
        } else if ((half & 7) == 0) {
            // the chunk lies in one half (half a multiple of 8) and its partners form one
            // aligned chunk half a rotated width away; its 8 angles are two 16-byte loads
            const bool first = j0 < half;
            const int i0 = first ? j0 : j0 - half;
            const bf16x8 xp = *reinterpret_cast<const bf16x8*>(row + qkv_col(p, which, h, first ? j0 + half : j0 - half));
            const f32x4* cp = reinterpret_cast<const f32x4*>(p.rope_cos + (int64_t)s * half + i0);
            const f32x4* sp = reinterpret_cast<const f32x4*>(p.rope_sin + (int64_t)s * half + i0);
            const f32x4 c0 = cp[0], c1 = cp[1], s0 = sp[0], s1 = sp[1];
            const float cv[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
            const float sv[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float y = (float)x[e], yp = (float)xp[e];
                o[e] = (__bf16)(first ? y * cv[e] - yp * sv[e] : y * cv[e] + yp * sv[e]);
            }
        } else if (p.rd <= 8) {
            // rotated width up to 8 (so j0 = 0): the partners are in this chunk
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                if (e >= p.rd) {
                    o[e] = x[e];
                    continue;
                }
                const bool first = e < half;
                const int i = first ? e : e - half;
                const float yp = pick8(x, first ? e + half : e - half);
                const float cs = p.rope_cos[(int64_t)s * half + i], sn = p.rope_sin[(int64_t)s * half + i];
                const float y = (float)x[e];
                o[e] = (__bf16)(first ? y * cs - yp * sn : y * cs + yp * sn);
            }
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) o[e] = (__bf16)roped(p, row, which, h, j0 + e, (float)x[e], s);
        }
    }
    __builtin_nontemporal_store(o, reinterpret_cast<bf16x8*>(out) + cc);
}

struct Derived {
    int64_t kvh = 0, rd = 0, Fq = 0, q_chunks = 0, kv_chunks = 0;
};

int check(const split_rope_desc* d, Derived* out) {
    if (!d) return FUSED_PROJ_EINVAL;
    if (d->dtype != FUSED_PROJ_BF16 && d->dtype != FUSED_PROJ_F32) return FUSED_PROJ_EINVAL;
    if (d->batch < 0 || d->tokens < 1 || d->n_heads < 1 || d->head_dim < 1) return FUSED_PROJ_EINVAL;
    if (d->n_kv_heads < 0 || (d->n_kv_heads > 0 && d->n_heads % d->n_kv_heads != 0)) return FUSED_PROJ_EINVAL;
    if (d->qkv_order != FUSED_PROJ_QKV_CONTIGUOUS && d->qkv_order != FUSED_PROJ_QKV_GROUPED) return FUSED_PROJ_EINVAL;
    if (d->pos_offset < 0 || d->rope_dims < 0) return FUSED_PROJ_EINVAL;
    Derived r;
    r.kvh = d->n_kv_heads > 0 ? d->n_kv_heads : d->n_heads;
    r.rd = d->rope_dims > 0 ? d->rope_dims : d->head_dim;
    if (d->rope) {
        if (r.rd % 2 != 0 || r.rd > d->head_dim) return FUSED_PROJ_EINVAL;
        if (!(d->rope_base > 0.0) || !std::isfinite(d->rope_base)) return FUSED_PROJ_EINVAL;
    }
    if (d->dtype != FUSED_PROJ_BF16) return FUSED_PROJ_EUNSUPPORTED;
    if (d->head_dim % 8 != 0) return FUSED_PROJ_EUNSUPPORTED;
    if (d->k_transposed && d->tokens % 8 != 0) return FUSED_PROJ_EUNSUPPORTED;
    const int64_t lim = (int64_t(1) << 31) - 1;
    if (d->n_heads > lim / 8 || d->head_dim > 4096 || d->tokens > lim || d->tokens + d->pos_offset > lim)
        return FUSED_PROJ_EUNSUPPORTED;
    r.Fq = (d->n_heads + 2 * r.kvh) * d->head_dim;
    const double chunks = (double)d->batch * (double)d->tokens * (double)r.Fq / 8.0;
    if (chunks > (double)lim) return FUSED_PROJ_EUNSUPPORTED;
    r.q_chunks = d->batch * d->tokens * d->n_heads * d->head_dim / 8;
    r.kv_chunks = d->batch * d->tokens * r.kvh * d->head_dim / 8;
    if (out) *out = r;
    return FUSED_PROJ_OK;
}

struct Range {
    uintptr_t lo, hi;
};
bool overlap(const Range& a, const Range& b) { return a.lo < b.hi && b.lo < a.hi; }

}  // namespace

struct split_rope_plan {
    split_rope_desc d;
    Derived r;
    int device = -1;
    float* d_cos = nullptr;
    float* d_sin = nullptr;
};

extern "C" {

int split_rope_validate(const split_rope_desc* desc) { return check(desc, nullptr); }

int split_rope_create(const split_rope_desc* desc, split_rope_t* out) {
    if (!out) return FUSED_PROJ_EINVAL;
    *out = nullptr;
    Derived r;
    const int rc = check(desc, &r);
    if (rc) return rc;
    split_rope_plan* h = new (std::nothrow) split_rope_plan();
    if (!h) return FUSED_PROJ_EHIP;
    h->d = *desc;
    h->r = r;
    hipError_t e = hipGetDevice(&h->device);
    if (e == hipSuccess && desc->rope) {
        // cos/sin of (s + pos_offset) * base^(-2i/rd), computed in float64, stored fp32
        const int64_t half = r.rd / 2, T = desc->tokens;
        std::vector<float> hc((size_t)(T * half)), hs((size_t)(T * half));
        for (int64_t s = 0; s < T; ++s)
            for (int64_t i = 0; i < half; ++i) {
                const double phi = (double)(s + desc->pos_offset) *
                                   std::pow(desc->rope_base, -2.0 * (double)i / (double)r.rd);
                hc[(size_t)(s * half + i)] = (float)std::cos(phi);
                hs[(size_t)(s * half + i)] = (float)std::sin(phi);
            }
        const size_t bytes = hc.size() * sizeof(float);
        e = hipMalloc((void**)&h->d_cos, bytes);
        if (e == hipSuccess) e = hipMalloc((void**)&h->d_sin, bytes);
        if (e == hipSuccess) e = hipMemcpy(h->d_cos, hc.data(), bytes, hipMemcpyHostToDevice);
        if (e == hipSuccess) e = hipMemcpy(h->d_sin, hs.data(), bytes, hipMemcpyHostToDevice);
    }
    if (e != hipSuccess) {
        fp::set_last_hip_error(e);
        split_rope_destroy(h);
        return FUSED_PROJ_EHIP;
    }
    *out = h;
    return FUSED_PROJ_OK;
}

int split_rope_run(split_rope_t h, const void* qkv, void* q, void* k, void* v, void* stream) {
    if (!h) return FUSED_PROJ_EINVAL;
    const Derived& r = h->r;
    const int64_t total = r.q_chunks + 2 * r.kv_chunks;
    if (total == 0) return FUSED_PROJ_OK;  // no tokens
    if (!qkv || !q || !k || !v) return FUSED_PROJ_EINVAL;
    for (const void* ptr : {qkv, (const void*)q, (const void*)k, (const void*)v})
        if (reinterpret_cast<uintptr_t>(ptr) & 15u) return FUSED_PROJ_EALIGN;
    const Range in{(uintptr_t)qkv, (uintptr_t)qkv + (uintptr_t)(total * 16)};
    const Range outs[3] = {{(uintptr_t)q, (uintptr_t)q + (uintptr_t)(r.q_chunks * 16)},
                           {(uintptr_t)k, (uintptr_t)k + (uintptr_t)(r.kv_chunks * 16)},
                           {(uintptr_t)v, (uintptr_t)v + (uintptr_t)(r.kv_chunks * 16)}};
    for (int i = 0; i < 3; ++i) {
        if (overlap(outs[i], in)) return FUSED_PROJ_EALIAS;
        for (int j = i + 1; j < 3; ++j)
            if (overlap(outs[i], outs[j])) return FUSED_PROJ_EALIAS;
    }
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        fp::set_last_hip_error(e);
        return FUSED_PROJ_EHIP;
    }
    if (dev != h->device) return FUSED_PROJ_EINVAL;
    SplitRopeArgs a;
    std::memset(&a, 0, sizeof(a));
    a.qkv = static_cast<const __bf16*>(qkv);
    a.q = static_cast<__bf16*>(q);
    a.k = static_cast<__bf16*>(k);
    a.v = static_cast<__bf16*>(v);
    a.rope_cos = h->d_cos;
    a.rope_sin = h->d_sin;
    a.Fq = r.Fq;
    a.q_chunks = r.q_chunks;
    a.kv_chunks = r.kv_chunks;
    a.T = (int32_t)h->d.tokens;
    a.H = (int32_t)h->d.n_heads;
    a.KVH = (int32_t)r.kvh;
    a.hd = (int32_t)h->d.head_dim;
    a.grouped = h->d.qkv_order == FUSED_PROJ_QKV_GROUPED ? 1 : 0;
    a.rope = h->d.rope ? 1 : 0;
    a.rd = (int32_t)r.rd;
    a.k_transposed = h->d.k_transposed ? 1 : 0;
    a.div_c8 = fp::make_fastdiv_u31((uint32_t)(a.hd / 8));
    a.div_t = fp::make_fastdiv_u31((uint32_t)a.T);
    a.div_h = fp::make_fastdiv_u31((uint32_t)a.H);
    a.div_kvh = fp::make_fastdiv_u31((uint32_t)a.KVH);
    a.div_t8 = fp::make_fastdiv_u31((uint32_t)(a.T / 8));
    a.div_hd = fp::make_fastdiv_u31((uint32_t)a.hd);
    const int64_t blocks = (total + 255) / 256;
    hipLaunchKernelGGL(split_rope_kernel, dim3((unsigned)blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                       a);
    e = hipGetLastError();
    if (e != hipSuccess) {
        fp::set_last_hip_error(e);
        return FUSED_PROJ_EHIP;
    }
    return FUSED_PROJ_OK;
}

int split_rope_destroy(split_rope_t h) {
    if (!h) return FUSED_PROJ_OK;
    hipError_t e1 = h->d_cos ? hipFree(h->d_cos) : hipSuccess;
    hipError_t e2 = h->d_sin ? hipFree(h->d_sin) : hipSuccess;
    delete h;
    if (e1 != hipSuccess || e2 != hipSuccess) {
        fp::set_last_hip_error(e1 != hipSuccess ? e1 : e2);
        return FUSED_PROJ_EHIP;
    }
    return FUSED_PROJ_OK;
}

}  // extern "C"
