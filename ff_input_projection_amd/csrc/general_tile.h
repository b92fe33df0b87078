// Building blocks of the 128 x 128 MFMA tile kernels (the general forward kernel and
// the backward kernels): 16-byte global loads staged through registers into
// XOR-swizzled LDS tiles, MFMA operand fetches from those tiles, the K loop, and
// 16-byte output stores.
//
// Layouts. A tile is K-major ([rows][BK], 16-byte chunks along k) when its operand is
// contiguous along the contraction, and M/N-major ([BK][rows], chunks along the rows)
// when it is contiguous along the rows; bf16 M/N-major operands are transposed on the
// way out of LDS by ds_read_b64_tr_b16. Both XOR-swizzle 16-byte chunks so that the
// MFMA operand reads spread over the LDS banks.
#pragma once
#include "device_common.h"
#include "fused_proj_kernels.h"

namespace fp {
namespace gt {

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kThreads = 256;

template <typename T> struct Traits;
template <> struct Traits<__bf16> {
    static constexpr int VW = 8;     // elements per 16-byte chunk
    static constexpr int KSTEP = 16; // k per MFMA
};
template <> struct Traits<float> {
    static constexpr int VW = 4;
    static constexpr int KSTEP = 2;
};

// ---------------------------------------------------------------- LDS tile addressing
// K-major tile: R rows (m or n), BK consecutive k per row; 16-byte chunk c of row r
// is stored at chunk position c ^ ((r/2) mod chunks-per-row).
template <int BK, int VW>
__device__ __forceinline__ int kmaj_chunk(int r, int c) {
    constexpr int CPR = BK / VW;
    return r * CPR + (c ^ ((r >> 1) & (CPR - 1)));
}
// MN-major tile: BK rows (k), R consecutive m (or n) per row; chunk c of row k is
// stored at c ^ (4 * (k mod 4)) so the four k rows read by one transposing load
// land on different 64-byte bank groups.
template <int R, int VW>
__device__ __forceinline__ int mnmaj_chunk(int k, int c) {
    constexpr int CPR = R / VW;
    static_assert(CPR >= 16, "MN-major tiles need at least 16 chunks per row");
    return k * CPR + (c ^ ((k & 3) << 2));
}

// ---------------------------------------------------------------- global -> LDS loaders
// A loader owns PER 16-byte chunks of a tile per thread. It keeps one pointer per
// chunk and advances it by one K step after every load.
template <typename T, bool KMAJOR, int R, int BK>
struct TileLoader {
    static constexpr int VW = Traits<T>::VW;
    static constexpr int CPR = KMAJOR ? BK / VW : R / VW;  // chunks per LDS row
    static constexpr int PER = R * BK / VW / kThreads;
    static_assert(PER * kThreads * VW == R * BK, "tile must split evenly over the workgroup");
    const T* ptr[PER];
    int kpos[PER];   // k offset of the chunk within the K step
    int dst[PER];    // chunk index in the LDS tile
    bool ok[PER];    // row (m or n) inside the problem
    int64_t step;    // elements to the next K step
    u32x4 reg[PER];

    __device__ __forceinline__ void load(int k0, int K) {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            u32x4 v = {0u, 0u, 0u, 0u};
            if (ok[i] && k0 + kpos[i] < K) v = *reinterpret_cast<const u32x4*>(ptr[i]);
            reg[i] = v;
            ptr[i] += step;
        }
    }
    __device__ __forceinline__ void store(T* tile) const {
#pragma unroll
        for (int i = 0; i < PER; ++i) reinterpret_cast<u32x4*>(tile)[dst[i]] = reg[i];
    }
};

// Activation x: token m = bi*S + s at x + bi*sb + s*ss + c*sc.
template <typename T, bool KMAJOR, int BM, int BK>
__device__ __forceinline__ void init_x_loader(TileLoader<T, KMAJOR, BM, BK>& L, const KernelArgs& p,
                                              int m0, int tid) {
    using LT = TileLoader<T, KMAJOR, BM, BK>;
    const T* x = static_cast<const T*>(p.x);
#pragma unroll
    for (int i = 0; i < LT::PER; ++i) {
        const int id = tid + i * kThreads;
        const int row = id / LT::CPR, c = id % LT::CPR;
        int m, krow;
        if (KMAJOR) { m = m0 + row; krow = c * LT::VW; L.dst[i] = kmaj_chunk<BK, LT::VW>(row, c); }
        else        { m = m0 + c * LT::VW; krow = row; L.dst[i] = mnmaj_chunk<BM, LT::VW>(row, c); }
        L.ok[i] = m < p.M;
        L.kpos[i] = krow;
        const int mm = L.ok[i] ? m : 0;
        const int bi = mm / p.S, s = mm - bi * p.S;
        L.ptr[i] = x + (int64_t)bi * p.x_sb + (int64_t)s * p.x_ss + (int64_t)krow * p.x_sc;
    }
    L.step = KMAJOR ? (int64_t)BK : (int64_t)BK * p.x_sc;
}

// Weight W: [C,F] (N-contiguous) when !KMAJOR, [F,C] (K-contiguous) when KMAJOR.
template <typename T, bool KMAJOR, int BN, int BK>
__device__ __forceinline__ void init_w_loader(TileLoader<T, KMAJOR, BN, BK>& L, const KernelArgs& p,
                                              int n0, int tid) {
    using LT = TileLoader<T, KMAJOR, BN, BK>;
    const T* w = static_cast<const T*>(p.w);
#pragma unroll
    for (int i = 0; i < LT::PER; ++i) {
        const int id = tid + i * kThreads;
        const int row = id / LT::CPR, c = id % LT::CPR;
        int n, krow;
        if (KMAJOR) { n = n0 + row; krow = c * LT::VW; L.dst[i] = kmaj_chunk<BK, LT::VW>(row, c); }
        else        { n = n0 + c * LT::VW; krow = row; L.dst[i] = mnmaj_chunk<BN, LT::VW>(row, c); }
        L.ok[i] = n < p.N;
        L.kpos[i] = krow;
        const int nn = L.ok[i] ? n : 0;
        L.ptr[i] = KMAJOR ? w + (int64_t)nn * p.K + krow : w + (int64_t)krow * p.N + nn;
    }
    L.step = KMAJOR ? (int64_t)BK : (int64_t)BK * p.N;
}

// ---------------------------------------------------------------- MFMA operand fetch
// 32x32 MFMA operand for rows rb..rb+31 (m for A, n for B) at k step kk.
// Lane l holds row rb + l%32; bf16 operands hold k = 16kk + 8(l/32) + [0..7],
// fp32 operands k = 2kk + l/32.
template <bool KMAJOR, int R, int BK>
__device__ __forceinline__ bf16x8 fetch_bf16(const __bf16* tile, int rb, int kk, int lane) {
    if constexpr (KMAJOR) {
        const int r = rb + (lane & 31);
        const int c = kk * 2 + (lane >> 5);
        const u32x4 v = reinterpret_cast<const u32x4*>(tile)[kmaj_chunk<BK, 8>(r, c)];
        return __builtin_bit_cast(bf16x8, v);
    } else {
        // ds_read_b64_tr_b16: in each 16-lane group, lane 4r+c names row r, columns
        // 4c..4c+3 of a 4 x 16 block; lane i receives column i of the 4 rows.
        const int g = lane >> 4, q = lane & 15;
        const int m = rb + (g & 1) * 16 + (q & 3) * 4;
        const int k = kk * 16 + (g >> 1) * 8 + (q >> 2);
        const short* base = reinterpret_cast<const short*>(tile);
        const int e1 = mnmaj_chunk<R, 8>(k, m >> 3) * 8 + (m & 7);
        const int e2 = mnmaj_chunk<R, 8>(k + 4, m >> 3) * 8 + (m & 7);
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + e1));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + e2));
        typedef short i16x8 __attribute__((ext_vector_type(8)));
        const i16x8 v = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
        return __builtin_bit_cast(bf16x8, v);
    }
}

template <bool KMAJOR, int R, int BK>
__device__ __forceinline__ float fetch_f32(const float* tile, int rb, int kk, int lane) {
    const int r = rb + (lane & 31);
    const int k = kk * 2 + (lane >> 5);
    if constexpr (KMAJOR) return tile[kmaj_chunk<BK, 4>(r, k >> 2) * 4 + (k & 3)];
    else                  return tile[mnmaj_chunk<R, 4>(k, r >> 2) * 4 + (r & 3)];
}

// ---------------------------------------------------------------- epilogue helpers
using dev::gelu_erf;
using dev::gelu_tanh;
using dev::relu_squared;
using dev::tile_coords;

// 16-byte output stores, non-temporal: every output is written once and not read here.
template <typename T> __device__ __forceinline__ void store16(T* dst, const float* y);
template <> __device__ __forceinline__ void store16<__bf16>(__bf16* dst, const float* y) {
    typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
    bf16x8_t o;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = (__bf16)y[e];  // round to nearest even
    __builtin_nontemporal_store(__builtin_bit_cast(u32x4, o), reinterpret_cast<u32x4*>(dst));
}
template <> __device__ __forceinline__ void store16<float>(float* dst, const float* y) {
    __builtin_nontemporal_store(f32x4{y[0], y[1], y[2], y[3]}, reinterpret_cast<f32x4*>(dst));
}

template <typename T> __device__ __forceinline__ float to_f32(T v) { return (float)v; }

// The K loop of one BM x BN tile: double-buffered LDS stages, one barrier per K step,
// the next step's global loads in flight while this step's MFMAs run. LA / LB are
// loaders with load(k0, K) (global -> registers, zeros outside the problem) and
// store(tile) (registers -> LDS); the first step must already be in LDS (stage 0).
// Waves are 2 x 2, each owning a (BM/2) x (BN/2) block of acc.
template <typename T, bool A_KM, bool B_KM, int BM, int BN, int BK, class LA, class LB, int TM, int TN>
__device__ __forceinline__ void gemm_k_loop(f32x16 (&acc)[TM][TN], LA& la, LB& lb, T* stage0, int K, int wm,
                                            int wn, int lane) {
    constexpr int KSTEP = Traits<T>::KSTEP;
    constexpr int A_ELEMS = BM * BK, B_ELEMS = BN * BK;
    constexpr int STAGE_ELEMS = A_ELEMS + B_ELEMS;
    constexpr int WM = BM / 2, WN = BN / 2;
    const int KT = (K + BK - 1) / BK;
    for (int kt = 0; kt < KT; ++kt) {
        T* const cur = stage0 + (kt & 1) * STAGE_ELEMS;
        T* const nxt = stage0 + ((kt + 1) & 1) * STAGE_ELEMS;
        const bool more = kt + 1 < KT;
        if (more) {
            la.load((kt + 1) * BK, K);
            lb.load((kt + 1) * BK, K);
        }
        const T* As = cur;
        const T* Bs = cur + A_ELEMS;
#pragma unroll
        for (int kk = 0; kk < BK / KSTEP; ++kk) {
            if constexpr (sizeof(T) == 2) {
                bf16x8 a[TM], b[TN];
#pragma unroll
                for (int i = 0; i < TM; ++i) a[i] = fetch_bf16<A_KM, BM, BK>(As, wm * WM + i * 32, kk, lane);
#pragma unroll
                for (int j = 0; j < TN; ++j) b[j] = fetch_bf16<B_KM, BN, BK>(Bs, wn * WN + j * 32, kk, lane);
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int j = 0; j < TN; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
            } else {
                float a[TM], b[TN];
#pragma unroll
                for (int i = 0; i < TM; ++i) a[i] = fetch_f32<A_KM, BM, BK>(As, wm * WM + i * 32, kk, lane);
#pragma unroll
                for (int j = 0; j < TN; ++j) b[j] = fetch_f32<B_KM, BN, BK>(Bs, wn * WN + j * 32, kk, lane);
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int j = 0; j < TN; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i], b[j], acc[i][j], 0, 0, 0);
            }
        }
        if (more) {
            la.store(nxt);
            lb.store(nxt + A_ELEMS);
        }
        __syncthreads();
    }
}

// Accumulators (+ a per-column value, e.g. the bias) -> an fp32 LDS tile [BM][CST]:
// acc[i][j][e] of wave (wm, wn) is row wm*BM/2 + 32i + 8(e/4) + 4(lane/32) + e%4,
// column wn*BN/2 + 32j + lane%32.
template <int BM, int BN, int CST, int TM, int TN>
__device__ __forceinline__ void acc_to_lds(float* Cs, const f32x16 (&acc)[TM][TN], const float (&colv)[TN], int wm,
                                           int wn, int lane) {
    constexpr int WM = BM / 2, WN = BN / 2;
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        const int col = wn * WN + j * 32 + (lane & 31);
#pragma unroll
        for (int i = 0; i < TM; ++i) {
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int row = wm * WM + i * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
                Cs[row * CST + col] = acc[i][j][e] + colv[j];
            }
        }
    }
}

// The slice of fused output column f0 (the first of a group of V columns, never
// straddling a head since head_dim is a multiple of V): kind 0 ff, 1 q, 2 k, 3 v, its
// head h and the element j0 of f0 in that head. The q/k/v columns are either contiguous
// (all q heads, the k heads, the v heads) or grouped per k/v head (its q heads, then k,
// then v).
__device__ __forceinline__ void column_group(const KernelArgs& p, int f0, int& kind, int& h, int& j0) {
    kind = 0;
    h = 0;
    j0 = 0;
    if (f0 < p.ff_dim) return;
    const int hd = p.head_dim, kvh = p.n_kv_heads;
    const int r = f0 - p.ff_dim;
    if (!p.qkv_grouped) {
        const int kvw = kvh * hd;
        const int which = r < p.qw ? 0 : r < p.qw + kvw ? 1 : 2;
        const int rem = which == 0 ? r : r - p.qw - (which - 1) * kvw;
        h = rem / hd;
        j0 = rem - h * hd;
        kind = 1 + which;
    } else {
        const int qpk = p.n_heads / kvh, gw = (qpk + 2) * hd;
        const int grp = r / gw, within = r - grp * gw, slot = within / hd;
        j0 = within - slot * hd;
        kind = slot < qpk ? 1 : slot == qpk ? 2 : 3;
        h = slot < qpk ? grp * qpk + slot : grp;
    }
}

}  // namespace gt
}  // namespace fp
