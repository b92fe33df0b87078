// Backward pass of the fused input projection (gfx950).
//
// The gradient of y = act(x W^T + b) dispatched into ff/q/k/v (xformers PR "Fused
// linear: small FW cleanup and much better perfs", follow-up comments on the backward
// pass; the forward op itself is described in fused_proj_kernels.hip), by the chain rule
// through the forward steps in reverse:
//
//   dy[t, f] = d_ff[t, f] * act'(y[t, f])                 ff columns (y recomputed)
//   dy[t, head columns] = R_p^T (upstream head gradient)   q and k (RoPE transposed)
//   dy[t, v head columns] = upstream v gradient
//   dx = dy W^T (in x's layout), dW = X^T dy, db = column sums of dy.
//
// Launches, all on the caller's stream (the fast kernel's variants take some of them
// for bf16; the C-ABI layer plans which):
//   1. dy's ff columns: the fast kernel's grad epilogue (bf16, an activation, token-major
//      d_ff; it writes their column sums too), or bwd_dy_kernel: 128 x 128
//      tiles over [M, F]; tiles holding ff columns with an activation recompute y with
//      the same MFMA K loop as the forward general kernel; the epilogue turns each tile
//      into dy in LDS (loading the upstream gradients as 16-byte chunks), stores it
//      token-major into the workspace and writes the tile's fp32 column sums (for db).
//   2. dy's q/k/v columns: bwd_dy_heads_kernel (bf16; a streaming kernel, no product),
//      or bwd_dy_kernel's tiles.
//   3. dx: a forward projection planned by the C-ABI layer (dy as a token-major
//      activation, W read transposed, the result as an "ff" slice laid out like x). When
//      its tiles would leave most CUs idle in a last round, the last token tiles are
//      contracted in ranges of the fused columns into fp32 partial sums, and
//      bwd_reduce_tiles_kernel sums them into dx.
//   4. dW: the fast kernel's (row tile, token range) units (bf16), or bwd_dw_kernel:
//      128 x 128 tiles over [C, F] contracted over tokens, split into token ranges when
//      the tiles alone cannot fill the CUs; x is read in place in its own layout
//      (channels-first: 16-byte runs of tokens; token-major: runs of channels), dy as
//      [tokens, F].
//   5. bwd_reduce_tiles_kernel (the fast kernel's partial sums, in its accumulator order)
//      or bwd_reduce_dw_kernel (the dW tile kernel's [splits, C, F]) into dW in W's layout,
//      and bwd_reduce_db_kernel: the column sums into db.
#include "general_tile.h"

namespace fp {
namespace {

using namespace gt;
using dev::gelu_erf_grad;
using dev::gelu_tanh_grad;
using dev::relu_squared_grad;
using dev::tile_coords;

constexpr int BT = 128;   // tile rows and columns of every backward kernel

// 16 bytes of the storage type at p, as fp32 values.
template <typename T> __device__ __forceinline__ void load16(const T* p, float* out);
template <> __device__ __forceinline__ void load16<__bf16>(const __bf16* p, float* out) {
    const bf16x8 v = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
#pragma unroll
    for (int e = 0; e < 8; ++e) out[e] = (float)v[e];
}
template <> __device__ __forceinline__ void load16<float>(const float* p, float* out) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(p);
    out[0] = v.x; out[1] = v.y; out[2] = v.z; out[3] = v.w;
}

// Four fp32 values stored as the storage type (8 bytes of bf16, 16 of fp32).
template <typename T> __device__ __forceinline__ void store4(T* dst, const float* v);
template <> __device__ __forceinline__ void store4<__bf16>(__bf16* dst, const float* v) {
    dev::bf16x4 o;
#pragma unroll
    for (int u = 0; u < 4; ++u) o[u] = (__bf16)v[u];
    *reinterpret_cast<dev::u32x2*>(dst) = __builtin_bit_cast(dev::u32x2, o);
}
template <> __device__ __forceinline__ void store4<float>(float* dst, const float* v) {
    *reinterpret_cast<f32x4*>(dst) = f32x4{v[0], v[1], v[2], v[3]};
}

__device__ __forceinline__ float act_grad(int act, float y) {
    return act == 1 ? gelu_erf_grad(y) : act == 2 ? gelu_tanh_grad(y) : act == 3 ? relu_squared_grad(y) : 1.0f;
}

// LDS footprint shared by the tile kernels: two operand stages or the fp32 result tile.
template <typename T, int BK>
struct TileLds {
    static constexpr int CST = BT + 8;   // floats per result row (padding spreads the banks)
    static constexpr int OPER = 2 * 2 * BT * BK * (int)sizeof(T);
    static constexpr int C = BT * CST * 4;
    static constexpr int BYTES = OPER > C ? OPER : C;
};

// ---------------------------------------------------------------- 1. dy
template <typename T, bool A_KM, bool B_KM, int BK>
__global__ __launch_bounds__(kThreads, 2) void bwd_dy_kernel(BwdArgs b) {
    constexpr int VW = Traits<T>::VW, OV = VW;
    constexpr int CST = TileLds<T, BK>::CST;
    constexpr int TM = BT / 2 / 32, TN = BT / 2 / 32;
    __shared__ __attribute__((aligned(16))) unsigned char smem[TileLds<T, BK>::BYTES];
    T* const stage0 = reinterpret_cast<T*>(smem);
    float* const Cs = reinterpret_cast<float*>(smem);
    const KernelArgs& p = b.f;

    int tm, tn;
    tile_coords(blockIdx.x, p.tiles_m, b.dy_col_tile1 - b.dy_col_tile0, p.group_m, tm, tn);
    tn += b.dy_col_tile0;
    const int m0 = tm * BT, n0 = tn * BT;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int M = (int)p.M, N = p.N, S = p.S;

    // y = x W + b of the tile, needed where an activation's derivative is taken
    const bool need_y = p.act != 0 && n0 < p.ff_dim;   // uniform over the workgroup
    if (need_y) {
        TileLoader<T, A_KM, BT, BK> la;
        TileLoader<T, B_KM, BT, BK> lb;
        init_x_loader(la, p, m0, tid);
        init_w_loader(lb, p, n0, tid);
        f32x16 acc[TM][TN];
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) acc[i][j] = f32x16{};
        la.load(0, p.K);
        lb.load(0, p.K);
        la.store(stage0);
        lb.store(stage0 + BT * BK);
        __syncthreads();
        gemm_k_loop<T, A_KM, B_KM, BT, BT, BK>(acc, la, lb, stage0, p.K, wm, wn, lane);
        const T* bias = static_cast<const T*>(p.bias);
        float bv[TN];
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int col = wn * (BT / 2) + j * 32 + (lane & 31);
            bv[j] = (bias != nullptr && n0 + col < N) ? (float)bias[n0 + col] : 0.0f;
        }
        acc_to_lds<BT, BT, CST>(Cs, acc, bv, wm, wn, lane);
        __syncthreads();
    }

    // ---- phase A: dy of the tile, written over y in LDS. Thread (g, rsub) takes column
    // group g (OV columns) of rows rsub, rsub + RPP, ...
    constexpr int GPR = BT / OV, RPP = kThreads / GPR;
    const int g = tid % GPR, rsub = tid / GPR;
    const int f0 = n0 + g * OV;
    const bool col_ok = f0 < N;
    int kind = 0, h = 0, j0 = 0;
    if (col_ok) column_group(p, f0, kind, h, j0);
    const int act = p.act, hd = p.head_dim;
    if (col_ok && kind == 0 && b.ff_cf) {
        // d_ff[bi, f, s]: OV consecutive tokens of one column per 16-byte load (rows start at
        // multiples of OV and S is a multiple of OV, so they lie in one slab)
        const T* dff = static_cast<const T*>(b.d_ff);
        for (int rc = rsub; rc < BT / OV; rc += RPP) {
            const int m = m0 + rc * OV;
            if (m >= M) break;
            const int bi = m / S, s0 = m - bi * S;
#pragma unroll
            for (int c = 0; c < OV; ++c) {
                float up[OV];
                load16<T>(dff + ((int64_t)bi * p.ff_dim + f0 + c) * S + s0, up);
#pragma unroll
                for (int e = 0; e < OV; ++e) {
                    float* const cell = Cs + (rc * OV + e) * CST + g * OV + c;
                    *cell = need_y ? up[e] * act_grad(act, *cell) : up[e];
                }
            }
        }
    } else if (col_ok && kind == 0) {
        const T* dff = static_cast<const T*>(b.d_ff);
        for (int row = rsub; row < BT; row += RPP) {
            const int m = m0 + row;
            if (m >= M) break;
            float up[OV];
            load16<T>(dff + (int64_t)m * p.ff_dim + f0, up);
            float* const c = Cs + row * CST + g * OV;
#pragma unroll
            for (int e = 0; e < OV; ++e) c[e] = need_y ? up[e] * act_grad(act, c[e]) : up[e];
        }
    } else if (col_ok) {
        // a q/k/v head: its upstream gradient, rotated back (R_p^T, the rotation by -phi)
        // over the first rope_dims elements of q and k
        const int heads = kind == 1 ? p.n_heads : p.n_kv_heads;
        const T* src = static_cast<const T*>(kind == 1 ? b.dq : kind == 2 ? b.dk : b.dv);
        const int rd = p.rope_dims, half = rd >> 1;
        const bool do_rope = p.rope && kind != 3 && j0 < rd;
        const bool vec_rope = do_rope && half % OV == 0;
        const bool first_half = j0 < half;
        const int i0 = first_half ? j0 : j0 - half;
        for (int row = rsub; row < BT; row += RPP) {
            const int m = m0 + row;
            if (m >= M) break;
            const int bi = m / S, s = m - bi * S;
            const T* const hrow = src + ((int64_t)(bi * heads + h) * S + s) * hd;
            float gv[OV];
            load16<T>(hrow + j0, gv);
            float out[OV];
            if (vec_rope) {
                // the partner chunk half a rotated width away, one angle per pair
                float pv[OV];
                load16<T>(hrow + (first_half ? j0 + half : j0 - half), pv);
                const float* cs = p.rope_cos + (int64_t)s * half + i0;
                const float* sn = p.rope_sin + (int64_t)s * half + i0;
#pragma unroll
                for (int e = 0; e < OV; ++e) {
                    // first half:  g_i c + g_{i+half} s;  second half: g_{i+half} c - g_i s
                    out[e] = first_half ? gv[e] * cs[e] + pv[e] * sn[e] : gv[e] * cs[e] - pv[e] * sn[e];
                }
            } else {
#pragma unroll
                for (int e = 0; e < OV; ++e) {
                    const int j = j0 + e;
                    out[e] = gv[e];
                    if (do_rope && j < rd) {
                        const bool fh = j < half;
                        const int i = fh ? j : j - half;
                        const float pe = (float)hrow[fh ? j + half : j - half];
                        const float c = p.rope_cos[(int64_t)s * half + i];
                        const float sv = p.rope_sin[(int64_t)s * half + i];
                        out[e] = fh ? gv[e] * c + pe * sv : gv[e] * c - pe * sv;
                    }
                }
            }
            float* const c = Cs + row * CST + g * OV;
#pragma unroll
            for (int e = 0; e < OV; ++e) c[e] = out[e];
        }
    }
    __syncthreads();

    // ---- phase B: dy rows out (16 bytes per thread), and the tile's column sums for db
    if (col_ok) {
        T* const dy = static_cast<T*>(b.dy);
        for (int row = rsub; row < BT; row += RPP) {
            const int m = m0 + row;
            if (m >= M) break;
            float y[OV];
            const float* src = Cs + row * CST + g * OV;
#pragma unroll
            for (int e = 0; e < OV; ++e) y[e] = src[e];
            store16<T>(dy + (int64_t)m * N + f0, y);
        }
    }
    if (b.dbp != nullptr && tid < BT && n0 + tid < N) {
        // one dbp row per 32 tokens (the rows that exist)
        const int rows = M - m0 < BT ? M - m0 : BT;
        for (int q = 0; q * 32 < rows; ++q) {
            float sum = 0.0f;
            const int rend = rows < 32 * q + 32 ? rows : 32 * q + 32;
            for (int r = 32 * q; r < rend; ++r) sum += Cs[r * CST + tid];
            b.dbp[(int64_t)(m0 / 32 + q) * N + n0 + tid] = sum;
        }
    }
}

// dy's q/k/v columns [col0, F) alone (bf16): the upstream head gradients rotated back,
// no product and no LDS tile. Workgroup: 128 tokens x 128 columns; thread (token lane tl,
// group gi) takes the 8 columns col0 + 128 blockIdx.x + 8 gi of the 8 tokens 8 tl .. 8 tl
// + 7 (16 threads store a token's 256 contiguous bytes), then the column sums of each
// 32-token block meet in LDS (one dbp row per 32 tokens, as everywhere).
__global__ __launch_bounds__(256) void bwd_dy_heads_kernel(BwdArgs b, int col0) {
    using T = __bf16;
    constexpr int OV = 8;
    __shared__ float part[16][BT + 4];
    const KernelArgs& p = b.f;
    const int gi = threadIdx.x & 15, tl = threadIdx.x >> 4;
    const int M = (int)p.M, N = p.N, S = p.S;
    const int f0 = col0 + (int)blockIdx.x * BT + gi * OV;
    const int m0 = (int)blockIdx.y * BT;
    const bool col_ok = f0 < N;
    float sum[OV];
#pragma unroll
    for (int e = 0; e < OV; ++e) sum[e] = 0.0f;
    if (col_ok) {
        int kind = 0, h = 0, j0 = 0;
        column_group(p, f0, kind, h, j0);
        const int hd = p.head_dim, heads = kind == 1 ? p.n_heads : p.n_kv_heads;
        const T* src = static_cast<const T*>(kind == 1 ? b.dq : kind == 2 ? b.dk : b.dv);
        const int rd = p.rope_dims, half = rd >> 1;
        const bool do_rope = p.rope && kind != 3 && j0 < rd;
        const bool vec_rope = do_rope && half % OV == 0;
        const bool first_half = j0 < half;
        const int i0 = first_half ? j0 : j0 - half;
        T* const dy = static_cast<T*>(b.dy);
        for (int k = 0; k < BT / 16; ++k) {
            const int m = m0 + 8 * tl + k;
            if (m >= M) break;
            const int bi = m / S, s = m - bi * S;
            const T* const hrow = src + ((int64_t)(bi * heads + h) * S + s) * hd;
            float gv[OV], out[OV];
            load16<T>(hrow + j0, gv);
            if (vec_rope) {
                // the partner chunk half a rotated width away, one angle per pair
                float pv[OV];
                load16<T>(hrow + (first_half ? j0 + half : j0 - half), pv);
                const f32x4* cs = reinterpret_cast<const f32x4*>(p.rope_cos + (int64_t)s * half + i0);
                const f32x4* sn = reinterpret_cast<const f32x4*>(p.rope_sin + (int64_t)s * half + i0);
                const f32x4 c0 = cs[0], c1 = cs[1], s0 = sn[0], s1 = sn[1];
                const float cv[OV] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
                const float sv[OV] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
                for (int e = 0; e < OV; ++e)
                    out[e] = first_half ? gv[e] * cv[e] + pv[e] * sv[e] : gv[e] * cv[e] - pv[e] * sv[e];
            } else {
#pragma unroll
                for (int e = 0; e < OV; ++e) {
                    const int j = j0 + e;
                    out[e] = gv[e];
                    if (do_rope && j < rd) {
                        const bool fh = j < half;
                        const int i = fh ? j : j - half;
                        const float pe = (float)hrow[fh ? j + half : j - half];
                        const float c = p.rope_cos[(int64_t)s * half + i];
                        const float sv = p.rope_sin[(int64_t)s * half + i];
                        out[e] = fh ? gv[e] * c + pe * sv : gv[e] * c - pe * sv;
                    }
                }
            }
            store16<T>(dy + (int64_t)m * N + f0, out);
#pragma unroll
            for (int e = 0; e < OV; ++e) sum[e] += out[e];
        }
    }
    if (b.dbp == nullptr) return;
#pragma unroll
    for (int e = 0; e < OV; ++e) part[tl][gi * OV + e] = sum[e];
    __syncthreads();
    // thread (q, c): column c of 32-token block q (token lanes 4q .. 4q + 3)
    const int c = (int)threadIdx.x & (BT - 1), q = (int)threadIdx.x >> 7;
    const int f = col0 + (int)blockIdx.x * BT + c;
    if (f < N) {
        for (int qq = q; qq < 4; qq += 2) {
            if (m0 + 32 * qq >= M) break;
            const float t = (part[4 * qq][c] + part[4 * qq + 1][c]) + (part[4 * qq + 2][c] + part[4 * qq + 3][c]);
            b.dbp[(int64_t)(m0 / 32 + qq) * N + f] = t;
        }
    }
}

// ---------------------------------------------------------------- 3. dW
// Loader of the transposed activation X^T [C, tokens] for token range [t0, t0 + K): rows
// are channels, the contraction runs over tokens. KMAJOR (channels-first x): each chunk
// is VW consecutive tokens of one channel; otherwise (token-major x) VW consecutive
// channels of one token. Token addresses are recomputed per K step (slabs break the
// stride); chunks past the range or past C read nothing (zeros).
template <typename T, bool KMAJOR, int BK>
struct XtLoader {
    static constexpr int VW = Traits<T>::VW;
    static constexpr int CPR = KMAJOR ? BK / VW : BT / VW;
    static constexpr int PER = BT * BK / VW / kThreads;
    static_assert(PER * kThreads * VW == BT * BK, "tile must split evenly over the workgroup");
    const T* x;
    int64_t rowoff[PER];   // channel offset of the chunk's row
    int kpos[PER];         // token offset of the chunk within the K step
    int dst[PER];
    bool ok[PER];
    int t0, S;
    int64_t sb, ss;
    u32x4 reg[PER];

    __device__ __forceinline__ void init(const KernelArgs& p, int c0, int t_begin, int tid) {
        x = static_cast<const T*>(p.x);
        t0 = t_begin;
        S = p.S;
        sb = p.x_sb;
        ss = p.x_ss;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int id = tid + i * kThreads;
            const int row = id / CPR, c = id % CPR;
            int ch, k;
            if (KMAJOR) { ch = c0 + row; k = c * VW; dst[i] = kmaj_chunk<BK, VW>(row, c); }
            else        { ch = c0 + c * VW; k = row; dst[i] = mnmaj_chunk<BT, VW>(row, c); }
            ok[i] = ch < p.K;
            kpos[i] = k;
            rowoff[i] = (int64_t)(ok[i] ? ch : 0) * p.x_sc;
        }
    }
    __device__ __forceinline__ void load(int k0, int K) {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            u32x4 v = {0u, 0u, 0u, 0u};
            if (ok[i] && k0 + kpos[i] < K) {
                const int t = t0 + k0 + kpos[i];
                const int bi = t / S, s = t - bi * S;
                v = *reinterpret_cast<const u32x4*>(x + (int64_t)bi * sb + (int64_t)s * ss + rowoff[i]);
            }
            reg[i] = v;
        }
    }
    __device__ __forceinline__ void store(T* tile) const {
#pragma unroll
        for (int i = 0; i < PER; ++i) reinterpret_cast<u32x4*>(tile)[dst[i]] = reg[i];
    }
};

// dy [tokens, F] from token t0 on, as the M/N-major operand of the dW tile at column n0.
template <typename T, int BK>
__device__ __forceinline__ void init_dy_loader(TileLoader<T, false, BT, BK>& L, const void* dy, int N, int n0,
                                               int t0, int tid) {
    using LT = TileLoader<T, false, BT, BK>;
    const T* base = static_cast<const T*>(dy) + (int64_t)t0 * N;
#pragma unroll
    for (int i = 0; i < LT::PER; ++i) {
        const int id = tid + i * kThreads;
        const int row = id / LT::CPR, c = id % LT::CPR;
        const int n = n0 + c * LT::VW;
        L.dst[i] = mnmaj_chunk<BT, LT::VW>(row, c);
        L.ok[i] = n < N;
        L.kpos[i] = row;
        L.ptr[i] = base + (int64_t)row * N + (L.ok[i] ? n : 0);
    }
    L.step = (int64_t)BK * N;
}

template <typename T, bool X_KM, int BK>
__global__ __launch_bounds__(kThreads, 2) void bwd_dw_kernel(BwdArgs b) {
    constexpr int VW = Traits<T>::VW, OV = VW;
    constexpr int CST = TileLds<T, BK>::CST;
    constexpr int TM = BT / 2 / 32, TN = BT / 2 / 32;
    __shared__ __attribute__((aligned(16))) unsigned char smem[TileLds<T, BK>::BYTES];
    T* const stage0 = reinterpret_cast<T*>(smem);
    float* const Cs = reinterpret_cast<float*>(smem);
    const KernelArgs& p = b.f;
    const int C = p.K, N = p.N, M = (int)p.M;

    int tm, tn;
    tile_coords(blockIdx.x, b.dw_tiles_m, b.dw_tiles_n, 8, tm, tn);
    const int c0 = tm * BT, n0 = tn * BT;
    const int z = blockIdx.y;
    const int t_begin = z * b.chunk;
    const int t_end = t_begin + b.chunk < M ? t_begin + b.chunk : M;
    const int K = t_end > t_begin ? t_end - t_begin : 0;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;

    XtLoader<T, X_KM, BK> la;
    TileLoader<T, false, BT, BK> lb;
    la.init(p, c0, t_begin, tid);
    init_dy_loader(lb, b.dy, N, n0, t_begin, tid);
    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = f32x16{};
    la.load(0, K);
    lb.load(0, K);
    la.store(stage0);
    lb.store(stage0 + BT * BK);
    __syncthreads();
    gemm_k_loop<T, X_KM, false, BT, BT, BK>(acc, la, lb, stage0, K, wm, wn, lane);
    const float zero[TN] = {};
    acc_to_lds<BT, BT, CST>(Cs, acc, zero, wm, wn, lane);
    __syncthreads();

    constexpr int GPR = BT / OV, RPP = kThreads / GPR;
    const int g = tid % GPR, rsub = tid / GPR;
    if (b.splits > 1) {
        // fp32 partial sums [z][C][F], OV columns per thread and row
        float* const out = b.dwp + (int64_t)z * C * N;
        const int f0 = n0 + g * OV;
        if (f0 >= N) return;
        for (int row = rsub; row < BT; row += RPP) {
            const int c = c0 + row;
            if (c >= C) break;
            const float* src = Cs + row * CST + g * OV;
#pragma unroll
            for (int e = 0; e < OV; e += 4)
                __builtin_nontemporal_store(f32x4{src[e], src[e + 1], src[e + 2], src[e + 3]},
                                            reinterpret_cast<f32x4*>(out + (int64_t)c * N + f0 + e));
        }
        return;
    }
    T* const dw = static_cast<T*>(b.dw);
    if (!b.w_fc) {
        // dW [C, F]: rows of the tile
        const int f0 = n0 + g * OV;
        if (f0 >= N) return;
        for (int row = rsub; row < BT; row += RPP) {
            const int c = c0 + row;
            if (c >= C) break;
            float y[OV];
#pragma unroll
            for (int e = 0; e < OV; ++e) y[e] = Cs[row * CST + g * OV + e];
            store16<T>(dw + (int64_t)c * N + f0, y);
        }
    } else {
        // dW [F, C]: OV consecutive channels of one column per store (C is a multiple of OV)
        for (int u = tid; u < BT * (BT / OV); u += kThreads) {
            const int col = u % BT, cg = u / BT;
            const int f = n0 + col, c = c0 + cg * OV;
            if (f >= N || c >= C) continue;
            float y[OV];
#pragma unroll
            for (int e = 0; e < OV; ++e) y[e] = Cs[(cg * OV + e) * CST + col];
            store16<T>(dw + (int64_t)f * C + c, y);
        }
    }
}

// ---------------------------------------------------------------- 4. reductions
// dW from its split partial sums: 64 x 64 blocks of [C, F]; each thread sums 16
// consecutive columns of one row over the splits (four 16-byte loads per split), then
// stores them as [C, F] rows or, through LDS, as [F, C] rows.
template <typename T>
__global__ __launch_bounds__(256) void bwd_reduce_dw_kernel(BwdArgs b) {
    __shared__ float tile[64][65];
    const int C = b.f.K, N = b.f.N;
    const int c0 = blockIdx.x * 64, f0 = blockIdx.y * 64;
    const int tid = threadIdx.x;
    const int cl = tid >> 2, fl = (tid & 3) * 16;
    const int c = c0 + cl;
    float sum[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) sum[e] = 0.0f;
    if (c < C) {
        for (int z = 0; z < b.splits; ++z) {
            const float* src = b.dwp + ((int64_t)z * C + c) * N + f0 + fl;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if (f0 + fl + 4 * q < N) {   // N is a multiple of 4
                    const f32x4 v = *reinterpret_cast<const f32x4*>(src + 4 * q);
                    sum[4 * q] += v.x; sum[4 * q + 1] += v.y; sum[4 * q + 2] += v.z; sum[4 * q + 3] += v.w;
                }
            }
        }
    }
    T* const dw = static_cast<T*>(b.dw);
    if (!b.w_fc) {
        if (c < C) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int f = f0 + fl + 4 * q;
                if (f < N) store4<T>(dw + (int64_t)c * N + f, sum + 4 * q);
            }
        }
        return;
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) tile[cl][fl + e] = sum[e];
    __syncthreads();
    // [F, C]: thread (fr, cq) writes 16 consecutive channels of column f0 + fr
    const int fr = tid >> 2, cq = (tid & 3) * 16;
    const int f = f0 + fr;
    if (f >= N) return;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int cc = c0 + cq + 4 * q;   // C is a multiple of 4
        if (cc >= C) continue;
        float v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = tile[cq + 4 * q + u][fr];
        store4<T>(dw + (int64_t)f * C + cc, v);
    }
}

// Partial sums in the fast kernel's accumulator order (its range units: [range][row tile]
// [column tile] blocks of 256 x 256 floats, 1 KB chunks ((wave * 4 + a) * 2 + j) * 4 + q
// of 64 lanes x 4 floats, lane l at row 64 wt + 32 j + l % 32 and columns 128 wf + 32 a +
// 8 q + 4 (l / 32) .. of the block, wave = 4 wf + wt) summed over the ranges. Workgroup:
// a 64 x 64 block of [rows, cols], i.e. 16 chunks of one wave; each thread reads 4 lanes'
// 64 contiguous bytes per range, the sums meet in LDS and leave as rows, transposed rows
// or a channels-first dx (64 tokens of one slab).
struct TileReduce {
    const float* part;
    void* out;
    int64_t range_floats;   // floats per range
    int32_t rows, cols;     // the problem's extent (the blocks may overhang it)
    int32_t tiles_c;        // column tiles per row tile
    int32_t splits;
    int32_t mode;           // 0: out[row][col]; 1: out[col][row]; 2: dx [b, C, S] from tokens
    int32_t ld;             // row stride (modes 0 and 1) or S (mode 2)
    int32_t row0;           // first token (mode 2)
};

template <typename T>
__global__ __launch_bounds__(256) void bwd_reduce_tiles_kernel(TileReduce tr) {
    __shared__ float tile[64][65];
    const int tid = threadIdx.x;
    const int r0 = blockIdx.x * 64, c0 = blockIdx.y * 64;
    const int wt = (r0 & 255) >> 6, wf = (c0 & 255) >> 7, a0 = (c0 & 127) >> 5;
    const int ci = tid >> 4, l0 = (tid & 15) * 4;
    const int a = a0 + (ci >> 3), j = (ci >> 2) & 1, q = ci & 3;
    const int chunk = (((wf * 4 + wt) * 4 + a) * 2 + j) * 4 + q;
    const float* src = tr.part + ((int64_t)(r0 >> 8) * tr.tiles_c + (c0 >> 8)) * 65536 + chunk * 256 + l0 * 4;
    f32x4 sum[4] = {};
    for (int z = 0; z < tr.splits; ++z) {
#pragma unroll
        for (int k = 0; k < 4; ++k) sum[k] += *reinterpret_cast<const f32x4*>(src + 4 * k);
        src += tr.range_floats;
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int l = l0 + k;
        const int row = 32 * j + (l & 31), col = 32 * (a - a0) + 8 * q + 4 * (l >> 5);
#pragma unroll
        for (int u = 0; u < 4; ++u) tile[row][col + u] = sum[k][u];
    }
    __syncthreads();
    T* const out = static_cast<T*>(tr.out);
    if (tr.mode == 0) {
        // thread (r, cq): 16 consecutive columns of row r0 + r
        const int r = tid >> 2, cq = (tid & 3) * 16;
        if (r0 + r >= tr.rows) return;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int c = c0 + cq + 4 * k;   // cols is a multiple of 4
            if (c < tr.cols) store4<T>(out + (int64_t)(r0 + r) * tr.ld + c, &tile[r][cq + 4 * k]);
        }
        return;
    }
    // thread (cr, rq): 16 consecutive rows of column c0 + cr (rows is a multiple of 4)
    const int cr = tid >> 2, rq = (tid & 3) * 16;
    const int c = c0 + cr;
    if (c >= tr.cols) return;
    T* base;
    if (tr.mode == 1) {
        base = out + (int64_t)c * tr.ld + r0;
    } else {
        const int t0 = tr.row0 + r0, bi = t0 / tr.ld;
        base = out + ((int64_t)bi * tr.cols + c) * tr.ld + (t0 - bi * tr.ld);
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int rr = rq + 4 * k;
        if (r0 + rr >= tr.rows) continue;
        float v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = tile[rr + u][cr];
        store4<T>(base + rr, v);
    }
}

// db from the column sums per 32 tokens: 16 columns per workgroup; thread (row group g,
// quad q) adds the 16-byte column quad q of rows g, g + 64, ..., then the 64 row groups'
// sums meet in LDS (a fixed order: the result does not depend on timing).
template <typename T>
__global__ __launch_bounds__(256) void bwd_reduce_db_kernel(BwdArgs b) {
    __shared__ f32x4 part[64][4];
    const int N = b.f.N;
    const int q = threadIdx.x & 3, g = threadIdx.x >> 2;
    const int f = blockIdx.x * 16 + 4 * q;   // N is a multiple of 4
    f32x4 sum = {};
    if (f < N) {
#pragma unroll 4
        for (int r = g; r < b.db_tiles; r += 64) sum += *reinterpret_cast<const f32x4*>(b.dbp + (int64_t)r * N + f);
    }
    part[g][q] = sum;
    __syncthreads();
    // 16 threads finish the 16 columns: column 4 qq + u of the quad
    if (threadIdx.x < 16) {
        const int qq = threadIdx.x >> 2, u = threadIdx.x & 3;
        const int fc = blockIdx.x * 16 + threadIdx.x;
        float t = 0.0f;
        for (int r = 0; r < 64; ++r) t += part[r][qq][u];
        if (fc < N) static_cast<T*>(b.db)[fc] = (T)t;
    }
}

__global__ __launch_bounds__(256) void zero_fill_kernel(unsigned* p, size_t n) {
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) p[i] = 0u;
}

template <typename T, bool A_KM, bool B_KM>
hipError_t launch_dy_one(const BwdArgs& b, hipStream_t s) {
    constexpr int BK = sizeof(T) == 2 ? 64 : 32;
    const unsigned grid = (unsigned)b.f.tiles_m * (unsigned)(b.dy_col_tile1 - b.dy_col_tile0);
    if (grid == 0) return hipSuccess;
    hipLaunchKernelGGL((bwd_dy_kernel<T, A_KM, B_KM, BK>), dim3(grid), dim3(kThreads), 0, s, b);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_dy_layouts(bool x_tl, bool w_fc, const BwdArgs& b, hipStream_t s) {
    if (x_tl) return w_fc ? launch_dy_one<T, true, true>(b, s) : launch_dy_one<T, true, false>(b, s);
    return w_fc ? launch_dy_one<T, false, true>(b, s) : launch_dy_one<T, false, false>(b, s);
}

template <typename T>
hipError_t launch_dw_layouts(bool x_tl, const BwdArgs& b, hipStream_t s) {
    constexpr int BK = sizeof(T) == 2 ? 64 : 32;
    const dim3 grid((unsigned)(b.dw_tiles_m * b.dw_tiles_n), (unsigned)b.splits);
    // channels-first x: tokens contiguous (K-major rows of X^T); token-major: channels
    if (x_tl)
        hipLaunchKernelGGL((bwd_dw_kernel<T, false, BK>), grid, dim3(kThreads), 0, s, b);
    else
        hipLaunchKernelGGL((bwd_dw_kernel<T, true, BK>), grid, dim3(kThreads), 0, s, b);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_reduce_tiles(const TileReduce& tr, hipStream_t s) {
    if (tr.rows <= 0 || tr.cols <= 0) return hipSuccess;
    const dim3 grid((unsigned)((tr.rows + 63) / 64), (unsigned)((tr.cols + 63) / 64));
    hipLaunchKernelGGL((bwd_reduce_tiles_kernel<T>), grid, dim3(256), 0, s, tr);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_reduce_t(const BwdArgs& b, hipStream_t s) {
    if (b.dw_partials && b.f.K > 0) {
        // the fast kernel's units: [splits][C tiles][F tiles] blocks into dW ([C, F] rows, or
        // [F, C] as transposed rows)
        TileReduce tr{};
        tr.part = b.dwp;
        tr.out = b.dw;
        tr.rows = b.f.K;
        tr.cols = b.f.N;
        tr.tiles_c = (b.f.N + 255) / 256;
        tr.range_floats = (int64_t)((b.f.K + 255) / 256) * tr.tiles_c * 65536;
        tr.splits = b.splits;
        tr.mode = b.w_fc ? 1 : 0;
        tr.ld = b.w_fc ? b.f.K : b.f.N;
        const hipError_t e = launch_reduce_tiles<T>(tr, s);
        if (e != hipSuccess) return e;
    } else if (b.splits > 1 && b.f.K > 0) {
        const dim3 grid((unsigned)((b.f.K + 63) / 64), (unsigned)((b.f.N + 63) / 64));
        hipLaunchKernelGGL((bwd_reduce_dw_kernel<T>), grid, dim3(256), 0, s, b);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (b.db != nullptr && b.dbp != nullptr) {
        hipLaunchKernelGGL((bwd_reduce_db_kernel<T>), dim3((unsigned)((b.f.N + 15) / 16)), dim3(256), 0, s, b);
        return hipGetLastError();
    }
    return hipSuccess;
}

}  // namespace

int tile_bk(DType dt) { return dt == DType::BF16 ? 64 : 32; }

hipError_t launch_bwd_dy(DType dt, bool x_tl, bool w_fc, const BwdArgs& b, hipStream_t s) {
    return dt == DType::BF16 ? launch_dy_layouts<__bf16>(x_tl, w_fc, b, s) : launch_dy_layouts<float>(x_tl, w_fc, b, s);
}

hipError_t launch_bwd_dw(DType dt, bool x_tl, const BwdArgs& b, hipStream_t s) {
    return dt == DType::BF16 ? launch_dw_layouts<__bf16>(x_tl, b, s) : launch_dw_layouts<float>(x_tl, b, s);
}

hipError_t launch_bwd_reduce(DType dt, const BwdArgs& b, hipStream_t s) {
    return dt == DType::BF16 ? launch_reduce_t<__bf16>(b, s) : launch_reduce_t<float>(b, s);
}

hipError_t launch_bwd_reduce_dx(const BwdArgs& b, hipStream_t s) {
    if (b.dx_splits <= 1 || b.dx_rows <= 0) return hipSuccess;
    // the tail's units: [splits][token tiles][C tiles] blocks into dx's last tokens
    TileReduce tr{};
    tr.part = b.dxp;
    tr.rows = b.dx_rows;
    tr.cols = b.f.K;
    tr.tiles_c = (b.f.K + 255) / 256;
    tr.range_floats = (int64_t)((b.dx_rows + 255) / 256) * tr.tiles_c * 65536;
    tr.splits = b.dx_splits;
    if (b.dx_cf) {
        tr.out = b.dx;
        tr.mode = 2;
        tr.ld = b.f.S;
        tr.row0 = b.dx_row0;
    } else {
        tr.out = static_cast<__bf16*>(b.dx) + (int64_t)b.dx_row0 * b.f.K;
        tr.mode = 0;
        tr.ld = b.f.K;
    }
    return launch_reduce_tiles<__bf16>(tr, s);
}

hipError_t launch_bwd_dy_heads(const BwdArgs& b, int col0, hipStream_t s) {
    if (col0 >= b.f.N || b.f.M <= 0) return hipSuccess;
    const dim3 grid((unsigned)((b.f.N - col0 + BT - 1) / BT), (unsigned)((b.f.M + BT - 1) / BT));
    hipLaunchKernelGGL(bwd_dy_heads_kernel, grid, dim3(256), 0, s, b, col0);
    return hipGetLastError();
}


hipError_t launch_zero_fill(void* p, size_t n, hipStream_t s) {
    const size_t words = n / 4;
    if (words == 0) return hipSuccess;
    const size_t blocks = (words + 255) / 256;
    hipLaunchKernelGGL(zero_fill_kernel, dim3((unsigned)(blocks < 1024 ? blocks : 1024)), dim3(256), 0, s,
                       static_cast<unsigned*>(p), words);
    return hipGetLastError();
}

}  // namespace fp
