// gfx950 kernels of the fused input projection.
//
// One workgroup computes a BM x BN tile of y = x W (+ bias) with 32x32 MFMA
// tiles (bf16: v_mfma_f32_32x32x16_bf16; fp32: v_mfma_f32_32x32x2f32, true
// fp32 products and sums), then runs the epilogue on that tile: GELU on ff
// columns, rotate-half RoPE on q/k heads, and the scatter into the ff
// ([b,S,ff]) and head-major q/k/v ([b*H,S,hd]) buffers.
//
// Operand staging. Tiles are copied global -> registers -> LDS (double
// buffered, one barrier per K step) with 16-byte loads along whichever axis
// is contiguous in memory:
//   - a token-major activation [b,s,c] and an [F,C] weight are K-contiguous;
//     their LDS tiles are [rows][BK] and MFMA operands are 16-byte LDS reads;
//   - a channels-first activation [b,c,h,w,d] (Walrus PR "Make fused_ff_qkv
//     contiguous": tokens are the h,w,d positions, channel c is S elements
//     apart) and a [C,F] weight are M/N-contiguous; their LDS tiles are
//     [BK][rows], and bf16 operands are transposed on the way out of LDS by
//     ds_read_b64_tr_b16 (two per operand), so no rearranged copy of x is ever
//     made, in memory or in LDS.
// Both LDS layouts XOR-swizzle 16-byte chunks to spread MFMA-operand reads
// over the banks. This kernel serves fp32 and the bf16 shapes the fast kernel
// does not take (RoPE head sizes other than 32, 64 or 128).
//
// Epilogue. The fp32 accumulators (+ bias) are restaged through LDS so that
// each thread owns 16 consecutive bytes of one output row: RoPE needs the
// partner element j +- hd/2 (both in the tile, since a tile holds whole
// heads), and the head-major buffers want 16-byte stores along j with
// consecutive tokens adjacent. The cos/sin of the RoPE angle come from a small
// fp32 table [S, hd/2] built in float64 on the host.
//
// Workgroup order. Workgroups are dispatched round-robin over the 8 XCDs, each
// with its own L2; the linear block id is remapped so that every XCD walks a
// contiguous range of tiles, in groups of group_m tile rows that sweep the
// columns together, so an XCD's L2 holds the x and W panels its CUs share.
#include "general_tile.h"

namespace fp {
namespace {

using namespace gt;

// ---------------------------------------------------------------- the kernel
template <typename T, bool A_KM, bool B_KM, int BM, int BN, int BK>
__global__ __launch_bounds__(kThreads, 2) void fused_proj_tile_kernel(KernelArgs p) {
    constexpr int VW = Traits<T>::VW;
    constexpr int A_ELEMS = BM * BK, B_ELEMS = BN * BK;
    constexpr int STAGE_ELEMS = A_ELEMS + B_ELEMS;
    constexpr int CPAD = 8;                 // floats of padding per epilogue row
    constexpr int CST = BN + CPAD;
    constexpr int OPER_BYTES = 2 * STAGE_ELEMS * (int)sizeof(T);
    constexpr int C_BYTES = BM * CST * 4;
    constexpr int LDS_BYTES = OPER_BYTES > C_BYTES ? OPER_BYTES : C_BYTES;
    constexpr int WM = BM / 2, WN = BN / 2;  // 2 x 2 waves
    constexpr int TM = WM / 32, TN = WN / 32;
    static_assert(TM >= 1 && TN >= 1, "wave tile must hold whole 32x32 MFMA tiles");
    __shared__ __attribute__((aligned(16))) unsigned char smem[LDS_BYTES];
    T* const stage0 = reinterpret_cast<T*>(smem);

    int tm, tn;
    tile_coords(blockIdx.x, p.tiles_m, p.tiles_n, p.group_m, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;

    TileLoader<T, A_KM, BM, BK> la;
    TileLoader<T, B_KM, BN, BK> lb;
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
    lb.store(stage0 + A_ELEMS);
    __syncthreads();
    gemm_k_loop<T, A_KM, B_KM, BM, BN, BK>(acc, la, lb, stage0, p.K, wm, wn, lane);

    // ---- epilogue, phase 1: accumulators + bias -> LDS tile [BM][CST] (fp32)
    float* const Cs = reinterpret_cast<float*>(smem);
    const T* bias = static_cast<const T*>(p.bias);
    float bv[TN];
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        const int col = wn * WN + j * 32 + (lane & 31);
        bv[j] = (bias != nullptr && n0 + col < p.N) ? to_f32(bias[n0 + col]) : 0.0f;
    }
    acc_to_lds<BM, BN, CST>(Cs, acc, bv, wm, wn, lane);
    __syncthreads();

    // ---- epilogue, phase 2: activation / RoPE, 16-byte stores into ff or q/k/v
    constexpr int OV = VW;            // outputs per 16-byte store
    constexpr int GPR = BN / OV;      // column groups per tile row
    constexpr int RPP = kThreads / GPR;
    static_assert(RPP * GPR == kThreads, "epilogue mapping");
    const int g = tid % GPR, rsub = tid / GPR;
    const int f0 = n0 + g * OV;
    if (f0 >= p.N) return;
    int kind, h, j0;
    column_group(p, f0, kind, h, j0);
    const int hd = p.head_dim, kvh = p.n_kv_heads;
    // RoPE over the first rope_dims elements of each q/k head: the partner of element j is
    // j +- rope_dims/2 in the same head, which lies in this tile (the host keeps heads whole
    // in 128-column tiles). When the group lies in one half of the rotated width the whole
    // group shares one partner offset (vector path); otherwise (partial rotation narrower
    // than two groups, or a group crossing rope_dims) each element finds its own.
    const int rd = p.rope_dims, half = rd >> 1;
    const bool do_rope = p.rope && (kind == 1 || kind == 2) && j0 < rd;
    const bool vec_rope = do_rope && half % OV == 0;
    const bool first_half = j0 < half;
    const int i0 = first_half ? j0 : j0 - half;
    const int pcol = g * OV + (first_half ? half : -half);
    const int heads = kind == 1 ? p.n_heads : kvh;
    T* const dst = static_cast<T*>(kind == 0 ? p.ff : kind == 1 ? p.q : kind == 2 ? p.k : p.v);
    auto activate = [&](float (&y)[OV]) __attribute__((always_inline)) {
        if (p.act == 1) {
#pragma unroll
            for (int e = 0; e < OV; ++e) y[e] = gelu_erf(y[e]);
        } else if (p.act == 2) {
#pragma unroll
            for (int e = 0; e < OV; ++e) y[e] = gelu_tanh(y[e]);
        } else if (p.act == 3) {
#pragma unroll
            for (int e = 0; e < OV; ++e) y[e] = relu_squared(y[e]);
        }
    };

    if (kind == 0 && p.ff_channels_first) {
        // ff[bi, f, s] (the 1x1x1-convolution layout): each store holds OV consecutive tokens
        // of one column. Rows start at multiples of OV and S is a multiple of OV (checked on
        // the host), so those tokens lie in one slab and all exist once the first does.
        for (int rc = rsub; rc < BM / OV; rc += RPP) {
            const int m = m0 + rc * OV;
            if (m >= p.M) break;
            const int bi = m / p.S, s0 = m - bi * p.S;
#pragma unroll
            for (int c = 0; c < OV; ++c) {
                float y[OV];
#pragma unroll
                for (int e = 0; e < OV; ++e) y[e] = Cs[(rc * OV + e) * CST + g * OV + c];
                activate(y);
                store16<T>(dst + ((int64_t)bi * p.ff_dim + f0 + c) * p.S + s0, y);
            }
        }
        return;
    }

    for (int row = rsub; row < BM; row += RPP) {
        const int m = m0 + row;
        if (m >= p.M) break;
        float y[OV];
        const float* src = Cs + row * CST + g * OV;
#pragma unroll
        for (int e = 0; e < OV; e += 4) {
            const f32x4 t = *reinterpret_cast<const f32x4*>(src + e);
            y[e] = t.x; y[e + 1] = t.y; y[e + 2] = t.z; y[e + 3] = t.w;
        }
        if (kind == 0) {
            activate(y);
            store16<T>(dst + (int64_t)m * p.ff_dim + f0, y);
        } else {
            const int bi = m / p.S, s = m - bi * p.S;
            if (vec_rope) {
                const float* ps = Cs + row * CST + pcol;
                const float* cs = p.rope_cos + (int64_t)s * half + i0;
                const float* sn = p.rope_sin + (int64_t)s * half + i0;
#pragma unroll
                for (int e = 0; e < OV; e += 4) {
                    const f32x4 yp = *reinterpret_cast<const f32x4*>(ps + e);
                    const f32x4 c = *reinterpret_cast<const f32x4*>(cs + e);
                    const f32x4 sv = *reinterpret_cast<const f32x4*>(sn + e);
                    const float ypv[4] = {yp.x, yp.y, yp.z, yp.w};
                    const float cv[4] = {c.x, c.y, c.z, c.w};
                    const float svv[4] = {sv.x, sv.y, sv.z, sv.w};
#pragma unroll
                    for (int u = 0; u < 4; ++u)
                        y[e + u] = first_half ? y[e + u] * cv[u] - ypv[u] * svv[u]
                                              : y[e + u] * cv[u] + ypv[u] * svv[u];
                }
            } else if (do_rope) {
#pragma unroll
                for (int e = 0; e < OV; ++e) {
                    const int j = j0 + e;
                    if (j >= rd) continue;
                    const bool fh = j < half;
                    const int i = fh ? j : j - half;
                    const float yp = Cs[row * CST + g * OV + e + (fh ? half : -half)];
                    const float c = p.rope_cos[(int64_t)s * half + i];
                    const float sv = p.rope_sin[(int64_t)s * half + i];
                    y[e] = fh ? y[e] * c - yp * sv : y[e] * c + yp * sv;
                }
            }
            const int64_t off = ((int64_t)(bi * heads + h) * p.S + s) * hd + j0;
            store16<T>(dst + off, y);
        }
    }
}

template <typename T, bool A_KM, bool B_KM, int BM, int BN, int BK>
hipError_t launch_one(const KernelArgs& a, hipStream_t stream) {
    const unsigned grid = (unsigned)a.tiles_m * (unsigned)a.tiles_n;
    hipLaunchKernelGGL((fused_proj_tile_kernel<T, A_KM, B_KM, BM, BN, BK>), dim3(grid), dim3(kThreads), 0,
                       stream, a);
    return hipGetLastError();
}

template <typename T, int BM, int BN, int BK>
hipError_t dispatch_layouts(bool x_tl, bool w_fc, const KernelArgs& a, hipStream_t s) {
    if (x_tl) return w_fc ? launch_one<T, true, true, BM, BN, BK>(a, s) : launch_one<T, true, false, BM, BN, BK>(a, s);
    return w_fc ? launch_one<T, false, true, BM, BN, BK>(a, s) : launch_one<T, false, false, BM, BN, BK>(a, s);
}

}  // namespace

bool plan_supported(DType dt, const TilePlan& pl) {
    if (dt == DType::BF16) return pl.bm == 128 && pl.bn == 128 && pl.bk == 64;
    return pl.bm == 128 && pl.bn == 128 && pl.bk == 32;
}

hipError_t launch_fused_proj(DType dt, bool x_tokens_last, bool w_fc, const TilePlan& pl, const KernelArgs& a,
                             hipStream_t stream) {
    if (!plan_supported(dt, pl)) return hipErrorInvalidValue;
    if (dt == DType::BF16) return dispatch_layouts<__bf16, 128, 128, 64>(x_tokens_last, w_fc, a, stream);
    return dispatch_layouts<float, 128, 128, 32>(x_tokens_last, w_fc, a, stream);
}

}  // namespace fp
