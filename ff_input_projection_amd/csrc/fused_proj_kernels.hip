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
#include "device_common.h"
#include "fused_proj_kernels.h"

namespace fp {
namespace {

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

// ---------------------------------------------------------------- the kernel
template <typename T, bool A_KM, bool B_KM, int BM, int BN, int BK>
__global__ __launch_bounds__(kThreads, 2) void fused_proj_tile_kernel(KernelArgs p) {
    constexpr int VW = Traits<T>::VW;
    constexpr int KSTEP = Traits<T>::KSTEP;
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

    const int KT = (p.K + BK - 1) / BK;
    la.load(0, p.K);
    lb.load(0, p.K);
    la.store(stage0);
    lb.store(stage0 + A_ELEMS);
    __syncthreads();

    for (int kt = 0; kt < KT; ++kt) {
        T* const cur = stage0 + (kt & 1) * STAGE_ELEMS;
        T* const nxt = stage0 + ((kt + 1) & 1) * STAGE_ELEMS;
        const bool more = kt + 1 < KT;
        if (more) {
            la.load((kt + 1) * BK, p.K);
            lb.load((kt + 1) * BK, p.K);
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

    // ---- epilogue, phase 1: accumulators + bias -> LDS tile [BM][CST] (fp32)
    float* const Cs = reinterpret_cast<float*>(smem);
    const T* bias = static_cast<const T*>(p.bias);
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        const int col = wn * WN + j * 32 + (lane & 31);
        const float bv = (bias != nullptr && n0 + col < p.N) ? to_f32(bias[n0 + col]) : 0.0f;
#pragma unroll
        for (int i = 0; i < TM; ++i) {
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int row = wm * WM + i * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
                Cs[row * CST + col] = acc[i][j][e] + bv;
            }
        }
    }
    __syncthreads();

    // ---- epilogue, phase 2: activation / RoPE, 16-byte stores into ff or q/k/v
    constexpr int OV = VW;            // outputs per 16-byte store
    constexpr int GPR = BN / OV;      // column groups per tile row
    constexpr int RPP = kThreads / GPR;
    static_assert(RPP * GPR == kThreads, "epilogue mapping");
    const int g = tid % GPR, rsub = tid / GPR;
    const int f0 = n0 + g * OV;
    if (f0 >= p.N) return;
    // The group's slice (0 ff, 1 q, 2 k, 3 v), head h and element j0 in the head. The q/k/v
    // columns are either contiguous (all q heads, the k heads, the v heads) or grouped per
    // k/v head (its q heads, then k, then v). A group never straddles heads (head_dim is a
    // multiple of OV).
    int kind = 0, h = 0, j0 = 0;
    const int hd = p.head_dim, kvh = p.n_kv_heads;
    if (f0 >= p.ff_dim) {
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
