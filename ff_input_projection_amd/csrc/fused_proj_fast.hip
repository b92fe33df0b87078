// Fast bf16 kernel of the fused input projection (gfx950).
//
// Orientation. The MFMA computes the transposed tile y^T = W^T x^T: MFMA rows
// are output columns f, MFMA columns are tokens. Each lane's accumulators then
// hold one token and runs of 4 consecutive output columns, so the whole
// epilogue runs in registers:
//   - bias, and exact-erf GELU on ff columns (xformers PR "Fused linear: small
//     FW cleanup and much better perfs": y = act(x W^T + b));
//   - rotate-half RoPE on q/k (NVIDIA/Fuser issue "Improve performance on RoPE
//     (and code around it)", rope_one_entry): the partner column j +- hd/2 sits
//     in the same lane, hd/32 MFMA row tiles (or hd/16 column groups) away;
//   - 8-byte stores straight into ff [b,S,ff] and the head-major q/k/v buffers
//     [b*H,S,hd] (memory-efficient-attention issue "Improve performance via
//     batched-matmul and fused multiplies"), with consecutive tokens adjacent
//     in q/k/v.
// Every branch of the epilogue depends only on the column group, which is the
// same for the whole wave, so it never diverges.
//
// Operands. x is read straight from its channels-first [b,c,spatial] or
// token-major [b,s,c] layout (Walrus PR "Make fused_ff_qkv contiguous": no
// rearranged copy), W from [C,F] or [F,C]. K steps of BK are copied from global
// memory into LDS by global_load_lds_dwordx4 (16 bytes per lane straight into
// LDS, no staging registers) three stages deep, one barrier per K step: before
// reading stage k a wave waits (vmcnt) for its own loads of that stage only,
// then the barrier makes every wave's loads visible. Each
// lane's source chunk is chosen so that the LDS image comes out XOR-swizzled.
// M/N-contiguous tiles feed the MFMA through ds_read_b64_tr_b16, K-contiguous
// ones through ds_read_b128. Chunks outside the problem (ragged M, N or K) are
// read from a small zero block instead, so no access leaves the operands.
//
// Occupancy. 256 threads as 2 x 2 waves, each wave a 128 (f) x 64 (token) tile
// (128 accumulators); two workgroups per CU, i.e. two waves per SIMD, so one
// wave's VALU-heavy epilogue co-issues with the other wave's MFMAs.
#include "device_common.h"
#include "fused_proj_kernels.h"

namespace fp {
namespace {

using namespace dev;
constexpr int kThreads = 256;

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    if constexpr (N == 0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    else if constexpr (N == 2) asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
    else if constexpr (N == 3) asm volatile("s_waitcnt vmcnt(3)" ::: "memory");
    else if constexpr (N == 4) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
    else if constexpr (N == 6) asm volatile("s_waitcnt vmcnt(6)" ::: "memory");
    else if constexpr (N == 8) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
    else if constexpr (N == 12) asm volatile("s_waitcnt vmcnt(12)" ::: "memory");
    else static_assert(N == 0, "add this vmcnt value");
}

__device__ __forceinline__ void store4_bf16(__bf16* dst, const float* o) {
    bf16x4 v;
    v[0] = (__bf16)o[0];
    v[1] = (__bf16)o[1];
    v[2] = (__bf16)o[2];
    v[3] = (__bf16)o[3];
    *reinterpret_cast<u32x2*>(dst) = __builtin_bit_cast(u32x2, v);
}

__device__ __forceinline__ void load4_bias(const __bf16* bias, int f, float* b) {
    if (bias == nullptr) {
        b[0] = b[1] = b[2] = b[3] = 0.0f;
        return;
    }
    const bf16x4 v = __builtin_bit_cast(bf16x4, *reinterpret_cast<const u32x2*>(bias + f));
    b[0] = (float)v[0];
    b[1] = (float)v[1];
    b[2] = (float)v[2];
    b[3] = (float)v[3];
}

// LDS reads at integer byte addresses: base + compile-time constant folds into the
// instruction's offset field, so the K loop spends no VALU on operand addresses.
__device__ __forceinline__ i16x4 lds_tr16(unsigned addr) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(size_t)addr);
}
__device__ __forceinline__ u32x4 lds_b128(unsigned addr) {
    return *(const __attribute__((address_space(3))) u32x4*)(size_t)addr;
}
__device__ __forceinline__ bf16x8 join_tr(i16x4 lo, i16x4 hi) {
    const i16x8 v = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    return __builtin_bit_cast(bf16x8, v);
}

// Per-lane byte offset (stage 0, k step 0) of a transposing-read operand for MFMA rows
// rb..rb+31 in an M/N-major tile of CPR chunks per k row: the swizzle term depends only
// on k mod 4, which is the same for every k step and for the second read (k + 4).
template <int CPR>
__device__ __forceinline__ unsigned mn_operand_base(int rb, int lane) {
    const int g = lane >> 4, q = lane & 15;
    const int m = rb + (g & 1) * 16 + (q & 3) * 4;
    const int kl = (g >> 1) * 8 + (q >> 2);
    return (unsigned)((kl * CPR + ((m >> 3) ^ ((kl & 3) << 2))) * 16 + (m & 7) * 2);
}
// Per-lane byte offset of a 16-byte operand read in a K-major tile, for k step kk.
template <int CPR>
__device__ __forceinline__ unsigned k_operand_base(int rb, int kk, int lane) {
    const int r = rb + (lane & 31);
    const int c = kk * 2 + (lane >> 5);
    return (unsigned)((r * CPR + (c ^ ((r * CPR / 16) % CPR))) * 16);
}

template <bool X_TL, bool W_FC, int BF, int BT, int BK>
struct FastCfg {
    static constexpr int STAGES = 3;
    static constexpr int WF = BF / 2, WT = BT / 2;   // 2 x 2 waves
    static constexpr int TI = WF / 32, TJ = WT / 32;
    static constexpr int NG = TI * 4;                // 8-column groups per wave
    static constexpr int KK = BK / 16;               // MFMA k steps per K step
    static constexpr int W_BYTES = BF * BK * 2, X_BYTES = BT * BK * 2;
    static constexpr int X_REGION = STAGES * W_BYTES;
    static constexpr int LDS_BYTES = STAGES * (W_BYTES + X_BYTES);
    static constexpr int W_CPR = W_FC ? BK / 8 : BF / 8;
    static constexpr int X_CPR = X_TL ? BK / 8 : BT / 8;
    static constexpr int W_INSTR = BF * BK / 8 / 64 / 4;   // direct loads per wave per K step
    static constexpr int X_INSTR = BT * BK / 8 / 64 / 4;
    static constexpr int NLOAD = W_INSTR + X_INSTR;
    static_assert(W_INSTR * 8 * 64 * 4 == BF * BK && X_INSTR * 8 * 64 * 4 == BT * BK, "tile split");
    static_assert(BK % 16 == 0, "BK");
    // immediate LDS offsets (stage + k step) must fit the 16-bit offset field
    static_assert(STAGES * W_BYTES <= 65536 && STAGES * X_BYTES <= 65536, "16-bit LDS offsets");
};

// Operand state of one wave: read bases and direct-load sources.
template <bool X_TL, bool W_FC, int BF, int BT, int BK>
struct FastPipe {
    using C = FastCfg<X_TL, W_FC, BF, BT, BK>;
    unsigned wbase[C::TI][W_FC ? C::KK : 1];   // LDS read bases of the W^T operands
    unsigned xbase[C::TJ][X_TL ? C::KK : 1];   // and of the x operands
    unsigned voff[C::NLOAD];                   // per-lane byte offset of each direct-load chunk
    int kofs[C::NLOAD];                        // its k offset inside the K step
    const char* wsrc;                          // W and x byte addresses of K step 0
    const char* xsrc;
    int64_t wstep, xstep;                      // bytes per K step
    unsigned lds0;                             // LDS byte address of the tile storage
    int wave;

    // Issue the direct loads of K step kt into stage ST. `tail`: K step kt runs past K;
    // its chunks beyond K are read from the zero block instead.
    template <int ST>
    __device__ __forceinline__ void issue(int kt, int K, bool tail, const char* zeros) const {
        const char* ws = wsrc + (int64_t)kt * wstep;
        const char* xs = xsrc + (int64_t)kt * xstep;
#pragma unroll
        for (int q = 0; q < C::NLOAD; ++q) {
            const bool isw = q < C::W_INSTR;
            const unsigned dst = lds0 + (isw ? ST * C::W_BYTES + (wave * C::W_INSTR + q) * 1024
                                             : C::X_REGION + ST * C::X_BYTES + (wave * C::X_INSTR + (q - C::W_INSTR)) * 1024);
            const char* base = isw ? ws : xs;
            if (!tail) {
                // SGPR base + 32-bit lane offset: no per-load VALU
                asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(voff[q]), "s"(base), "{m0}"(dst) : "memory");
            } else {
                const char* a = (kt * BK + kofs[q] < K) ? base + voff[q] : zeros;
                asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(a), "{m0}"(dst) : "memory");
            }
        }
    }

    // All MFMA k steps of stage ST.
    template <int ST>
    __device__ __forceinline__ void compute(f32x16 (&acc)[C::TI][C::TJ]) const {
        bf16x8 a[C::KK][C::TI], b[C::KK][C::TJ];
#pragma unroll
        for (int kk = 0; kk < C::KK; ++kk) {
#pragma unroll
            for (int i = 0; i < C::TI; ++i) {
                if constexpr (W_FC) {
                    a[kk][i] = __builtin_bit_cast(bf16x8, lds_b128(wbase[i][kk] + ST * C::W_BYTES));
                } else {
                    const unsigned o = wbase[i][0] + ST * C::W_BYTES + kk * 16 * C::W_CPR * 16;
                    a[kk][i] = join_tr(lds_tr16(o), lds_tr16(o + 4 * C::W_CPR * 16));
                }
            }
#pragma unroll
            for (int j = 0; j < C::TJ; ++j) {
                if constexpr (X_TL) {
                    b[kk][j] = __builtin_bit_cast(bf16x8, lds_b128(xbase[j][kk] + ST * C::X_BYTES));
                } else {
                    const unsigned o = xbase[j][0] + ST * C::X_BYTES + kk * 16 * C::X_CPR * 16;
                    b[kk][j] = join_tr(lds_tr16(o), lds_tr16(o + 4 * C::X_CPR * 16));
                }
            }
        }
#pragma unroll
        for (int kk = 0; kk < C::KK; ++kk)
#pragma unroll
            for (int i = 0; i < C::TI; ++i)
#pragma unroll
                for (int j = 0; j < C::TJ; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[kk][i], b[kk][j], acc[i][j], 0, 0, 0);
    }
};

// One K step: wait for this wave's loads of stage ST, barrier (all waves' loads landed,
// all waves done with the stage about to be refilled), refill it two steps ahead, compute.
template <int ST, class Pipe, class Acc>
__device__ __forceinline__ void k_step(const Pipe& pp, Acc& acc, int kt, int KT, int K, int KT_full,
                                       const char* zeros) {
    using C = typename Pipe::C;
    if (kt + 1 < KT) wait_vmcnt<C::NLOAD>();
    else wait_vmcnt<0>();
    __syncthreads();
    if (kt + 2 < KT) pp.template issue<(ST + 2) % C::STAGES>(kt + 2, K, kt + 2 >= KT_full, zeros);
    pp.template compute<ST>(acc);
}

// X_TL: x token-major [b,s,c] (else channels-first). W_FC: W [F,C] (else [C,F]).
// DG: RoPE partner distance in 8-column groups (hd/16), 0 = no RoPE in this kernel.
template <bool X_TL, bool W_FC, int BF, int BT, int BK, int DG>
__global__ __launch_bounds__(kThreads, 2) void fused_proj_fast_kernel(KernelArgs p) {
    using C = FastCfg<X_TL, W_FC, BF, BT, BK>;
    constexpr int WF = C::WF, WT = C::WT, TI = C::TI, TJ = C::TJ, NG = C::NG;
    __shared__ __attribute__((aligned(1024))) unsigned char smem[C::LDS_BYTES];
    __shared__ __attribute__((aligned(16))) float bias_s[BF];   // this tile's bias, fp32

    int tt, tf;
    tile_coords(blockIdx.x, p.tiles_m, p.tiles_n, p.group_m, tt, tf);
    const int m0 = tt * BT, n0 = tf * BF;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
    const int wf = wave >> 1, wt = wave & 1;
    const int K = p.K, N = p.N, M = (int)p.M, S = p.S;
    const char* const zeros = static_cast<const char*>(p.zeros);

    FastPipe<X_TL, W_FC, BF, BT, BK> pp;
    pp.wave = wave;
    pp.lds0 = (unsigned)(size_t)(lds_void*)smem;
#pragma unroll
    for (int i = 0; i < TI; ++i) {
        if constexpr (W_FC) {
#pragma unroll
            for (int kk = 0; kk < C::KK; ++kk) pp.wbase[i][kk] = pp.lds0 + k_operand_base<C::W_CPR>(wf * WF + 32 * i, kk, lane);
        } else {
            pp.wbase[i][0] = pp.lds0 + mn_operand_base<C::W_CPR>(wf * WF + 32 * i, lane);
        }
    }
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
        if constexpr (X_TL) {
#pragma unroll
            for (int kk = 0; kk < C::KK; ++kk)
                pp.xbase[j][kk] = pp.lds0 + C::X_REGION + k_operand_base<C::X_CPR>(wt * WT + 32 * j, kk, lane);
        } else {
            pp.xbase[j][0] = pp.lds0 + C::X_REGION + mn_operand_base<C::X_CPR>(wt * WT + 32 * j, lane);
        }
    }
    // Direct-load chunk of each lane: the LDS image comes out swizzled because lane l of
    // instruction q fills physical chunk (wave*INSTR + q)*64 + l.
#pragma unroll
    for (int q = 0; q < C::W_INSTR; ++q) {
        const int pch = (wave * C::W_INSTR + q) * 64 + lane;
        const int row = pch / C::W_CPR, pc = pch % C::W_CPR;
        int64_t off;
        int krow;
        if constexpr (W_FC) {
            const int c = pc ^ ((row * C::W_CPR / 16) % C::W_CPR);
            const int n = n0 + row;
            krow = c * 8;
            off = (int64_t)(n < N ? n : 0) * K + krow;   // rows past N read row 0: never stored
        } else {
            const int c = pc ^ ((row & 3) << 2);
            const int n = n0 + c * 8;
            krow = row;
            off = (int64_t)krow * N + (n < N ? n : 0);
        }
        pp.voff[q] = (unsigned)(off * 2);
        pp.kofs[q] = krow;
    }
#pragma unroll
    for (int q = 0; q < C::X_INSTR; ++q) {
        const int pch = (wave * C::X_INSTR + q) * 64 + lane;
        const int row = pch / C::X_CPR, pc = pch % C::X_CPR;
        int m, krow;
        if constexpr (X_TL) {
            const int c = pc ^ ((row * C::X_CPR / 16) % C::X_CPR);
            m = m0 + row;
            krow = c * 8;
        } else {
            const int c = pc ^ ((row & 3) << 2);
            m = m0 + c * 8;
            krow = row;
        }
        const int mm = m < M ? m : 0;                  // tokens past M read token 0: never stored
        const int bi = mm / S, s = mm - bi * S;
        const int64_t off = (int64_t)bi * p.x_sb + (int64_t)s * p.x_ss + (int64_t)krow * p.x_sc;
        pp.voff[C::W_INSTR + q] = (unsigned)(off * 2);
        pp.kofs[C::W_INSTR + q] = krow;
    }
    pp.wsrc = static_cast<const char*>(p.w);
    pp.xsrc = static_cast<const char*>(p.x);
    pp.wstep = (W_FC ? (int64_t)BK : (int64_t)BK * N) * 2;
    pp.xstep = (X_TL ? (int64_t)BK : (int64_t)BK * p.x_sc) * 2;

    // The tile's bias goes to LDS once (fp32; zero past N or without bias): the epilogue
    // then reads it without global loads, which would otherwise queue behind its stores.
    if (tid < BF / 4) {
        const int f = n0 + 4 * tid;
        float b4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        if (p.bias != nullptr && f < N) load4_bias(static_cast<const __bf16*>(p.bias), f, b4);
        *reinterpret_cast<f32x4*>(bias_s + 4 * tid) = f32x4{b4[0], b4[1], b4[2], b4[3]};
    }

    f32x16 acc[TI][TJ];
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j) acc[i][j] = f32x16{};

    const int KT = (K + BK - 1) / BK;
    const int KT_full = K / BK;  // K steps with no chunk past K
    if (KT > 0) pp.template issue<0>(0, K, 0 >= KT_full, zeros);
    if (KT > 1) pp.template issue<1>(1, K, 1 >= KT_full, zeros);
    for (int kt = 0; kt < KT; kt += 3) {
        k_step<0>(pp, acc, kt, KT, K, KT_full, zeros);
        if (kt + 1 < KT) k_step<1>(pp, acc, kt + 1, KT, K, KT_full, zeros);
        if (kt + 2 < KT) k_step<2>(pp, acc, kt + 2, KT, K, KT_full, zeros);
    }

    if (KT == 0) __syncthreads();  // (with K steps, their barriers publish bias_s)

    // ---- epilogue in registers. acc[i][j][e]: column f = 32i + 8(e/4) + 4(lane/32) + e%4,
    // token 32j + lane%32 (both relative to the wave tile). The outputs never overlap the
    // inputs (checked on the host), so loads may be hoisted above stores.
    const int hl = lane >> 5;
    __bf16* __restrict__ const out_ff = static_cast<__bf16*>(p.ff);
    __bf16* __restrict__ const out_q = static_cast<__bf16*>(p.q);
    __bf16* __restrict__ const out_k = static_cast<__bf16*>(p.k);
    __bf16* __restrict__ const out_v = static_cast<__bf16*>(p.v);
    const float* __restrict__ const rope_cos = p.rope_cos;
    const float* __restrict__ const rope_sin = p.rope_sin;
    const int ff_dim = p.ff_dim, qw = p.qw, hd = p.head_dim;
    const int n_heads = p.n_heads, act = p.act, rope = p.rope;
    const int half = hd >> 1;
    const int64_t head_stride = (int64_t)S * hd;   // elements between heads of one slab
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
        const int t = m0 + wt * WT + 32 * j + (lane & 31);
        const bool tv = t < M;
        const int bi = t / S, s = t - bi * S;
        __bf16* const ff_row = out_ff + (int64_t)t * ff_dim;
        const int64_t tok = (int64_t)bi * n_heads * head_stride + (int64_t)s * hd;   // head 0 of this token
        const float* const cs_row = rope_cos + (int64_t)s * half;
        const float* const sn_row = rope_sin + (int64_t)s * half;
#pragma unroll
        for (int G = 0; G < NG; ++G) {
            const int f8 = n0 + wf * WF + 8 * G;  // wave-uniform column group
            if (f8 >= N) continue;
            const int f = f8 + 4 * hl;
            const int fl = wf * WF + 8 * G + 4 * hl;   // column inside the tile
            float y[4];
            const f32x4 bv = *reinterpret_cast<const f32x4*>(bias_s + fl);
#pragma unroll
            for (int u = 0; u < 4; ++u) y[u] = acc[G >> 2][j][4 * (G & 3) + u] + bv[u];
            if (f8 < ff_dim) {
                if (act == 1) {
#pragma unroll
                    for (int u = 0; u < 4; ++u) y[u] = gelu_erf_fast(y[u]);
                }
                if (tv) store4_bf16(ff_row + f, y);
                continue;
            }
            const int r = f8 - ff_dim;
            const int which = r / qw;
            const int rem = r - which * qw;
            const int h = rem / hd;
            const int jh8 = rem - h * hd;   // wave-uniform group start inside the head
            const int jh = jh8 + 4 * hl;    // this lane's first column
            __bf16* const dst = (which == 0 ? out_q : which == 1 ? out_k : out_v) + tok + h * head_stride;
            if (DG > 0 && rope && which < 2) {
                // first-half group: compute it and its partner DG groups on (same head,
                // hence inside this wave's tile); the partner's own iteration skips.
                if (jh8 >= half || G + DG >= NG) continue;
                const int G2 = (G + DG < NG) ? G + DG : G;  // constant after unrolling
                float y2[4];
                const f32x4 b2 = *reinterpret_cast<const f32x4*>(bias_s + fl + half);
#pragma unroll
                for (int u = 0; u < 4; ++u) y2[u] = acc[G2 >> 2][j][4 * (G2 & 3) + u] + b2[u];
                const f32x4 c = *reinterpret_cast<const f32x4*>(cs_row + jh);
                const f32x4 sn = *reinterpret_cast<const f32x4*>(sn_row + jh);
                float o1[4], o2[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    o1[u] = y[u] * c[u] - y2[u] * sn[u];
                    o2[u] = y2[u] * c[u] + y[u] * sn[u];
                }
                if (tv) {
                    store4_bf16(dst + jh, o1);
                    store4_bf16(dst + jh + half, o2);
                }
                continue;
            }
            if (tv) store4_bf16(dst + jh, y);
        }
    }
}

template <bool X_TL, bool W_FC, int BF, int BT, int BK, int DG>
hipError_t launch_fast_one(const KernelArgs& a, hipStream_t stream) {
    const unsigned grid = (unsigned)a.tiles_m * (unsigned)a.tiles_n;
    hipLaunchKernelGGL((fused_proj_fast_kernel<X_TL, W_FC, BF, BT, BK, DG>), dim3(grid), dim3(kThreads), 0, stream,
                       a);
    return hipGetLastError();
}

template <int BF, int BT, int BK, int DG>
hipError_t dispatch_fast_layouts(bool x_tl, bool w_fc, const KernelArgs& a, hipStream_t s) {
    if (x_tl) return w_fc ? launch_fast_one<true, true, BF, BT, BK, DG>(a, s) : launch_fast_one<true, false, BF, BT, BK, DG>(a, s);
    return w_fc ? launch_fast_one<false, true, BF, BT, BK, DG>(a, s) : launch_fast_one<false, false, BF, BT, BK, DG>(a, s);
}

}  // namespace

int fast_rope_groups(int head_dim, bool rope) {
    if (!rope) return 0;
    const int dg = head_dim / 16;
    return (head_dim % 16 == 0 && (dg == 2 || dg == 4 || dg == 8)) ? dg : -1;
}

hipError_t launch_fused_proj_fast(bool x_tokens_last, bool w_fc, int dg, const TilePlan& pl, const KernelArgs& a,
                                  hipStream_t stream) {
    if (pl.bm != 128 || pl.bn != 256 || pl.bk != 32) return hipErrorInvalidValue;
    switch (dg) {
        case 0: return dispatch_fast_layouts<256, 128, 32, 0>(x_tokens_last, w_fc, a, stream);
        case 2: return dispatch_fast_layouts<256, 128, 32, 2>(x_tokens_last, w_fc, a, stream);
        case 4: return dispatch_fast_layouts<256, 128, 32, 4>(x_tokens_last, w_fc, a, stream);
        case 8: return dispatch_fast_layouts<256, 128, 32, 8>(x_tokens_last, w_fc, a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace fp
