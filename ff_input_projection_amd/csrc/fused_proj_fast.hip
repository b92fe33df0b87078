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
// LDS, no staging registers), one barrier per K step: before reading stage k a
// wave waits (vmcnt) for its own loads of that stage only, then the barrier
// makes every wave's loads visible. Each
// lane's source chunk is chosen so that the LDS image comes out XOR-swizzled.
// M/N-contiguous tiles feed the MFMA through ds_read_b64_tr_b16, K-contiguous
// ones through ds_read_b128. Chunks outside the problem (ragged M, N or K) are
// read from a small zero block instead, so no access leaves the operands.
//
// Schedule. The kernel is persistent: one workgroup of 8 waves per CU, each
// workgroup walking a list of 256 x 256 tiles (2 x 4 waves of 128 (f) x 64
// (tokens), 128 accumulators each, two waves per SIMD). The direct-load
// pipeline is four stages deep and runs straight on into the next tile: the
// first K steps of tile i+1 are in flight while tile i finishes its last K
// steps and its epilogue. Larger tiles halve the panel traffic from L2 per
// flop compared with 128-token tiles (the L2->CU path, about 54 B/clk per CU
// measured, is the scarce resource), and the workgroup's tiles are taken from
// a contiguous, grouped range of the XCD it runs on.
#include "device_common.h"
#include "fused_proj_kernels.h"

namespace fp {
namespace {

using namespace dev;

// s_waitcnt vmcnt(N): at most N of this wave's vector memory operations outstanding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
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

// Tile geometry: BF output columns x BT tokens per workgroup, NWF x NWT waves.
template <bool X_TL, bool W_FC, int BF, int BT, int NWF, int NWT, int BK, int STAGES>
struct FastCfg {
    static constexpr int NW = NWF * NWT, THREADS = 64 * NW;
    static constexpr int WF = BF / NWF, WT = BT / NWT;   // wave tile
    static constexpr int TI = WF / 32, TJ = WT / 32;
    static constexpr int NG = TI * 4;                    // 8-column groups per wave
    static constexpr int KK = BK / 16;                   // MFMA k steps per K step
    static constexpr int W_BYTES = BF * BK * 2, X_BYTES = BT * BK * 2;
    static constexpr int X_REGION = STAGES * W_BYTES;
    static constexpr int LDS_BYTES = STAGES * (W_BYTES + X_BYTES);
    static constexpr int W_CPR = W_FC ? BK / 8 : BF / 8;
    static constexpr int X_CPR = X_TL ? BK / 8 : BT / 8;
    static constexpr int W_INSTR = BF * BK / 8 / 64 / NW;   // direct loads per wave per K step
    static constexpr int X_INSTR = BT * BK / 8 / 64 / NW;
    static constexpr int NLOAD = W_INSTR + X_INSTR;
    static_assert(W_INSTR * 8 * 64 * NW == BF * BK && X_INSTR * 8 * 64 * NW == BT * BK, "tile split");
    static_assert(TI >= 1 && TJ >= 1 && BK % 16 == 0 && STAGES >= 3, "geometry");
    // the largest immediate LDS offset (stage + k step) must fit the 16-bit field
    static constexpr int W_MAX_IMM = (STAGES - 1) * W_BYTES + (W_FC ? 0 : ((KK - 1) * 16 + 4) * W_CPR * 16);
    static constexpr int X_MAX_IMM = (STAGES - 1) * X_BYTES + (X_TL ? 0 : ((KK - 1) * 16 + 4) * X_CPR * 16);
    static_assert(W_MAX_IMM < 65536 && X_MAX_IMM < 65536, "16-bit LDS offsets");
    static_assert((STAGES - 2) * NLOAD < 64, "vmcnt range");
};

// Wave-constant operand state: LDS read bases and the direct-load chunk map.
template <class C, bool X_TL, bool W_FC, int BK>
struct FastPipe {
    unsigned wbase[C::TI][W_FC ? C::KK : 1];   // LDS read bases of the W^T operands
    unsigned xbase[C::TJ][X_TL ? C::KK : 1];   // and of the x operands
    int kofs[C::NLOAD];                        // k offset of each direct-load chunk in its K step
    unsigned lds0;
    int wave;
    const char* wsrc;                          // W and x byte addresses of K step 0
    const char* xsrc;
    int64_t wstep, xstep;                      // bytes per K step

    // Issue the direct loads of K step ks (of the tile whose chunk offsets are voff) into
    // stage ST. Chunks at or past K (a ragged last step, or the steps that pad the step
    // count to a multiple of the stage count) are read from the zero block.
    template <int ST>
    __device__ __forceinline__ void issue(const unsigned (&voff)[C::NLOAD], int ks, int K,
                                          const char* zeros) const {
        const char* ws = wsrc + (int64_t)ks * wstep;
        const char* xs = xsrc + (int64_t)ks * xstep;
        const bool tail = (ks + 1) * BK > K;
#pragma unroll
        for (int q = 0; q < C::NLOAD; ++q) {
            const bool isw = q < C::W_INSTR;
            const unsigned dst = lds0 + (isw ? ST * C::W_BYTES + (wave * C::W_INSTR + q) * 1024
                                             : C::X_REGION + ST * C::X_BYTES +
                                                   (wave * C::X_INSTR + (q - C::W_INSTR)) * 1024);
            const char* base = isw ? ws : xs;
            if (!tail) {
                // SGPR base + 32-bit lane offset: no per-load VALU. Inline asm keeps the
                // compiler from waiting on every stage in flight before each LDS read.
                asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(voff[q]), "s"(base), "{m0}"(dst) : "memory");
            } else {
                const char* a = (ks * BK + kofs[q] < K) ? base + voff[q] : zeros;
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

// Byte offset of each lane's direct-load chunks for the tile at (m0, n0). Lane l of
// instruction q fills physical LDS chunk (wave*INSTR + q)*64 + l, so choosing the
// source chunk through the inverse swizzle makes the LDS image come out swizzled.
// Rows past N and tokens past M read row / token 0 instead (in bounds, never stored).
template <class C, bool X_TL, bool W_FC>
__device__ __forceinline__ void tile_offsets(unsigned (&voff)[C::NLOAD], int (&kofs)[C::NLOAD], int m0, int n0,
                                             int wave, int lane, int K, int N, int M, int S, int64_t sb,
                                             int64_t ss, int64_t sc) {
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
            off = (int64_t)(n < N ? n : 0) * K + krow;
        } else {
            const int c = pc ^ ((row & 3) << 2);
            const int n = n0 + c * 8;
            krow = row;
            off = (int64_t)krow * N + (n < N ? n : 0);
        }
        voff[q] = (unsigned)(off * 2);
        kofs[q] = krow;
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
        const int mm = m < M ? m : 0;
        const int bi = mm / S, s = mm - bi * S;
        const int64_t off = (int64_t)bi * sb + (int64_t)s * ss + (int64_t)krow * sc;
        voff[C::W_INSTR + q] = (unsigned)(off * 2);
        kofs[C::W_INSTR + q] = krow;
    }
}

// k-th tile of this workgroup. The tiles of the grid's linear order are split into 8
// contiguous ranges, one per XCD (workgroup b runs on XCD b mod 8); inside its range a
// workgroup takes every (workgroups per XCD)-th tile. Linear order: groups of group_m
// token tiles sweep the column tiles together.
__device__ __forceinline__ bool block_tile(int k, int tiles_t, int tiles_f, int group_m, int& tt, int& tf) {
    const int total = tiles_t * tiles_f;
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3, per_xcd = gridDim.x >> 3;
    const int q = total >> 3, r = total & 7;
    const int count = q + (xcd < r ? 1 : 0);
    const int li = slot + k * per_xcd;
    if (li >= count) return false;
    const int lin = xcd * q + (xcd < r ? xcd : r) + li;
    const int per_group = group_m * tiles_f;
    const int grp = lin / per_group;
    const int first = grp * group_m;
    const int gsz = (tiles_t - first) < group_m ? (tiles_t - first) : group_m;
    const int in = lin - grp * per_group;
    tt = first + in % gsz;
    tf = in / gsz;
    return true;
}

// X_TL: x token-major [b,s,c] (else channels-first). W_FC: W [F,C] (else [C,F]).
// DG: RoPE partner distance in 8-column groups (hd/16), 0 = no RoPE.
template <bool X_TL, bool W_FC, int BF, int BT, int NWF, int NWT, int BK, int STAGES, int DG>
__global__ __launch_bounds__(64 * NWF * NWT, 1) void fused_proj_fast_kernel(KernelArgs p) {
    using C = FastCfg<X_TL, W_FC, BF, BT, NWF, NWT, BK, STAGES>;
    constexpr int WF = C::WF, WT = C::WT, TI = C::TI, TJ = C::TJ, NG = C::NG, NLOAD = C::NLOAD;
    __shared__ __attribute__((aligned(1024))) unsigned char smem[C::LDS_BYTES];
    __shared__ __attribute__((aligned(16))) float bias_s[2][BF];   // tile bias (fp32), double-buffered

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
    const int wf = wave / NWT, wt = wave % NWT;
    const int K = p.K, N = p.N, M = (int)p.M, S = p.S;
    const char* const zeros = static_cast<const char*>(p.zeros);
    const __bf16* const bias = static_cast<const __bf16*>(p.bias);

    int tt, tf;
    if (!block_tile(0, p.tiles_m, p.tiles_n, p.group_m, tt, tf)) return;

    FastPipe<C, X_TL, W_FC, BK> pp;
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
    pp.wsrc = static_cast<const char*>(p.w);
    pp.xsrc = static_cast<const char*>(p.x);
    pp.wstep = (W_FC ? (int64_t)BK : (int64_t)BK * N) * 2;
    pp.xstep = (X_TL ? (int64_t)BK : (int64_t)BK * p.x_sc) * 2;

    unsigned voff_cur[NLOAD], voff_nxt[NLOAD];
    tile_offsets<C, X_TL, W_FC>(voff_cur, pp.kofs, tt * BT, tf * BF, wave, lane, K, N, M, S, p.x_sb, p.x_ss,
                                p.x_sc);

    // bias of the first tile (the barriers of its first K step publish it)
    auto stage_bias = [&](int buf, int n0) __attribute__((always_inline)) {
        if (tid < BF / 4) {
            const int f = n0 + 4 * tid;
            float b4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
            if (bias != nullptr && f < N) load4_bias(bias, f, b4);
            *reinterpret_cast<f32x4*>(&bias_s[buf][4 * tid]) = f32x4{b4[0], b4[1], b4[2], b4[3]};
        }
    };
    stage_bias(0, tf * BF);

    // K steps per tile, padded to a multiple of the stage count so that step s of every
    // tile uses stage s mod STAGES (the padding steps read zeros). At least one step.
    const int KT = K > 0 ? (K + BK - 1) / BK : 1;
    const int KTp = (KT + STAGES - 1) / STAGES * STAGES;

    // prologue: the first STAGES-1 steps of the first tile
    pp.template issue<0>(voff_cur, 0, K, zeros);
    pp.template issue<1>(voff_cur, 1, K, zeros);
    if constexpr (STAGES > 3) pp.template issue<2>(voff_cur, 2, K, zeros);
    if constexpr (STAGES > 4) pp.template issue<3>(voff_cur, 3, K, zeros);
    static_assert(STAGES <= 5, "prologue");

    // epilogue constants
    const int hl = lane >> 5;
    __bf16* __restrict__ const out_ff = static_cast<__bf16*>(p.ff);
    __bf16* __restrict__ const out_q = static_cast<__bf16*>(p.q);
    __bf16* __restrict__ const out_k = static_cast<__bf16*>(p.k);
    __bf16* __restrict__ const out_v = static_cast<__bf16*>(p.v);
    const float* __restrict__ const rope_cos = p.rope_cos;
    const float* __restrict__ const rope_sin = p.rope_sin;
    const int ff_dim = p.ff_dim, qw = p.qw, hd = p.head_dim, n_heads = p.n_heads, act = p.act;
    const int64_t head_stride = (int64_t)S * hd;   // elements between heads of one slab

    for (int k_tile = 0;; ++k_tile) {
        const int m0 = tt * BT, n0 = tf * BF;
        int ntt = 0, ntf = 0;
        const bool has_next = block_tile(k_tile + 1, p.tiles_m, p.tiles_n, p.group_m, ntt, ntf);
        if (has_next)
            tile_offsets<C, X_TL, W_FC>(voff_nxt, pp.kofs, ntt * BT, ntf * BF, wave, lane, K, N, M, S, p.x_sb,
                                        p.x_ss, p.x_sc);

        f32x16 acc[TI][TJ];
#pragma unroll
        for (int i = 0; i < TI; ++i)
#pragma unroll
            for (int j = 0; j < TJ; ++j) acc[i][j] = f32x16{};

        // One K step: wait for this wave's loads of the step (the loads of up to STAGES-2
        // later steps may stay in flight), barrier (every wave's loads landed; every wave is
        // done with the stage about to be refilled), refill it STAGES-1 steps ahead --
        // from the next tile once this one runs out -- then compute.
        auto k_step = [&](auto stc, int kt) __attribute__((always_inline)) {
            constexpr int ST = decltype(stc)::value;
            const int later = (KTp - 1 - kt) + (has_next ? KTp : 0);  // steps after kt still to run
            if (later >= STAGES - 2) wait_vmcnt<(STAGES - 2) * NLOAD>();
            else if (STAGES > 3 && later == 1) wait_vmcnt<NLOAD>();
            else wait_vmcnt<0>();
            __syncthreads();
            const int s_next = kt + STAGES - 1;
            constexpr int SN = (ST + STAGES - 1) % STAGES;
            if (s_next < KTp) pp.template issue<SN>(voff_cur, s_next, K, zeros);
            else if (has_next) pp.template issue<SN>(voff_nxt, s_next - KTp, K, zeros);
            pp.template compute<ST>(acc);
        };
        for (int kt = 0; kt < KTp; kt += STAGES) {
            k_step(std::integral_constant<int, 0>{}, kt);
            k_step(std::integral_constant<int, 1>{}, kt + 1);
            k_step(std::integral_constant<int, 2>{}, kt + 2);
            if constexpr (STAGES > 3) k_step(std::integral_constant<int, 3>{}, kt + 3);
            if constexpr (STAGES > 4) k_step(std::integral_constant<int, 4>{}, kt + 4);
        }

        // ---- epilogue in registers. acc[i][j][e]: column f = 32i + 8(e/4) + 4(lane/32) +
        // e%4, token 32j + lane%32 (both relative to the wave tile). Outputs never overlap
        // the inputs (checked on the host), so loads may be hoisted above stores.
        const float* const bias_t = bias_s[k_tile & 1];
#pragma unroll
        for (int j = 0; j < TJ; ++j) {
            const int t = m0 + wt * WT + 32 * j + (lane & 31);
            const bool tv = t < M;
            const int bi = t / S, s = t - bi * S;
            __bf16* const ff_row = out_ff + (int64_t)t * ff_dim;
            const int64_t tok = (int64_t)bi * n_heads * head_stride + (int64_t)s * hd;   // head 0 of this token
            const float* const cs_row = rope_cos + (int64_t)s * (DG * 8);
            const float* const sn_row = rope_sin + (int64_t)s * (DG * 8);
#pragma unroll
            for (int G = 0; G < NG; ++G) {
                const int f8 = n0 + wf * WF + 8 * G;  // wave-uniform column group
                if (f8 >= N) continue;
                const int fl = wf * WF + 8 * G + 4 * hl;   // this lane's first column inside the tile
                float y[4];
                const f32x4 bv = *reinterpret_cast<const f32x4*>(bias_t + fl);
#pragma unroll
                for (int u = 0; u < 4; ++u) y[u] = acc[G >> 2][j][4 * (G & 3) + u] + bv[u];
                if (f8 < ff_dim) {
                    if (act == 1) {
#pragma unroll
                        for (int u = 0; u < 4; ++u) y[u] = gelu_erf_fast(y[u]);
                    }
                    if (tv) store4_bf16(ff_row + n0 + fl, y);
                    continue;
                }
                const int r = f8 - ff_dim;
                const int which = r / qw;
                const int rem = r - which * qw;
                const int h = rem / hd;
                __bf16* const dst = (which == 0 ? out_q : which == 1 ? out_k : out_v) + tok + h * head_stride;
                if (DG > 0 && which < 2) {
                    // Heads start on head_dim boundaries of this wave's columns, so the
                    // group's place inside its head is a compile-time constant. A
                    // first-half group is computed together with its partner DG groups on;
                    // the partner's own iteration skips.
                    constexpr int HD = DG > 0 ? 16 * DG : 16, HALF = HD / 2;
                    const int jh8 = (8 * G) % HD;
                    if (jh8 >= HALF || G + DG >= NG) continue;
                    const int G2 = (G + DG < NG) ? G + DG : G;  // constant after unrolling
                    const int jh = jh8 + 4 * hl;
                    float y2[4];
                    const f32x4 b2 = *reinterpret_cast<const f32x4*>(bias_t + fl + HALF);
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
                        store4_bf16(dst + jh + HALF, o2);
                    }
                    continue;
                }
                const int jh = rem - h * hd + 4 * hl;
                if (tv) store4_bf16(dst + jh, y);
            }
        }
        if (!has_next) break;
        // the next tile's bias goes to the other buffer (last read two tiles ago)
        stage_bias((k_tile + 1) & 1, ntf * BF);
#pragma unroll
        for (int q = 0; q < NLOAD; ++q) voff_cur[q] = voff_nxt[q];
        tt = ntt;
        tf = ntf;
    }
}

// Tile shapes compiled for the fast kernel.
constexpr int kBF = 256, kBT = 256, kNWF = 2, kNWT = 4, kBK = 32, kStages = 4;

template <bool X_TL, bool W_FC, int DG>
hipError_t launch_fast_one(const KernelArgs& a, int grid, hipStream_t stream) {
    hipLaunchKernelGGL((fused_proj_fast_kernel<X_TL, W_FC, kBF, kBT, kNWF, kNWT, kBK, kStages, DG>), dim3(grid),
                       dim3(64 * kNWF * kNWT), 0, stream, a);
    return hipGetLastError();
}

template <int DG>
hipError_t dispatch_fast_layouts(bool x_tl, bool w_fc, const KernelArgs& a, int grid, hipStream_t s) {
    if (x_tl) return w_fc ? launch_fast_one<true, true, DG>(a, grid, s) : launch_fast_one<true, false, DG>(a, grid, s);
    return w_fc ? launch_fast_one<false, true, DG>(a, grid, s) : launch_fast_one<false, false, DG>(a, grid, s);
}

}  // namespace

int fast_rope_groups(int head_dim, bool rope) {
    if (!rope) return 0;
    const int dg = head_dim / 16;
    return (head_dim % 16 == 0 && (dg == 2 || dg == 4 || dg == 8)) ? dg : -1;
}

TilePlan fast_plan(int64_t M, int64_t F, int num_cus) {
    TilePlan t{kBT, kBF, kBK, 8, 0};
    const int64_t tiles = ((M + kBT - 1) / kBT) * ((F + kBF - 1) / kBF);
    int64_t grid = num_cus > 0 ? num_cus : 256;           // one persistent workgroup per CU
    if (grid > tiles) grid = tiles;
    t.grid = (int)((grid + 7) / 8 * 8);                   // a multiple of the 8 XCDs
    return t;
}

hipError_t launch_fused_proj_fast(bool x_tokens_last, bool w_fc, int dg, const TilePlan& pl, const KernelArgs& a,
                                  hipStream_t stream) {
    if (pl.bm != kBT || pl.bn != kBF || pl.bk != kBK || pl.grid <= 0 || pl.grid % 8) return hipErrorInvalidValue;
    switch (dg) {
        case 0: return dispatch_fast_layouts<0>(x_tokens_last, w_fc, a, pl.grid, stream);
        case 2: return dispatch_fast_layouts<2>(x_tokens_last, w_fc, a, pl.grid, stream);
        case 4: return dispatch_fast_layouts<4>(x_tokens_last, w_fc, a, pl.grid, stream);
        case 8: return dispatch_fast_layouts<8>(x_tokens_last, w_fc, a, pl.grid, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace fp
