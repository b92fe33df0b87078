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
//   - stores into ff [b,S,ff] and the head-major q/k/v buffers [b*H,S,hd]
//     (memory-efficient-attention issue "Improve performance via batched-matmul
//     and fused multiplies"), with consecutive tokens adjacent in q/k/v,
//     restaged through LDS into whole 256-byte token rows.
// Every branch of the compute part of the epilogue depends only on the column
// group, which is the same for the whole wave, so it never diverges.
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
// Schedule. Two tile shapes (see LargeTile / SmallTile below). Large: 256 x 256
// tiles, 8 waves of 128 (f) x 64 (token) outputs, two per SIMD, one persistent
// workgroup per CU walking a list of tiles from a contiguous, grouped range of the
// XCD it runs on; the direct-load pipeline runs three K steps of 32 ahead through four
// stages, straight on into the next tile. Small (problems with fewer large tiles than
// CUs): 128 x 128 tiles, 4 waves of 128 x 32, one tile per workgroup, two workgroups per
// CU, loads four K steps ahead through five stages. Either way the operands of the next
// K step are read from LDS while the MFMAs of the current one run.
#include "device_common.h"
#include "fused_proj_kernels.h"

namespace fp {
namespace {

using namespace dev;

// Wait states that every inline-asm memory instruction below starts with. The compiler
// inserts the wait states its own instructions need, but it cannot see inside inline
// asm: right before one it may restore a spilled SGPR with v_readlane (a VALU write of
// an SGPR) or set M0 with an SALU move. On gfx9-family chips a VMEM instruction that
// reads an SGPR written by VALU needs 5 wait states first (the compiler itself puts
// s_nop 4 there for its own loads), and an LDS-DMA load needs 1 after an SALU write of
// M0. Without them the load can use a stale base address.
#define HAZARD_NOPS "s_nop 4\n\t"

// s_waitcnt vmcnt(N): at most N of this wave's vector memory operations outstanding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Four fp32 values rounded to bf16, as 8 bytes.
__device__ __forceinline__ u32x2 pack4_bf16(const float* o) {
    bf16x4 v;
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = (__bf16)o[u];
    return __builtin_bit_cast(u32x2, v);
}
// Four bf16 bias values from LDS, as fp32.
__device__ __forceinline__ f32x4 bias4(const __bf16* p) {
    const bf16x4 v = __builtin_bit_cast(bf16x4, *reinterpret_cast<const u32x2*>(p));
    return f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
}

// Sixteen consecutive dwords of read-only memory at a wave-uniform address, through the
// scalar unit. A vector load here would make the compiler wait (vmcnt) for every older
// vector memory operation, including the direct-to-LDS loads of the next tile in flight;
// the scalar load has its own counter, waited for right away.
// The address is passed through readfirstlane so that it is in SGPRs even where the
// compiler cannot prove it uniform (it is uniform by construction). readfirstlane returns
// int: each half goes through uint32_t before widening, else the low half would be
// sign-extended into the high one.
__device__ __forceinline__ u32x16 scalar_load16(const unsigned* p) {
    const uint64_t a = reinterpret_cast<uint64_t>(p);
    const uint64_t ua = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((unsigned)(a >> 32)) << 32) |
                        (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((unsigned)a);
    u32x16 v;
    asm volatile(HAZARD_NOPS "s_load_dwordx16 %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)"
                 : "=s"(v)
                 : "s"(reinterpret_cast<const unsigned*>(ua)));
    return v;
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
template <bool X_TL, bool W_FC, int BF, int BT, int NWF, int NWT, int BK, int STAGES, int PAD>
struct FastCfg {
    static constexpr int NW = NWF * NWT, THREADS = 64 * NW;
    static constexpr int WF = BF / NWF, WT = BT / NWT;   // wave tile
    static constexpr int TI = WF / 32, TJ = WT / 32;
    static constexpr int NG = TI * 4;                    // 8-column groups per wave
    static constexpr int KK = BK / 16;                   // MFMA k steps per K step
    static constexpr int W_BYTES = BF * BK * 2, X_BYTES = BT * BK * 2;
    // W stages, PAD spare bytes, X stages, PAD spare bytes
    static constexpr int X_REGION = STAGES * W_BYTES + PAD;
    static constexpr int LDS_BYTES = STAGES * (W_BYTES + X_BYTES) + 2 * PAD;
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
// KUNITS: the tile's K steps start at step kb of the operands (a range of the contraction,
// for contractions split over workgroups); SLABK: x's K steps cross slabs (a contraction
// over the tokens of a channels-first x), each K step lying in one slab.
template <class C, bool X_TL, bool W_FC, int BK, bool TAILK, bool KUNITS = false, bool SLABK = false>
struct FastPipe {
    unsigned wbase[C::TI][W_FC ? C::KK : 1];   // LDS read bases of the W^T operands
    unsigned xbase[C::TJ][X_TL ? C::KK : 1];   // and of the x operands
    int kofs[C::NLOAD];                        // k offset of each direct-load chunk in its K step
    unsigned lds0;
    int wave;
    const char* wsrc;                          // W and x byte addresses of K step 0
    const char* xsrc;
    int64_t wstep, xstep;                      // bytes per K step
    int ksps = 1;                              // SLABK: K steps per slab of x
    FastDivU31 div_ksps{};                     // SLABK: division by ksps
    int64_t slab_bytes = 0;                    // SLABK: bytes between slabs of x

    // Issue the direct loads of K step ks (of the tile whose chunk offsets are voff) into
    // stage ST. Chunks at or past K (a ragged last step, or the steps that pad the step
    // count to a multiple of the stage count) are read from the zero block; without
    // TAILK every step is whole.
    template <int ST>
    __device__ __forceinline__ void issue(const unsigned (&voff)[C::NLOAD], int ks, int K,
                                          const char* zeros, int kb = 0) const {
        const int ka = KUNITS ? kb + ks : ks;   // the step in the operands
        const char* ws = wsrc + (int64_t)ka * wstep;
        const char* xs;
        if constexpr (SLABK) {
            const int sl = (int)fastdiv_u31((uint32_t)ka, div_ksps);
            xs = xsrc + (int64_t)sl * slab_bytes + (int64_t)(ka - sl * ksps) * xstep;
        } else {
            xs = xsrc + (int64_t)ka * xstep;
        }
        const bool tail = TAILK && (ks + 1) * BK > K;
        auto dst_of = [&](int q) __attribute__((always_inline)) {
            return lds0 + (q < C::W_INSTR ? ST * C::W_BYTES + (wave * C::W_INSTR + q) * 1024
                                          : C::X_REGION + ST * C::X_BYTES +
                                                (wave * C::X_INSTR + (q - C::W_INSTR)) * 1024);
        };
        // one branch around all of the step's loads (one per load, as the compiler would
        // otherwise lay it out, costs a K step of the small tiles about a tenth)
        if (!tail) {
#pragma unroll
            for (int q = 0; q < C::NLOAD; ++q) {
                // SGPR base + 32-bit lane offset: no per-load VALU. Inline asm keeps the
                // compiler from waiting on every stage in flight before each LDS read.
                asm volatile(HAZARD_NOPS "global_load_lds_dwordx4 %0, %1" ::"v"(voff[q]),
                             "s"(q < C::W_INSTR ? ws : xs), "{m0}"(dst_of(q))
                             : "memory");
            }
        } else {
#pragma unroll
            for (int q = 0; q < C::NLOAD; ++q) {
                const char* a = (ks * BK + kofs[q] < K) ? (q < C::W_INSTR ? ws : xs) + voff[q] : zeros;
                asm volatile(HAZARD_NOPS "global_load_lds_dwordx4 %0, off" ::"v"(a), "{m0}"(dst_of(q)) : "memory");
            }
        }
    }

    // MFMA operands of one 16-deep k step: TI W^T row blocks and TJ token blocks.
    struct Ops {
        bf16x8 a[C::TI];
        bf16x8 b[C::TJ];
    };

    // LDS reads of k step KK of stage ST.
    template <int ST, int KK>
    __device__ __forceinline__ Ops read() const {
        Ops o;
#pragma unroll
        for (int i = 0; i < C::TI; ++i) {
            if constexpr (W_FC) {
                o.a[i] = __builtin_bit_cast(bf16x8, lds_b128(wbase[i][KK] + ST * C::W_BYTES));
            } else {
                const unsigned a = wbase[i][0] + ST * C::W_BYTES + KK * 16 * C::W_CPR * 16;
                o.a[i] = join_tr(lds_tr16(a), lds_tr16(a + 4 * C::W_CPR * 16));
            }
        }
#pragma unroll
        for (int j = 0; j < C::TJ; ++j) {
            if constexpr (X_TL) {
                o.b[j] = __builtin_bit_cast(bf16x8, lds_b128(xbase[j][KK] + ST * C::X_BYTES));
            } else {
                const unsigned a = xbase[j][0] + ST * C::X_BYTES + KK * 16 * C::X_CPR * 16;
                o.b[j] = join_tr(lds_tr16(a), lds_tr16(a + 4 * C::X_CPR * 16));
            }
        }
        return o;
    }

    static __device__ __forceinline__ void mma(f32x16 (&acc)[C::TI][C::TJ], const Ops& o) {
#pragma unroll
        for (int i = 0; i < C::TI; ++i)
#pragma unroll
            for (int j = 0; j < C::TJ; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(o.a[i], o.b[j], acc[i][j], 0, 0, 0);
    }
};

// Byte offset of each lane's direct-load chunks for the tile at (m0, n0). Lane l of
// instruction q fills physical LDS chunk (wave*INSTR + q)*64 + l, so choosing the
// source chunk through the inverse swizzle makes the LDS image come out swizzled.
// Rows past N and tokens past M read row / token 0 instead (in bounds, never stored).
template <class C, bool X_TL, bool W_FC>
__device__ __forceinline__ void tile_offsets(unsigned (&voff)[C::NLOAD], int (&kofs)[C::NLOAD], int m0, int n0,
                                             int wave, int lane, int K, int N, int M, int S, FastDivU31 ds,
                                             int64_t sb, int64_t ss, int64_t sc, int wld) {
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
            off = (int64_t)(n < N ? n : 0) * wld + krow;
        } else {
            const int c = pc ^ ((row & 3) << 2);
            const int n = n0 + c * 8;
            krow = row;
            off = (int64_t)krow * wld + (n < N ? n : 0);
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
        const int bi = (int)fastdiv_u31((uint32_t)mm, ds), s = mm - bi * S;
        const int64_t off = (int64_t)bi * sb + (int64_t)s * ss + (int64_t)krow * sc;
        voff[C::W_INSTR + q] = (unsigned)(off * 2);
        kofs[C::W_INSTR + q] = krow;
    }
}

// k-th tile of this workgroup. The tiles of the grid's linear order are split into 8
// contiguous ranges, one per XCD (workgroup b runs on XCD b mod 8); inside its range a
// workgroup takes every (workgroups per XCD)-th tile. Linear order: groups of group_m
// token tiles sweep the column tiles together.
// Wave-uniform; the division by the group size is a host-computed multiply-high, and the
// groups of group_m token tiles (a power of two except possibly the last group) are
// walked with shifts.
__device__ __forceinline__ bool block_tile(int k, const KernelArgs& p, int& tt, int& tf) {
    const int tiles_t = p.tiles_m, tiles_f = p.tiles_n, group_m = p.group_m;
    const int total = tiles_t * tiles_f;
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3, per_xcd = gridDim.x >> 3;
    const int q = total >> 3, r = total & 7;
    const int count = q + (xcd < r ? 1 : 0);
    const int li = slot + k * per_xcd;
    if (li >= count) return false;
    const int lin = xcd * q + (xcd < r ? xcd : r) + li;
    const int per_group = group_m * tiles_f;
    const int grp = (int)fastdiv_u31((uint32_t)lin, p.div_group);
    const int first = grp * group_m;
    const int gsz = (tiles_t - first) < group_m ? (tiles_t - first) : group_m;
    const int in = lin - grp * per_group;
    if ((gsz & (gsz - 1)) == 0) {
        const int sh = __builtin_ctz((unsigned)gsz);
        tt = first + (in & (gsz - 1));
        tf = in >> sh;
    } else {
        tt = first + in % gsz;
        tf = in / gsz;
    }
    return true;
}

// Tile shapes compiled for the fast kernel, BF output columns x BT tokens per workgroup
// with NWF x NWT waves (WPE per SIMD); K steps of BK through STAGES LDS stages for both,
// loads issued PF K steps ahead.
//  - large: 256 x 256 by 2 x 4 waves of 128 x 64, one workgroup per CU (130 KB of LDS).
//    The loads run three K steps ahead, which three stages carry; the fourth is idle at the
//    end of a tile, where the epilogue restages its stores, and the tile bias is
//    double-buffered after the stages.
//  - small: 128 x 128 by 1 x 4 waves of 128 x 32, two workgroups per CU, for problems with
//    fewer large tiles than CUs (short K, few tokens): four times the tiles. SINGLE: every
//    workgroup gets at most one tile (the host launches one per tile), so the K steps are
//    not padded to a multiple of the stage count and no loads run ahead into a next tile.
//    Such problems are bound by load latency rather than by the MFMAs, so the loads run
//    four K steps ahead through five stages: 80 KB, exactly half the CU's LDS. The bias and
//    the restaged stores live inside the stage area (a stage no load has reached yet, and
//    the idle stages after the last K step).
struct LargeTile {
    static constexpr int BF = 256, BT = 256, NWF = 2, NWT = 4, PER_CU = 1, STAGES = 4, PF = 3, WPE = 2;
    static constexpr bool SINGLE = false;
};
struct SmallTile {
    static constexpr int BF = 128, BT = 128, NWF = 1, NWT = 4, PER_CU = 2, STAGES = 5, PF = 4, WPE = 2;
    static constexpr bool SINGLE = true;
};

constexpr int kBK = 32;
// Restaged epilogue rows: 16 tokens x (128 bf16 columns + 16 bytes of padding).
constexpr int kRestageRows = 16, kRestageRow = 272;
// Channels-first ff restage: 32 token rows of 64 columns (8 bytes of padding per row).
constexpr int kCfRow = 136;
static_assert(32 * kCfRow <= kRestageRows * kRestageRow, "channels-first restage fits the wave's rows");
// Epilogue variants: exact-erf GELU or none with token-major stores; tanh GELU or squared
// ReLU (no RoPE); a channels-first ff output (no RoPE).
constexpr int kEpiDefault = 0, kEpiOtherAct = 1, kEpiFfChannelsFirst = 2;
// As the default, with RoPE on the first 8 columns of each q/k head only (partial rotary):
// a rotated group's pairs lie 4 columns apart, in the two half-waves, and the descriptor's
// bit 29 marks the group.
constexpr int kEpiRope8 = 3;
// Contractions split into ranges: tiles are (row tile, K range) units, each storing its fp32
// partial sums [range][M][N] straight from the accumulators (no activation, bias, RoPE or
// restage). The weight gradient (dW = X^T dy over token ranges, rows are channels), and the
// input gradient's last token tiles (dx = dy W^T over ranges of the fused columns).
constexpr int kEpiDwPartial = 4;
// The weight gradient in one token range: the same units' pipeline, stored straight into
// dW in bf16 by the restaged token-major store ([C, F] rows; no activation) or by the
// channels-first store ([F, C]: column f's channels as one run).
constexpr int kEpiDwRows = 6, kEpiDwCols = 7;
// The backward pass's dy over the ff columns: the forward product y recomputed, then
// dy = d_ff * act'(y) (d_ff token-major, read 8 bytes per lane and group) stored token-major
// with row stride ff_ld (no RoPE).
constexpr int kEpiGrad = 5;

// X_TL: x token-major [b,s,c] (else channels-first). W_FC: W [F,C] (else [C,F]).
// DG: RoPE partner distance in 8-column groups (hd/16), 0 = no RoPE. TAILK: K is not a
// multiple of T::STAGES * BK (some K steps are partial or padding).
template <bool X_TL, bool W_FC, int DG, bool TAILK, class T, int EPI>
__global__ __launch_bounds__(64 * T::NWF * T::NWT, T::PER_CU) __attribute__((amdgpu_waves_per_eu(T::WPE, T::WPE))) void
fused_proj_fast_kernel(KernelArgs p) {
    constexpr int BF = T::BF, BT = T::BT, BK = kBK, STAGES = T::STAGES, PF = T::PF, kNWT = T::NWT;
    // restaged epilogues: each wave owns kRestageRows rows of kRestageRow bytes -- with a next
    // tile in flight, in the idle last stage and the spare bytes after it; single-tile
    // workgroups anywhere in the (then idle) stage area
    constexpr int RGN_ALL = T::NWF * T::NWT / 2 * kRestageRows * kRestageRow, W_STAGE = BF * kBK * 2;
    constexpr int PAD = !T::SINGLE && RGN_ALL > W_STAGE ? RGN_ALL - W_STAGE : 0;
    using C = FastCfg<X_TL, W_FC, BF, BT, T::NWF, kNWT, BK, STAGES, PAD>;
    // range units (the weight gradient's, dx's last tiles): their pipeline, and whether the
    // epilogue stores fp32 partial sums
    constexpr bool DW = EPI == kEpiDwPartial || EPI == kEpiDwRows || EPI == kEpiDwCols;
    constexpr bool DWP = EPI == kEpiDwPartial;
    // the channels-first ff store
    constexpr bool CF_STORE = EPI == kEpiFfChannelsFirst || EPI == kEpiDwCols;
    using Pipe = FastPipe<C, X_TL, W_FC, BK, TAILK, DW, DW && X_TL>;
    using Ops = typename Pipe::Ops;
    constexpr int WF = C::WF, WT = C::WT, TI = C::TI, TJ = C::TJ, NG = C::NG, NLOAD = C::NLOAD;
    static_assert(C::KK == 2, "two MFMA k steps per K step");
    static_assert(T::SINGLE || (PF == 3 && (STAGES == 3 || STAGES == 4)),
                  "the multi-tile wait counts below are written for three steps ahead");
    static_assert(!T::SINGLE || (PF >= 2 && PF <= 5 && STAGES == PF + 1), "single-tile pipeline depth");
    static_assert(T::SINGLE || STAGES == 4, "the restaged epilogue uses the idle fourth stage");
    static_assert(!T::SINGLE || C::NW * kRestageRows * kRestageRow <= C::LDS_BYTES, "single-tile restage rows");
    static_assert(NG == 16, "one 16-entry column descriptor load per wave");
    // LDS: the stages, then (multi-tile workgroups) the tile bias, double-buffered. A
    // single-tile workgroup keeps its bias in stage PF, which no load reaches before the
    // first K step's barrier, after which the bias has been read.
    constexpr int BIAS_OFS = T::SINGLE ? PF * C::W_BYTES : C::LDS_BYTES;
    __shared__ __attribute__((aligned(1024))) unsigned char smem[C::LDS_BYTES + (T::SINGLE ? 0 : 2 * BF * 2)];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wf = wave / kNWT, wt = wave % kNWT;
    const int K = p.K, N = p.N, M = (int)p.M, S = p.S;
    const char* const zeros = static_cast<const char*>(p.zeros);
    const __bf16* const bias = static_cast<const __bf16*>(p.bias);

    int tt, tf;
    if (!block_tile(0, p, tt, tf)) return;

    Pipe pp;
    pp.wave = wave;
    pp.lds0 = (unsigned)(size_t)(lds_void*)smem;
    // LDS read bases: K-major operands need one per MFMA k step (the swizzle depends on
    // the chunk), M/N-major ones a single one (the k step goes into the immediate offset).
#pragma unroll
    for (int i = 0; i < TI; ++i) {
        if constexpr (W_FC) {
#pragma unroll
            for (int kk = 0; kk < C::KK; ++kk)
                pp.wbase[i][kk] = pp.lds0 + k_operand_base<C::W_CPR>(wf * WF + 32 * i, kk, lane);
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
    // W's row stride: [K, N] rows are N long except for the grad epilogue's product, which
    // reads the ff columns of a wider [C, F] weight; [N, K] rows are K long except for
    // contraction ranges (the input gradient's range units), which cover part of each row
    const int wld = W_FC ? (DW ? p.w_ld : K) : EPI == kEpiGrad ? p.w_ld : N;
    pp.wstep = (W_FC ? (int64_t)BK : (int64_t)BK * wld) * 2;
    pp.xstep = (X_TL ? (int64_t)BK : (int64_t)BK * p.x_sc) * 2;
    if constexpr (DW && X_TL) {
        pp.ksps = p.k_slab_steps;
        pp.div_ksps = p.div_kslab;
        pp.slab_bytes = p.x_sb * 2;
    }
    // a unit of the weight gradient: row tile and token range of "tile row" tt
    auto unit_of = [&](int t, int& trow, int& kb) __attribute__((always_inline)) {
        if constexpr (DW) {
            const int z = (int)fastdiv_u31((uint32_t)t, p.div_dwt);
            trow = t - z * p.dw_tiles_t;
            kb = z * (K / BK);   // the token range is K long, a whole number of K steps
        } else {
            trow = t;
            kb = 0;
        }
    };

    // The bias slice of a tile, copied into bias buffer buf by the first wave's first lanes
    // with the same direct-to-LDS loads as the operands (from the zero block where there
    // is no bias). It is issued right after the tile's step 0, so the waits and barriers
    // that make step 0 visible also cover it.
    const unsigned bias_lds = (unsigned)(size_t)(lds_void*)(smem + BIAS_OFS);
    auto issue_bias = [&](int buf, int n0) __attribute__((always_inline)) {
        if (wave == 0 && lane < BF / 8) {
            const int f = n0 + 8 * lane;
            const char* src = (bias != nullptr && f < N) ? reinterpret_cast<const char*>(bias + f) : zeros;
            const unsigned dst = bias_lds + (unsigned)buf * (BF * 2);
            asm volatile(HAZARD_NOPS "global_load_lds_dwordx4 %0, off" ::"v"(src), "{m0}"(dst) : "memory");
        }
    };

    // K steps per tile, padded to a multiple of the stage count so that step s of every
    // tile uses stage s mod STAGES (the padding steps read zeros). At least one group.
    // Single-tile workgroups run just the K steps there are.
    const int KT = K > 0 ? (K + BK - 1) / BK : 1;
    const int KTp = T::SINGLE ? KT : (KT + STAGES - 1) / STAGES * STAGES;

    // epilogue constants
    const int hl = lane >> 5;
    const float* __restrict__ const rope_cos = p.rope_cos;
    const float* __restrict__ const rope_sin = p.rope_sin;
    const int ff_dim = p.ff_dim, hd = p.head_dim, act = p.act;
    const int ffr = EPI == kEpiGrad ? p.ff_ld : ff_dim;   // row stride of the ff output
    // q/k/v elements of one slab (all heads of the slice): q, and k or v
    const int64_t slab_q = (int64_t)S * p.qw, slab_kv = (int64_t)S * p.n_kv_heads * hd;
    constexpr bool R8 = EPI == kEpiRope8;
    // epilogues whose every wave issues exactly TJ * 8 stores per tile (the restaged ones)
    constexpr bool RELAX = EPI == kEpiDefault || EPI == kEpiOtherAct || EPI == kEpiRope8 || EPI == kEpiDwRows;

    unsigned voff_cur[NLOAD], voff_nxt[NLOAD];
    int trow_cur, kb_cur;
    unit_of(tt, trow_cur, kb_cur);
    tile_offsets<C, X_TL, W_FC>(voff_cur, pp.kofs, trow_cur * BT, tf * BF, wave, lane, K, N, M, S, p.div_s, p.x_sb,
                                p.x_ss, p.x_sc, wld);
    // Wait until this wave's loads of all but the `later` most recently issued K steps have
    // landed (the vector memory counter counts in issue order).
    auto wait_steps = [&](int later) __attribute__((always_inline)) {
        static_assert(PF - 1 <= 3, "wait counts cover up to three later steps");
        if (later >= 3) wait_vmcnt<3 * NLOAD>();
        else if (later == 2) wait_vmcnt<2 * NLOAD>();
        else if (later == 1) wait_vmcnt<NLOAD>();
        else wait_vmcnt<0>();
    };
    // Prologue: the first PF K steps of the first tile and its bias in flight; once step 0
    // has landed (the later ones may still be in flight), read its operands. Single-tile
    // workgroups issue only the steps that exist, so that no load is in flight after the
    // last K step (their epilogue reuses the whole stage area) -- except in the ragged-K
    // form (UNIFORM), where a step past the last one reads the zero block like any chunk
    // past K: every K step then has the same code and waits (no branches on the step), and
    // the epilogue first waits for all loads. (On a whole-K shape the extra loads and that
    // wait cost more than the branches: small-K 11.3 against 11.0 us; grouped-query 10.3
    // against 10.65.)
    constexpr bool UNIFORM = T::SINGLE && TAILK;
    const bool exists1 = !T::SINGLE || UNIFORM || 1 < KTp, exists2 = !T::SINGLE || UNIFORM || 2 < KTp;
    const bool exists3 = !T::SINGLE || UNIFORM || 3 < KTp, exists4 = !T::SINGLE || UNIFORM || 4 < KTp;
    pp.template issue<0>(voff_cur, 0, K, zeros, kb_cur);
    issue_bias(0, tf * BF);
    if (exists1) pp.template issue<1>(voff_cur, 1, K, zeros, kb_cur);
    if (exists2) pp.template issue<2>(voff_cur, 2, K, zeros, kb_cur);
    if constexpr (PF >= 4) if (exists3) pp.template issue<3>(voff_cur, 3, K, zeros, kb_cur);
    if constexpr (PF >= 5) if (exists4) pp.template issue<4>(voff_cur, 4, K, zeros, kb_cur);
    wait_steps(T::SINGLE && !UNIFORM ? min(PF - 1, KTp - 1) : PF - 1);
    __syncthreads();
    Ops c0 = pp.template read<0, 0>();
    Ops c1 = pp.template read<0, 1>();

    for (int k_tile = 0;; ++k_tile) {
        const int m0 = trow_cur * BT, n0 = tf * BF;
        int ntt = 0, ntf = 0, trow_nxt = 0, kb_nxt = kb_cur;
        const bool has_next = block_tile(k_tile + 1, p, ntt, ntf);
        if (has_next) {
            unit_of(ntt, trow_nxt, kb_nxt);
            tile_offsets<C, X_TL, W_FC>(voff_nxt, pp.kofs, trow_nxt * BT, ntf * BF, wave, lane, K, N, M, S, p.div_s,
                                        p.x_sb, p.x_ss, p.x_sc, wld);
        } else {
            // past the last tile the loads repeat this tile's first steps (in bounds, never
            // read), which keeps the K loop free of branches
            ntf = tf;
#pragma unroll
            for (int q = 0; q < NLOAD; ++q) voff_nxt[q] = voff_cur[q];
        }

        // The accumulators start from the bias (in LDS since the last barrier): acc[a][j][e]
        // holds column 32a + 8(e/4) + 4(lane/32) + e%4 of the wave tile.
        const __bf16* const bias_t =
            reinterpret_cast<const __bf16*>(smem + BIAS_OFS) + (k_tile & 1) * BF + wf * WF + 4 * hl;
        f32x16 acc[TI][TJ];
#pragma unroll
        for (int a = 0; a < TI; ++a) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const f32x4 b = bias4(bias_t + 32 * a + 8 * q);
#pragma unroll
                for (int j = 0; j < TJ; ++j)
#pragma unroll
                    for (int u = 0; u < 4; ++u) acc[a][j][4 * q + u] = b[u];
            }
        }

        // One K step kt, whose operands c0/c1 (its two MFMA k steps) are already in
        // registers: wait for this wave's loads of step kt+1 (those of kt+2 may stay in
        // flight), barrier (every wave's loads of kt+1 landed; every wave has read the
        // stages of kt and kt-1), fill the stage of kt+3, and read step kt+1's operands
        // while the MFMAs of kt run. Once kt+3 is past the tile the loads are the next
        // tile's first steps (its bias right after its step 0), and the last step reads the
        // next tile's step 0 ahead. Every step has the same code -- no step is peeled -- so
        // the accumulators stay in the accumulation registers. The scheduling fences keep
        // every instruction inside its step (the compiler would otherwise move MFMAs across
        // the barrier and recycle operand registers); inside a step the compiler orders the
        // LDS reads and MFMAs itself (forcing all reads first measured slower).
        auto k_step = [&](auto stc, int kt) __attribute__((always_inline)) {
            constexpr int ST = decltype(stc)::value;
            constexpr int SN = (ST + 1) % STAGES, SL = (ST + PF) % STAGES;
            __builtin_amdgcn_sched_barrier(0);
            const int s_load = kt + PF;
            if constexpr (UNIFORM) {
                // steps issued so far: 0 .. kt+PF-1; those after kt+1 may stay in flight
                wait_steps(PF - 2);
                __syncthreads();
                pp.template issue<SL>(voff_cur, s_load, K, zeros, kb_cur);
            } else if constexpr (T::SINGLE) {
                // steps issued so far: 0 .. kt+PF-1 while they exist (by the prologue and
                // the steps before); those after kt+1 may stay in flight
                wait_steps(min(kt + PF - 1, KTp - 1) - kt - 1);
                __syncthreads();
                if (s_load < KTp) pp.template issue<SL>(voff_cur, s_load, K, zeros, kb_cur);
            } else {
                // After an epilogue of the restaged kind, its TJ * 8 stores follow the loads
                // of the tile's steps 1 and 2: those two steps need not wait for them.
                if (RELAX && kt < 2 && k_tile > 0) wait_vmcnt<NLOAD + TJ * 8>();
                else wait_vmcnt<NLOAD>();
                __syncthreads();
                const bool ahead = s_load >= KTp;   // wave-uniform
                unsigned vo[NLOAD];
#pragma unroll
                for (int q = 0; q < NLOAD; ++q) vo[q] = ahead ? voff_nxt[q] : voff_cur[q];
                pp.template issue<SL>(vo, ahead ? s_load - KTp : s_load, K, zeros, ahead ? kb_nxt : kb_cur);
                if (s_load == KTp) issue_bias((k_tile + 1) & 1, ntf * BF);
            }
            const Ops n0 = pp.template read<SN, 0>();
            Pipe::mma(acc, c0);
            const Ops n1 = pp.template read<SN, 1>();
            Pipe::mma(acc, c1);
            c0 = n0;
            c1 = n1;
            __builtin_amdgcn_sched_barrier(0);
        };
        // (a do-while: KTp >= STAGES, and a loop the compiler thinks may run zero times
        // makes it keep a spilled copy of the initial accumulators for that path)
        int kt = 0;
        if constexpr (T::SINGLE) {
            static_assert(STAGES >= 3 && STAGES <= 6, "the unrolling below covers 3 to 6 stages");
            for (; kt + STAGES <= KTp; kt += STAGES) {
                k_step(std::integral_constant<int, 0>{}, kt);
                k_step(std::integral_constant<int, 1>{}, kt + 1);
                k_step(std::integral_constant<int, 2>{}, kt + 2);
                if constexpr (STAGES >= 4) k_step(std::integral_constant<int, 3 % STAGES>{}, kt + 3);
                if constexpr (STAGES >= 5) k_step(std::integral_constant<int, 4 % STAGES>{}, kt + 4);
                if constexpr (STAGES >= 6) k_step(std::integral_constant<int, 5 % STAGES>{}, kt + 5);
            }
            // the last KTp mod STAGES steps
            if (kt < KTp) k_step(std::integral_constant<int, 0>{}, kt);
            if (kt + 1 < KTp) k_step(std::integral_constant<int, 1>{}, kt + 1);
            if constexpr (STAGES >= 4) if (kt + 2 < KTp) k_step(std::integral_constant<int, 2>{}, kt + 2);
            if constexpr (STAGES >= 5) if (kt + 3 < KTp) k_step(std::integral_constant<int, 3 % STAGES>{}, kt + 3);
            if constexpr (STAGES >= 6) if (kt + 4 < KTp) k_step(std::integral_constant<int, 4 % STAGES>{}, kt + 4);
            if constexpr (UNIFORM) {
                // the loads past the last step, before the epilogue takes over the stage area
                wait_vmcnt<0>();
                __syncthreads();
            }
        } else {
            do {
                k_step(std::integral_constant<int, 0>{}, kt);
                k_step(std::integral_constant<int, 1>{}, kt + 1);
                k_step(std::integral_constant<int, 2>{}, kt + 2);
                if constexpr (STAGES == 4) k_step(std::integral_constant<int, 3>{}, kt + 3);
                kt += STAGES;
            } while (kt < KTp);
        }

        // ---- epilogue. acc[a][j][e] (bias included): column f = 32a + 8(e/4) + 4(lane/32)
        // + e%4, token 32j + lane%32 (both relative to the wave tile). Outputs never overlap
        // the inputs (checked on the host), so loads may be hoisted above stores. GELU on ff
        // columns and RoPE on q/k columns run in registers; the bf16 results of each 32-token
        // block are restaged through LDS into whole 256-byte token rows and stored with
        // non-temporal 16-byte stores (the outputs are written once and not read back here:
        // they should neither evict the operand panels from the XCD's L2 nor sit dirty
        // there for the write-back at the end of the kernel).
        const int tw0 = m0 + wt * WT;   // the wave's first token
        if constexpr (DWP) {
            // fp32 partial sums of this unit in the accumulators' own order, so that every
            // store writes 1 KB contiguous: the unit's BT x BF block [range][row tile]
            // [column tile] is 256-float chunks ((wave * TI + a) * TJ + j) * 4 + q, lane l
            // holding floats 4l..4l+3 = acc[a][j][4q..4q+3] (row 32j + l%32 of the wave tile,
            // columns 32a + 8q + 4(l/32) ..). Rows and columns outside the problem are stored
            // too (the block is whole); the reduction skips them.
            const int z = (int)fastdiv_u31((uint32_t)tt, p.div_dwt);
            float* const blk = static_cast<float*>(p.ff) +
                               (((int64_t)z * p.dw_tiles_t + trow_cur) * p.tiles_n + tf) * (int64_t)(BT * BF);
#pragma unroll
            for (int a = 0; a < TI; ++a) {
#pragma unroll
                for (int j = 0; j < TJ; ++j) {
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int chunk = ((wave * TI + a) * TJ + j) * 4 + q;
                        const f32x4 v = {acc[a][j][4 * q], acc[a][j][4 * q + 1], acc[a][j][4 * q + 2],
                                         acc[a][j][4 * q + 3]};
                        __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(blk + chunk * 256 + lane * 4));
                    }
                }
            }
        } else {
        // The wave's 16 column groups: kind (0 ff, 1 q, 2 k, 3 v) in bits 30-31 and the
        // element offset of the group's first column in the low bits (ff: column; q/k/v:
        // head * S * hd + place in head; bit 29 marks the rotated groups of the 8-column
        // RoPE), all sixteen in one scalar load.
        const int fw = n0 + wf * WF;
        const u32x16 desc = scalar_load16(p.col_desc + (unsigned)fw / 8u);
        constexpr unsigned OFS_MASK = R8 ? 0x1fffffffu : 0x3fffffffu;
        // cos/sin registers: the 4 columns of each first-half group of a head this lane
        // rotates (8-column RoPE: the 4 pairs of the rotated group)
        constexpr int HD = DG > 0 ? 16 * DG : 16, HALF = HD / 2, NR = R8 ? 1 : HALF / 8, NRB = NR > 4 ? 4 : NR;

        // The stores: written straight from the accumulator layout, a store instruction
        // touches 32 token rows with 16 bytes each; restaged, each one writes 4 token rows of
        // 256 contiguous bytes (the wave's 128 columns). The wave owns 16 rows of 272 bytes
        // (a token's 128 bf16 columns and 16 bytes of padding, which keep both the row
        // writes and the 16-byte chunk reads free of bank conflicts) in the stage no K step
        // uses until the next tile's first barrier and the spare bytes after it. Every LDS
        // address is a per-lane base plus a constant.
        static_assert(T::SINGLE ||
                          (C::W_BYTES == C::X_BYTES && C::W_BYTES + PAD >= C::NW / 2 * kRestageRows * kRestageRow),
                      "restage regions");
        constexpr int RGN = kRestageRows * kRestageRow;
        // single-tile workgroups: no load is in flight after the last K step's wait (or the
        // wait after it) and every wave has passed its barrier, so the whole stage area is free
        const unsigned wave_lds = T::SINGLE          ? pp.lds0 + wave * RGN
                                  : wave < C::NW / 2 ? pp.lds0 + (STAGES - 1) * C::W_BYTES + wave * RGN
                                                     : pp.lds0 + C::X_REGION + (STAGES - 1) * C::X_BYTES +
                                                           (wave - C::NW / 2) * RGN;
        // The lane index again, recomputed per tile where the compiler cannot see it: the
        // LDS addresses and column selects below depend only on it, and hoisted out of the
        // tile loop they would hold registers through the K loop (spilled to scratch, whose
        // reload waits for every load in flight).
        int lane_e;
        asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(lane_e));
        // writer: token row lane%16 of a 16-token half block, column half lane/32 of each
        // group; reader: 16-byte chunk (column group) gl of token rows r0 + 4 rr
        const int gl = lane_e & 15, r0 = lane_e >> 4;
        const unsigned wr_lds = wave_lds + (lane_e & 15) * kRestageRow + (lane_e >> 5) * 8;
        const unsigned rd_lds = wave_lds + r0 * kRestageRow + gl * 16;
        // channels-first ff stores: the writer of token row lane%32 and column half lane/32 of
        // each 8-column group; the transposing reader, lane l of 16-lane group g naming row
        // 8g + (l%16)/4 and columns 4(l%4).. of a 4 x 16 block and receiving column l%16 of
        // its 4 rows
        const unsigned cf_wr = wave_lds + (lane_e & 31) * kCfRow + (lane_e >> 5) * 8;
        const unsigned cf_rd = wave_lds + (8 * (lane_e >> 4) + ((lane_e & 15) >> 2)) * kCfRow + (lane_e & 3) * 8;
        // this lane's chunk: its destination buffer and element offset, and the bytes
        // between consecutive tokens there
        unsigned dl = desc[0];
#pragma unroll
        for (int g = 1; g < 16; ++g) dl = gl == g ? desc[g] : dl;
        const unsigned kind_l = dl >> 30;
        char* const base_l = static_cast<char*>(kind_l == 0 ? p.ff : kind_l == 1 ? p.q : kind_l == 2 ? p.k : p.v) +
                             (size_t)(dl & OFS_MASK) * 2;
        const int64_t slab_l = kind_l == 1 ? slab_q : slab_kv;
        const unsigned stride_l = kind_l == 0 ? (unsigned)(2 * ffr) : (unsigned)(2 * hd);
        char* const row0_l = base_l + r0 * stride_l;
        const bool col_ok = fw + 8 * gl < N;
        char* const sink_l = static_cast<char*>(p.sink) + 16 * gl;
        // the wave's tokens usually lie in one slab: then a token's offset is linear in it
        const int bi_first = (int)fastdiv_u31((uint32_t)tw0, p.div_s);
        const bool one_slab =
            (int)fastdiv_u31((uint32_t)(tw0 + WT - 1 < M ? tw0 + WT - 1 : M - 1), p.div_s) == bi_first;
        auto token_off = [&](int t) __attribute__((always_inline)) {
            const int bi = (int)fastdiv_u31((uint32_t)t, p.div_s);
            const int s = t - bi * S;
            return kind_l == 0 ? (unsigned)t * (unsigned)(2 * ffr)
                               : (unsigned)(((int64_t)bi * slab_l + (int64_t)s * hd) * 2);
        };

        // cos/sin of this lane's token at its 4 columns of each first-half group of a head;
        // every head of the wave uses the same ones -- all at once for head sizes up to 64,
        // in two halves for 128 (registers). Those of the next token block are loaded
        // before this block's stores: a load issued after a store would wait for it too
        // (the vector memory counter counts in order). Every wave loads them, rotating or
        // not: loads under a branch leave the compiler unsure which loads are still in
        // flight, and it then waits for this block's stores before the next block's RoPE.
        f32x4 rc[NRB], rsn[NRB];
        auto load_rope = [&](int j, int r0) __attribute__((always_inline)) {
            const int t = tw0 + 32 * j + (lane_e & 31);
            const int tc = t < M ? t : 0;
            const int s = tc - (int)fastdiv_u31((uint32_t)tc, p.div_s) * S;
            // the table holds rd/2 values per token: a lane's 4 start at 4 * (lane / 32) of
            // each group of 8 (8-column RoPE: both half-waves read the token's 4)
            const unsigned rp_off = R8 ? (unsigned)(s * 16) : (unsigned)((s * (DG * 8) + 4 * (lane_e >> 5)) * 4);
            if constexpr (DG > 0 || R8) {
#pragma unroll
                for (int r = 0; r < NRB; ++r) {
                    const char* const c = reinterpret_cast<const char*>(rope_cos + 8 * (r0 + r)) + rp_off;
                    const char* const sn = reinterpret_cast<const char*>(rope_sin + 8 * (r0 + r)) + rp_off;
                    rc[r] = *reinterpret_cast<const f32x4*>(c);
                    rsn[r] = *reinterpret_cast<const f32x4*>(sn);
                }
                if constexpr (R8) {
                    // the first half of a pair takes -sin times its partner, the second +sin
                    const float sg = (lane_e >> 5) ? 1.0f : -1.0f;
#pragma unroll
                    for (int u = 0; u < 4; ++u) rsn[0][u] *= sg;
                }
            }
        };
        load_rope(0, 0);
#pragma unroll
        for (int j = 0; j < TJ; ++j) {
            // grad epilogue: column sums of the stored dy over this lane's rows of the block
            // (its 8-column chunk gl of token rows r0, r0 + 4, ... of both half blocks), for db
            float csum[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) csum[e] = 0.0f;
            // every group's outputs rounded to bf16 (each branch packs its own results:
            // results written back into acc under these branches would cost a register
            // copy per value where the branches join)
            u32x2 pk[NG];
#pragma unroll
            for (int G = 0; G < NG; ++G) pk[G] = u32x2{0u, 0u};
#pragma unroll
            for (int G = 0; G < NG; ++G) {
                if (fw + 8 * G >= N) continue;   // ragged last column tile (not stored)
                const unsigned kind = desc[G] >> 30;
                float y[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) y[u] = acc[G >> 2][j][4 * (G & 3) + u];
                if (kind == 0) {
                    if constexpr (EPI == kEpiGrad) {
                        // dy = d_ff * act'(y) for this lane's token and 4 columns
                        const int tg = tw0 + 32 * j + (lane_e & 31);
                        const u32x2 gv = *reinterpret_cast<const u32x2*>(
                            static_cast<const __bf16*>(p.grad_in) + (int64_t)(tg < M ? tg : 0) * ff_dim + fw +
                            8 * G + 4 * hl);
                        const bf16x4 g4 = __builtin_bit_cast(bf16x4, gv);
#pragma unroll
                        for (int u = 0; u < 4; ++u) {
                            const float d = act == 1 ? gelu_erf_grad_poly(y[u])
                                            : act == 2 ? gelu_tanh_grad(y[u])
                                            : act == 3 ? relu_squared_grad(y[u]) : 1.0f;
                            y[u] = (float)g4[u] * d;
                        }
                        pk[G] = pack4_bf16(y);
                        continue;
                    }
                    if constexpr (EPI == kEpiOtherAct) {
                        if (act == 2) {
#pragma unroll
                            for (int u = 0; u < 4; ++u) y[u] = gelu_tanh(y[u]);
                        } else {
#pragma unroll
                            for (int u = 0; u < 4; ++u) y[u] = relu_squared(y[u]);
                        }
                    } else if (act == 1) {
#pragma unroll
                        for (int u = 0; u < 4; ++u) y[u] = gelu_erf_poly(y[u]);
                    }
                    pk[G] = pack4_bf16(y);
                    continue;
                }
                if constexpr (R8) {
                    if (desc[G] & (1u << 29)) {
                        // the first 8 columns of a q/k head: columns c and c + 4 form pair c,
                        // held for the same token by this lane and the one 32 lanes away
                        float o[4];
#pragma unroll
                        for (int u = 0; u < 4; ++u) {
                            const float partner = __shfl_xor(y[u], 32);
                            o[u] = y[u] * rc[0][u] + partner * rsn[0][u];
                        }
                        pk[G] = pack4_bf16(o);
                        continue;
                    }
                }
                if (DG > 0 && kind != 3) {
                    // Heads start on head_dim boundaries of the wave's columns, so the
                    // group's place in its head is a compile-time constant. A first-half
                    // group is rotated together with its partner DG groups on, which it
                    // also packs.
                    const int jh8 = (8 * G) % HD;
                    if (jh8 >= HALF || G + DG >= NG) continue;
                    const int G2 = (G + DG < NG) ? G + DG : G;   // constant after unrolling
                    if (NR > NRB && jh8 == 8 * NRB) load_rope(j, NRB);   // second half (head size 128)
                    const f32x4 c = rc[(jh8 / 8) % NRB], sn = rsn[(jh8 / 8) % NRB];
                    float o1[4], o2[4];
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const float y2 = acc[G2 >> 2][j][4 * (G2 & 3) + u];
                        o1[u] = y[u] * c[u] - y2 * sn[u];
                        o2[u] = y2 * c[u] + y[u] * sn[u];
                    }
                    pk[G] = pack4_bf16(o1);
                    pk[G2] = pack4_bf16(o2);
                    continue;
                }
                pk[G] = pack4_bf16(y);
            }
            // the next block's cos/sin, ahead of this block's stores
            if (j + 1 < TJ) load_rope(j + 1, 0);
            if constexpr (CF_STORE) {
                if (fw < ff_dim) {
                    // channels-first ff [b, ff, S] (ff_dim is a multiple of the wave's 128
                    // columns, so the whole wave is ff): the block goes through LDS one column
                    // half at a time as 32 token rows of 64 columns; two transposing reads give
                    // each lane 8 consecutive tokens of one column, and the 16-lane groups take
                    // the block's four 8-token runs, so every column is stored as one 64-byte run
#pragma unroll
                    for (int hc = 0; hc < 2; ++hc) {
#pragma unroll
                        for (int G = 0; G < NG / 2; ++G)
                            *(__attribute__((address_space(3))) u32x2*)(size_t)(cf_wr + G * 16) = pk[NG / 2 * hc + G];
                        const int t = tw0 + 32 * j + 8 * (lane_e >> 4);   // in one slab (S % 8 == 0)
                        const unsigned bi = fastdiv_u31((uint32_t)(t < M ? t : 0), p.div_s);
                        const unsigned sidx = (unsigned)(t < M ? t : 0) - bi * (unsigned)S;
#pragma unroll
                        for (int cb = 0; cb < 4; ++cb) {
                            const unsigned a = cf_rd + (unsigned)(32 * cb);
                            const bf16x8 v = join_tr(lds_tr16(a), lds_tr16(a + 4 * kCfRow));
                            if (t < M) {
                                const unsigned col = (unsigned)(fw + 64 * hc + 16 * cb + (lane_e & 15));
                                char* const dst = static_cast<char*>(p.ff) +
                                                  ((bi * (unsigned)ff_dim + col) * (unsigned)S + sidx) * 2u;
                                __builtin_nontemporal_store(__builtin_bit_cast(u32x4, v), reinterpret_cast<u32x4*>(dst));
                            }
                        }
                    }
                    continue;
                }
            }
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                // the lanes whose token is in this half of the token block write its rows
                if (((lane_e & 31) >> 4) == h) {
#pragma unroll
                    for (int G = 0; G < NG; ++G)
                        *(__attribute__((address_space(3))) u32x2*)(size_t)(wr_lds + G * 16) = pk[G];
                }
                const int t0 = tw0 + 32 * j + 16 * h;   // the half block's first token
                const int rows = M - t0;                 // its rows that exist
                // in one slab: row r of this lane's chunk at row0_l + u + (r - r0) * stride_l
                const unsigned u = kind_l == 0 ? (unsigned)t0 * (unsigned)(2 * ffr)
                                               : (unsigned)(((int64_t)bi_first * slab_l +
                                                             (int64_t)(t0 - bi_first * S) * hd) * 2);
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    const int r = r0 + 4 * rr;   // token row of the half block
                    const u32x4 v = *(const __attribute__((address_space(3))) u32x4*)(size_t)(
                        rd_lds + rr * 4 * kRestageRow);
                    // every lane stores, rows or columns outside the problem into the sink: with
                    // a fixed store count the compiler's waits (and the K loop's) can count them
                    char* const dst = !(r < rows && col_ok) ? sink_l
                                      : one_slab            ? row0_l + (u + (unsigned)(4 * rr) * stride_l)
                                                            : base_l + token_off(t0 + r);
                    __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(dst));
                    if constexpr (EPI == kEpiGrad) {
                        if (r < rows) {
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                csum[2 * e] += __uint_as_float(v[e] << 16);
                                csum[2 * e + 1] += __uint_as_float(v[e] & 0xffff0000u);
                            }
                        }
                    }
                }
            }
            if constexpr (EPI == kEpiGrad) {
                // the four lanes of a chunk (lane bits 4 and 5) add up their rows: the block's
                // 32 tokens; lanes 0-15 store the chunk's 8 sums into the block's row
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    csum[e] += __shfl_xor(csum[e], 16);
                    csum[e] += __shfl_xor(csum[e], 32);
                }
                const int c0 = fw + 8 * gl, tb = tw0 + 32 * j;
                if (p.colsum != nullptr && r0 == 0 && tb < M && c0 < p.colsum_cols) {
                    float* const dst = p.colsum + (int64_t)(tb / 32) * ffr + c0;
                    *reinterpret_cast<f32x4*>(dst) = f32x4{csum[0], csum[1], csum[2], csum[3]};
                    *reinterpret_cast<f32x4*>(dst + 4) = f32x4{csum[4], csum[5], csum[6], csum[7]};
                }
            }
        }
        }
        if (!has_next) break;
#pragma unroll
        for (int q = 0; q < NLOAD; ++q) voff_cur[q] = voff_nxt[q];
        tt = ntt;
        tf = ntf;
        trow_cur = trow_nxt;
        kb_cur = kb_nxt;
    }
    wait_vmcnt<0>();   // the trailing loads into LDS
}

template <bool X_TL, bool W_FC, int DG, class T, int EPI>
hipError_t launch_fast_one(const KernelArgs& a, int grid, hipStream_t stream) {
    const dim3 block(64 * T::NWF * T::NWT);
    if (a.K > 0 && a.K % (kBK * T::STAGES) == 0)
        hipLaunchKernelGGL((fused_proj_fast_kernel<X_TL, W_FC, DG, false, T, EPI>), dim3(grid), block, 0, stream, a);
    else
        hipLaunchKernelGGL((fused_proj_fast_kernel<X_TL, W_FC, DG, true, T, EPI>), dim3(grid), block, 0, stream, a);
    return hipGetLastError();
}

template <int DG, class T, int EPI>
hipError_t dispatch_fast_layouts(bool x_tl, bool w_fc, const KernelArgs& a, int grid, hipStream_t s) {
    if (x_tl)
        return w_fc ? launch_fast_one<true, true, DG, T, EPI>(a, grid, s)
                    : launch_fast_one<true, false, DG, T, EPI>(a, grid, s);
    return w_fc ? launch_fast_one<false, true, DG, T, EPI>(a, grid, s)
                : launch_fast_one<false, false, DG, T, EPI>(a, grid, s);
}

// The kernel's instantiations are spread over five translation units of this file: the
// build compiles it once per FP_FAST_PART value (0-4, in parallel); without FP_FAST_PART one
// unit holds them all. Part 0 also holds the host functions below.
//   0: default epilogue, no RoPE or partner distance 2     1: default, distances 4 and 8
//   2: tanh GELU / squared ReLU, channels-first ff         3: 8-column RoPE, backward dy
//   4: range units (partial sums, or the weight gradient stored directly)
#ifdef FP_FAST_PART
#define FP_PART(k) (FP_FAST_PART == (k))
#else
#define FP_PART(k) 1
#endif

constexpr int fast_part_of(int epi, int dg) {
    return epi == kEpiDefault ? (dg <= 2 ? 0 : 1)
           : (epi == kEpiOtherAct || epi == kEpiFfChannelsFirst) ? 2
           : (epi == kEpiDwPartial || epi == kEpiDwRows || epi == kEpiDwCols) ? 4 : 3;
}

// The variants one part compiles, for tile shape T: an unsupported combination is an error.
template <int P, class T>
hipError_t dispatch_part(int dg, int epi, bool x_tl, bool w_fc, const KernelArgs& a, int grid, hipStream_t s) {
    if constexpr (P == 0) {
        if (epi == kEpiDefault && dg == 0) return dispatch_fast_layouts<0, T, kEpiDefault>(x_tl, w_fc, a, grid, s);
        if (epi == kEpiDefault && dg == 2) return dispatch_fast_layouts<2, T, kEpiDefault>(x_tl, w_fc, a, grid, s);
    } else if constexpr (P == 1) {
        if (epi == kEpiDefault && dg == 4) return dispatch_fast_layouts<4, T, kEpiDefault>(x_tl, w_fc, a, grid, s);
        if (epi == kEpiDefault && dg == 8) return dispatch_fast_layouts<8, T, kEpiDefault>(x_tl, w_fc, a, grid, s);
    } else if constexpr (P == 2) {
        // compiled without RoPE only
        if (dg == 0 && epi == kEpiOtherAct) return dispatch_fast_layouts<0, T, kEpiOtherAct>(x_tl, w_fc, a, grid, s);
        if (dg == 0 && epi == kEpiFfChannelsFirst)
            return dispatch_fast_layouts<0, T, kEpiFfChannelsFirst>(x_tl, w_fc, a, grid, s);
    } else if constexpr (P == 3) {
        // the 8-column RoPE is marked in the descriptors; dy has no RoPE
        if (dg == 0 && epi == kEpiRope8) return dispatch_fast_layouts<0, T, kEpiRope8>(x_tl, w_fc, a, grid, s);
        if (dg == 0 && epi == kEpiGrad) return dispatch_fast_layouts<0, T, kEpiGrad>(x_tl, w_fc, a, grid, s);
    } else {
        // [N, K] weights: the input gradient's contraction ranges (x token-major)
        if (dg == 0 && epi == kEpiDwPartial) {
            if (w_fc) return x_tl ? launch_fast_one<true, true, 0, T, kEpiDwPartial>(a, grid, s) : hipErrorInvalidValue;
            return x_tl ? launch_fast_one<true, false, 0, T, kEpiDwPartial>(a, grid, s)
                        : launch_fast_one<false, false, 0, T, kEpiDwPartial>(a, grid, s);
        }
        // the weight gradient stored directly (large tiles only)
        if constexpr (!T::SINGLE) {
            if (dg == 0 && epi == kEpiDwRows && !w_fc)
                return x_tl ? launch_fast_one<true, false, 0, T, kEpiDwRows>(a, grid, s)
                            : launch_fast_one<false, false, 0, T, kEpiDwRows>(a, grid, s);
            if (dg == 0 && epi == kEpiDwCols && !w_fc)
                return x_tl ? launch_fast_one<true, false, 0, T, kEpiDwCols>(a, grid, s)
                            : launch_fast_one<false, false, 0, T, kEpiDwCols>(a, grid, s);
        }
    }
    return hipErrorInvalidValue;
}

}  // namespace

// One launcher per part, each defined in its own part and declared in every one.
template <int P>
hipError_t fast_launch_part(bool large, int dg, int epi, bool x_tl, bool w_fc, const KernelArgs& a, int grid,
                            hipStream_t s);
template <>
hipError_t fast_launch_part<0>(bool, int, int, bool, bool, const KernelArgs&, int, hipStream_t);
template <>
hipError_t fast_launch_part<1>(bool, int, int, bool, bool, const KernelArgs&, int, hipStream_t);
template <>
hipError_t fast_launch_part<2>(bool, int, int, bool, bool, const KernelArgs&, int, hipStream_t);
template <>
hipError_t fast_launch_part<3>(bool, int, int, bool, bool, const KernelArgs&, int, hipStream_t);
template <>
hipError_t fast_launch_part<4>(bool, int, int, bool, bool, const KernelArgs&, int, hipStream_t);
#define FP_DEFINE_PART(P)                                                                                        \
    template <>                                                                                                  \
    hipError_t fast_launch_part<P>(bool large, int dg, int epi, bool x_tl, bool w_fc, const KernelArgs& a,       \
                                   int grid, hipStream_t s) {                                                    \
        return large ? dispatch_part<P, LargeTile>(dg, epi, x_tl, w_fc, a, grid, s)                              \
                     : dispatch_part<P, SmallTile>(dg, epi, x_tl, w_fc, a, grid, s);                             \
    }
#if FP_PART(0)
FP_DEFINE_PART(0)
#endif
#if FP_PART(1)
FP_DEFINE_PART(1)
#endif
#if FP_PART(2)
FP_DEFINE_PART(2)
#endif
#if FP_PART(3)
FP_DEFINE_PART(3)
#endif
#if FP_PART(4)
FP_DEFINE_PART(4)
#endif
#undef FP_DEFINE_PART

#if FP_PART(0)

int fast_rope_groups(int head_dim, bool rope) {
    if (!rope) return 0;
    const int dg = head_dim / 16;
    return (head_dim % 16 == 0 && (dg == 2 || dg == 4 || dg == 8)) ? dg : -1;
}

TilePlan fast_plan(int64_t M, int64_t F, int num_cus) {
    const int cus = num_cus > 0 ? num_cus : 256;
    const int64_t large = ((M + LargeTile::BT - 1) / LargeTile::BT) * ((F + LargeTile::BF - 1) / LargeTile::BF);
    if (large >= cus) {
        // persistent: one workgroup per CU walks the large tiles
        TilePlan t{LargeTile::BT, LargeTile::BF, kBK, 8, 0, kFastLarge};
        t.grid = cus;
        t.grid = (t.grid + 7) / 8 * 8;   // a multiple of the 8 XCDs
        return t;
    }
    // too few large tiles to fill the CUs: small tiles, one per workgroup
    TilePlan t{SmallTile::BT, SmallTile::BF, kBK, 8, 0, kFastSmall};
    const int64_t small = ((M + SmallTile::BT - 1) / SmallTile::BT) * ((F + SmallTile::BF - 1) / SmallTile::BF);
    t.grid = (int)((small + 7) / 8 * 8);
    return t;
}

bool fast_addressable(int64_t M, int64_t S, int64_t ff_dim, int64_t qw) {
    const int64_t lim32 = int64_t(1) << 32, lim30 = int64_t(1) << 30;
    return M * ff_dim * 2 < lim32 && M * qw * 2 < lim32 && ff_dim < lim30 && S * qw < lim30;
}

// Entries for whole large column tiles, which also covers whole small ones.
int64_t fast_col_desc_entries(int64_t F) { return (F + LargeTile::BF - 1) / LargeTile::BF * (LargeTile::BF / 8); }

void fast_col_desc(int64_t S, int64_t ff_dim, int64_t n_heads, int64_t n_kv_heads, int64_t head_dim, bool grouped,
                   bool rope8, int64_t F, unsigned* out, int64_t entries) {
    const int64_t hd = head_dim, qw = n_heads * hd, kvw = n_kv_heads * hd;
    for (int64_t g = 0; g < entries; ++g) {
        const int64_t f = 8 * g;
        unsigned d = 0;
        if (f < F) {
            if (f < ff_dim) {
                d = (unsigned)f;
            } else {
                // the group's slice (1 q, 2 k, 3 v), head and place in the head
                const int64_t r = f - ff_dim;
                int64_t kind, h, jh;
                if (!grouped) {
                    const int64_t which = r < qw ? 0 : r < qw + kvw ? 1 : 2;
                    const int64_t rem = which == 0 ? r : r - qw - (which - 1) * kvw;
                    h = rem / hd;
                    jh = rem - h * hd;
                    kind = 1 + which;
                } else {
                    // per k/v head: its n_heads / n_kv_heads q heads, then k, then v
                    const int64_t qpk = n_heads / n_kv_heads, gw = (qpk + 2) * hd;
                    const int64_t grp = r / gw, within = r - grp * gw, slot = within / hd;
                    jh = within - slot * hd;
                    kind = slot < qpk ? 1 : slot == qpk ? 2 : 3;
                    h = slot < qpk ? grp * qpk + slot : grp;
                }
                d = ((unsigned)kind << 30) | (unsigned)(h * S * hd + jh);
                if (rope8 && kind != 3 && jh == 0) d |= 1u << 29;
            }
        }
        out[g] = d;
    }
}

hipError_t launch_fused_proj_fast(bool x_tokens_last, bool w_fc, int dg, int epi, const TilePlan& pl, const KernelArgs& a,
                                  hipStream_t stream) {
    if (pl.bk != kBK || pl.grid <= 0 || pl.grid % 8) return hipErrorInvalidValue;
    auto is = [&](auto t) { return pl.bm == decltype(t)::BT && pl.bn == decltype(t)::BF; };
    bool large;
    switch (pl.shape) {
        case kFastLarge:
            if (!is(LargeTile{})) return hipErrorInvalidValue;
            large = true;
            break;
        case kFastSmall:
            // one tile per workgroup at most: each XCD's share of the tiles fits its workgroups
            static_assert(SmallTile::SINGLE, "small tiles are planned one per workgroup");
            if ((int64_t)a.tiles_m * a.tiles_n > (int64_t)(pl.grid / 8) * 8) return hipErrorInvalidValue;
            if (!is(SmallTile{})) return hipErrorInvalidValue;
            large = false;
            break;
        default: return hipErrorInvalidValue;
    }
    switch (fast_part_of(epi, dg)) {
        case 0: return fast_launch_part<0>(large, dg, epi, x_tokens_last, w_fc, a, pl.grid, stream);
        case 1: return fast_launch_part<1>(large, dg, epi, x_tokens_last, w_fc, a, pl.grid, stream);
        case 2: return fast_launch_part<2>(large, dg, epi, x_tokens_last, w_fc, a, pl.grid, stream);
        case 3: return fast_launch_part<3>(large, dg, epi, x_tokens_last, w_fc, a, pl.grid, stream);
        default: return fast_launch_part<4>(large, dg, epi, x_tokens_last, w_fc, a, pl.grid, stream);
    }
}
#endif  // FP_PART(0)

}  // namespace fp
