// Internal interface between the C-ABI layer and the gfx950 kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp {

// Division by a divisor d >= 1 fixed at plan time, for dividends 0 <= n < 2^31, as one
// multiply-high, an add and a shift (Granlund and Montgomery, "Division by invariant
// integers using multiplication", 1994): with l = ceil(log2 d) and
// m = ceil(2^(32+l) / d), m - 2^32 fits 32 bits and n / d = (umulhi(n, m - 2^32) + n) >> l.
// Exact: m d - 2^(32+l) < d <= 2^l, so n m / 2^(32+l) exceeds n / d by less than 1 / (2d).
struct FastDivU31 {
    uint32_t mul;    // m - 2^32
    uint32_t shift;  // l
};
inline FastDivU31 make_fastdiv_u31(uint32_t d) {
    if (d == 0) d = 1;
    uint32_t l = 0;
    while ((uint64_t(1) << l) < d) ++l;
    const uint64_t p = uint64_t(1) << (32 + l);
    const uint64_t m = p / d + (p % d != 0 ? 1 : 0);
    return FastDivU31{(uint32_t)(m - (uint64_t(1) << 32)), l};
}
__host__ __device__ inline uint32_t fastdiv_u31(uint32_t n, FastDivU31 f) {
    return (uint32_t)((((uint64_t)n * f.mul) >> 32) + n) >> f.shift;
}

// Everything a launch needs, passed by value as the kernel argument.
struct KernelArgs {
    const void* x;       // activation (storage type)
    const void* w;       // weight [C,F] or [F,C]
    const void* bias;    // [F] or nullptr
    void* ff;            // [b, S, ff_dim]
    void* q;             // [b*H, S, hd]
    void* k;
    void* v;
    const float* rope_cos;  // [S, hd/2] fp32, row s holds angle (s + pos_offset) * theta_i
    const float* rope_sin;
    int64_t x_sb;        // element stride between slabs
    int64_t x_ss;        // element stride between consecutive tokens of a slab
    int64_t x_sc;        // element stride between channels
    int64_t M;           // tokens = b * S
    int32_t S;           // tokens per slab
    int32_t K;           // channels (contraction length)
    int32_t N;           // fused columns F
    int32_t ff_dim;
    int32_t n_heads;
    int32_t head_dim;
    int32_t qw;          // n_heads * head_dim (columns of the q slice)
    int32_t n_kv_heads;  // k and v heads (n_heads unless grouped-query)
    int32_t qkv_grouped; // 0: q, k, v columns contiguous; 1: grouped per k/v head
    int32_t rope_dims;   // rotated width of each q/k head (head_dim unless partial)
    int32_t ff_channels_first;  // 1: ff stored [b, ff_dim, S] (the fast kernel: its epilogue variant)
    int32_t act;         // ff slice: 0 none, 1 exact-erf GELU, 2 tanh GELU, 3 squared ReLU
    int32_t rope;        // 1: RoPE on q and k
    int32_t tiles_m;
    int32_t tiles_n;
    int32_t group_m;     // tile rows per raster group
    const void* zeros;   // >= 16 zero bytes: source of operand chunks outside the problem
    void* sink;          // 256 bytes that the fast kernel's stores outside the problem go to (never read)
    // Fast kernel only: one entry per 8 output columns, covering every column tile in
    // full. Bits 30-31: 0 ff, 1 q, 2 k, 3 v; bits 0-29: element offset of the group's
    // first column (ff: its column; q/k/v: head * S * head_dim + place in the head), whose
    // bit 29 instead marks a rotated group when RoPE covers the first 8 columns of a head.
    const unsigned* col_desc;
    // Fast kernel only: division by S (token -> slab) and by group_m * tiles_n (tile order).
    FastDivU31 div_s;
    FastDivU31 div_group;
    // Fast kernel, weight-gradient units only: row tiles per token range (tile rows count
    // (row tile, range) units), division by it, and for a channels-first x the K steps per
    // slab and division by them.
    int32_t dw_tiles_t;
    FastDivU31 div_dwt;
    int32_t k_slab_steps;
    FastDivU31 div_kslab;
    // Fast kernel, backward dy only: row stride of a [C, F] weight whose first N columns are
    // read, row stride of the ff output, and the upstream gradient of ff ([M, ff_dim]).
    int32_t w_ld;
    int32_t ff_ld;
    const void* grad_in;
    // ... and where dy's column sums go: [M/32 rows, ff_ld] fp32, one row per 32 tokens,
    // for columns below colsum_cols (null: none)
    float* colsum;
    int32_t colsum_cols;
};

// Tile plan chosen on the host.
struct TilePlan {
    int bm, bn, bk;
    int group_m;         // tiles along M that share a column sweep (L2 reuse)
    int grid;            // workgroups launched (0: one per tile)
    int shape = 0;       // fast kernel: which compiled tile shape (FastShape)
};

// Tile shapes of the fast kernel.
enum FastShape { kFastLarge = 0, kFastSmall = 1 };

// Kernel variants: storage type x activation layout x weight layout.
enum class DType { BF16 = 0, F32 = 1 };

// Records the HIP error that fused_proj_strerror reports for FUSED_PROJ_EHIP (both C-ABI
// files report through it).
void set_last_hip_error(hipError_t e);

// Launches one fused projection. Returns hipSuccess or the launch error.
hipError_t launch_fused_proj(DType dt, bool x_tokens_last, bool w_fc, const TilePlan& plan,
                             const KernelArgs& args, hipStream_t stream);

// Whether a tile plan is compiled for this combination.
bool plan_supported(DType dt, const TilePlan& plan);

// Fast bf16 kernel (F-major MFMA orientation, register epilogue; persistent 256 x 256
// tiles, or 128 x 128 tiles two per CU when the large ones cannot fill the CUs).
// fast_rope_groups returns the RoPE partner distance in 8-column groups it needs (0
// without RoPE) or -1 when the head size is not supported by it. fast_plan picks the
// tile shape and grid (a multiple of 8).
int fast_rope_groups(int head_dim, bool rope);
TilePlan fast_plan(int64_t M, int64_t F, int num_cus);
// Whether the fast kernel can address this problem with its 32-bit per-lane output
// offsets and 30-bit column offsets.
bool fast_addressable(int64_t M, int64_t S, int64_t ff_dim, int64_t qw);
// Column descriptor table of the fast kernel (entries for ceil(F / 256) full column tiles):
// each 8-column group's slice and element offset, for q/k/v columns either contiguous or
// grouped per k/v head; with rope8 (RoPE on the first 8 columns of each q/k head) bit 29
// marks those groups.
void fast_col_desc(int64_t S, int64_t ff_dim, int64_t n_heads, int64_t n_kv_heads, int64_t head_dim, bool grouped,
                   bool rope8, int64_t F, unsigned* out, int64_t entries);
int64_t fast_col_desc_entries(int64_t F);
// epi: 0 exact-erf GELU or no activation, token-major ff; 1 tanh GELU or squared ReLU;
// 2 channels-first ff (1 and 2 without RoPE, dg == 0); 3 as 0 with RoPE on the first 8
// columns of each q/k head only (the groups bit 29 of the descriptor marks, dg == 0); 5 the backward pass's dy over the ff
// columns (dg == 0); 4 the weight gradient's fp32
// partial sums over token ranges (dg == 0, W read as [K, N]; x_tokens_last selects K-major
// rows with K steps crossing slabs).
hipError_t launch_fused_proj_fast(bool x_tokens_last, bool w_fc, int dg, int epi, const TilePlan& plan,
                                  const KernelArgs& args, hipStream_t stream);

// ---------------------------------------------------------------- backward pass
// Arguments of the backward kernels. f is the forward problem (operands, layouts,
// heads, RoPE table), with its tile counts set for the 128 x 128 tiles of the dy
// kernel over [M, F].
struct BwdArgs {
    KernelArgs f;
    const void* d_ff;    // upstream gradients: [b, S, ff] (or [b, ff, S] with ff_cf)
    const void* dq;      // [b*H, S, hd]
    const void* dk;      // [b*KVH, S, hd]
    const void* dv;
    void* dy;            // workspace: gradient of the fused output, [M, F] token-major, storage type
    float* dbp;          // workspace: [db_tiles, F] fp32 column sums of dy per 32 tokens, or null
    void* dw;            // dW in W's layout (written by the dW kernel when splits == 1)
    float* dwp;          // workspace: fp32 partial sums of dW: [splits, C, F] from the dW tile kernel
                         // (splits > 1), whole 256 x 256 blocks in accumulator order from the fast one
    void* db;            // [F] or null
    int32_t ff_cf;       // d_ff channels-first
    int32_t w_fc;        // W (and dW) stored [F, C]
    int32_t splits;      // token ranges of the dW contraction
    int32_t chunk;       // tokens per range (a multiple of the K step)
    int32_t dw_tiles_m;  // 128 x 128 tiles over [C, F]
    int32_t dw_tiles_n;
    int32_t db_tiles;    // rows of dbp (32-token blocks)
    int32_t dw_partials; // dW goes through dwp in the fast kernel's block order
    int32_t dy_col_tile0;// the dy tile kernel's 128-column tiles [dy_col_tile0, dy_col_tile1): the fast
    int32_t dy_col_tile1;// kernel did the ones before, the heads kernel (bf16) the q/k/v ones after
    // dx's last tokens when their tiles go through contraction ranges (dx_splits > 1)
    float* dxp;          // workspace: fp32 partial sums, [dx_splits][token tiles][C tiles] blocks
    void* dx;            // dx in x's layout
    int32_t dx_row0;     // the first of those tokens (a whole number of slabs for a channels-first x)
    int32_t dx_rows;     // how many (a multiple of 64 for a channels-first x)
    int32_t dx_splits;
    int32_t dx_cf;       // x and dx channels-first (then S is a multiple of 64)
};

// K step of the 128 x 128 tile kernels for a storage type.
int tile_bk(DType dt);
// The dy kernel: 128 x 128 tiles over [M, F], column tiles [dy_col_tile0, dy_col_tile1).
// The heads kernel (bf16): dy's q/k/v columns [col0, F) from the head gradients alone.
hipError_t launch_bwd_dy(DType dt, bool x_tokens_last, bool w_fc, const BwdArgs& b, hipStream_t stream);
hipError_t launch_bwd_dy_heads(const BwdArgs& b, int col0, hipStream_t stream);
// The dW kernel: grid (dw_tiles_m x dw_tiles_n, splits).
hipError_t launch_bwd_dw(DType dt, bool x_tokens_last, const BwdArgs& b, hipStream_t stream);
// Sums dx's partial sums into its last tokens (bf16).
hipError_t launch_bwd_reduce_dx(const BwdArgs& b, hipStream_t stream);
// Sums the dW partials (splits > 1) into dW and the dy column sums into db (when db).
hipError_t launch_bwd_reduce(DType dt, const BwdArgs& b, hipStream_t stream);
// Writes zeros to n bytes at p (n a multiple of 4; a kernel, not a memset node).
hipError_t launch_zero_fill(void* p, size_t n, hipStream_t stream);

}  // namespace fp
