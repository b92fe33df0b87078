// C ABI of the fused input projection: descriptor checks, plan and RoPE table,
// argument checks and the launch. The arithmetic all runs in the HIP kernels.
#include "../../include/fused_proj.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <vector>

#include "fused_proj_kernels.h"

namespace {

thread_local hipError_t g_last_hip = hipSuccess;
thread_local char g_msg[256];

constexpr int64_t kMaxOffset = int64_t(1) << 62;
constexpr int64_t kMaxIndex = (int64_t(1) << 31) - 1;

// a*b, or -1 when it would leave [0, kMaxOffset)
int64_t mul_cap(int64_t a, int64_t b) {
    if (a < 0 || b < 0) return -1;
    if (a == 0 || b == 0) return 0;
    if (a > kMaxOffset / b) return -1;
    return a * b;
}
int64_t add_cap(int64_t a, int64_t b) {
    if (a < 0 || b < 0 || a > kMaxOffset - b) return -1;
    return a + b;
}

struct Derived {
    int64_t S = 0, M = 0, F = 0, qw = 0, V = 8;
    int64_t kvh = 0, kvw = 0, rd = 0;  // k/v heads and columns per k/v slice, rotated width
    int64_t sb = 0, ss = 0, sc = 0;  // canonical strides: slab, token, channel
    int64_t x_span = 0;              // 1 + largest element offset of x (0 when empty)
};

// Full descriptor check; fills the canonical strides on success.
int check_desc(const fused_proj_desc* d, Derived* out) {
    if (!d) return FUSED_PROJ_EINVAL;
    if (d->dtype != FUSED_PROJ_BF16 && d->dtype != FUSED_PROJ_F32) return FUSED_PROJ_EINVAL;
    if (d->x_layout != FUSED_PROJ_X_CHANNELS_FIRST && d->x_layout != FUSED_PROJ_X_TOKENS_LAST) return FUSED_PROJ_EINVAL;
    if (d->w_layout != FUSED_PROJ_W_CF && d->w_layout != FUSED_PROJ_W_FC) return FUSED_PROJ_EINVAL;
    if (d->ff_act != FUSED_PROJ_ACT_NONE && d->ff_act != FUSED_PROJ_ACT_GELU_ERF &&
        d->ff_act != FUSED_PROJ_ACT_GELU_TANH && d->ff_act != FUSED_PROJ_ACT_RELU_SQUARED)
        return FUSED_PROJ_EINVAL;
    if (d->batch < 0 || d->channels < 0 || d->ff_dim < 0 || d->n_heads < 0 || d->head_dim < 0) return FUSED_PROJ_EINVAL;
    if ((d->n_heads > 0) != (d->head_dim > 0)) return FUSED_PROJ_EINVAL;
    if (d->n_kv_heads < 0 || (d->n_heads == 0 && d->n_kv_heads != 0)) return FUSED_PROJ_EINVAL;
    if (d->n_kv_heads > 0 && d->n_heads % d->n_kv_heads != 0) return FUSED_PROJ_EINVAL;
    if (d->qkv_order != FUSED_PROJ_QKV_CONTIGUOUS && d->qkv_order != FUSED_PROJ_QKV_GROUPED) return FUSED_PROJ_EINVAL;
    if (d->rope_dims < 0) return FUSED_PROJ_EINVAL;
    if (d->ff_layout != FUSED_PROJ_FF_TOKENS_LAST && d->ff_layout != FUSED_PROJ_FF_CHANNELS_FIRST)
        return FUSED_PROJ_EINVAL;
    if (d->x_layout == FUSED_PROJ_X_TOKENS_LAST ? d->n_spatial != 1 : (d->n_spatial < 1 || d->n_spatial > 3))
        return FUSED_PROJ_EINVAL;
    if (d->x_stride_batch < 0 || d->x_stride_channel < 0) return FUSED_PROJ_EINVAL;
    for (int i = 0; i < d->n_spatial; ++i)
        if (d->spatial[i] < 0 || d->x_stride_spatial[i] < 0) return FUSED_PROJ_EINVAL;
    if (d->pos_offset < 0) return FUSED_PROJ_EINVAL;
    if (d->rope) {
        if (d->head_dim % 2 != 0) return FUSED_PROJ_EINVAL;
        const int64_t rd = d->rope_dims > 0 ? d->rope_dims : d->head_dim;
        if (rd % 2 != 0 || rd > d->head_dim) return FUSED_PROJ_EINVAL;
        if (!(d->rope_base > 0.0) || !std::isfinite(d->rope_base)) return FUSED_PROJ_EINVAL;
    }
    Derived r;
    r.V = d->dtype == FUSED_PROJ_BF16 ? 8 : 4;
    r.qw = mul_cap(d->n_heads, d->head_dim);
    if (r.qw < 0 || r.qw > kMaxIndex) return FUSED_PROJ_EUNSUPPORTED;
    r.kvh = d->n_kv_heads > 0 ? d->n_kv_heads : d->n_heads;
    r.kvw = mul_cap(r.kvh, d->head_dim);
    r.rd = d->rope_dims > 0 ? d->rope_dims : d->head_dim;
    if (r.kvw < 0 || r.kvw > kMaxIndex) return FUSED_PROJ_EUNSUPPORTED;
    r.F = add_cap(add_cap(d->ff_dim, r.qw), mul_cap(2, r.kvw));
    if (r.F == 0) return FUSED_PROJ_EINVAL;
    if (r.F < 0 || r.F > kMaxIndex || d->channels > kMaxIndex) return FUSED_PROJ_EUNSUPPORTED;
    int64_t S = 1;
    for (int i = 0; i < d->n_spatial; ++i) {
        S = mul_cap(S, d->spatial[i]);
        if (S < 0) return FUSED_PROJ_EUNSUPPORTED;
    }
    r.S = S;
    r.M = mul_cap(d->batch, S);
    if (r.M < 0 || r.M > kMaxIndex || S > kMaxIndex) return FUSED_PROJ_EUNSUPPORTED;

    // Supported shapes.
    const int64_t V = r.V;
    if (d->channels % V || d->ff_dim % V || d->head_dim % V) return FUSED_PROJ_EUNSUPPORTED;
    if (d->rope && r.qw > 0) {
        const int64_t hd = d->head_dim;
        if (128 % hd) return FUSED_PROJ_EUNSUPPORTED;         // a 128-column tile holds whole heads
        if (d->ff_dim % hd) return FUSED_PROJ_EUNSUPPORTED;   // heads start on head boundaries
        if (add_cap(S, d->pos_offset) < 0 || S + d->pos_offset > kMaxIndex) return FUSED_PROJ_EUNSUPPORTED;
    }
    // a channels-first ff output is stored V tokens of one column at a time
    if (d->ff_layout == FUSED_PROJ_FF_CHANNELS_FIRST && d->ff_dim > 0 && S % V) return FUSED_PROJ_EUNSUPPORTED;
    // Canonical strides. x is read only when it holds elements (C > 0 and b*S > 0); an
    // empty x may report any strides (an empty tensor's carry no layout), so they are
    // checked only then.
    const bool x_read = d->channels > 0 && r.M > 0;
    r.sb = d->x_stride_batch;
    r.sc = d->x_stride_channel;
    if (d->x_layout == FUSED_PROJ_X_TOKENS_LAST) {
        r.ss = d->x_stride_spatial[0];
        if (x_read && d->channels > 1 && r.sc != 1) return FUSED_PROJ_EUNSUPPORTED;
        r.sc = 1;
        if (x_read && ((S > 1 && r.ss % V) || (d->batch > 1 && r.sb % V))) return FUSED_PROJ_EUNSUPPORTED;
    } else {
        // spatial dims must flatten into one unit-stride token index
        int64_t expect = 1;
        for (int i = d->n_spatial - 1; i >= 0; --i) {
            if (x_read && d->spatial[i] > 1 && d->x_stride_spatial[i] != expect) return FUSED_PROJ_EUNSUPPORTED;
            expect = mul_cap(expect, d->spatial[i]);
            if (expect < 0) return FUSED_PROJ_EUNSUPPORTED;
        }
        r.ss = 1;
        if (S % V) return FUSED_PROJ_EUNSUPPORTED;
        if (x_read && ((d->channels > 1 && r.sc % V) || (d->batch > 1 && r.sb % V))) return FUSED_PROJ_EUNSUPPORTED;
    }
    // Offsets must stay below 2^62.
    if (r.M > 0 && d->channels > 0) {
        int64_t span = add_cap(mul_cap(d->batch - 1, r.sb), mul_cap(S - 1, r.ss));
        span = add_cap(span, mul_cap(d->channels - 1, r.sc));
        span = add_cap(span, 1);
        if (span < 0) return FUSED_PROJ_EUNSUPPORTED;
        r.x_span = span;
    }
    if (mul_cap(d->channels, r.F) < 0 || mul_cap(r.M, r.F) < 0) return FUSED_PROJ_EUNSUPPORTED;
    // one workgroup per 128 x 128 output tile; the grid must fit a 31-bit count
    if (mul_cap((r.M + 127) / 128, (r.F + 127) / 128) > kMaxIndex) return FUSED_PROJ_EUNSUPPORTED;
    if (out) *out = r;
    return FUSED_PROJ_OK;
}

struct Range {
    uintptr_t lo, hi;  // [lo, hi)
};
bool overlap(const Range& a, const Range& b) { return a.lo < b.hi && b.lo < a.hi; }

}  // namespace

void fp::set_last_hip_error(hipError_t e) { g_last_hip = e; }

// ---------------------------------------------------------------- static scratch
// The workspace of fused_proj_backward_noalloc: a fixed device array (each GPU the library
// runs on holds its own copy until the process ends). In host code `scratch` names a
// host-side stand-in, never the device memory: its device address is looked up once per
// device (hipGetSymbolAddress, at plan creation with that device current) and only that
// address is ever passed to kernels.
namespace {
constexpr size_t kScratchBytes = size_t(64) << 20;
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
// Looks up this device's scratch address once (device current); FUSED_PROJ_OK or EHIP.
int scratch_setup(int device) {
    if (device < 0 || device >= kMaxDevices) return FUSED_PROJ_EUNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[device] != nullptr) return FUSED_PROJ_OK;
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr) {
        g_last_hip = e != hipSuccess ? e : hipErrorInvalidSymbol;
        return FUSED_PROJ_EHIP;
    }
    g_scratch_ptr[device] = ptr;
    return FUSED_PROJ_OK;
}
void* scratch_ptr(int device) {
    if (device < 0 || device >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    return g_scratch_ptr[device];
}
}  // namespace

struct fused_proj_plan {
    fused_proj_desc d;
    Derived r;
    fp::DType dt;
    bool x_tl, w_fc;
    fp::TilePlan tile;
    fp::KernelArgs base;
    bool fast = false;  // fast bf16 kernel (else the general kernel)
    int dg = 0;         // its RoPE partner distance in 8-column groups
    int epi = 0;        // its epilogue variant
    float* d_cos = nullptr;
    float* d_sin = nullptr;
    void* d_zeros = nullptr;
    unsigned* d_desc = nullptr;  // fast kernel: column descriptors
    // Forward tail: when the large tiles' last round would leave most CUs idle, the tokens
    // from tail_m0 on (whole slabs) run on small tiles in a second launch (0: no tail).
    int64_t tail_m0 = 0;
    fp::TilePlan tail_tile{};
    fp::KernelArgs tail_args{};          // the tail's arguments but the per-call pointers
    int device = 0;
    int num_cus = 0;
    bool debug_sync = false;
    // backward pass
    fused_proj_plan* dx_plan = nullptr;  // dx = dy W^T as a forward projection (null when C == 0)
    fp::BwdArgs bwd{};                   // everything but the per-call pointers
    bool fast_dy = false;                // dy's ff columns on the fast kernel (grad epilogue)
    fp::KernelArgs dy_args{};            // its arguments but the per-call pointers
    fp::TilePlan dy_tile{};
    unsigned* d_desc_dy = nullptr;       // its column descriptors
    int dw_epi = 4;                      // the fast dW's epilogue: 4 partial sums, 6 or 7 dW itself
    unsigned* d_desc_dw = nullptr;       // column descriptors when it stores dW itself
    bool dy_heads = false;               // dy's q/k/v columns by the heads kernel
    bool fast_dw = false;                // dW on the fast kernel (else the dW tile kernel)
    bool dw_x_kmajor = false;            // ... reading x as K-major rows (channels-first x)
    fp::KernelArgs dw_args{};            // its arguments but the per-call pointers
    fp::TilePlan dw_tile{};
    // dx in two parts when its tiles would leave most CUs idle in a last round: the first
    // dx_head_m tokens through the nested plan's kernel, the rest in ranges of the fused
    // columns (fp32 partial sums) and a reduction
    bool dx_split = false;
    int64_t dx_head_m = 0;
    fp::KernelArgs dxt_args{};           // the range units' arguments but the per-call pointers
    fp::TilePlan dxt_tile{};
    size_t ws_dbp = 0, ws_dwp = 0;       // workspace offsets (dy at 0)
    size_t ws_dxp = 0;
    size_t ws_bytes = 0;                 // workspace size
};

namespace {

int create_plan(const fused_proj_desc* desc, fused_proj_t* out, bool with_backward);

constexpr size_t kWsAlign = 256;
size_t ws_round(size_t n) { return (n + kWsAlign - 1) / kWsAlign * kWsAlign; }

// The forward's tail. Large tiles are walked by one persistent workgroup per CU, so a last
// round of a few tiles leaves most CUs idle. Then the tokens of the last slabs (enough for
// the head to end one round earlier) go to a second launch on small tiles, at most two per
// CU (one round of them). The tail starts on a slab boundary, so its inputs and outputs
// are the whole problem's with every pointer advanced by its first token and the same
// column descriptors and rotary table. The estimate charges the last large round in full
// (a tile's MFMA time at about 55% of a CU's share of the bf16 peak), the small tiles 0.55
// (one per CU) to 0.7 (two per CU) of it, and a launch. Measured, a part-filled last round
// costs less than a full one (its few tiles contend less: at K = 768, 18 us against 27 us
// for a quarter-filled round), about what the small tiles take, so the split gains a few
// percent: 73.6 -> 71.3 us on 16384 tokens x 2304 columns, 100.7 -> 99.2 us on 24576 x 2304.
// FUSED_PROJ_TAIL=0 never splits, =1 splits wherever a tail fits.
void plan_fwd_tail(fused_proj_plan* h) {
    const Derived& r = h->r;
    if (!h->fast || h->tile.shape != fp::kFastLarge || r.M <= 0 || r.S <= 0 || h->d.channels <= 0) return;
    const char* env = std::getenv("FUSED_PROJ_TAIL");
    const int force = env && env[0] == '0' ? 0 : env && env[0] == '1' ? 1 : -1;
    if (force == 0) return;
    const int64_t cus = h->num_cus, K = h->d.channels;
    const int64_t tn = (r.F + 255) / 256, tiles = h->base.tiles_m * tn;
    const int64_t rounds = (tiles + cus - 1) / cus;
    if (rounds < 2) return;
    // the most whole slabs whose tiles fit one round fewer
    const int64_t head_rows = (rounds - 1) * cus / tn;         // 256-token rows
    const int64_t n1 = std::min(head_rows * 256 / r.S, r.M / r.S - 1);
    if (n1 <= 0) return;
    const int64_t m0 = n1 * r.S, mt = r.M - m0;
    const int64_t small = ((mt + 127) / 128) * ((r.F + 127) / 128);
    if (small > 2 * cus) return;
    const double round_s = 2.0 * 256 * 256 * (double)K / (2.5e15 / (double)cus * 0.55);
    const double t_split = (double)(((m0 + 255) / 256 * tn + cus - 1) / cus) * round_s +
                           (small <= cus ? 0.55 : 0.7) * round_s + 3e-6;
    if (force != 1 && t_split >= 0.97 * (double)rounds * round_s) return;
    fp::KernelArgs t = h->base;
    t.M = mt;
    t.tiles_m = (int32_t)((mt + 127) / 128);
    t.tiles_n = (int32_t)((r.F + 127) / 128);
    t.group_m = 8;
    t.div_group = fp::make_fastdiv_u31((uint32_t)(8 * t.tiles_n));
    h->tail_args = t;
    h->tail_tile = fp::TilePlan{128, 128, 32, 8, (int)((small + 7) / 8 * 8), fp::kFastSmall};
    h->tail_m0 = m0;
}

// dx = dy W^T on large tiles takes rounds of tiles over the CUs; when the last round is
// mostly idle (Walrus: 288 tiles on 256 CUs), the last token tiles are instead split into
// (tile, range of the fused columns) units that fill one round, each storing fp32 partial
// sums that a reduction adds into dx. The head keeps a whole number of slabs (channels-first
// x, whose dx is stored per slab). The split (tail tiles, ranges) minimises an estimated
// time: rounds of tiles times a tile's MFMA time (at about 55% of a CU's share of the bf16
// peak), plus writing and reading back the partial sums (about 4 TB/s) and two launches.
void plan_dx_split(fused_proj_plan* h) {
    const fused_proj_desc& d = h->d;
    const Derived& r = h->r;
    const fused_proj_plan* xp = h->dx_plan;
    const char* force = std::getenv("FUSED_PROJ_KERNEL");
    if (!xp || !xp->fast || xp->tile.shape != fp::kFastLarge || xp->epi > 2 || r.M <= 0 || r.F % 32 != 0 ||
        (force && std::strcmp(force, "general") == 0))
        return;
    const bool cf = d.x_layout == FUSED_PROJ_X_CHANNELS_FIRST;
    if (cf && r.S % 64 != 0) return;
    const int64_t bt = 256, tm = xp->base.tiles_m, tn = xp->base.tiles_n, cus = h->num_cus;
    const int64_t ksteps = r.F / 32, C = d.channels;
    // head tile rows come in multiples of g (a whole number of slabs)
    int64_t g = 1;
    if (cf) {
        int64_t a = r.S, b2 = bt;
        while (b2) {
            const int64_t t = a % b2;
            a = b2;
            b2 = t;
        }
        g = r.S / a;
    }
    const double tile_s = 2.0 * 256 * 256 * (double)r.F / (2.5e15 / (double)cus * 0.55);
    const double base = (double)((tm * tn + cus - 1) / cus) * tile_s;
    double best = base * 0.97;   // worth a split only when clearly faster
    int64_t best_head = -1, best_r = 1;
    for (int64_t head = (tm - 1) / g * g; head >= 0; head -= g) {
        const int64_t rows = r.M - head * bt;   // tail tokens
        const int64_t rt = tm - head;
        for (int64_t rs = 2; rs <= 16; ++rs) {
            if (ksteps % rs) continue;
            const double t = (double)((head * tn + cus - 1) / cus) * tile_s +
                             (double)((rt * tn * rs + cus - 1) / cus) * tile_s / (double)rs +
                             (double)rs * (double)rows * (double)C * 8.0 / 4e12 + 5e-6;
            if (t < best) {
                best = t;
                best_head = head;
                best_r = rs;
            }
        }
        if (head == 0) break;
    }
    if (best_head < 0) return;
    const int64_t rt = tm - best_head, rows = r.M - best_head * bt;
    fp::KernelArgs t = xp->base;
    t.M = rows;
    t.S = (int32_t)rows;
    t.div_s = fp::make_fastdiv_u31((uint32_t)rows);
    t.x_sb = rows * r.F;
    t.K = (int32_t)(r.F / best_r);
    t.N = (int32_t)C;
    t.tiles_m = (int32_t)(rt * best_r);
    t.tiles_n = (int32_t)tn;
    t.group_m = 8;
    t.div_group = fp::make_fastdiv_u31((uint32_t)(8 * tn));
    t.dw_tiles_t = (int32_t)rt;
    t.div_dwt = fp::make_fastdiv_u31((uint32_t)rt);
    t.k_slab_steps = (int32_t)ksteps;   // dy's rows are one "slab": no K step crosses one
    t.div_kslab = fp::make_fastdiv_u31((uint32_t)ksteps);
    t.w_ld = (int32_t)(xp->w_fc ? r.F : C);
    t.bias = nullptr;
    h->dxt_args = t;
    h->dxt_tile = fp::TilePlan{256, 256, 32, 8, (int)((cus + 7) / 8 * 8), fp::kFastLarge};
    h->dx_split = true;
    h->dx_head_m = best_head * bt;
    fp::BwdArgs& b = h->bwd;
    b.dx_row0 = (int32_t)(best_head * bt);
    b.dx_rows = (int32_t)rows;
    b.dx_splits = (int32_t)best_r;
    b.dx_cf = cf ? 1 : 0;
}

// Backward plan: the dx sub-projection, the dy and dW tilings and the workspace layout.
int plan_backward(fused_proj_plan* h) {
    const fused_proj_desc& d = h->d;
    const Derived& r = h->r;
    const int64_t es = h->dt == fp::DType::BF16 ? 2 : 4;
    if (d.channels > 0) {
        // dx[t, c] = sum_f dy[t, f] W[c, f]: dy [b, S, F] token-major is the activation, W is
        // read the other way round, and the result is an ff slice of width C laid out like x
        fused_proj_desc s{};
        s.dtype = d.dtype;
        s.x_layout = FUSED_PROJ_X_TOKENS_LAST;
        s.batch = d.batch;
        s.channels = r.F;
        s.n_spatial = 1;
        s.spatial[0] = r.S;
        s.x_stride_batch = r.S * r.F;
        s.x_stride_channel = 1;
        s.x_stride_spatial[0] = r.F;
        s.w_layout = d.w_layout == FUSED_PROJ_W_CF ? FUSED_PROJ_W_FC : FUSED_PROJ_W_CF;
        s.has_bias = 0;
        s.ff_dim = d.channels;
        s.ff_act = FUSED_PROJ_ACT_NONE;
        s.rope_base = 10000.0;
        s.ff_layout = d.x_layout == FUSED_PROJ_X_CHANNELS_FIRST ? FUSED_PROJ_FF_CHANNELS_FIRST
                                                                 : FUSED_PROJ_FF_TOKENS_LAST;
        const int rc = create_plan(&s, &h->dx_plan, false);
        if (rc) return rc;
    }
    fp::BwdArgs& b = h->bwd;
    b.f = h->base;
    const int bk = fp::tile_bk(h->dt);
    b.f.tiles_m = (int32_t)((r.M + 127) / 128);
    b.f.tiles_n = (int32_t)((r.F + 127) / 128);
    b.f.group_m = 8;
    b.ff_cf = d.ff_layout == FUSED_PROJ_FF_CHANNELS_FIRST ? 1 : 0;
    b.w_fc = d.w_layout == FUSED_PROJ_W_FC ? 1 : 0;
    b.dw_tiles_m = (int32_t)((d.channels + 127) / 128);
    b.dw_tiles_n = b.f.tiles_n;
    b.db_tiles = (int32_t)((r.M + 31) / 32);   // one row of column sums per 32 tokens
    // dW contracts over the tokens: split them into ranges when the dW tiles alone
    // cannot fill the CUs (two workgroups each), at most 16 ranges
    const int64_t dw_tiles = (int64_t)b.dw_tiles_m * b.dw_tiles_n;
    const int64_t ksteps = (r.M + bk - 1) / bk;
    int64_t splits = 1;
    if (dw_tiles > 0 && ksteps > 0) {
        splits = (2 * (int64_t)h->num_cus + dw_tiles - 1) / dw_tiles;
        if (splits > 16) splits = 16;
        if (splits > ksteps) splits = ksteps;
        if (splits < 1) splits = 1;
    }
    const int64_t chunk = ksteps > 0 ? (ksteps + splits - 1) / splits * bk : bk;
    splits = r.M > 0 ? (r.M + chunk - 1) / chunk : 1;
    b.splits = (int32_t)splits;
    b.chunk = (int32_t)chunk;

    const char* force = std::getenv("FUSED_PROJ_KERNEL");
    const bool want_general = force && std::strcmp(force, "general") == 0;
    const bool cf = d.x_layout == FUSED_PROJ_X_CHANNELS_FIRST;
    const int64_t lim32 = int64_t(1) << 32;
    // dy's ff columns on the fast kernel (bf16, an activation to differentiate, token-major
    // d_ff): the forward product over the first ff_dim columns, then dy = d_ff * act'(y)
    // stored into dy's rows (stride F). The 128-column tiles it covers entirely are then left
    // out of the dy tile kernel, and their column sums (db) taken from dy afterwards.
    if (h->dt == fp::DType::BF16 && d.ff_dim > 0 && d.ff_act != FUSED_PROJ_ACT_NONE && r.M > 0 &&
        d.channels > 0 && d.ff_layout == FUSED_PROJ_FF_TOKENS_LAST && !want_general &&
        r.x_span * 2 < lim32 && d.channels * r.F * 2 < lim32 && r.M * r.F * 2 < lim32 &&
        fp::fast_addressable(r.M, r.S, d.ff_dim, 0)) {
        fp::KernelArgs a = h->base;
        a.N = (int32_t)d.ff_dim;
        a.ff_dim = (int32_t)d.ff_dim;
        a.n_heads = a.head_dim = a.qw = 0;
        a.n_kv_heads = 0;
        a.rope = 0;
        a.rope_cos = a.rope_sin = nullptr;
        a.ff_channels_first = 0;
        a.w_ld = (int32_t)r.F;
        a.ff_ld = (int32_t)r.F;
        const fp::TilePlan tp = fp::fast_plan(r.M, d.ff_dim, h->num_cus);
        a.tiles_m = (int32_t)((r.M + tp.bm - 1) / tp.bm);
        a.tiles_n = (int32_t)((d.ff_dim + tp.bn - 1) / tp.bn);
        a.group_m = tp.group_m;
        a.div_group = fp::make_fastdiv_u31((uint32_t)((int64_t)a.group_m * a.tiles_n));
        const int64_t n = fp::fast_col_desc_entries(d.ff_dim);
        std::vector<unsigned> hd((size_t)n);
        fp::fast_col_desc(r.S, d.ff_dim, 0, 0, 0, false, false, d.ff_dim, hd.data(), n);
        hipError_t e = hipMalloc((void**)&h->d_desc_dy, (size_t)n * sizeof(unsigned));
        if (e == hipSuccess)
            e = hipMemcpy(h->d_desc_dy, hd.data(), (size_t)n * sizeof(unsigned), hipMemcpyHostToDevice);
        if (e != hipSuccess) {
            g_last_hip = e;
            return FUSED_PROJ_EHIP;
        }
        a.col_desc = h->d_desc_dy;
        h->dy_args = a;
        h->dy_tile = tp;
        h->fast_dy = true;
        b.dy_col_tile0 = (int32_t)(d.ff_dim / 128);
        // it writes the column sums of the 128-column tiles it covers entirely
        h->dy_args.colsum_cols = b.dy_col_tile0 * 128;
    }
    // dy's q/k/v columns (bf16) from the head gradients alone, in a streaming kernel: the
    // tile kernel keeps the column tiles holding ff columns
    b.dy_col_tile1 = b.f.tiles_n;
    h->dy_heads = h->dt == fp::DType::BF16 && r.qw > 0 && !want_general;
    if (h->dy_heads) b.dy_col_tile1 = (int32_t)((d.ff_dim + 127) / 128);

    // dW on the fast kernel (bf16): rows are channels, the contraction runs over the tokens,
    // and the work is split into (256-row tile, token range) units whose fp32 partial sums
    // the reduction adds up. A channels-first x is read as K-major rows whose K steps (32
    // tokens) each lie in one slab (S a multiple of 32); a token-major x as M-major rows
    // with one token stride across slabs.
    bool fast_dw = h->dt == fp::DType::BF16 && d.channels > 0 && r.M > 0 && !want_general &&
                   (cf ? r.S % 32 == 0 : (d.batch == 1 || r.sb == r.S * r.ss)) && r.x_span * 2 < lim32 &&
                   r.M * r.F * 2 < lim32 && d.channels * r.F < (int64_t(1) << 31);
    if (fast_dw) {
        const int64_t tiles_t = (d.channels + 255) / 256, tiles_f = (r.F + 255) / 256;
        const int64_t tiles = tiles_t * tiles_f, cus = h->num_cus;
        // token ranges: a divisor of the K-step count (equal whole ranges), at most 16, that
        // minimises the estimated time: rounds of units over the CUs times a unit's MFMA time
        // (at about 40% of a CU's share of the bf16 peak), plus writing and reading back
        // each range's fp32 partial sums (at about 4 TB/s)
        int64_t best = 1;
        if (r.M % 32 == 0) {
            const int64_t steps = r.M / 32;
            const double tile_s = 2.0 * 256 * 256 * (double)r.M / (2.5e15 / (double)cus * 0.4);
            const double partial_s = (double)d.channels * (double)r.F * 8.0 / 4e12;
            auto cost = [&](int64_t sp) {
                return (double)((tiles * sp + cus - 1) / cus) / (double)sp * tile_s + (double)sp * partial_s;
            };
            double best_cost = cost(1);
            for (int64_t sp = 2; sp <= 16; ++sp) {
                if (steps % sp) continue;
                if (cost(sp) < best_cost) {
                    best_cost = cost(sp);
                    best = sp;
                }
            }
        }
        fp::KernelArgs& a = h->dw_args;
        std::memset(&a, 0, sizeof(a));
        a.M = d.channels;          // rows: channels
        a.S = (int32_t)d.channels; // one "slab" of rows
        a.K = (int32_t)(r.M / best);
        a.N = (int32_t)r.F;
        a.ff_dim = (int32_t)r.F;
        if (cf) {                  // K-major rows: channel stride, tokens contiguous, slabs apart
            a.x_sb = r.sb;
            a.x_ss = r.sc;
            a.x_sc = 1;
            a.k_slab_steps = (int32_t)(r.S / 32);
            a.div_kslab = fp::make_fastdiv_u31((uint32_t)(r.S / 32));
        } else {                   // M-major rows: channels contiguous, one token stride
            a.x_sb = 0;
            a.x_ss = 1;
            a.x_sc = r.ss;
        }
        a.tiles_m = (int32_t)(tiles_t * best);
        a.tiles_n = (int32_t)tiles_f;
        a.group_m = 8;
        a.div_s = fp::make_fastdiv_u31((uint32_t)d.channels);
        a.div_group = fp::make_fastdiv_u31((uint32_t)(8 * tiles_f));
        a.dw_tiles_t = (int32_t)tiles_t;
        a.div_dwt = fp::make_fastdiv_u31((uint32_t)tiles_t);
        a.zeros = h->d_zeros;
        a.sink = static_cast<char*>(h->d_zeros) + 256;
        h->dw_tile = fp::TilePlan{256, 256, 32, 8, (int)((cus + 7) / 8 * 8), fp::kFastLarge};
        h->dw_x_kmajor = cf;
        h->fast_dw = true;
        splits = best;
        b.splits = (int32_t)best;
        b.chunk = (int32_t)(r.M / best);
        b.dw_partials = 1;
        // one token range: the units store dW itself in bf16 (no partial sums, no
        // reduction), [C, F] as token-major rows of a "forward" with C tokens and F ff
        // columns, [F, C] as its channels-first ff (whole 128-column waves: F % 128 == 0)
        if (best == 1 && (d.w_layout == FUSED_PROJ_W_CF || r.F % 128 == 0)) {
            const int64_t n = fp::fast_col_desc_entries(r.F);
            std::vector<unsigned> hd((size_t)n);
            fp::fast_col_desc(d.channels, r.F, 0, 0, 0, false, false, r.F, hd.data(), n);
            hipError_t e = hipMalloc((void**)&h->d_desc_dw, (size_t)n * sizeof(unsigned));
            if (e == hipSuccess)
                e = hipMemcpy(h->d_desc_dw, hd.data(), (size_t)n * sizeof(unsigned), hipMemcpyHostToDevice);
            if (e != hipSuccess) {
                g_last_hip = e;
                return FUSED_PROJ_EHIP;
            }
            a.col_desc = h->d_desc_dw;
            a.ff_dim = (int32_t)r.F;
            h->dw_epi = d.w_layout == FUSED_PROJ_W_CF ? 6 : 7;
            b.dw_partials = 0;
        }
    }
    plan_dx_split(h);
    // workspace: dy, then the column sums of dy per token tile (bias), then the dW partials,
    // then dx's partials
    size_t off = ws_round((size_t)(r.M * r.F * es));
    h->ws_dbp = off;
    if (d.has_bias) off += ws_round((size_t)b.db_tiles * (size_t)r.F * 4);
    // (the fast kernel's partial sums are whole 256 x 256 blocks)
    auto up256 = [](int64_t v) { return (size_t)((v + 255) / 256 * 256); };
    h->ws_dwp = off;
    if (h->fast_dw && h->dw_epi == 4) off += ws_round((size_t)splits * up256(d.channels) * up256(r.F) * 4);
    else if (splits > 1) off += ws_round((size_t)splits * (size_t)d.channels * (size_t)r.F * 4);
    h->ws_dxp = off;
    if (h->dx_split) off += ws_round((size_t)b.dx_splits * up256(b.dx_rows) * up256(d.channels) * 4);
    h->ws_bytes = r.M > 0 ? off : 0;
    return FUSED_PROJ_OK;
}

}  // namespace

extern "C" {

int fused_proj_validate(const fused_proj_desc* desc) { return check_desc(desc, nullptr); }

int fused_proj_create(const fused_proj_desc* desc, fused_proj_t* out) { return create_plan(desc, out, true); }

}  // extern "C"

namespace {

int create_plan(const fused_proj_desc* desc, fused_proj_t* out, bool with_backward) {
    if (!out) return FUSED_PROJ_EINVAL;
    *out = nullptr;
    Derived r;
    int rc = check_desc(desc, &r);
    if (rc) return rc;
    fused_proj_plan* h = new (std::nothrow) fused_proj_plan();
    if (!h) return FUSED_PROJ_EHIP;
    h->d = *desc;
    h->r = r;
    h->dt = desc->dtype == FUSED_PROJ_BF16 ? fp::DType::BF16 : fp::DType::F32;
    h->x_tl = desc->x_layout == FUSED_PROJ_X_TOKENS_LAST;
    h->w_fc = desc->w_layout == FUSED_PROJ_W_FC;
    const char* dbg = std::getenv("FUSED_PROJ_DEBUG_SYNC");
    h->debug_sync = dbg && dbg[0] == '1';
    hipError_t e = hipGetDevice(&h->device);
    int num_cus = 0;
    if (e == hipSuccess) e = hipDeviceGetAttribute(&num_cus, hipDeviceAttributeMultiprocessorCount, h->device);
    h->num_cus = num_cus > 0 ? num_cus : 256;
    // FUSED_PROJ_CUS=n (8 <= n <= the device's CUs) plans for n CUs: the tests use it to
    // reach the persistent walk and the tail split at small sizes
    if (const char* cu_env = std::getenv("FUSED_PROJ_CUS")) {
        const int n = std::atoi(cu_env);
        if (n >= 8 && n <= h->num_cus) h->num_cus = n;
    }
    if (e != hipSuccess) {
        g_last_hip = e;
        delete h;
        return FUSED_PROJ_EHIP;
    }
    // Kernel choice. The fast bf16 kernel needs RoPE over a whole head of 32, 64 or 128
    // columns or over the first 8 columns of each head (or no RoPE), and x and W spans under
    // 4 GiB (it addresses them with 32-bit offsets). Every other shape goes to the general
    // kernel.
    // FUSED_PROJ_KERNEL=general forces the general kernel (the tests use it to cover both);
    // FUSED_PROJ_KERNEL=fast takes the fast kernel on any shape it can address.
    const char* force = std::getenv("FUSED_PROJ_KERNEL");
    const bool want_general = force && std::strcmp(force, "general") == 0;
    const bool want_fast = force && std::strcmp(force, "fast") == 0;
    const bool roped = desc->rope && r.qw > 0;
    // RoPE on 8 columns of each head: rotated within one 8-column group (a separate epilogue)
    const bool rope8 = roped && r.rd == 8;
    const int dg = rope8 ? 0 : r.rd == desc->head_dim ? fp::fast_rope_groups((int)desc->head_dim, roped) : -1;
    const bool fits32 = r.x_span * 2 < (int64_t(1) << 32) && desc->channels * r.F * 2 < (int64_t(1) << 32);
    const fp::TilePlan fp_plan = fp::fast_plan(r.M, r.F, h->num_cus);
    // Both tile shapes take any token, column and channel count: tokens past M read token
    // 0 and columns past F read row 0 of W and the zero block for the bias, and neither is
    // stored (a channels-first x has S, hence M, a multiple of the 8-token load chunk);
    // channels past C (a partial last K step, and on large tiles the steps that pad the K
    // loop to a multiple of its four stages) read the zero block. Measured against the
    // general kernel on such shapes (C 320, 72, 200 on large tiles): faster or equal.
    // Without channels (C = 0, bias only) there is no contraction to pipeline: the general
    // kernel's empty K loop is the plain choice, and the fast kernel (one K step read from
    // its zero block) runs only when forced.
    const bool has_channels = desc->channels > 0;
    // (the 8-column RoPE's descriptors keep bit 29 for the rotated groups)
    const bool addressable = fp::fast_addressable(r.M, r.S, desc->ff_dim, r.qw) &&
                             (!rope8 || r.S * r.qw < (int64_t(1) << 29));
    // The fast kernel's epilogue takes any q/k/v layout (fewer k/v heads, grouped columns:
    // both are in its column descriptors) and applies every ff activation. Its variants:
    // tanh GELU and squared ReLU, and a channels-first ff output (when ff_dim is a multiple
    // of the wave's 128 columns, with exact GELU or no activation), are compiled without
    // RoPE; the 8-column RoPE with exact GELU or no activation and a token-major ff.
    const bool ff_cf = desc->ff_dim > 0 && desc->ff_layout == FUSED_PROJ_FF_CHANNELS_FIRST;
    const bool other_act = desc->ff_dim > 0 && (desc->ff_act == FUSED_PROJ_ACT_GELU_TANH ||
                                                desc->ff_act == FUSED_PROJ_ACT_RELU_SQUARED);
    h->epi = ff_cf ? 2 : other_act ? 1 : rope8 ? 3 : 0;
    const bool fast_epi = h->epi == 0 || h->epi == 3 ||
                          (!roped && (h->epi == 1 || (!other_act && desc->ff_dim % 128 == 0)));
    h->fast = h->dt == fp::DType::BF16 && dg >= 0 && fits32 && addressable && fast_epi && (has_channels || want_fast) &&
              !want_general;
    h->dg = dg < 0 ? 0 : dg;
    h->tile = h->fast ? fp_plan : fp::TilePlan{128, 128, h->dt == fp::DType::BF16 ? 64 : 32, 8, 0};

    fp::KernelArgs& a = h->base;
    std::memset(&a, 0, sizeof(a));
    a.x_sb = r.sb;
    a.x_ss = r.ss;
    a.x_sc = r.sc;
    a.M = r.M;
    a.S = (int32_t)r.S;
    a.K = (int32_t)desc->channels;
    a.N = (int32_t)r.F;
    a.ff_dim = (int32_t)desc->ff_dim;
    a.n_heads = (int32_t)desc->n_heads;
    a.head_dim = (int32_t)desc->head_dim;
    a.qw = (int32_t)r.qw;
    a.n_kv_heads = (int32_t)r.kvh;
    a.qkv_grouped = desc->qkv_order == FUSED_PROJ_QKV_GROUPED ? 1 : 0;
    a.rope_dims = (int32_t)r.rd;
    a.ff_channels_first = desc->ff_layout == FUSED_PROJ_FF_CHANNELS_FIRST ? 1 : 0;
    a.act = desc->ff_act == FUSED_PROJ_ACT_GELU_ERF      ? 1
            : desc->ff_act == FUSED_PROJ_ACT_GELU_TANH     ? 2
            : desc->ff_act == FUSED_PROJ_ACT_RELU_SQUARED ? 3
                                                           : 0;
    a.rope = (desc->rope && r.qw > 0) ? 1 : 0;
    a.tiles_m = (int32_t)((r.M + h->tile.bm - 1) / h->tile.bm);  // token tiles
    a.tiles_n = (int32_t)((r.F + h->tile.bn - 1) / h->tile.bn);
    a.group_m = h->tile.group_m;
    a.div_s = fp::make_fastdiv_u31((uint32_t)r.S);
    a.div_group = fp::make_fastdiv_u31((uint32_t)((int64_t)a.group_m * a.tiles_n));

    if (a.rope && r.S > 0) {
        // cos/sin of (s + pos_offset) * base^(-2i/rd) for the rotated width rd (the head
        // size unless partial), computed in float64, stored fp32
        const int64_t half = r.rd / 2;
        const size_t n = (size_t)r.S * (size_t)half;
        std::vector<float> hc(n), hs(n);
        std::vector<double> theta((size_t)half);
        for (int64_t i = 0; i < half; ++i)
            theta[(size_t)i] = std::pow(desc->rope_base, -2.0 * (double)i / (double)r.rd);
        for (int64_t s = 0; s < r.S; ++s) {
            const double p = (double)(s + desc->pos_offset);
            for (int64_t i = 0; i < half; ++i) {
                const double phi = p * theta[(size_t)i];
                hc[(size_t)(s * half + i)] = (float)std::cos(phi);
                hs[(size_t)(s * half + i)] = (float)std::sin(phi);
            }
        }
        e = hipMalloc((void**)&h->d_cos, n * sizeof(float));
        if (e == hipSuccess) e = hipMalloc((void**)&h->d_sin, n * sizeof(float));
        if (e == hipSuccess) e = hipMemcpy(h->d_cos, hc.data(), n * sizeof(float), hipMemcpyHostToDevice);
        if (e == hipSuccess) e = hipMemcpy(h->d_sin, hs.data(), n * sizeof(float), hipMemcpyHostToDevice);
        if (e != hipSuccess) {
            g_last_hip = e;
            fused_proj_destroy(h);
            return FUSED_PROJ_EHIP;
        }
    }
    a.rope_cos = h->d_cos;
    a.rope_sin = h->d_sin;
    // a zero block: operand chunks outside the problem are read from its first 256 bytes;
    // the fast kernel's stores outside the problem go to the other 256
    e = hipMalloc(&h->d_zeros, 512);
    if (e == hipSuccess) e = hipMemset(h->d_zeros, 0, 512);
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (e != hipSuccess) {
        g_last_hip = e;
        fused_proj_destroy(h);
        return FUSED_PROJ_EHIP;
    }
    a.zeros = h->d_zeros;
    a.sink = static_cast<char*>(h->d_zeros) + 256;
    if (h->fast) {
        const int64_t n = fp::fast_col_desc_entries(r.F);
        std::vector<unsigned> hd((size_t)n);
        fp::fast_col_desc(r.S, desc->ff_dim, desc->n_heads, r.kvh, desc->head_dim,
                          desc->qkv_order == FUSED_PROJ_QKV_GROUPED, h->epi == 3, r.F, hd.data(), n);
        e = hipMalloc((void**)&h->d_desc, (size_t)n * sizeof(unsigned));
        if (e == hipSuccess) e = hipMemcpy(h->d_desc, hd.data(), (size_t)n * sizeof(unsigned), hipMemcpyHostToDevice);
        if (e != hipSuccess) {
            g_last_hip = e;
            fused_proj_destroy(h);
            return FUSED_PROJ_EHIP;
        }
    }
    a.col_desc = h->d_desc;
    plan_fwd_tail(h);
    if (with_backward) {
        rc = plan_backward(h);
        if (rc == FUSED_PROJ_OK) rc = scratch_setup(h->device);
        if (rc) {
            fused_proj_destroy(h);
            return rc;
        }
    }
    *out = h;
    return FUSED_PROJ_OK;
}

}  // namespace

extern "C" {

int fused_proj_run(fused_proj_t h, const void* x, const void* w, const void* bias, void* ff, void* q, void* k,
                   void* v, void* stream) {
    if (!h) return FUSED_PROJ_EINVAL;
    const Derived& r = h->r;
    if (r.M == 0) return FUSED_PROJ_OK;  // no tokens: nothing to do
    const bool need_xw = h->d.channels > 0;
    if (need_xw && (!x || !w)) return FUSED_PROJ_EINVAL;
    if (h->d.has_bias && !bias) return FUSED_PROJ_EINVAL;
    if (h->d.ff_dim > 0 && !ff) return FUSED_PROJ_EINVAL;
    if (r.qw > 0 && (!q || !k || !v)) return FUSED_PROJ_EINVAL;
    const void* ptrs[] = {need_xw ? x : nullptr, need_xw ? w : nullptr, h->d.has_bias ? bias : nullptr,
                          h->d.ff_dim > 0 ? ff : nullptr, r.qw > 0 ? q : nullptr, r.qw > 0 ? k : nullptr,
                          r.qw > 0 ? v : nullptr};
    for (const void* p : ptrs)
        if (p && (reinterpret_cast<uintptr_t>(p) & 15u)) return FUSED_PROJ_EALIGN;

    // Outputs may overlap neither each other nor an input (at most 3 inputs and 4 outputs:
    // fixed arrays, nothing allocated).
    const uintptr_t es = h->dt == fp::DType::BF16 ? 2 : 4;
    Range ins[3], outs[4];
    int n_in = 0, n_out = 0;
    if (need_xw) {
        ins[n_in++] = {(uintptr_t)x, (uintptr_t)x + (uintptr_t)r.x_span * es};
        ins[n_in++] = {(uintptr_t)w, (uintptr_t)w + (uintptr_t)(h->d.channels * r.F) * es};
    }
    if (h->d.has_bias) ins[n_in++] = {(uintptr_t)bias, (uintptr_t)bias + (uintptr_t)r.F * es};
    if (h->d.ff_dim > 0) outs[n_out++] = {(uintptr_t)ff, (uintptr_t)ff + (uintptr_t)(r.M * h->d.ff_dim) * es};
    if (r.qw > 0) {
        outs[n_out++] = {(uintptr_t)q, (uintptr_t)q + (uintptr_t)(r.M * r.qw) * es};
        outs[n_out++] = {(uintptr_t)k, (uintptr_t)k + (uintptr_t)(r.M * r.kvw) * es};
        outs[n_out++] = {(uintptr_t)v, (uintptr_t)v + (uintptr_t)(r.M * r.kvw) * es};
    }
    for (int i = 0; i < n_out; ++i) {
        for (int j = i + 1; j < n_out; ++j)
            if (overlap(outs[i], outs[j])) return FUSED_PROJ_EALIAS;
        for (int j = 0; j < n_in; ++j)
            if (overlap(outs[i], ins[j])) return FUSED_PROJ_EALIAS;
    }

    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        g_last_hip = e;
        return FUSED_PROJ_EHIP;
    }
    if (dev != h->device) return FUSED_PROJ_EINVAL;

    fp::KernelArgs a = h->base;
    a.x = x;
    a.w = w;
    a.bias = h->d.has_bias ? bias : nullptr;
    a.ff = ff;
    a.q = q;
    a.k = k;
    a.v = v;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (h->tail_m0 > 0) {
        // the head's tokens on the large tiles, then the tail's (whole slabs from tail_m0)
        // on small tiles: every pointer advanced by the tail's first token
        fp::KernelArgs t = h->tail_args;
        const int64_t m0 = h->tail_m0, n1 = m0 / r.S;
        t.x = static_cast<const char*>(x) + (size_t)(n1 * r.sb) * es;
        t.w = w;
        t.bias = a.bias;
        t.ff = ff ? static_cast<char*>(ff) + (size_t)(m0 * h->d.ff_dim) * es : nullptr;
        t.q = q ? static_cast<char*>(q) + (size_t)(m0 * r.qw) * es : nullptr;
        t.k = k ? static_cast<char*>(k) + (size_t)(m0 * r.kvw) * es : nullptr;
        t.v = v ? static_cast<char*>(v) + (size_t)(m0 * r.kvw) * es : nullptr;
        a.M = m0;
        a.tiles_m = (int32_t)((m0 + h->tile.bm - 1) / h->tile.bm);
        e = fp::launch_fused_proj_fast(h->x_tl, h->w_fc, h->dg, h->epi, h->tile, a, s);
        if (e == hipSuccess) e = fp::launch_fused_proj_fast(h->x_tl, h->w_fc, h->dg, h->epi, h->tail_tile, t, s);
    } else {
        e = h->fast ? fp::launch_fused_proj_fast(h->x_tl, h->w_fc, h->dg, h->epi, h->tile, a, s)
                    : fp::launch_fused_proj(h->dt, h->x_tl, h->w_fc, h->tile, a, s);
    }
    if (e == hipSuccess && h->debug_sync) {
        e = hipStreamSynchronize(s);
        if (e == hipSuccess) e = hipGetLastError();
    }
    if (e != hipSuccess) {
        g_last_hip = e;
        return FUSED_PROJ_EHIP;
    }
    return FUSED_PROJ_OK;
}

int fused_proj_destroy(fused_proj_t h) {
    if (!h) return FUSED_PROJ_OK;
    const int rc_sub = fused_proj_destroy(h->dx_plan);
    if (h->d_desc_dy) (void)hipFree(h->d_desc_dy);
    if (h->d_desc_dw) (void)hipFree(h->d_desc_dw);
    hipError_t e1 = h->d_cos ? hipFree(h->d_cos) : hipSuccess;
    hipError_t e2 = h->d_sin ? hipFree(h->d_sin) : hipSuccess;
    hipError_t e3 = h->d_zeros ? hipFree(h->d_zeros) : hipSuccess;
    hipError_t e4 = h->d_desc ? hipFree(h->d_desc) : hipSuccess;
    if (e2 == hipSuccess) e2 = e3;
    if (e2 == hipSuccess) e2 = e4;
    delete h;
    if (e1 != hipSuccess || e2 != hipSuccess) {
        g_last_hip = e1 != hipSuccess ? e1 : e2;
        return FUSED_PROJ_EHIP;
    }
    return rc_sub;
}

int fused_proj_backward_noalloc(fused_proj_t h, const void* x, const void* w, const void* bias,
                                const void* d_ff, const void* dq, const void* dk, const void* dv, void* dx,
                                void* dw, void* db, void* stream) {
    if (!h) return FUSED_PROJ_EINVAL;
    if (h->ws_bytes > kScratchBytes) return FUSED_PROJ_ESCRATCH;
    void* ws = nullptr;
    if (h->ws_bytes > 0) {
        ws = scratch_ptr(h->device);
        if (ws == nullptr) return FUSED_PROJ_EHIP;
    }
    return fused_proj_backward(h, x, w, bias, d_ff, dq, dk, dv, dx, dw, db, ws, ws ? kScratchBytes : 0, stream);
}

size_t fused_proj_noalloc_scratch_bytes(void) { return kScratchBytes; }

int fused_proj_backward_workspace_size(fused_proj_t h, size_t* bytes) {
    if (!h || !bytes) return FUSED_PROJ_EINVAL;
    *bytes = h->ws_bytes;
    return FUSED_PROJ_OK;
}

int fused_proj_backward(fused_proj_t h, const void* x, const void* w, const void* bias, const void* d_ff,
                        const void* dq, const void* dk, const void* dv, void* dx, void* dw, void* db,
                        void* workspace, size_t workspace_bytes, void* stream) {
    if (!h) return FUSED_PROJ_EINVAL;
    const Derived& r = h->r;
    const fused_proj_desc& d = h->d;
    const bool has_c = d.channels > 0, has_m = r.M > 0;
    const bool has_ff = d.ff_dim > 0, has_h = r.qw > 0;
    // required pointers
    if (has_c && ((has_m && (!x || !dx)) || !w || !dw)) return FUSED_PROJ_EINVAL;
    if (d.has_bias && (!bias || !db)) return FUSED_PROJ_EINVAL;
    if (has_m && ((has_ff && !d_ff) || (has_h && (!dq || !dk || !dv)))) return FUSED_PROJ_EINVAL;
    if (h->ws_bytes > 0 && (!workspace || workspace_bytes < h->ws_bytes)) return FUSED_PROJ_EINVAL;
    const uintptr_t es = h->dt == fp::DType::BF16 ? 2 : 4;
    const uintptr_t M = (uintptr_t)r.M, C = (uintptr_t)d.channels, F = (uintptr_t)r.F;
    // inputs: x, w, bias, d_ff, dq, dk, dv; outputs: dx, dw, db, workspace (fixed arrays)
    Range ins[7], outs[4];
    int n_in = 0, n_out = 0;
    auto add = [](Range* arr, int& n, const void* p, uintptr_t bytes) {
        if (p && bytes > 0) arr[n++] = Range{(uintptr_t)p, (uintptr_t)p + bytes};
    };
    add(ins, n_in, has_c && has_m ? x : nullptr, (uintptr_t)r.x_span * es);
    add(ins, n_in, has_c ? w : nullptr, C * F * es);
    add(ins, n_in, d.has_bias ? bias : nullptr, F * es);
    add(ins, n_in, has_m && has_ff ? d_ff : nullptr, M * (uintptr_t)d.ff_dim * es);
    add(ins, n_in, has_m && has_h ? dq : nullptr, M * (uintptr_t)r.qw * es);
    add(ins, n_in, has_m && has_h ? dk : nullptr, M * (uintptr_t)r.kvw * es);
    add(ins, n_in, has_m && has_h ? dv : nullptr, M * (uintptr_t)r.kvw * es);
    add(outs, n_out, has_c && has_m ? dx : nullptr, M * C * es);
    add(outs, n_out, has_c ? dw : nullptr, C * F * es);
    add(outs, n_out, d.has_bias ? db : nullptr, F * es);
    add(outs, n_out, h->ws_bytes > 0 ? workspace : nullptr, h->ws_bytes);
    for (int i = 0; i < n_in; ++i)
        if (ins[i].lo & 15u) return FUSED_PROJ_EALIGN;
    for (int i = 0; i < n_out; ++i)
        if (outs[i].lo & 15u) return FUSED_PROJ_EALIGN;
    for (int i = 0; i < n_out; ++i) {
        for (int j = i + 1; j < n_out; ++j)
            if (overlap(outs[i], outs[j])) return FUSED_PROJ_EALIAS;
        for (int j = 0; j < n_in; ++j)
            if (overlap(outs[i], ins[j])) return FUSED_PROJ_EALIAS;
    }
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        g_last_hip = e;
        return FUSED_PROJ_EHIP;
    }
    if (dev != h->device) return FUSED_PROJ_EINVAL;
    hipStream_t s = static_cast<hipStream_t>(stream);

    if (!has_m) {
        // no tokens: the weight and bias gradients are zero
        if (has_c) e = fp::launch_zero_fill(dw, C * F * es, s);
        if (e == hipSuccess && d.has_bias) e = fp::launch_zero_fill(db, F * es, s);
    } else {
        fp::BwdArgs b = h->bwd;
        b.f.x = x;
        b.f.w = w;
        b.f.bias = d.has_bias ? bias : nullptr;
        b.d_ff = d_ff;
        b.dq = dq;
        b.dk = dk;
        b.dv = dv;
        char* ws = static_cast<char*>(workspace);
        b.dy = ws;
        b.dbp = d.has_bias ? reinterpret_cast<float*>(ws + h->ws_dbp) : nullptr;
        b.dwp = (b.splits > 1 || (h->fast_dw && h->dw_epi == 4)) ? reinterpret_cast<float*>(ws + h->ws_dwp)
                                                                    : nullptr;
        b.dw = dw;
        b.db = d.has_bias ? db : nullptr;
        if (h->fast_dy) {
            fp::KernelArgs a = h->dy_args;
            a.x = x;
            a.w = w;
            a.bias = d.has_bias ? bias : nullptr;
            a.ff = b.dy;
            a.grad_in = d_ff;
            a.colsum = b.dbp;
            e = fp::launch_fused_proj_fast(h->x_tl, h->w_fc, 0, 5, h->dy_tile, a, s);
        }
        if (e == hipSuccess) e = fp::launch_bwd_dy(h->dt, h->x_tl, h->w_fc, b, s);
        if (e == hipSuccess && h->dy_heads) e = fp::launch_bwd_dy_heads(b, b.dy_col_tile1 * 128, s);
        if (e == hipSuccess && has_c && !h->dx_split) {
            const int rc = fused_proj_run(h->dx_plan, b.dy, w, nullptr, dx, nullptr, nullptr, nullptr, stream);
            if (rc) return rc;
        } else if (e == hipSuccess && has_c) {
            // the head's tiles through the nested plan's kernel, the tail's range units, then
            // their reduction into dx
            const fused_proj_plan* xp = h->dx_plan;
            if (h->dx_head_m > 0) {
                fp::KernelArgs a = xp->base;
                a.M = h->dx_head_m;
                a.tiles_m = (int32_t)(h->dx_head_m / 256);
                a.x = b.dy;
                a.w = w;
                a.bias = nullptr;
                a.ff = dx;
                e = fp::launch_fused_proj_fast(xp->x_tl, xp->w_fc, xp->dg, xp->epi, xp->tile, a, s);
            }
            if (e == hipSuccess) {
                fp::KernelArgs a = h->dxt_args;
                a.x = static_cast<const char*>(b.dy) + (size_t)h->dx_head_m * (size_t)F * es;
                a.w = w;
                a.ff = ws + h->ws_dxp;
                e = fp::launch_fused_proj_fast(true, xp->w_fc, 0, 4, h->dxt_tile, a, s);
            }
            b.dxp = reinterpret_cast<float*>(ws + h->ws_dxp);
            b.dx = dx;
            if (e == hipSuccess) e = fp::launch_bwd_reduce_dx(b, s);
        }
        if (e == hipSuccess && has_c) {
            if (h->fast_dw) {
                fp::KernelArgs a = h->dw_args;
                a.x = x;
                a.w = b.dy;
                a.ff = h->dw_epi == 4 ? static_cast<void*>(b.dwp) : dw;
                e = fp::launch_fused_proj_fast(h->dw_x_kmajor, false, 0, h->dw_epi, h->dw_tile, a, s);
            } else {
                e = fp::launch_bwd_dw(h->dt, h->x_tl, b, s);
            }
        }
        if (e == hipSuccess) e = fp::launch_bwd_reduce(h->dt, b, s);
    }
    if (e == hipSuccess && h->debug_sync) {
        e = hipStreamSynchronize(s);
        if (e == hipSuccess) e = hipGetLastError();
    }
    if (e != hipSuccess) {
        g_last_hip = e;
        return FUSED_PROJ_EHIP;
    }
    return FUSED_PROJ_OK;
}

const char* fused_proj_strerror(int code) {
    switch (code) {
        case FUSED_PROJ_OK: return "success";
        case FUSED_PROJ_EINVAL: return "invalid argument";
        case FUSED_PROJ_EUNSUPPORTED: return "unsupported shape, layout or stride";
        case FUSED_PROJ_EALIGN: return "device pointer not 16-byte aligned";
        case FUSED_PROJ_EALIAS: return "output overlaps another output or an input";
        case FUSED_PROJ_ESCRATCH:
            return "the problem needs more scratch memory than the static buffer of the allocation-free entry "
                   "point holds (see fused_proj_noalloc_scratch_bytes)";
        case FUSED_PROJ_EHIP:
            std::snprintf(g_msg, sizeof(g_msg), "HIP error: %s", hipGetErrorString(g_last_hip));
            return g_msg;
        default: return "unknown status code";
    }
}

int fused_proj_describe(fused_proj_t h, char* buf, size_t len) {
    if (!h || !buf || len == 0) return FUSED_PROJ_EINVAL;
    std::snprintf(buf, len,
                  "kernel=%s dtype=%s x=%s w=%s tile=%dx%dx%d group_m=%d grid=%d tiles=%d "
                  "M=%lld K=%lld N=%lld",
                  h->fast ? "fused_proj_fast_kernel" : "fused_proj_tile_kernel",
                  h->dt == fp::DType::BF16 ? "bf16" : "f32", h->x_tl ? "tokens_last" : "channels_first",
                  h->w_fc ? "FC" : "CF", h->tile.bm, h->tile.bn, h->tile.bk, h->tile.group_m,
                  h->tile.grid > 0 ? h->tile.grid : h->base.tiles_m * h->base.tiles_n,
                  h->base.tiles_m * h->base.tiles_n, (long long)h->r.M, (long long)h->d.channels,
                  (long long)h->r.F);
    if (h->tail_m0 > 0) {
        const size_t n = std::strlen(buf);
        if (n + 1 < len)
            std::snprintf(buf + n, len - n, " tail=%lld+%lld tail_tile=%dx%d tail_grid=%d",
                          (long long)h->tail_m0, (long long)(h->r.M - h->tail_m0), h->tail_tile.bm,
                          h->tail_tile.bn, h->tail_tile.grid);
    }
    return FUSED_PROJ_OK;
}

}  // extern "C"
