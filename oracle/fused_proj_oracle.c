/*
 * Fused input projection: float64 CPU oracle.
 *
 * TEST INFRASTRUCTURE ONLY. This file is the plain, slow, obviously correct
 * definition of what the fused projection computes. Only the test suite, the
 * smoke check and the benchmark's CPU-baseline leg may load it. It shares no
 * code, header, table or constant with the GPU library, and it never reads
 * anything the GPU library produced.
 *
 * What it computes, and where each step is stated:
 *
 *  1. Token gather. Walrus PR "Make fused_ff_qkv contiguous" (first comment):
 *     the block takes a channels-first activation x[b,c,h,w,d], views it as
 *     channels-last [b,h,w,d,c] and projects every (b,h,w,d) position, i.e.
 *     one row per token, contracted over c. The same op on a token-major
 *     [b,s,c] activation is the plain linear layer. Tokens are numbered
 *     t = bi*S + s with s the row-major flattening of the spatial indices.
 *
 *  2. Contraction, bias and activation. xformers PR "Fused linear: small FW
 *     cleanup and much better perfs" (description and follow-up comments):
 *     the op is y = act(x W^T + b); for the attention projection it is the
 *     same op with no activation, written into three buffers.
 *     y[t,f] = sum_c x[t,c] * W[c,f] + b[f], summed in increasing c. With no
 *     channels (C = 0, which the pages never meet) the sum is empty: y = b.
 *
 *  3. Split. Walrus PR (second comment): the fused output is split into
 *     ff, q, k, v. Reading: contiguous column slices in that order, each of
 *     the q/k/v slices holding n_heads heads of head_dim columns, head-major.
 *
 *  4. Activation on the ff slice: exact-erf GELU, 0.5*y*(1+erf(y/sqrt 2)).
 *     (The pages name no GELU form; erf is the reading taken.) Two more
 *     activations on the same slice: the tanh form of GELU, from the paper
 *     that defines GELU (Hendrycks and Gimpel, "Gaussian Error Linear Units
 *     (GELUs)", 2016): 0.5*y*(1+tanh(sqrt(2/pi)*(y+0.044715*y^3))); and
 *     squared ReLU, max(y,0)^2, which the xformers PR discussion names among
 *     the activations a fused linear layer handles natively. Non-finite values
 *     (which the pages never meet) go through the formulas in IEEE arithmetic,
 *     and squared ReLU leaves a NaN in place as torch's relu does.
 *
 *  5. Head-major buffers. memory-efficient-attention issue "Improve
 *     performance via batched-matmul and fused multiplies" (first comment):
 *     q/k/v live as [batch*num_heads, tokens, channels_per_head]. This file
 *     writes token-major rows [t, h, j]; the Python side reorders them into
 *     [bi*H + h, s, j] with a plain array transpose.
 *
 *  6. RoPE on q and k. NVIDIA/Fuser issue "Improve performance on RoPE (and
 *     code around it)", rope_one_entry in the thunder example: split the head
 *     into halves x1, x2; the rotated vector is (-x2, x1); the output is
 *     x*cos + rotated*sin. Pairs are (i, i + head_dim/2). The page fills the
 *     cos/sin tables with random numbers, so the angle is the textbook
 *     phi = p * base^(-2i/head_dim) (a convention, not fixed by the pages:
 *     parity unpinned against the pages for the angles; the tests pin the
 *     rotation itself), with p = s + pos_offset, the token's position inside
 *     its slab.
 *
 *  7. The backward pass (oracle_fused_proj_backward below): the gradients of x,
 *     W and the bias by the chain rule through steps 1-6, in reverse order.
 *
 * No step is blocked, fused or reordered beyond that statement.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_OK 0
#define ORACLE_EINVAL (-1)

/* x element for token (bi, s), channel c.
 * The spatial index s is unflattened row-major over sp_size[0..nsp). */
static double x_at(const double *x, int64_t bi, int64_t s, int64_t c, int64_t sb, int64_t sc,
                   int nsp, const int64_t *sp_size, const int64_t *sp_stride)
{
    int64_t off = bi * sb + c * sc;
    int64_t rem = s;
    for (int d = nsp - 1; d >= 0; --d) {
        int64_t idx = rem % sp_size[d];
        rem /= sp_size[d];
        off += idx * sp_stride[d];
    }
    return x[off];
}

static double w_at(const double *w, int64_t c, int64_t f, int64_t C, int64_t F, int w_fc)
{
    /* w_fc == 0: W stored [C, F] (row c holds all outputs of channel c).
     * w_fc == 1: W stored [F, C] (nn.Linear weight, y = x W^T). */
    return w_fc ? w[f * C + c] : w[c * F + f];
}

static double gelu_erf(double y)
{
    return 0.5 * y * (1.0 + erf(y / sqrt(2.0)));
}

static double gelu_tanh(double y)
{
    const double k = sqrt(2.0 / 3.14159265358979323846);
    return 0.5 * y * (1.0 + tanh(k * (y + 0.044715 * y * y * y)));
}

/* max(y, 0)^2; a NaN is not clamped to 0 but passes through, as it does through
 * torch's relu (and through both GELU forms above in IEEE arithmetic). */
static double relu_squared(double y)
{
    const double r = (y > 0.0 || isnan(y)) ? y : 0.0;
    return r * r;
}

/* ff_act: 0 identity, 1 exact-erf GELU, 2 tanh GELU, 3 squared ReLU */
static double activate(int ff_act, double y)
{
    switch (ff_act) {
    case 1: return gelu_erf(y);
    case 2: return gelu_tanh(y);
    case 3: return relu_squared(y);
    default: return y;
    }
}

/* Rotate-half RoPE on the first rd elements of one head vector v at position p, in
 * place (rd even; rd equal to the head size is the full rotation). Elements from rd on
 * are left as they are (partial rotary, rope_one_entry with rope_n_elem in the nvFuser
 * RoPE issue: the angles belong to the rotated width rd). */
static void rope_rotate_half(double *v, int64_t rd, double p, double base)
{
    int64_t half = rd / 2;
    for (int64_t i = 0; i < half; ++i) {
        double theta = pow(base, -2.0 * (double)i / (double)rd);
        double phi = p * theta;
        double cs = cos(phi), sn = sin(phi);
        double x1 = v[i], x2 = v[i + half];
        v[i] = x1 * cs - x2 * sn;        /* x1*cos + (-x2)*sin */
        v[i + half] = x2 * cs + x1 * sn; /* x2*cos + ( x1)*sin */
    }
}

/* Destination of column r of the q/k/v part of the fused output (column ff_dim + r):
 * which (0 q, 1 k, 2 v), head and element j. Contiguous order: all q heads, then the k
 * heads, then the v heads. Grouped order (split_qkv in the nvFuser RoPE issue, the
 * lit-gpt layout): n_kv groups of q_per_kv q heads, one k head and one v head; q head i
 * of group g is head g*q_per_kv + i. */
static void qkv_column(int64_t r, int64_t n_heads, int64_t n_kv, int64_t hd, int grouped, int *which,
                       int64_t *head, int64_t *j)
{
    *j = r % hd;
    if (!grouped) {
        const int64_t qw = n_heads * hd, kvw = n_kv * hd;
        if (r < qw) {
            *which = 0;
            *head = r / hd;
        } else if (r < qw + kvw) {
            *which = 1;
            *head = (r - qw) / hd;
        } else {
            *which = 2;
            *head = (r - qw - kvw) / hd;
        }
    } else {
        const int64_t qpk = n_heads / n_kv, gw = (qpk + 2) * hd;
        const int64_t g = r / gw, slot = (r % gw) / hd;
        if (slot < qpk) {
            *which = 0;
            *head = g * qpk + slot;
        } else {
            *which = slot == qpk ? 1 : 2;
            *head = g;
        }
    }
}

/*
 * Computes the fused projection for the tokens listed in tokens[0..ntok).
 *
 *   x        float64 activation; element (bi, c, s) at
 *            bi*sb + c*sc + sum_d idx_d(s)*sp_stride[d]
 *   nb, C, S slabs, channels, tokens per slab (S = prod sp_size); C may be 0,
 *            an empty contraction: y is then the bias (or zero)
 *   w        float64 weight, [C,F] (w_fc=0) or [F,C] (w_fc=1)
 *   bias     float64 [F] or NULL
 *   ff_dim   width of the ff slice; F = ff_dim + 3*n_heads*head_dim
 *   ff_act   activation on the ff slice: 0 identity, 1 exact-erf GELU,
 *            2 tanh GELU, 3 squared ReLU
 *   n_kv     k and v heads (0: n_heads); must divide n_heads
 *   grouped  0: q/k/v columns in contiguous order, 1: grouped per k/v head
 *   rope_dims rotated width of each q and k head (0: head_dim); even
 *   rope     1: rotate-half RoPE on q and k
 *   tokens   global token indices t = bi*S + s, each in [0, nb*S)
 *   outputs  token-major rows: ff_rows [ntok, ff_dim],
 *            q_rows [ntok, n_heads*head_dim], k_rows/v_rows
 *            [ntok, n_kv*head_dim]; any may be NULL
 *            when its slice is empty.
 *   nthreads OpenMP threads (<= 0: runtime default)
 * Returns 0, or -1 on an invalid argument (nothing is written then).
 */
int oracle_fused_proj(const double *x, int64_t nb, int64_t C, int64_t S, int64_t sb, int64_t sc,
                      int nsp, const int64_t *sp_size, const int64_t *sp_stride,
                      const double *w, int64_t F, int w_fc, const double *bias,
                      int64_t ff_dim, int ff_act, int64_t n_heads, int64_t head_dim,
                      int64_t n_kv, int grouped, int64_t rope_dims,
                      int rope, double rope_base, int64_t pos_offset,
                      const int64_t *tokens, int64_t ntok,
                      double *ff_rows, double *q_rows, double *k_rows, double *v_rows,
                      int nthreads)
{
    if (!x || !w || !tokens || nb <= 0 || C < 0 || S <= 0 || nsp < 1 || nsp > 3 || ntok < 0)
        return ORACLE_EINVAL;
    int64_t prod = 1;
    for (int d = 0; d < nsp; ++d) {
        if (sp_size[d] <= 0) return ORACLE_EINVAL;
        prod *= sp_size[d];
    }
    if (prod != S) return ORACLE_EINVAL;
    if (ff_dim < 0 || n_heads < 0 || head_dim < 0) return ORACLE_EINVAL;
    if (ff_act < 0 || ff_act > 3) return ORACLE_EINVAL;
    if (n_kv == 0) n_kv = n_heads;
    if (n_kv < 0 || (n_heads > 0 && (n_kv == 0 || n_heads % n_kv != 0)) || (grouped != 0 && grouped != 1))
        return ORACLE_EINVAL;
    const int64_t qw = n_heads * head_dim, kvw = n_kv * head_dim;
    if (F != ff_dim + qw + 2 * kvw || F <= 0) return ORACLE_EINVAL;
    const int64_t rd = rope_dims > 0 ? rope_dims : head_dim;
    if (rope && (rd % 2 != 0 || rd > head_dim)) return ORACLE_EINVAL;
    if (ff_dim > 0 && !ff_rows) return ORACLE_EINVAL;
    if (qw > 0 && (!q_rows || !k_rows || !v_rows)) return ORACLE_EINVAL;
    for (int64_t i = 0; i < ntok; ++i)
        if (tokens[i] < 0 || tokens[i] >= nb * S) return ORACLE_EINVAL;

#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif

    int status = ORACLE_OK;
#pragma omp parallel
    {
        double *y = (double *)malloc((size_t)F * sizeof(double));
        double *xr = (double *)malloc((size_t)(C > 0 ? C : 1) * sizeof(double));
        if (!y || !xr) {
#pragma omp atomic write
            status = ORACLE_EINVAL;
        }
#pragma omp for schedule(dynamic, 16)
        for (int64_t i = 0; i < ntok; ++i) {
            if (!y || !xr) continue;
            const int64_t t = tokens[i];
            const int64_t bi = t / S, s = t % S;
            /* 1. gather the token's row */
            for (int64_t c = 0; c < C; ++c)
                xr[c] = x_at(x, bi, s, c, sb, sc, nsp, sp_size, sp_stride);
            /* 2. contraction, sequential in c for every output column */
            for (int64_t f = 0; f < F; ++f) y[f] = 0.0;
            if (!w_fc) {
                for (int64_t c = 0; c < C; ++c) {
                    const double xc = xr[c];
                    const double *wr = w + c * F;
                    for (int64_t f = 0; f < F; ++f) y[f] += xc * wr[f];
                }
            } else {
                for (int64_t f = 0; f < F; ++f) {
                    double acc = 0.0;
                    for (int64_t c = 0; c < C; ++c) acc += xr[c] * w_at(w, c, f, C, F, 1);
                    y[f] = acc;
                }
            }
            /* bias */
            if (bias)
                for (int64_t f = 0; f < F; ++f) y[f] += bias[f];
            /* 3+4. ff slice with activation */
            for (int64_t f = 0; f < ff_dim; ++f)
                ff_rows[i * ff_dim + f] = activate(ff_act, y[f]);
            /* 3+6. q, k, v slices; RoPE on q and k per head */
            if (qw > 0) {
                double *dst[3] = {q_rows + i * qw, k_rows + i * kvw, v_rows + i * kvw};
                for (int64_t r = 0; r < qw + 2 * kvw; ++r) {
                    int which;
                    int64_t head, j;
                    qkv_column(r, n_heads, n_kv, head_dim, grouped, &which, &head, &j);
                    dst[which][head * head_dim + j] = y[ff_dim + r];
                }
                for (int which = 0; rope && which < 2; ++which)
                    for (int64_t h = 0; h < (which == 0 ? n_heads : n_kv); ++h)
                        rope_rotate_half(dst[which] + h * head_dim, rd, (double)(s + pos_offset), rope_base);
            }
        }
        free(y);
        free(xr);
    }
    return status;
}

/*
 * Split + RoPE of an already projected q/k/v tensor (the nvFuser RoPE issue's
 * split_qkv followed by rope_one_entry on q and k): qkv [nb, T, (H + 2*KVH)*hd]
 * token-major, columns in contiguous or grouped order (qkv_column). Outputs:
 * q [nb*H, T, hd], v [nb*KVH, T, hd], and k [nb*KVH, T, hd], or [nb*KVH, hd, T]
 * with k_transposed = 1 (the pre-transposed key of the memory-efficient-attention
 * issue). RoPE on the first rope_dims elements of each q and k head at position
 * s + pos_offset. Returns 0, or -1 on an invalid argument.
 */
int oracle_split_rope(const double *qkv, int64_t nb, int64_t T, int64_t n_heads, int64_t n_kv, int64_t hd,
                      int grouped, int rope, int64_t rope_dims, double rope_base, int64_t pos_offset,
                      int k_transposed, double *q, double *k, double *v)
{
    if (!qkv || !q || !k || !v || nb <= 0 || T <= 0 || n_heads <= 0 || hd <= 0) return ORACLE_EINVAL;
    if (n_kv == 0) n_kv = n_heads;
    if (n_kv < 0 || n_heads % n_kv != 0 || (grouped != 0 && grouped != 1)) return ORACLE_EINVAL;
    const int64_t rd = rope_dims > 0 ? rope_dims : hd;
    if (rope && (rd % 2 != 0 || rd > hd)) return ORACLE_EINVAL;
    const int64_t Fq = (n_heads + 2 * n_kv) * hd;
    double *head = (double *)malloc((size_t)hd * sizeof(double));
    if (!head) return ORACLE_EINVAL;
    for (int64_t bi = 0; bi < nb; ++bi) {
        for (int64_t s = 0; s < T; ++s) {
            const double *row = qkv + (bi * T + s) * Fq;
            /* every head of this token: gather its hd columns, rotate, store */
            for (int which = 0; which < 3; ++which) {
                const int64_t heads = which == 0 ? n_heads : n_kv;
                for (int64_t h = 0; h < heads; ++h) {
                    for (int64_t r = 0; r < Fq; ++r) {
                        int wh;
                        int64_t hh, j;
                        qkv_column(r, n_heads, n_kv, hd, grouped, &wh, &hh, &j);
                        if (wh == which && hh == h) head[j] = row[r];
                    }
                    if (rope && which < 2) rope_rotate_half(head, rd, (double)(s + pos_offset), rope_base);
                    for (int64_t j = 0; j < hd; ++j) {
                        const int64_t slab = bi * heads + h;
                        if (which == 0) q[(slab * T + s) * hd + j] = head[j];
                        else if (which == 2) v[(slab * T + s) * hd + j] = head[j];
                        else if (!k_transposed) k[(slab * T + s) * hd + j] = head[j];
                        else k[(slab * hd + j) * T + s] = head[j];
                    }
                }
            }
        }
    }
    free(head);
    return ORACLE_OK;
}

/* ---------------------------------------------------------------- backward pass
 *
 * The gradient of the fused projection (the backward pass the xformers PR "Fused
 * linear: small FW cleanup and much better perfs" discusses in its follow-up comments:
 * the weight and input gradients of y = act(x W^T + b)), by the chain rule through the
 * forward steps above, in their reverse order. Given the upstream gradients of the
 * four outputs (d_ff, dq, dk, dv, laid out like the outputs):
 *
 *  a. dy[t, f], the gradient of the fused pre-activation output y[t, f]:
 *     - ff column f: d_ff[t, f] * act'(y[t, f]), with y recomputed as in the forward;
 *     - q/k head: RoPE is a rotation R_p of each pair (i, i + rd/2), so the gradient of
 *       the head before the rotation is R_p^T (the rotation by -phi) applied to the
 *       head's upstream gradient; elements from rd on, and v, pass through;
 *  b. dx[t, c] = sum_f dy[t, f] * W[c, f]   (summed in increasing f);
 *  c. dW[c, f] = sum_t x[t, c] * dy[t, f]   (summed in increasing t);
 *  d. db[f]    = sum_t dy[t, f].
 *
 * act' in float64: exact GELU  Phi(y) + y phi(y);
 *                  tanh GELU   0.5 (1 + tanh u) + 0.5 y (1 - tanh^2 u) u'(y),
 *                              u = sqrt(2/pi) (y + 0.044715 y^3);
 *                  squared ReLU 2 max(y, 0);  identity 1.
 */
static double activate_grad(int ff_act, double y)
{
    switch (ff_act) {
    case 1: {
        const double pdf = exp(-0.5 * y * y) / sqrt(2.0 * 3.14159265358979323846);
        return 0.5 * (1.0 + erf(y / sqrt(2.0))) + y * pdf;
    }
    case 2: {
        const double k = sqrt(2.0 / 3.14159265358979323846);
        const double u = k * (y + 0.044715 * y * y * y);
        const double th = tanh(u);
        const double du = k * (1.0 + 3.0 * 0.044715 * y * y);
        return 0.5 * (1.0 + th) + 0.5 * y * (1.0 - th * th) * du;
    }
    case 3: return y > 0.0 ? 2.0 * y : 0.0;
    default: return 1.0;
    }
}

/* The transpose of rope_rotate_half: rotate each pair (i, i + rd/2) of g by -phi. */
static void rope_rotate_half_transposed(double *g, int64_t rd, double p, double base)
{
    int64_t half = rd / 2;
    for (int64_t i = 0; i < half; ++i) {
        double theta = pow(base, -2.0 * (double)i / (double)rd);
        double phi = p * theta;
        double cs = cos(phi), sn = sin(phi);
        double g1 = g[i], g2 = g[i + half];
        g[i] = g1 * cs + g2 * sn;
        g[i + half] = g2 * cs - g1 * sn;
    }
}

/*
 * Backward pass for every token of the batch. Arguments as oracle_fused_proj, plus:
 *   ff_cf    layout of d_ff: 0 [nb, S, ff_dim], 1 [nb, ff_dim, S]
 *   d_ff     float64 upstream gradient of ff (NULL when ff_dim == 0)
 *   dq       float64 [nb*n_heads, S, head_dim]; dk, dv [nb*n_kv, S, head_dim]
 *            (NULL when there are no heads)
 * Outputs (float64, all written):
 *   dy       [nb*S, F] token-major: the gradient of the fused output y
 *   dx_rows  [nb*S, C] token-major rows of the input gradient
 *   dw       [C, F] (whatever the layout of w)
 *   db       [F], or NULL
 * Returns 0, or -1 on an invalid argument.
 */
int oracle_fused_proj_backward(const double *x, int64_t nb, int64_t C, int64_t S, int64_t sb, int64_t sc,
                               int nsp, const int64_t *sp_size, const int64_t *sp_stride,
                               const double *w, int64_t F, int w_fc, const double *bias,
                               int64_t ff_dim, int ff_act, int64_t n_heads, int64_t head_dim,
                               int64_t n_kv, int grouped, int64_t rope_dims,
                               int rope, double rope_base, int64_t pos_offset, int ff_cf,
                               const double *d_ff, const double *dq, const double *dk, const double *dv,
                               double *dy, double *dx_rows, double *dw, double *db, int nthreads)
{
    if (!x || !w || !dy || !dx_rows || !dw || nb <= 0 || C < 0 || S <= 0 || nsp < 1 || nsp > 3)
        return ORACLE_EINVAL;
    int64_t prod = 1;
    for (int d = 0; d < nsp; ++d) {
        if (sp_size[d] <= 0) return ORACLE_EINVAL;
        prod *= sp_size[d];
    }
    if (prod != S) return ORACLE_EINVAL;
    if (ff_dim < 0 || n_heads < 0 || head_dim < 0 || ff_act < 0 || ff_act > 3) return ORACLE_EINVAL;
    if (n_kv == 0) n_kv = n_heads;
    if (n_kv < 0 || (n_heads > 0 && (n_kv == 0 || n_heads % n_kv != 0)) || (grouped != 0 && grouped != 1))
        return ORACLE_EINVAL;
    const int64_t qw = n_heads * head_dim, kvw = n_kv * head_dim;
    if (F != ff_dim + qw + 2 * kvw || F <= 0) return ORACLE_EINVAL;
    const int64_t rd = rope_dims > 0 ? rope_dims : head_dim;
    if (rope && (rd % 2 != 0 || rd > head_dim)) return ORACLE_EINVAL;
    if (ff_dim > 0 && !d_ff) return ORACLE_EINVAL;
    if (qw > 0 && (!dq || !dk || !dv)) return ORACLE_EINVAL;
    const int64_t M = nb * S;

#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif

    int status = ORACLE_OK;
    /* a + b: per token, the gradient of y, then the input gradient */
#pragma omp parallel
    {
        double *y = (double *)malloc((size_t)F * sizeof(double));
        double *xr = (double *)malloc((size_t)(C > 0 ? C : 1) * sizeof(double));
        double *g = (double *)malloc((size_t)(head_dim > 0 ? head_dim : 1) * sizeof(double));
        if (!y || !xr || !g) {
#pragma omp atomic write
            status = ORACLE_EINVAL;
        }
#pragma omp for schedule(dynamic, 16)
        for (int64_t t = 0; t < M; ++t) {
            if (!y || !xr || !g) continue;
            const int64_t bi = t / S, s = t % S;
            double *dyt = dy + t * F;
            /* the forward pre-activation output of the ff slice */
            if (ff_dim > 0 && ff_act != 0) {
                for (int64_t c = 0; c < C; ++c)
                    xr[c] = x_at(x, bi, s, c, sb, sc, nsp, sp_size, sp_stride);
                for (int64_t f = 0; f < ff_dim; ++f) {
                    double acc = 0.0;
                    for (int64_t c = 0; c < C; ++c) acc += xr[c] * w_at(w, c, f, C, F, w_fc);
                    y[f] = acc + (bias ? bias[f] : 0.0);
                }
            }
            for (int64_t f = 0; f < ff_dim; ++f) {
                const double up = ff_cf ? d_ff[(bi * ff_dim + f) * S + s] : d_ff[t * ff_dim + f];
                dyt[f] = up * activate_grad(ff_act, ff_act != 0 ? y[f] : 0.0);
            }
            /* q, k, v heads: each head's upstream gradient, rotated back for q and k,
             * scattered to its fused columns */
            for (int which = 0; qw > 0 && which < 3; ++which) {
                const int64_t heads = which == 0 ? n_heads : n_kv;
                const double *src = which == 0 ? dq : which == 1 ? dk : dv;
                for (int64_t h = 0; h < heads; ++h) {
                    for (int64_t j = 0; j < head_dim; ++j)
                        g[j] = src[((bi * heads + h) * S + s) * head_dim + j];
                    if (rope && which < 2)
                        rope_rotate_half_transposed(g, rd, (double)(s + pos_offset), rope_base);
                    for (int64_t r = 0; r < qw + 2 * kvw; ++r) {
                        int wh;
                        int64_t hh, j;
                        qkv_column(r, n_heads, n_kv, head_dim, grouped, &wh, &hh, &j);
                        if (wh == which && hh == h) dyt[ff_dim + r] = g[j];
                    }
                }
            }
            /* b. dx[t, c] = sum_f dy[t, f] W[c, f] */
            for (int64_t c = 0; c < C; ++c) {
                double acc = 0.0;
                for (int64_t f = 0; f < F; ++f) acc += dyt[f] * w_at(w, c, f, C, F, w_fc);
                dx_rows[t * C + c] = acc;
            }
        }
        free(y);
        free(xr);
        free(g);
    }
    if (status != ORACLE_OK) return status;
    /* c. dW[c, f] = sum_t x[t, c] dy[t, f] */
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t c = 0; c < C; ++c) {
        double *row = dw + c * F;
        for (int64_t f = 0; f < F; ++f) row[f] = 0.0;
        for (int64_t t = 0; t < M; ++t) {
            const double xv = x_at(x, t / S, t % S, c, sb, sc, nsp, sp_size, sp_stride);
            const double *dyt = dy + t * F;
            for (int64_t f = 0; f < F; ++f) row[f] += xv * dyt[f];
        }
    }
    /* d. db[f] = sum_t dy[t, f] */
    if (db) {
        for (int64_t f = 0; f < F; ++f) db[f] = 0.0;
        for (int64_t t = 0; t < M; ++t)
            for (int64_t f = 0; f < F; ++f) db[f] += dy[t * F + f];
    }
    return ORACLE_OK;
}

/* Threads the OpenMP runtime would use by default (for reporting). */
int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
