/*
 * fused_proj.h — C ABI of the MI355X (gfx950) fused input projection.
 *
 * The operation (one call = one kernel launch):
 *
 *   For every token t = bi*S + s of a batch of activations, gather its row
 *   x[t, 0..C) straight from a channels-first [b, c, spatial...] or a
 *   token-major [b, s, c] tensor (no rearranged copy), and compute
 *
 *     y[t, f] = sum_c x[t, c] * W[c, f] + bias[f],        f in [0, F)
 *
 *   as one [tokens, C] x [C, F] product. The columns split into an ff slice
 *   [0, ff_dim), then H q heads and KVH k and v heads of head_dim columns each
 *   (F = ff_dim + (H + 2*KVH)*hd). In the default contiguous order the q slice
 *   comes first (head h, element j at slice column h*hd + j), then the k slice,
 *   then the v slice; FUSED_PROJ_QKV_GROUPED groups them per k/v head instead.
 *
 *     ff[bi, s, f]            = act(y[t, f])                    act: see FUSED_PROJ_ACT_*
 *                               (or ff[bi, f, s], see FUSED_PROJ_FF_*)
 *     q[bi*H + h, s, j]       = RoPE_p(q head h of y[t, .])[j]  p = s + pos_offset
 *     k[bi*KVH + g, s, j]     = RoPE_p(k head g of y[t, .])[j]
 *     v[bi*KVH + g, s, j]     = v head g of y[t, .], element j
 *
 *   RoPE is rotate-half over the first rd = rope_dims (default hd) elements of a
 *   head: for i < rd/2, with phi = p * base^(-2i/rd),
 *     out[i]        = y[i] cos(phi) - y[i + rd/2] sin(phi)
 *     out[i + rd/2] = y[i + rd/2] cos(phi) + y[i] sin(phi),
 *   and elements from rd on pass through.
 *   Accumulation, bias, the activation and RoPE run in fp32; each output is
 *   rounded once to the storage type (round to nearest even).
 *
 * Where each part is defined:
 *   - gather + single GEMM instead of one GEMV per token: Walrus PR
 *     "Make fused_ff_qkv contiguous", first comment (the rearrange from
 *     channels-first to channels-last and the [tokens, fused_dims] product);
 *   - y = act(x W^T + b), and the attention projection as the same op with no
 *     activation written into three buffers: xformers PR "Fused linear: small
 *     FW cleanup and much better perfs", description and follow-up comments;
 *   - the ff, q, k, v split of the fused output: Walrus PR, second comment;
 *   - head-major [batch*heads, tokens, head_dim] buffers: memory-efficient-
 *     attention issue "Improve performance via batched-matmul and fused
 *     multiplies", first comment;
 *   - rotate-half RoPE: NVIDIA/Fuser issue "Improve performance on RoPE (and
 *     code around it)", rope_one_entry in the thunder example. The angle
 *     convention base^(-2i/hd) is the textbook one (the page's tables are
 *     random numbers).
 *
 * Threading: a handle may be used from several host threads and streams at
 * once; fused_proj_run only reads it. Create and destroy are not concurrent
 * with runs on the same handle.
 */
#ifndef FUSED_PROJ_H
#define FUSED_PROJ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes (every call returns one; 0 is success). */
#define FUSED_PROJ_OK 0
#define FUSED_PROJ_EINVAL (-1)       /* malformed descriptor or argument (NULL, negative size, F mismatch) */
#define FUSED_PROJ_EUNSUPPORTED (-2) /* well formed, but outside what the kernels handle (see validate) */
#define FUSED_PROJ_EALIGN (-3)       /* a device pointer is not 16-byte aligned */
#define FUSED_PROJ_EALIAS (-4)       /* an output overlaps another output or an input */
#define FUSED_PROJ_EHIP (-5)         /* a HIP runtime call failed (allocation, copy, launch) */
#define FUSED_PROJ_ESCRATCH (-6)     /* fused_proj_backward_noalloc: the workspace this problem needs
                                        exceeds the static scratch buffer */

/* Storage type of x, W, bias and every output. Accumulation is always fp32. */
#define FUSED_PROJ_BF16 0
#define FUSED_PROJ_F32 1

/* Activation layout. */
#define FUSED_PROJ_X_CHANNELS_FIRST 0 /* [b, c, spatial...]: tokens are the row-major flattening of the
                                         1-3 spatial dims; channel c of token s is x_stride_channel apart */
#define FUSED_PROJ_X_TOKENS_LAST 1    /* [b, s, c]: one spatial dim (s); channels contiguous */

/* Weight layout (both dense, row-major). */
#define FUSED_PROJ_W_CF 0 /* W[C, F]: W[c*F + f] */
#define FUSED_PROJ_W_FC 1 /* W[F, C] (torch nn.Linear weight, y = x W^T): W[f*C + c] */

/* Activation on the ff slice. Non-finite values come out as the formulas below give them
 * in IEEE arithmetic: a NaN anywhere in a token's row of x, in a column of W or in the
 * bias stays NaN through the contraction, every activation and RoPE (squared ReLU keeps
 * NaN too); GELU(+inf) = +inf and GELU(-inf) = NaN in both forms; max(-inf, 0)^2 = 0.
 * No NaN becomes a finite value. A non-finite x element reaches only its own token's
 * outputs; one in W or the bias only its own column's (and, with RoPE, its partner's). */
#define FUSED_PROJ_ACT_NONE 0
#define FUSED_PROJ_ACT_GELU_ERF 1 /* 0.5 y (1 + erf(y / sqrt 2)) */
/* 0.5 y (1 + tanh(sqrt(2/pi) (y + 0.044715 y^3))): the tanh form of GELU from the paper that
 * defines GELU (Hendrycks and Gimpel, "Gaussian Error Linear Units (GELUs)", 2016). */
#define FUSED_PROJ_ACT_GELU_TANH 2
/* max(y, 0)^2: squared ReLU, which the xformers PR "Fused linear: small FW cleanup and much
 * better perfs" discussion names among the activations a fused linear layer handles
 * natively. */
#define FUSED_PROJ_ACT_RELU_SQUARED 3

/* Order of the q, k and v columns after the ff slice. */
#define FUSED_PROJ_QKV_CONTIGUOUS 0 /* all q heads, then the k heads, then the v heads */
/* n_kv_heads groups, each holding n_heads/n_kv_heads q heads, then one k head and one v head;
 * q head i of group g is head g*(n_heads/n_kv_heads) + i (split_qkv in the NVIDIA/Fuser issue
 * "Improve performance on RoPE (and code around it)", the lit-gpt layout). k and v are written
 * once per group, not repeated for every q head. */
#define FUSED_PROJ_QKV_GROUPED 1

/* Layout of the ff output. */
#define FUSED_PROJ_FF_TOKENS_LAST 0   /* ff[bi, s, f] */
/* ff[bi, f, s]: channels-first like x, the output of the equivalent 1x1x1 convolution (the
 * Walrus PR compares the fused linear with a 1x1x1 Conv3d). */
#define FUSED_PROJ_FF_CHANNELS_FIRST 1

typedef struct fused_proj_desc {
    int32_t dtype;             /* FUSED_PROJ_BF16 | FUSED_PROJ_F32 */
    int32_t x_layout;          /* FUSED_PROJ_X_* */
    int64_t batch;             /* b >= 0 (slabs; time steps may be folded in); with b = 0
                                  fused_proj_run does nothing */
    int64_t channels;          /* C >= 0, the contraction length; with C = 0 every output
                                  is computed from the bias alone (y = bias) */
    int32_t n_spatial;         /* 1..3 for channels-first, exactly 1 for tokens-last */
    int64_t spatial[3];        /* sizes of the spatial dims; S = their product */
    int64_t x_stride_batch;    /* element strides of x, all >= 0; their layout is checked
                                  only when x holds elements (C > 0 and b*S > 0) */
    int64_t x_stride_channel;
    int64_t x_stride_spatial[3];
    int32_t w_layout;          /* FUSED_PROJ_W_* */
    int32_t has_bias;          /* 1: bias[F] (storage type) is added to every column */
    int64_t ff_dim;            /* width of the ff slice, >= 0 */
    int32_t ff_act;            /* FUSED_PROJ_ACT_* */
    int64_t n_heads;           /* H >= 0; q holds H*head_dim columns, k and v KVH*head_dim */
    int64_t head_dim;          /* hd >= 0 */
    int32_t rope;              /* 1: rotate-half RoPE on q and k */
    double rope_base;          /* > 0; 10000 is customary */
    int64_t pos_offset;        /* >= 0; position of token s is s + pos_offset */
    /* Fields below are zero in a zero-initialised descriptor, which keeps the plain
     * multi-head layout: as many k/v heads as q heads, contiguous order, full rotation. */
    int64_t n_kv_heads;        /* k and v heads, dividing n_heads; 0 means n_heads */
    int32_t qkv_order;         /* FUSED_PROJ_QKV_* */
    int64_t rope_dims;         /* rotated width of each q/k head: even, <= head_dim; 0 means
                                  head_dim. Elements from rope_dims on pass through; the
                                  angles are (s + pos_offset) * base^(-2i/rope_dims)
                                  (rope_one_entry with rope_n_elem in the same issue). */
    int32_t ff_layout;         /* FUSED_PROJ_FF_*; channels-first needs S a multiple of V */
} fused_proj_desc;

typedef struct fused_proj_plan *fused_proj_t;

/*
 * Checks a descriptor on the host; touches no GPU and allocates nothing.
 * Returns FUSED_PROJ_OK, FUSED_PROJ_EINVAL (malformed: a size < 0, F = ff_dim +
 * (H + 2*KVH)*hd == 0, n_spatial out of range, unknown enum, KVH not dividing H,
 * rope_dims odd or above hd with RoPE, base <= 0) or FUSED_PROJ_EUNSUPPORTED.
 * Supported, with V = 8 for bf16 and 4 for fp32:
 *   C, ff_dim and head_dim multiples of V; with RoPE, 128 a multiple of head_dim
 *   and ff_dim a multiple of head_dim;
 *   channels-first: spatial strides that flatten into one unit-stride token
 *   index (stride of the last spatial dim 1, each outer stride the product of the
 *   inner sizes), S, x_stride_channel and x_stride_batch multiples of V;
 *   tokens-last: x_stride_channel 1, token and batch strides multiples of V
 *   (the stride rules of both layouts apply only when x holds elements: C > 0
 *   and b*S > 0; S stays a multiple of V for channels-first);
 *   every element offset of x, W and the outputs below 2^62.
 */
int fused_proj_validate(const fused_proj_desc *desc);

/*
 * Validates, picks the kernel and tile plan, and (with RoPE) builds the cos/sin
 * table for positions pos_offset .. pos_offset+S-1 in float64, rounds it to fp32
 * and uploads it to the current HIP device (synchronous; this is the only call
 * that allocates or synchronises). On success *out owns that table.
 * Errors: as validate, FUSED_PROJ_EINVAL for out == NULL, FUSED_PROJ_EHIP.
 */
int fused_proj_create(const fused_proj_desc *desc, fused_proj_t *out);

/*
 * Enqueues the projection on `stream` (a hipStream_t; NULL = the legacy default
 * stream of the current device) and returns without waiting. Allocates nothing
 * and never synchronises, so it may be captured into a HIP graph.
 *
 *   x     device, storage type, laid out as the descriptor says
 *   w     device, [C,F] or [F,C] dense
 *   bias  device [F] when has_bias, else ignored (may be NULL)
 *   ff    device [b, S, ff_dim] dense token-major; required when ff_dim > 0
 *   q,k,v device [b*H, S, hd] dense head-major; required when H*hd > 0
 * The caller owns every buffer and keeps them alive until the work completes.
 * Every pointer must be 16-byte aligned (FUSED_PROJ_EALIGN); outputs may not
 * overlap each other or any input (FUSED_PROJ_EALIAS); a NULL required pointer
 * is FUSED_PROJ_EINVAL. A failed launch returns FUSED_PROJ_EHIP; faults inside
 * the kernel surface at the caller's next synchronisation, as for any launch.
 * With FUSED_PROJ_DEBUG_SYNC=1 in the environment the call synchronises the
 * stream and reports kernel errors as FUSED_PROJ_EHIP (debugging only).
 */
int fused_proj_run(fused_proj_t plan, const void *x, const void *w, const void *bias, void *ff, void *q,
                   void *k, void *v, void *stream);

/* Frees the plan and its table. NULL is accepted. Not concurrent with runs in flight
 * on the plan: synchronise their streams first. */
int fused_proj_destroy(fused_proj_t plan);

/* Human-readable text for a status code (static storage). For FUSED_PROJ_EHIP the
 * text of the last HIP error seen by this library on the calling thread follows. */
const char *fused_proj_strerror(int code);

/*
 * Backward pass. Given the upstream gradients of the four outputs, computes the
 * gradients of x, W and the bias (the backward pass of y = act(x W^T + b) that the
 * xformers PR "Fused linear: small FW cleanup and much better perfs" discusses in its
 * follow-up comments), by the chain rule through the forward steps in reverse:
 *
 *   dy[t, f]  = d_ff[t, f] * act'(y[t, f])          ff columns (y recomputed from x, W, b)
 *   dy[t, ..] = R_p^T dq (dk) of the head             q and k: RoPE's rotation transposed
 *                                                     (rotation by -phi) over the first
 *                                                     rope_dims elements, the rest copied
 *   dy[t, ..] = dv of the head                        v
 *   dx[t, c]  = sum_f dy[t, f] W[c, f]
 *   dW[c, f]  = sum_t x[t, c] dy[t, f]
 *   db[f]     = sum_t dy[t, f]
 *
 * Accumulation in fp32; dy is rounded once to the storage type (it lives in the
 * workspace), every gradient once more when stored.
 *
 * fused_proj_backward_workspace_size: bytes of device workspace fused_proj_backward
 * needs for this plan (0 when there are no tokens). Returns FUSED_PROJ_OK or
 * FUSED_PROJ_EINVAL (NULL argument).
 */
int fused_proj_backward_workspace_size(fused_proj_t plan, size_t *bytes);

/*
 * Enqueues the backward pass on `stream` (asynchronous; allocates nothing, never
 * synchronises, so it may be captured into a HIP graph).
 *
 *   x, w, bias  the forward inputs (device, as for fused_proj_run); bias required when
 *               has_bias
 *   d_ff        device, laid out like ff ([b, S, ff_dim], or [b, ff_dim, S] with
 *               FUSED_PROJ_FF_CHANNELS_FIRST); required when ff_dim > 0
 *   dq          device [b*H, S, hd]; dk, dv [b*KVH, S, hd]; required when H*hd > 0
 *   dx          device, dense in x's logical shape: [b, C, spatial...] for a
 *               channels-first x, [b, S, C] for a token-major one (whatever x's strides)
 *   dw          device, in W's layout ([C, F] or [F, C])
 *   db          device [F] when has_bias, else ignored
 *   workspace   device, at least fused_proj_backward_workspace_size bytes; its contents
 *               on entry do not matter and are undefined afterwards. Calls that share
 *               a workspace must not overlap in time.
 * With no tokens (b = 0) dw and db are set to zero. Every pointer must be 16-byte
 * aligned (FUSED_PROJ_EALIGN); outputs and the workspace may not overlap each other or
 * any input (FUSED_PROJ_EALIAS); a missing required pointer or a short workspace is
 * FUSED_PROJ_EINVAL; a failed launch FUSED_PROJ_EHIP.
 */
int fused_proj_backward(fused_proj_t plan, const void *x, const void *w, const void *bias, const void *d_ff,
                        const void *dq, const void *dk, const void *dv, void *dx, void *dw, void *db,
                        void *workspace, size_t workspace_bytes, void *stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): fused_proj_backward with the
 * library's own static device scratch buffer as the workspace, so neither the library
 * nor the caller allocates anything. The buffer holds fused_proj_noalloc_scratch_bytes()
 * bytes (64 MiB) on each GPU the library runs on, for the whole life of the process; a
 * plan whose fused_proj_backward_workspace_size exceeds it is rejected with
 * FUSED_PROJ_ESCRATCH. Arguments, results and the other errors are those of
 * fused_proj_backward. Every call on one GPU shares that GPU's buffer and leaves its last
 * contents there (the kernels write every scratch byte they read, so nothing needs to
 * start at zero): calls that overlap in time on one GPU, from any thread or stream, race
 * and must be serialised by the caller.
 */
int fused_proj_backward_noalloc(fused_proj_t plan, const void *x, const void *w, const void *bias,
                                const void *d_ff, const void *dq, const void *dk, const void *dv, void *dx,
                                void *dw, void *db, void *stream);

/* Size in bytes of the static scratch buffer of fused_proj_backward_noalloc. */
size_t fused_proj_noalloc_scratch_bytes(void);

/* Writes a one-line description of the chosen kernel and tiling into buf
 * (NUL-terminated, truncated to len). Returns FUSED_PROJ_OK or FUSED_PROJ_EINVAL. */
int fused_proj_describe(fused_proj_t plan, char *buf, size_t len);

#ifdef __cplusplus
}
#endif

#endif /* FUSED_PROJ_H */
