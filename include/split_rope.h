/*
 * split_rope.h — C ABI of the standalone split + RoPE on MI355X (gfx950).
 *
 * The operation (one call = one kernel launch), for a q/k/v projection computed
 * elsewhere, qkv[b, T, (H + 2*KVH)*hd] (token-major, contiguous):
 *
 *   split the columns of every token into H q heads and KVH k and v heads, in the
 *   contiguous or the grouped order of fused_proj.h (FUSED_PROJ_QKV_*), and write
 *     q[bi*H + h, s, j]   = RoPE_p(q head h)[j]
 *     k[bi*KVH + g, s, j] = RoPE_p(k head g)[j]      (or k[bi*KVH + g, j, s] when transposed)
 *     v[bi*KVH + g, s, j] = v head g [j]
 *   with p = s + pos_offset and rotate-half RoPE over the first rope_dims elements of
 *   each q and k head (angles p * base^(-2i/rope_dims)); the other elements pass
 *   through. RoPE runs in fp32 and each output is rounded once to bf16.
 *
 * Where it is defined: the NVIDIA/Fuser issue "Improve performance on RoPE (and code
 * around it)" (split_qkv and rope_one_entry in the thunder example, and the pointwise
 * kernels it measures); the transposed key is the pre-transposed key of the
 * memory-efficient-attention issue "Improve performance via batched-matmul and fused
 * multiplies" (key_needs_transpose). k and v are written once per k/v head.
 *
 * Memory: the caller owns every device buffer; the plan owns its cos/sin table.
 * Errors are the FUSED_PROJ_* codes; fused_proj_strerror() describes them.
 */
#ifndef SPLIT_ROPE_H
#define SPLIT_ROPE_H

#include <stddef.h>
#include <stdint.h>

#include "fused_proj.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct split_rope_desc {
    int32_t dtype;        /* FUSED_PROJ_BF16 (the only storage type supported) */
    int64_t batch;        /* b >= 0 sequences */
    int64_t tokens;       /* T >= 1 tokens per sequence */
    int64_t n_heads;      /* H >= 1 q heads */
    int64_t n_kv_heads;   /* k and v heads, dividing H; 0 means H */
    int64_t head_dim;     /* hd, a multiple of 8 */
    int32_t qkv_order;    /* FUSED_PROJ_QKV_CONTIGUOUS | FUSED_PROJ_QKV_GROUPED */
    int32_t rope;         /* 1: RoPE on q and k */
    int64_t rope_dims;    /* rotated width, even, <= hd; 0 means hd */
    double rope_base;     /* > 0 */
    int64_t pos_offset;   /* >= 0 */
    int32_t k_transposed; /* 1: k written as [b*KVH, hd, T] (T a multiple of 8) */
} split_rope_desc;

typedef struct split_rope_plan *split_rope_t;

/* Host-only check. FUSED_PROJ_OK, FUSED_PROJ_EINVAL (malformed: sizes, enums, KVH not
 * dividing H, rope_dims odd or above hd, base <= 0) or FUSED_PROJ_EUNSUPPORTED (not
 * bf16, hd not a multiple of 8, a transposed key with T not a multiple of 8, or more
 * than 2^31 - 1 output chunks of 8 elements). */
int split_rope_validate(const split_rope_desc *desc);

/* Validates and (with RoPE) builds the cos/sin table for positions pos_offset ..
 * pos_offset + T - 1 in float64, stored fp32 on the current device (synchronous; the
 * only call that allocates). Errors: as validate, FUSED_PROJ_EINVAL for out == NULL,
 * FUSED_PROJ_EHIP. */
int split_rope_create(const split_rope_desc *desc, split_rope_t *out);

/* Enqueues the op on `stream` (a hipStream_t; NULL = the legacy default stream) and
 * returns; allocates nothing and never synchronises. qkv [b, T, (H+2KVH)*hd]; q
 * [b*H, T, hd]; k [b*KVH, T, hd] (or [b*KVH, hd, T]); v [b*KVH, T, hd]; all bf16,
 * contiguous, 16-byte aligned, on the plan's device. Errors: FUSED_PROJ_EINVAL (NULL
 * pointer or another device current), FUSED_PROJ_EALIGN, FUSED_PROJ_EALIAS (an output
 * overlapping another or the input), FUSED_PROJ_EHIP (launch failure). */
int split_rope_run(split_rope_t plan, const void *qkv, void *q, void *k, void *v, void *stream);

/* Frees the plan and its table. NULL is accepted. */
int split_rope_destroy(split_rope_t plan);

#ifdef __cplusplus
}
#endif

#endif /* SPLIT_ROPE_H */
