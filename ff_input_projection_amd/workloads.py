"""Seeded synthetic workloads for the fused input projection.

This module holds shapes, seeds and the random-number recipe only: none of the
projection's arithmetic. Both the GPU path's tests/benchmark and the float64
oracle take their inputs from here, so they see the same stored values.

Recipe: NumPy ``default_rng(seed)`` draws x, then W, then the bias in float64
from standard normals; W is scaled to variance 1/C and the bias to variance
0.02; each tensor is then rounded once to the storage dtype (bf16 by
round-to-nearest-even through fp32). The float64 copies returned alongside are
exact images of the stored values.

Shapes stand in for the workloads on the pages: the Walrus processor block
(Walrus PR "Make fused_ff_qkv contiguous": a 32x32x1 latent grid, 6 steps,
batch 4, folded into 24 slabs), a BERT-base linear + GELU and its QKV
projection (xformers PR "Fused linear: small FW cleanup and much better
perfs", follow-up comments), a 32-head decoder QKV with rotate-half RoPE
(NVIDIA/Fuser issue "Improve performance on RoPE (and code around it)"), and
the SD-2.1 attention projection at 4096 tokens, 5 heads, batch 2
(memory-efficient-attention issue "Improve performance via batched-matmul and
fused multiplies"). No dataset or trained weight is involved.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    dtype: str              # "bf16" or "f32": storage type of x, W, bias and outputs
    layout: str             # "channels_first" ([b,c,spatial...]) or "tokens_last" ([b,s,c])
    x_shape: tuple
    ff_dim: int
    ff_act: str             # "none", "gelu" (exact erf), "gelu_tanh" or "relu2" (squared ReLU)
    n_heads: int
    head_dim: int
    has_bias: bool
    rope: bool
    seed: int
    rope_base: float = 10000.0
    pos_offset: int = 0
    w_layout: str = "cf"    # "cf": W [C,F]; "fc": W [F,C]
    description: str = field(default="", compare=False)
    n_kv_heads: int = 0     # k/v heads (0: n_heads)
    qkv_order: str = "contiguous"   # or "grouped" (per k/v head: its q heads, k, v)
    rope_dims: int = 0      # rotated width of each q/k head (0: head_dim)
    ff_layout: str = "tokens_last"  # or "channels_first": ff [b, ff_dim, S] (1x1x1-convolution layout)

    @property
    def kvh(self) -> int:
        return self.n_kv_heads if self.n_kv_heads > 0 else self.n_heads

    @property
    def rd(self) -> int:
        return self.rope_dims if self.rope_dims > 0 else self.head_dim

    @property
    def C(self) -> int:
        return self.x_shape[1] if self.layout == "channels_first" else self.x_shape[2]

    @property
    def nb(self) -> int:
        return self.x_shape[0]

    @property
    def S(self) -> int:
        if self.layout == "channels_first":
            return int(np.prod(self.x_shape[2:]))
        return self.x_shape[1]

    @property
    def M(self) -> int:
        return self.nb * self.S

    @property
    def F(self) -> int:
        return self.ff_dim + (self.n_heads + 2 * self.kvh) * self.head_dim

    @property
    def flops(self) -> float:
        """Algorithmic flops of the contraction: 2*M*C*F."""
        return 2.0 * self.M * self.C * self.F

    @property
    def elem_bytes(self) -> int:
        return 2 if self.dtype == "bf16" else 4

    @property
    def alg_bytes(self) -> float:
        """Algorithmic HBM bytes: x once, W once, bias, RoPE table (fp32 cos+sin,
        [positions, head_dim/2]) and every output once."""
        e = self.elem_bytes
        b = self.M * self.C * e + self.C * self.F * e + self.M * self.F * e
        if self.has_bias:
            b += self.F * e
        if self.rope and self.n_heads > 0:
            b += 2 * 4 * self.S * (self.rd // 2)
        return float(b)


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny_f32", "f32", "channels_first", (1, 32, 8, 8, 1), 128, "gelu", 4, 8, True, True, 1,
                 description="tiny fp32: x [1,32,8,8,1], W [32,224], FF 128 GELU, Q/K/V 4x8, RoPE"),
        Workload("walrus_bf16", "bf16", "channels_first", (24, 768, 32, 32, 1), 3072, "gelu", 12, 64, True, True, 2,
                 description="Walrus-like bf16: x [24,768,32,32,1] (4 x 6 steps), W [768,5376], FF 3072 GELU, "
                             "Q/K/V 12x64, RoPE"),
        Workload("bert_ff_bf16", "bf16", "tokens_last", (32, 512, 768), 3072, "gelu", 0, 0, True, False, 3,
                 description="BERT-base FF bf16: x [32,512,768], W [768,3072], GELU"),
        Workload("bert_qkv_bf16", "bf16", "tokens_last", (32, 512, 768), 0, "none", 12, 64, True, False, 31,
                 description="BERT-base QKV bf16: x [32,512,768], W [768,2304], 3 x [384,512,64]"),
        Workload("decoder_qkv_rope_bf16", "bf16", "tokens_last", (2, 4096, 4096), 0, "none", 32, 128, False, True, 4,
                 description="decoder QKV+RoPE bf16: x [2,4096,4096], W [4096,12288], 3 x [64,4096,128]"),
        Workload("smallk_qkv_bf16", "bf16", "channels_first", (2, 320, 64, 64), 0, "none", 5, 64, False, False, 5,
                 description="small-K bf16: x [2,320,64,64] channels-first, W [320,960], 3 x [10,4096,64]"),
        # BERT-base FF with squared ReLU (an activation the xformers PR discussion names)
        Workload("bert_ff_relu2_bf16", "bf16", "tokens_last", (32, 512, 768), 3072, "relu2", 0, 0, True, False, 7,
                 description="BERT-base FF bf16 with squared ReLU: x [32,512,768], W [768,3072]"),
        # The nvFuser RoPE issue's lit-gpt block: bsz 2, T 1024, n_embd 512, 16 q heads in 4
        # query groups (k/v once per group), head size 32, RoPE on the first 8 elements,
        # q/k/v columns grouped per k/v head, no bias
        Workload("gqa_rope8_bf16", "bf16", "tokens_last", (2, 1024, 512), 0, "none", 16, 32, False, True, 8,
                 n_kv_heads=4, qkv_order="grouped", rope_dims=8,
                 description="lit-gpt GQA bf16: x [2,1024,512], W [512,768], 16 q heads / 4 k-v groups x 32, "
                             "grouped columns, RoPE on 8 of 32"),
        # The Walrus page's 1x1x1 Conv3d comparison: the temporal q/k/v projection of the
        # latent grid as a convolution, output channels-first [24, 2304, 32, 32, 1]
        Workload("conv1x1_walrus_bf16", "bf16", "channels_first", (24, 768, 32, 32, 1), 2304, "none", 0, 0, True,
                 False, 10, ff_layout="channels_first",
                 description="1x1x1 Conv3d-shaped bf16: x [24,768,32,32,1] -> [24,2304,32,32,1] channels-first"),
        # The Walrus block at the width its profiles imply (C = 1408, F = 7C: FF 4C and
        # Q/K/V C each): F is not a multiple of 256, so the last large column tile is ragged.
        Workload("walrus_c1408_bf16", "bf16", "channels_first", (24, 1408, 32, 32, 1), 5632, "gelu", 22, 64, True,
                 True, 6,
                 description="Walrus block at width 1408 bf16: x [24,1408,32,32,1] (4 x 6 steps), W [1408,9856], "
                             "FF 5632 GELU, Q/K/V 22x64, RoPE"),
    ]
}


def round_to(a64: np.ndarray, dtype: str) -> torch.Tensor:
    """Round a float64 array once to the storage dtype (RNE); returns a CPU tensor."""
    t = torch.from_numpy(np.ascontiguousarray(a64, dtype=np.float32)) if dtype == "f32" else \
        torch.from_numpy(np.ascontiguousarray(a64, dtype=np.float32)).to(torch.bfloat16)
    return t


def as_f64(t: torch.Tensor) -> np.ndarray:
    """Exact float64 image of a bf16/fp32 CPU tensor."""
    return t.to(torch.float64).numpy()


@dataclass
class Inputs:
    x: torch.Tensor          # storage dtype, CPU, contiguous in the workload's layout
    w: torch.Tensor          # [C,F] or [F,C]
    bias: torch.Tensor | None
    x64: np.ndarray
    w64: np.ndarray
    bias64: np.ndarray | None


def make_inputs(wl: Workload, seed: int | None = None) -> Inputs:
    """Draw x ~ N(0,1), W ~ N(0,1/C), bias ~ N(0,0.02) (second argument = variance).
    With C = 0 (no channels) W is empty and its scale is irrelevant."""
    rng = np.random.default_rng(wl.seed if seed is None else seed)
    C, F = wl.C, wl.F
    x = rng.standard_normal(wl.x_shape)
    w = rng.standard_normal((C, F)) * math.sqrt(1.0 / max(C, 1))
    if wl.w_layout == "fc":
        w = np.ascontiguousarray(w.T)
    b = rng.standard_normal(F) * math.sqrt(0.02) if wl.has_bias else None
    xt, wt = round_to(x, wl.dtype), round_to(w, wl.dtype)
    bt = round_to(b, wl.dtype) if b is not None else None
    return Inputs(xt, wt, bt, as_f64(xt), as_f64(wt), None if bt is None else as_f64(bt))


def with_shape(wl: Workload, name: str, **kw) -> Workload:
    """A variant of a workload (smaller or ragged shapes for tests)."""
    d = dict(wl.__dict__)
    d.update(kw)
    d["name"] = name
    return Workload(**d)


@dataclass(frozen=True)
class SplitRopeWorkload:
    """A projected q/k/v tensor [batch, tokens, (H + 2*KVH)*hd] ~ N(0,1), split into
    head-major q/k/v with RoPE (the standalone op of split_rope.h)."""
    name: str
    batch: int
    tokens: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    qkv_order: str
    rope_dims: int
    k_transposed: bool
    seed: int
    pos_offset: int = 0
    description: str = field(default="", compare=False)

    @property
    def Fq(self) -> int:
        return (self.n_heads + 2 * self.n_kv_heads) * self.head_dim

    @property
    def alg_bytes(self) -> float:
        """The input once, every output once (the same count), and the fp32 cos/sin table."""
        return 2.0 * 2 * self.batch * self.tokens * self.Fq + 2 * 4 * self.tokens * (self.rope_dims // 2)


SPLIT_ROPE_WORKLOADS = {
    w.name: w
    for w in [
        # the nvFuser RoPE issue's workload: bf16 [2, 1024, 768], 16 q heads in 4 groups of
        # head size 32, grouped columns, RoPE on the first 8 elements
        SplitRopeWorkload("splitrope_gqa_bf16", 2, 1024, 16, 4, 32, "grouped", 8, False, 9,
                          description="split+RoPE bf16 [2,1024,768]: 16 q / 4 k-v heads x 32, grouped, RoPE on 8"),
        SplitRopeWorkload("splitrope_gqa_kt_bf16", 2, 1024, 16, 4, 32, "grouped", 8, True, 9,
                          description="as splitrope_gqa_bf16 with the key written transposed [8, 32, 1024]"),
    ]
}


def make_qkv(batch: int, tokens: int, width: int, seed: int):
    """Seeded qkv ~ N(0,1) [batch, tokens, width]: the bf16 tensor and its exact float64 image."""
    a = np.random.default_rng(seed).standard_normal((batch, tokens, width))
    t = round_to(a, "bf16")
    return t, as_f64(t)


@dataclass
class Grads:
    """Seeded upstream gradients of the four outputs, laid out like the outputs: d_ff
    [b, S, FF] (or [b, FF, S] for a channels-first ff), dq [b*H, S, hd], dk and dv
    [b*KVH, S, hd]; storage type on the CPU, with their exact float64 images."""
    d_ff: torch.Tensor | None
    dq: torch.Tensor | None
    dk: torch.Tensor | None
    dv: torch.Tensor | None
    d_ff64: np.ndarray | None
    dq64: np.ndarray | None
    dk64: np.ndarray | None
    dv64: np.ndarray | None


def make_grads(wl: Workload, seed: int | None = None) -> Grads:
    """Upstream gradients ~ N(0,1), drawn after nothing else (their own generator, seeded
    with the workload's seed + 1000): d_ff, then dq, dk, dv; rounded once to the storage type."""
    rng = np.random.default_rng((wl.seed if seed is None else seed) + 1000)
    out, out64 = [], []
    ff_shape = None
    if wl.ff_dim > 0:
        ff_shape = (wl.nb, wl.ff_dim, wl.S) if wl.ff_layout == "channels_first" else (wl.nb, wl.S, wl.ff_dim)
    heads = wl.n_heads * wl.head_dim > 0
    shapes = [ff_shape,
              (wl.nb * wl.n_heads, wl.S, wl.head_dim) if heads else None,
              (wl.nb * wl.kvh, wl.S, wl.head_dim) if heads else None,
              (wl.nb * wl.kvh, wl.S, wl.head_dim) if heads else None]
    for s in shapes:
        if s is None:
            out.append(None)
            out64.append(None)
            continue
        t = round_to(rng.standard_normal(s), wl.dtype)
        out.append(t)
        out64.append(as_f64(t))
    return Grads(*out, *out64)
