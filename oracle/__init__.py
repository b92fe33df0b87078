"""Float64 CPU oracle of the fused input projection.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this package; the GPU library never does. It shares
no code with the GPU path. The arithmetic lives in ``fused_proj_oracle.c``
(plain loops, float64); this module only builds that file with gcc, marshals
NumPy arrays into it and reorders its token-major q/k/v rows into the
head-major ``[batch*heads, tokens, head_dim]`` buffers described in the
memory-efficient-attention issue "Improve performance via batched-matmul and
fused multiplies" (first comment), using a plain array transpose.

Parity pins: see ``tests/test_oracle_pins.py``. The RoPE angle convention
``phi = p * base**(-2i/head_dim)`` is the one point the pages leave open (their
tables are random); it is pinned to hand-derived closed forms, not to the pages.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fused_proj_oracle.c")
_LIB = os.path.join(_HERE, "liboracle_fused_proj.so")
_lib = None

# ff-slice activations: identity, exact-erf GELU, tanh GELU, squared ReLU
ACTIVATIONS = {"none": 0, "gelu": 1, "gelu_tanh": 2, "relu2": 3}

GCC_FLAGS = ["-O2", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared", "-std=c99"]


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no fused multiply-add contraction)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", *GCC_FLAGS, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        d = ctypes.POINTER(ctypes.c_double)
        i64 = ctypes.c_int64
        p64 = ctypes.POINTER(ctypes.c_int64)
        lib.oracle_fused_proj.restype = ctypes.c_int
        lib.oracle_fused_proj.argtypes = [
            d, i64, i64, i64, i64, i64, ctypes.c_int, p64, p64,
            d, i64, ctypes.c_int, d,
            i64, ctypes.c_int, i64, i64,
            i64, ctypes.c_int, i64,
            ctypes.c_int, ctypes.c_double, i64,
            p64, i64, d, d, d, d, ctypes.c_int,
        ]
        lib.oracle_split_rope.restype = ctypes.c_int
        lib.oracle_split_rope.argtypes = [d, i64, i64, i64, i64, i64, ctypes.c_int, ctypes.c_int, i64,
                                          ctypes.c_double, i64, ctypes.c_int, d, d, d]
        lib.oracle_fused_proj_backward.restype = ctypes.c_int
        lib.oracle_fused_proj_backward.argtypes = [
            d, i64, i64, i64, i64, i64, ctypes.c_int, p64, p64,
            d, i64, ctypes.c_int, d,
            i64, ctypes.c_int, i64, i64,
            i64, ctypes.c_int, i64,
            ctypes.c_int, ctypes.c_double, i64, ctypes.c_int,
            d, d, d, d,
            d, d, d, d, ctypes.c_int,
        ]
        lib.oracle_max_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def max_threads() -> int:
    return int(_load().oracle_max_threads())


@dataclass
class OracleResult:
    """Outputs in float64. Full runs: ff [nb, S, FF], q [nb*H, S, hd], k/v [nb*KVH, S, hd].
    Token-subset runs: ff [ntok, FF], q [ntok, H, hd], k/v [ntok, KVH, hd] (token-major)."""
    ff: np.ndarray | None
    q: np.ndarray | None
    k: np.ndarray | None
    v: np.ndarray | None


def _dptr(a: np.ndarray | None):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def fused_proj(x: np.ndarray, layout: str, w: np.ndarray, w_layout: str, bias: np.ndarray | None,
               ff_dim: int, ff_act: str, n_heads: int, head_dim: int, rope: bool,
               rope_base: float = 10000.0, pos_offset: int = 0, tokens: np.ndarray | None = None,
               nthreads: int = 0, n_kv_heads: int = 0, qkv_order: str = "contiguous",
               rope_dims: int = 0) -> OracleResult:
    """Float64 fused projection.

    x: float64 array, ``layout`` "channels_first" ([b,c,h,w,d] or [b,c,s...]:
       dim 0 batch, dim 1 channel, the rest spatial, flattened row-major) or
       "tokens_last" ([b,s,c]). Any strides (element strides are passed as-is).
    w: float64 [C,F] (w_layout "cf") or [F,C] (w_layout "fc").
    tokens: None for every token (full layouts returned) or an int64 array of
       global token indices bi*S + s (token-major rows returned).
    n_kv_heads: k/v heads (0: n_heads); qkv_order: "contiguous" ([q | k | v]) or
       "grouped" (per k/v head: its q heads, then k, then v); rope_dims: rotated
       width of each q/k head (0: head_dim).
    """
    lib = _load()
    x = np.asarray(x)
    if x.dtype != np.float64:
        raise TypeError("oracle takes float64 inputs")
    item = x.itemsize
    if layout == "channels_first":
        nb, C = x.shape[0], x.shape[1]
        sp = x.shape[2:]
        sp_stride = [st // item for st in x.strides[2:]]
        sb, sc = x.strides[0] // item, x.strides[1] // item
    elif layout == "tokens_last":
        nb, C = x.shape[0], x.shape[2]
        sp = (x.shape[1],)
        sp_stride = [x.strides[1] // item]
        sb, sc = x.strides[0] // item, x.strides[2] // item
    else:
        raise ValueError(layout)
    if not 1 <= len(sp) <= 3:
        raise ValueError("1 to 3 spatial dims")
    S = int(np.prod(sp))
    # base pointer of the view: strides may be arbitrary but non-negative
    if any(s < 0 for s in x.strides):
        raise ValueError("negative strides not supported by the oracle wrapper")
    w = np.ascontiguousarray(w, dtype=np.float64)
    if w_layout == "cf":
        assert w.shape[0] == C
        F = w.shape[1]
        w_fc = 0
    elif w_layout == "fc":
        assert w.shape[1] == C
        F = w.shape[0]
        w_fc = 1
    else:
        raise ValueError(w_layout)
    if bias is not None:
        bias = np.ascontiguousarray(bias, dtype=np.float64)
        assert bias.shape == (F,)
    full = tokens is None
    if full:
        tokens = np.arange(nb * S, dtype=np.int64)
    tokens = np.ascontiguousarray(tokens, dtype=np.int64)
    ntok = tokens.shape[0]
    kvh = n_kv_heads if n_kv_heads > 0 else n_heads
    grouped = {"contiguous": 0, "grouped": 1}[qkv_order]
    qw, kvw = n_heads * head_dim, kvh * head_dim
    ff_rows = np.empty((ntok, ff_dim)) if ff_dim > 0 else None
    q_rows = np.empty((ntok, qw)) if qw > 0 else None
    k_rows = np.empty((ntok, kvw)) if qw > 0 else None
    v_rows = np.empty((ntok, kvw)) if qw > 0 else None
    spz = (ctypes.c_int64 * len(sp))(*sp)
    sps = (ctypes.c_int64 * len(sp))(*sp_stride)
    act = ACTIVATIONS[ff_act]
    rc = lib.oracle_fused_proj(
        x.ctypes.data_as(ctypes.POINTER(ctypes.c_double)), nb, C, S, sb, sc, len(sp), spz, sps,
        _dptr(w), F, w_fc, _dptr(bias),
        ff_dim, act, n_heads, head_dim, int(n_kv_heads), grouped, int(rope_dims),
        int(bool(rope)), float(rope_base), int(pos_offset),
        tokens.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), ntok,
        _dptr(ff_rows), _dptr(q_rows), _dptr(k_rows), _dptr(v_rows), int(nthreads))
    if rc != 0:
        raise ValueError(f"oracle rejected its arguments (code {rc})")
    if not full:
        rs = (lambda a, h: None if a is None else a.reshape(ntok, h, head_dim))
        return OracleResult(ff_rows, rs(q_rows, n_heads), rs(k_rows, kvh), rs(v_rows, kvh))

    def head_major(a, h):
        if a is None:
            return None
        # [b, S, H, hd] -> [b, H, S, hd] -> [b*H, S, hd]
        return a.reshape(nb, S, h, head_dim).transpose(0, 2, 1, 3).reshape(nb * h, S, head_dim)

    ff = None if ff_rows is None else ff_rows.reshape(nb, S, ff_dim)
    return OracleResult(ff, head_major(q_rows, n_heads), head_major(k_rows, kvh), head_major(v_rows, kvh))


def _x_geometry(x: np.ndarray, layout: str):
    """(nb, C, spatial sizes, spatial element strides, batch stride, channel stride)."""
    item = x.itemsize
    if layout == "channels_first":
        nb, C = x.shape[0], x.shape[1]
        sp = x.shape[2:]
        sp_stride = [st // item for st in x.strides[2:]]
        sb, sc = x.strides[0] // item, x.strides[1] // item
    elif layout == "tokens_last":
        nb, C = x.shape[0], x.shape[2]
        sp = (x.shape[1],)
        sp_stride = [x.strides[1] // item]
        sb, sc = x.strides[0] // item, x.strides[2] // item
    else:
        raise ValueError(layout)
    if not 1 <= len(sp) <= 3:
        raise ValueError("1 to 3 spatial dims")
    if any(st < 0 for st in x.strides):
        raise ValueError("negative strides not supported by the oracle wrapper")
    return nb, C, tuple(sp), sp_stride, sb, sc


@dataclass
class BackwardResult:
    """Float64 gradients: dx in x's logical layout (dense), dw in w's layout, db [F] or
    None, and dy [nb*S, F], the gradient of the fused pre-activation output."""
    dx: np.ndarray
    dw: np.ndarray
    db: np.ndarray | None
    dy: np.ndarray


def fused_proj_backward(x: np.ndarray, layout: str, w: np.ndarray, w_layout: str, bias: np.ndarray | None,
                        ff_dim: int, ff_act: str, n_heads: int, head_dim: int, rope: bool,
                        d_ff: np.ndarray | None, dq: np.ndarray | None, dk: np.ndarray | None,
                        dv: np.ndarray | None, rope_base: float = 10000.0, pos_offset: int = 0,
                        n_kv_heads: int = 0, qkv_order: str = "contiguous", rope_dims: int = 0,
                        ff_layout: str = "tokens_last", nthreads: int = 0) -> BackwardResult:
    """Float64 backward pass of fused_proj (same arguments) for upstream gradients laid out
    like the outputs: d_ff [b, S, FF] (or [b, FF, S] with ff_layout "channels_first"),
    dq [b*H, S, hd], dk and dv [b*KVH, S, hd]. Every token is included."""
    lib = _load()
    x = np.asarray(x)
    if x.dtype != np.float64:
        raise TypeError("oracle takes float64 inputs")
    nb, C, sp, sp_stride, sb, sc = _x_geometry(x, layout)
    S = int(np.prod(sp))
    w = np.ascontiguousarray(w, dtype=np.float64)
    F = w.shape[1] if w_layout == "cf" else w.shape[0]
    w_fc = {"cf": 0, "fc": 1}[w_layout]
    if bias is not None:
        bias = np.ascontiguousarray(bias, dtype=np.float64)
    grads = [None if g is None else np.ascontiguousarray(g, dtype=np.float64) for g in (d_ff, dq, dk, dv)]
    M = nb * S
    dy = np.empty((M, F))
    dx_rows = np.empty((M, C))
    dw = np.empty((C, F))
    db = np.empty(F) if bias is not None else None
    spz = (ctypes.c_int64 * len(sp))(*sp)
    sps = (ctypes.c_int64 * len(sp))(*sp_stride)
    rc = lib.oracle_fused_proj_backward(
        x.ctypes.data_as(ctypes.POINTER(ctypes.c_double)), nb, C, S, sb, sc, len(sp), spz, sps,
        _dptr(w), F, w_fc, _dptr(bias),
        ff_dim, ACTIVATIONS[ff_act], n_heads, head_dim, int(n_kv_heads),
        {"contiguous": 0, "grouped": 1}[qkv_order], int(rope_dims),
        int(bool(rope)), float(rope_base), int(pos_offset), {"tokens_last": 0, "channels_first": 1}[ff_layout],
        *[_dptr(g) for g in grads], _dptr(dy), _dptr(dx_rows), _dptr(dw), _dptr(db), int(nthreads))
    if rc != 0:
        raise ValueError(f"oracle rejected its arguments (code {rc})")
    if layout == "channels_first":
        # token-major rows [b, S, C] -> [b, C, spatial...]
        dx = dx_rows.reshape(nb, S, C).transpose(0, 2, 1).reshape((nb, C) + sp)
    else:
        dx = dx_rows.reshape(nb, S, C)
    if w_layout == "fc":
        dw = np.ascontiguousarray(dw.T)
    return BackwardResult(np.ascontiguousarray(dx), dw, db, dy)


def split_rope(qkv: np.ndarray, n_heads: int, head_dim: int, n_kv_heads: int = 0, qkv_order: str = "contiguous",
               rope: bool = True, rope_dims: int = 0, rope_base: float = 10000.0, pos_offset: int = 0,
               k_transposed: bool = False):
    """Float64 split + RoPE of a projected q/k/v tensor qkv [b, T, (H + 2*KVH)*hd].
    Returns (q [b*H, T, hd], k [b*KVH, T, hd] or [b*KVH, hd, T], v [b*KVH, T, hd])."""
    lib = _load()
    qkv = np.ascontiguousarray(qkv, dtype=np.float64)
    nb, T, Fq = qkv.shape
    kvh = n_kv_heads if n_kv_heads > 0 else n_heads
    if Fq != (n_heads + 2 * kvh) * head_dim:
        raise ValueError("qkv width does not match the heads")
    q = np.empty((nb * n_heads, T, head_dim))
    v = np.empty((nb * kvh, T, head_dim))
    k = np.empty((nb * kvh, head_dim, T) if k_transposed else (nb * kvh, T, head_dim))
    rc = lib.oracle_split_rope(_dptr(qkv), nb, T, n_heads, int(n_kv_heads), head_dim,
                               {"contiguous": 0, "grouped": 1}[qkv_order], int(bool(rope)), int(rope_dims),
                               float(rope_base), int(pos_offset), int(bool(k_transposed)), _dptr(q), _dptr(k),
                               _dptr(v))
    if rc != 0:
        raise ValueError(f"oracle rejected its arguments (code {rc})")
    return q, k, v
