"""Per-element parity bar between the GPU outputs and the float64 oracle.

TEST INFRASTRUCTURE ONLY (used by the tests, the smoke check and the
benchmark's CPU-baseline leg).

The bar: |gpu - oracle| <= rel * scale, element by element, with
scale = ||x_t|| * ||w_col|| + |b_col|, rel = 4e-3 for bf16 storage and 1e-5
for fp32. For q/k elements after RoPE the output is itself a projection with
the effective column w_eff = cos(phi) W[:, j] -/+ sin(phi) W[:, j'], since RoPE is
linear; its norm is used. The bias enters such an element as two products,
cos(phi) b_j -/+ sin(phi) b_j', and its part of the scale is the sum of their
magnitudes (the usual bound for the rounding of a sum of products), which stays
apart from zero where the two cancel (with C = 0 the bias is the whole output). For GELU outputs
(either form) the pre-activation scale is used (both are under 1.13-Lipschitz).
Squared ReLU doubles an input error by |y| at y: its outputs o use the
pre-activation scale times (1 + 2 sqrt(o)), which bounds
|d(y^2)| <= 2|y||dy| + dy^2 while |dy| <= 1. With fewer k/v heads, the grouped
column order or partial rotary, the scales follow the column map of qkv_columns,
and RoPE mixes only the rotated width.

A second, tighter diagnostic bar is also reported for bf16: the output's own
rounding (2^-8 relative) plus 1e-4 * scale of accumulation error.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

REL = {"bf16": 4e-3, "f32": 1e-5}
# The backward pass rounds twice in the storage type: dy (it is held between launches),
# then each gradient. bf16 keeps 7 fraction bits, so each rounding moves a value by at most
# 2^-8 of itself: dy's rounding moves a sum by at most 2^-8 of its Cauchy-Schwarz bound,
# and the result's rounding the result (at most the bound) by 2^-8 again. 2 * 2^-8 (1 +
# 2^-8) < 8e-3. (The forward rounds once: 2^-8 < 4e-3.)
BACKWARD_REL = {"bf16": 8e-3, "f32": 1e-5}


def token_rows(x64: np.ndarray, layout: str, tokens: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Rows x[t, :] (float64) and in-slab positions s for the given global tokens."""
    if layout == "channels_first":
        nb, C = x64.shape[0], x64.shape[1]
        S = int(np.prod(x64.shape[2:]))
        xf = x64.reshape(nb, C, S)
        bi, s = np.divmod(tokens, S)
        rows = xf[bi, :, s]
    else:
        nb, S, C = x64.shape
        bi, s = np.divmod(tokens, S)
        rows = x64[bi, s, :]
    return np.ascontiguousarray(rows), s


@dataclass
class Scales:
    ff: np.ndarray | None   # [n, FF]
    q: np.ndarray | None    # [n, H, hd]
    k: np.ndarray | None
    v: np.ndarray | None


def qkv_columns(ff_dim: int, n_heads: int, head_dim: int, n_kv_heads: int = 0, qkv_order: str = "contiguous"):
    """Fused column of every q/k/v output element: three int arrays [heads, head_dim]
    (q with n_heads heads, k and v with n_kv_heads), following the contiguous
    [q | k | v] order or the grouped order (per k/v head: its q heads, then k, then v)."""
    kvh = n_kv_heads if n_kv_heads > 0 else n_heads
    j = np.arange(head_dim)
    if qkv_order == "contiguous":
        q = ff_dim + np.arange(n_heads)[:, None] * head_dim + j
        k = ff_dim + n_heads * head_dim + np.arange(kvh)[:, None] * head_dim + j
        v = k + kvh * head_dim
        return q, k, v
    qpk = n_heads // kvh
    gw = (qpk + 2) * head_dim
    h = np.arange(n_heads)
    q = ff_dim + (h // qpk)[:, None] * gw + (h % qpk)[:, None] * head_dim + j
    g = np.arange(kvh)[:, None]
    k = ff_dim + g * gw + qpk * head_dim + j
    return q, k, k + head_dim


def scales(rows: np.ndarray, positions: np.ndarray, w_cf: np.ndarray, bias: np.ndarray | None, ff_dim: int,
           n_heads: int, head_dim: int, rope: bool, rope_base: float = 10000.0, pos_offset: int = 0,
           ff_act: str = "none", ff_ref: np.ndarray | None = None, n_kv_heads: int = 0,
           qkv_order: str = "contiguous", rope_dims: int = 0) -> Scales:
    """Per-element scale for tokens with gathered rows [n, C]; w_cf is W as [C, F].
    For ff_act "relu2" the oracle's ff outputs ff_ref [n, FF] are needed. q is
    [n, H, hd], k and v [n, KVH, hd]; RoPE mixes the first rope_dims (0: head_dim)
    elements of each q/k head."""
    n = rows.shape[0]
    F = w_cf.shape[1]
    xn = np.linalg.norm(rows, axis=1)                         # [n]
    wn = np.linalg.norm(w_cf, axis=0)                         # [F]
    b = np.zeros(F) if bias is None else np.asarray(bias, dtype=np.float64)
    plain = xn[:, None] * wn[None, :] + np.abs(b)[None, :]    # [n, F]
    ff = plain[:, :ff_dim] if ff_dim > 0 else None
    if ff is not None and ff_act == "relu2":
        if ff_ref is None:
            raise ValueError("squared ReLU scales need the oracle's ff outputs")
        ff = ff * (1.0 + 2.0 * np.sqrt(np.maximum(np.asarray(ff_ref, dtype=np.float64).reshape(ff.shape), 0.0)))
    if n_heads * head_dim == 0:
        return Scales(ff, None, None, None)
    R = rope_dims if rope_dims > 0 else head_dim
    half = R // 2
    out = []
    for which, cols in enumerate(qkv_columns(ff_dim, n_heads, head_dim, n_kv_heads, qkv_order)):
        s_plain = plain[:, cols]                               # [n, heads, hd]
        if not (rope and which < 2):
            out.append(s_plain)
            continue
        Wh = w_cf[:, cols]                                     # [C, heads, hd]
        bh = b[cols]                                           # [heads, hd]
        w1, w2 = Wh[:, :, :half], Wh[:, :, half:R]             # [C, heads, half]
        n1, n2 = (w1 ** 2).sum(0), (w2 ** 2).sum(0)            # [heads, half]
        d12 = (w1 * w2).sum(0)
        theta = rope_base ** (-2.0 * np.arange(half) / R)
        phi = (positions.astype(np.float64) + pos_offset)[:, None] * theta[None, :]   # [n, half]
        c, s = np.cos(phi)[:, None, :], np.sin(phi)[:, None, :]                     # [n, 1, half]
        # first half: c w1 - s w2 ; second half: c w2 + s w1
        e1 = np.sqrt(np.maximum(c * c * n1 + s * s * n2 - 2 * c * s * d12, 0.0))
        e2 = np.sqrt(np.maximum(c * c * n2 + s * s * n1 + 2 * c * s * d12, 0.0))
        a1, a2 = np.abs(bh[None, :, :half]), np.abs(bh[None, :, half:R])
        b1 = np.abs(c) * a1 + np.abs(s) * a2
        b2 = np.abs(c) * a2 + np.abs(s) * a1
        sc = np.concatenate([xn[:, None, None] * e1 + b1, xn[:, None, None] * e2 + b2, s_plain[:, :, R:]], axis=2)
        out.append(sc)
    return Scales(ff, out[0], out[1], out[2])


@dataclass
class Verdict:
    ok: bool
    max_ratio: float        # max |err| / (rel * scale); <= 1 passes the bar
    max_tight_ratio: float  # diagnostic bar (bf16 only; equals max_ratio for fp32)
    max_abs_err: float
    n: int

    def __str__(self):
        return (f"ok={self.ok} max_err/tol={self.max_ratio:.3g} tight={self.max_tight_ratio:.3g} "
                f"max_abs_err={self.max_abs_err:.3g} n={self.n}")


def compare(got: list, ref: list, scl: list, dtype: str, rel: float | None = None, tight: bool = True) -> Verdict:
    """got/ref/scl: matching lists of arrays (None entries skipped); rel defaults to the
    forward bar of the storage type. tight=False reports the main bar in place of the bf16
    diagnostic bar (which models one rounding of a value computed in fp32)."""
    rel = REL[dtype] if rel is None else rel
    mr, mt, ma, n = 0.0, 0.0, 0.0, 0
    finite = True
    for g, r, s in zip(got, ref, scl):
        if r is None:
            continue
        g = np.asarray(g, dtype=np.float64)
        err = np.abs(g - r)
        finite &= bool(np.all(np.isfinite(g)))
        ratio = err / (rel * s + 1e-300)
        mr = max(mr, float(np.max(ratio)) if ratio.size else 0.0)
        if dtype == "bf16" and tight:
            tr = err / (2.0 ** -8 * np.abs(r) + 1e-4 * s + 1e-300)
        else:
            tr = ratio
        mt = max(mt, float(np.max(tr)) if tr.size else 0.0)
        ma = max(ma, float(np.max(err)) if err.size else 0.0)
        n += g.size
    if not finite:
        mr = mt = math.inf
    return Verdict(finite and mr <= 1.0, mr, mt, ma, n)


@dataclass
class BackwardScales:
    dx: np.ndarray   # [M, C] token-major rows
    dw: np.ndarray   # [C, F]
    db: np.ndarray   # [F]


def backward_scales(x_rows: np.ndarray, w_cf: np.ndarray, dy: np.ndarray) -> BackwardScales:
    """Per-element scales of the backward pass: each gradient element is one sum of
    products, and its scale is the Cauchy-Schwarz bound of that sum,
      dx[t, c] = sum_f dy[t, f] W[c, f]  ->  ||dy[t, :]|| ||W[c, :]||
      dW[c, f] = sum_t x[t, c] dy[t, f]  ->  ||x[:, c]|| ||dy[:, f]||
      db[f]    = sum_t dy[t, f]          ->  sqrt(M) ||dy[:, f]||,
    with dy the oracle's float64 gradient of the fused output ([M, F]) and x_rows the
    gathered activation [M, C]. Rounding dy once to the storage type moves each sum by at
    most 2^-8 of its bound (bf16), and each rounded output by 2^-8 of itself: the bar is
    BACKWARD_REL times these scales (compare_backward)."""
    dyn_t = np.linalg.norm(dy, axis=1)          # [M]
    dyn_f = np.linalg.norm(dy, axis=0)          # [F]
    wn_c = np.linalg.norm(w_cf, axis=1)         # [C]
    xn_c = np.linalg.norm(x_rows, axis=0)       # [C]
    M = dy.shape[0]
    return BackwardScales(dyn_t[:, None] * wn_c[None, :], xn_c[:, None] * dyn_f[None, :],
                          math.sqrt(M) * dyn_f)


def compare_backward(got: list, ref: list, scl: list, dtype: str) -> Verdict:
    """compare() with the backward pass's bar (two roundings in the storage type). The
    forward's diagnostic bar does not apply: dy's rounding moves a gradient element by a
    fraction of its Cauchy-Schwarz scale, not of the element itself, so the diagnostic
    reports the backward bar."""
    return compare(got, ref, scl, dtype, rel=BACKWARD_REL[dtype], tight=False)
