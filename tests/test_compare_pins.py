"""Pins of the per-element parity bar (oracle/compare.py) to a brute-force bar (CPU only).

The bar every GPU parity verdict rests on is |gpu - oracle| <= rel * scale with
scale = ||x_t|| * ||w_eff|| + |b_eff|, where w_eff and b_eff are the effective
column and bias of one output element: the plain W column and bias for ff and v
elements, and for q/k elements after RoPE (RoPE is linear) the rotation-mixed column
and bias at that token's position.

Here w_eff and b_eff are not computed from any formula: they are read off the float64
oracle itself, which is linear in x and in the bias when the ff activation is left
out. Running it on unit activation rows e_c (channel c set to 1, no bias) returns
w_eff[c] for every output element at every position; running it on a zero activation
with the bias returns b_eff. scales() must match the bar built from those, for both
column orders, fewer k/v heads, partial rotary, a position offset, squared ReLU (whose
bar is the pre-activation one times 1 + 2 sqrt(output)) and no bias.
compare() is pinned with planted errors just above and just below the bar, and with
non-finite values.
"""
import math

import numpy as np
import pytest

import oracle
from oracle import compare as cmp


def _rows(res, which):
    return {"ff": res.ff, "q": res.q, "k": res.k, "v": res.v}[which]


def brute_force_scales(x, w, b, S, ff_dim, H, hd, rope, pos_offset, kvh, order, rope_dims, ff_act):
    """Brute-force bar per output element for a token-major x [1, S, C] and W [C, F]."""
    C = x.shape[2]
    tokens = np.arange(S, dtype=np.int64)
    kw = dict(n_kv_heads=kvh, qkv_order=order, rope_dims=rope_dims, tokens=tokens)
    parts = ("ff", "q", "k", "v")
    weff = {p: [] for p in parts}
    for c in range(C):
        e = np.zeros((1, S, C))
        e[0, :, c] = 1.0
        r = oracle.fused_proj(e, "tokens_last", w, "cf", None, ff_dim, "none", H, hd, rope, 10000.0, pos_offset,
                              **kw)
        for p in parts:
            weff[p].append(_rows(r, p))
    bterm = {p: 0.0 for p in parts}
    if b is not None:
        # the bias's part: sum over bias entries j of |d out / d b_j| * |b_j|, each
        # derivative read from a run with a one-hot bias and x = 0
        for j in range(w.shape[1]):
            ej = np.zeros(w.shape[1])
            ej[j] = 1.0
            r = oracle.fused_proj(np.zeros((1, S, C)), "tokens_last", w, "cf", ej, ff_dim, "none", H, hd, rope,
                                  10000.0, pos_offset, **kw)
            for p in parts:
                if _rows(r, p) is not None:
                    bterm[p] = bterm[p] + np.abs(_rows(r, p)) * abs(b[j])
    xn = np.linalg.norm(x[0], axis=1)                              # [S]
    act_out = oracle.fused_proj(x, "tokens_last", w, "cf", b, ff_dim, ff_act, H, hd, rope, 10000.0, pos_offset,
                                **kw)
    out = {}
    for p in parts:
        if weff[p][0] is None:
            out[p] = None
            continue
        stack = np.stack(weff[p], axis=0)                          # [C, S, ...]
        wn = np.sqrt((stack ** 2).sum(axis=0))                     # [S, ...]
        xs = xn.reshape((S,) + (1,) * (wn.ndim - 1))
        bar = xs * wn + bterm[p]
        if p == "ff" and ff_act == "relu2":
            bar = bar * (1.0 + 2.0 * np.sqrt(np.maximum(act_out.ff, 0.0)))
        out[p] = bar
    return out, act_out


CASES = [
    # (name, C, S, ff_dim, H, hd, kvh, order, rope, rope_dims, pos_offset, bias, ff_act)
    ("contiguous_full_rope", 6, 5, 8, 2, 8, 0, "contiguous", True, 0, 0, True, "gelu"),
    ("contiguous_full_rope_offset", 5, 4, 0, 3, 4, 0, "contiguous", True, 0, 11, True, "none"),
    ("grouped_gqa_partial_rope", 7, 6, 0, 4, 8, 2, "grouped", True, 4, 3, True, "none"),
    ("contiguous_gqa_partial_rope_relu2", 6, 5, 12, 6, 8, 3, "contiguous", True, 6, 0, True, "relu2"),
    ("grouped_mqa_no_bias", 5, 4, 4, 2, 6, 1, "grouped", True, 0, 2, False, "gelu"),
    ("no_rope_relu2", 4, 3, 10, 1, 4, 0, "contiguous", False, 0, 0, True, "relu2"),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_scales_equal_brute_force_bar(case):
    """scales() == the bar built from the oracle's own effective columns and the
    magnitudes of the bias's terms. Catches the column norm over the wrong axis, the sign
    of the RoPE cross term, a bias mixed with the wrong partner, the partner taken over the
    head instead of the rotated width, and a wrong squared-ReLU factor."""
    name, C, S, ff_dim, H, hd, kvh, order, rope, rd, off, has_b, act = case
    K = kvh if kvh > 0 else H
    F = ff_dim + (H + 2 * K) * hd
    r = np.random.default_rng(sum(map(ord, name)))
    x = r.standard_normal((1, S, C))
    w = r.standard_normal((C, F)) / math.sqrt(C)
    b = r.standard_normal(F) * 0.5 if has_b else None
    ref, act_out = brute_force_scales(x, w, b, S, ff_dim, H, hd, rope, off, kvh, order, rd, act)
    rows, pos = cmp.token_rows(x, "tokens_last", np.arange(S, dtype=np.int64))
    sc = cmp.scales(rows, pos, w, b, ff_dim, H, hd, rope, 10000.0, off, ff_act=act, ff_ref=act_out.ff,
                    n_kv_heads=kvh, qkv_order=order, rope_dims=rd)
    for p in ("ff", "q", "k", "v"):
        got, exp = getattr(sc, p), ref[p]
        if exp is None:
            assert got is None, p
            continue
        assert got.shape == exp.shape, (p, got.shape, exp.shape)
        assert np.allclose(got, exp, rtol=1e-12, atol=1e-14), (p, np.max(np.abs(got - exp)))


def test_channels_first_token_rows():
    """token_rows() gathers channel c of token (bi, s) from x[bi, c, s...] for a
    channels-first x with two spatial dims, and returns the in-slab position s."""
    r = np.random.default_rng(7)
    x = r.standard_normal((3, 4, 2, 5))
    tokens = np.array([0, 4, 9, 10, 23, 29], dtype=np.int64)
    rows, pos = cmp.token_rows(x, "channels_first", tokens)
    for i, t in enumerate(tokens):
        bi, s = divmod(int(t), 10)
        assert pos[i] == s
        assert np.array_equal(rows[i], x[bi, :, s // 5, s % 5])


def _planted(dtype, factor, where=(1, 2)):
    r = np.random.default_rng(3)
    ref = r.standard_normal((4, 5))
    scl = np.abs(r.standard_normal((4, 5))) + 0.5
    got = ref.copy()
    got[where] += factor * cmp.REL[dtype] * scl[where]
    return got, ref, scl


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_compare_fails_just_above_the_bar(dtype):
    got, ref, scl = _planted(dtype, 1.01)
    v = cmp.compare([got], [ref], [scl], dtype)
    assert not v.ok and 1.009 < v.max_ratio < 1.011, v


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_compare_passes_just_below_the_bar(dtype):
    got, ref, scl = _planted(dtype, 0.99)
    v = cmp.compare([got], [ref], [scl], dtype)
    assert v.ok and 0.989 < v.max_ratio < 0.991, v
    # a negative error of the same size too
    got, ref, scl = _planted(dtype, -0.99, where=(3, 0))
    assert cmp.compare([got], [ref], [scl], dtype).ok


def test_compare_checks_every_array_and_skips_none():
    """An error in the last of several arrays still fails; None entries are skipped."""
    good = np.ones((2, 3))
    got, ref, scl = _planted("bf16", 1.5)
    v = cmp.compare([good, None, got], [good, None, ref], [good, None, scl], "bf16")
    assert not v.ok and v.n == good.size + got.size


@pytest.mark.parametrize("bad", [float("nan"), float("inf"), -float("inf")])
def test_compare_fails_on_non_finite(bad):
    got, ref, scl = _planted("bf16", 0.0)
    got[0, 0] = bad
    v = cmp.compare([got], [ref], [scl], "bf16")
    assert not v.ok and math.isinf(v.max_ratio)


def test_tight_bar_is_reported_for_bf16():
    """The diagnostic bar 2^-8 |ref| + 1e-4 scale: an error of 2^-8 |ref| alone sits at
    about 1 of it, while the main bar (4e-3 scale) is far from reached."""
    ref = np.array([[1.0, -2.0, 4.0]])
    scl = np.array([[100.0, 100.0, 100.0]])
    got = ref + 2.0 ** -8 * np.abs(ref)
    v = cmp.compare([got], [ref], [scl], "bf16")
    assert v.ok
    expect = max(2.0 ** -8 * abs(r) / (2.0 ** -8 * abs(r) + 1e-4 * 100.0) for r in ref[0])
    assert abs(v.max_tight_ratio - expect) < 1e-12


def test_backward_diagnostic_is_the_backward_bar():
    """compare_backward reports its own bar as the diagnostic: an error at 0.9 of the
    backward bar on a near-zero gradient element reads 0.9 twice (the forward's 2^-8 |ref|
    diagnostic would call the same element far over)."""
    ref = np.array([[1e-6, 3.0]])
    scl = np.array([[10.0, 10.0]])
    got = ref + np.array([[0.9 * cmp.BACKWARD_REL["bf16"] * 10.0, 0.0]])
    v = cmp.compare_backward([got], [ref], [scl], "bf16")
    assert v.ok and abs(v.max_ratio - 0.9) < 1e-9 and abs(v.max_tight_ratio - 0.9) < 1e-9
    f = cmp.compare([got], [ref], [scl], "bf16", rel=cmp.BACKWARD_REL["bf16"])
    assert f.max_tight_ratio > 10.0


def test_backward_scales_are_the_cauchy_schwarz_bounds():
    """backward_scales() against norms written out as loops: dx[t, c] scale
    sqrt(sum_f dy[t,f]^2) * sqrt(sum_f W[c,f]^2), dW[c, f] scale
    sqrt(sum_t x[t,c]^2) * sqrt(sum_t dy[t,f]^2), db[f] scale sqrt(M) * sqrt(sum_t dy[t,f]^2);
    and every oracle gradient element lies within its scale (the bound holds)."""
    r = np.random.default_rng(11)
    M, C, F = 5, 3, 4
    x = r.standard_normal((M, C))
    w = r.standard_normal((C, F))
    dy = r.standard_normal((M, F))
    sc = cmp.backward_scales(x, w, dy)
    for t in range(M):
        for c in range(C):
            e = math.sqrt(sum(dy[t, f] ** 2 for f in range(F))) * math.sqrt(sum(w[c, f] ** 2 for f in range(F)))
            assert abs(sc.dx[t, c] - e) <= 1e-12 * e
            assert abs(sum(dy[t, f] * w[c, f] for f in range(F))) <= sc.dx[t, c]
    for c in range(C):
        for f in range(F):
            e = math.sqrt(sum(x[t, c] ** 2 for t in range(M))) * math.sqrt(sum(dy[t, f] ** 2 for t in range(M)))
            assert abs(sc.dw[c, f] - e) <= 1e-12 * e
            assert abs(sum(x[t, c] * dy[t, f] for t in range(M))) <= sc.dw[c, f]
    for f in range(F):
        e = math.sqrt(M) * math.sqrt(sum(dy[t, f] ** 2 for t in range(M)))
        assert abs(sc.db[f] - e) <= 1e-12 * e
        assert abs(sum(dy[t, f] for t in range(M))) <= sc.db[f]


def _bf16(a):
    """Round float64 values to bf16 (round to nearest even) and back, through torch."""
    import torch

    return torch.from_numpy(np.asarray(a, dtype=np.float64)).float().to(torch.bfloat16).double().numpy()


def test_backward_bar_covers_two_bf16_roundings():
    """The backward bar is the arithmetic's: a dW element summed over 3 tokens from dy rounded
    to bf16 (its 7 fraction bits give each rounding up to 2^-8 of the value), then rounded
    itself, lands 0.62% of its Cauchy-Schwarz bound from the exact sum (one such element
    came out of a seeded backward case): more than the forward's 4e-3, less than the
    backward's 8e-3."""
    x = np.array([-0.02160645, 0.81640625, -0.546875])          # bf16 values
    dy = np.array([-0.18385676, 1.07453544, -2.13347303])       # exact float64 gradient
    exact = float(x @ dy)
    bound = float(np.linalg.norm(x) * np.linalg.norm(dy))
    got = float(_bf16(np.float32(x @ _bf16(dy))))
    err = abs(got - exact) / bound
    assert cmp.REL["bf16"] < err < cmp.BACKWARD_REL["bf16"], err


def test_backward_bar_bounds_random_double_roundings():
    """Random short and long sums with dy rounded to bf16 and the fp32 result rounded again:
    every error stays within 2 * 2^-8 (1 + 2^-8) of the bound, below BACKWARD_REL."""
    rng = np.random.default_rng(17)
    worst = 0.0
    for n in (1, 2, 3, 4, 8, 64):
        x = _bf16(rng.standard_normal((4000, n)))
        dy = rng.standard_normal((4000, n)) * rng.choice([0.25, 1.0, 3.0], size=(4000, 1))
        exact = np.einsum("ij,ij->i", x, dy)
        got = _bf16(np.einsum("ij,ij->i", x, _bf16(dy)).astype(np.float32))
        bound = np.linalg.norm(x, axis=1) * np.linalg.norm(dy, axis=1)
        worst = max(worst, float(np.max(np.abs(got - exact) / bound)))
    assert worst <= 2 * 2.0 ** -8 * (1 + 2.0 ** -8)
    assert worst < cmp.BACKWARD_REL["bf16"]
    # and the bar is that bound, not looser (within 5%)
    assert cmp.BACKWARD_REL["bf16"] <= 1.05 * 2 * 2.0 ** -8 * (1 + 2.0 ** -8)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_compare_backward_uses_the_backward_bar(dtype):
    """compare_backward() fails at 1.01x BACKWARD_REL and passes at 0.99x."""
    ref = np.array([1.0, -2.0, 0.5])
    scl = np.array([3.0, 4.0, 5.0])
    rel = cmp.BACKWARD_REL[dtype]
    assert not cmp.compare_backward([ref + 1.01 * rel * scl], [ref], [scl], dtype).ok
    assert cmp.compare_backward([ref + 0.99 * rel * scl], [ref], [scl], dtype).ok
