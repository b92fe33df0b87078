"""Pins of the float64 oracle to facts outside itself (CPU only).

Each test names the plausible mistake it would catch. Sources: Walrus PR "Make
fused_ff_qkv contiguous" (gather + single GEMM), xformers PR "Fused linear:
small FW cleanup and much better perfs" (y = act(xW^T + b), three-buffer QKV),
NVIDIA/Fuser issue "Improve performance on RoPE (and code around it)"
(rotate-half RoPE), memory-efficient-attention issue "Improve performance via
batched-matmul and fused multiplies" ([batch*heads, tokens, head_dim]).
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rng_inputs(seed, x_shape, C, F, bias=True):
    r = np.random.default_rng(seed)
    x = r.standard_normal(x_shape)
    w = r.standard_normal((C, F)) / math.sqrt(C)
    b = r.standard_normal(F) * math.sqrt(0.02) if bias else None
    return x, w, b


def gathered_rows(x, layout):
    """[M, C] token rows by the pages' rearrange 'b c h w d -> b h w d c' (numpy transpose)."""
    if layout == "channels_first":
        nd = x.ndim
        perm = (0,) + tuple(range(2, nd)) + (1,)
        return x.transpose(perm).reshape(-1, x.shape[1])
    return x.reshape(-1, x.shape[2])


def scale(xr, w, b):
    s = np.linalg.norm(xr, axis=1)[:, None] * np.linalg.norm(w, axis=0)[None, :]
    if b is not None:
        s = s + np.abs(b)[None, :]
    return s


# --------------------------------------------------------------------------- contraction + gather

@pytest.mark.parametrize("w_layout", ["cf", "fc"])
@pytest.mark.parametrize("layout,x_shape", [("channels_first", (2, 12, 3, 5, 2)),
                                             ("tokens_last", (3, 7, 12))])
def test_per_token_gemv_equals_batched_gemm(layout, x_shape, w_layout):
    """Per-token GEMV loop (oracle) == one batched GEMM (numpy @) on the gathered
    matrix. Catches a dropped c term, a transposed W, a wrong gather stride."""
    C = x_shape[1] if layout == "channels_first" else x_shape[2]
    FF, H, hd = 8, 2, 4
    F = FF + 3 * H * hd
    x, w, b = rng_inputs(11, x_shape, C, F)
    wa = w if w_layout == "cf" else np.ascontiguousarray(w.T)
    res = oracle.fused_proj(x, layout, wa, w_layout, b, FF, "none", H, hd, rope=False)
    X = gathered_rows(x, layout)
    Y = X @ w + b
    s = scale(X, w, b)
    nb = x.shape[0]
    S = X.shape[0] // nb
    ff = res.ff.reshape(-1, FF)
    assert np.all(np.abs(ff - Y[:, :FF]) <= 1e-12 * s[:, :FF])
    # q/k/v: explicit index definition dst[bi*H + h, s, j] = y[bi*S + s, off + h*hd + j]
    for which, dst in enumerate([res.q, res.k, res.v]):
        off = FF + which * H * hd
        for bi in range(nb):
            for h in range(H):
                for si in range(S):
                    t = bi * S + si
                    cols = slice(off + h * hd, off + (h + 1) * hd)
                    assert np.all(np.abs(dst[bi * H + h, si] - Y[t, cols]) <= 1e-12 * s[t, cols])


def test_one_hot_weight_returns_gathered_rows_exactly():
    """W = [I | 0]: the ff slice is the gathered row itself, bit for bit.
    Catches any error in the channels-first index order (h, w, d, c)."""
    x = np.random.default_rng(3).standard_normal((2, 6, 3, 4, 5))
    C = 6
    FF, H, hd = C, 1, 2
    w = np.zeros((C, FF + 3 * H * hd))
    w[:, :C] = np.eye(C)
    res = oracle.fused_proj(x, "channels_first", w, "cf", None, FF, "none", H, hd, rope=False)
    expect = np.ascontiguousarray(x.transpose(0, 2, 3, 4, 1)).reshape(2, 60, C)
    assert np.array_equal(res.ff, expect)
    assert np.all(res.q == 0) and np.all(res.k == 0) and np.all(res.v == 0)


def test_layout_invariance_channels_first_vs_contiguous_copy():
    """Only contiguity changes between a channels-first tensor and its channels-last
    copy, so the result must be bitwise identical (the page's whole point)."""
    x, w, b = rng_inputs(5, (3, 16, 4, 4, 2), 16, 8 + 3 * 2 * 8)
    cl = np.ascontiguousarray(x.transpose(0, 2, 3, 4, 1)).reshape(3, 32, 16)
    args = dict(w=w, w_layout="cf", bias=b, ff_dim=8, ff_act="gelu", n_heads=2, head_dim=8, rope=True)
    r1 = oracle.fused_proj(x, "channels_first", **args)
    r2 = oracle.fused_proj(cl, "tokens_last", **args)
    for a, c in zip([r1.ff, r1.q, r1.k, r1.v], [r2.ff, r2.q, r2.k, r2.v]):
        assert np.array_equal(a, c)


def test_ff_slice_equals_1x1x1_conv3d():
    """The ff slice of a channels-first input, laid out channels-first, is the 1x1x1
    Conv3d the Walrus PR compares the linear with: torch's conv3d in float64 (a library
    routine) with the weight W[:, :ff]^T as [ff, C, 1, 1, 1] and the bias."""
    x, w, b = rng_inputs(51, (2, 6, 3, 4, 2), 6, 10)
    res = oracle.fused_proj(x, "channels_first", w, "cf", b, 10, "none", 0, 0, rope=False)
    ff_cf = res.ff.reshape(2, 3, 4, 2, 10).transpose(0, 4, 1, 2, 3)           # [b, ff, h, w, d]
    conv = torch.nn.functional.conv3d(torch.from_numpy(x), torch.from_numpy(w.T.copy()).reshape(10, 6, 1, 1, 1),
                                      torch.from_numpy(b)).numpy()
    assert np.allclose(ff_cf, conv, rtol=0, atol=1e-13)


def test_strided_view_equals_contiguous_copy():
    """x as a channel slice of a larger tensor (non-unit batch stride) and a view with
    a transposed spatial order give the same result as contiguous copies."""
    big = np.random.default_rng(9).standard_normal((2, 20, 4, 6, 1))
    x = big[:, 3:15]                               # channel slice, strided batch
    C, FF, H, hd = 12, 4, 2, 4
    w = np.random.default_rng(10).standard_normal((C, FF + 3 * H * hd))
    args = dict(w=w, w_layout="cf", bias=None, ff_dim=FF, ff_act="none", n_heads=H, head_dim=hd, rope=True)
    r1 = oracle.fused_proj(x, "channels_first", **args)
    r2 = oracle.fused_proj(np.ascontiguousarray(x), "channels_first", **args)
    assert np.array_equal(r1.ff, r2.ff) and np.array_equal(r1.q, r2.q)


def test_token_subset_matches_full_run():
    x, w, b = rng_inputs(21, (2, 10, 3, 3, 1), 10, 6 + 3 * 3 * 4)
    args = dict(w=w, w_layout="cf", bias=b, ff_dim=6, ff_act="gelu", n_heads=3, head_dim=4, rope=True)
    full = oracle.fused_proj(x, "channels_first", **args)
    toks = np.array([0, 5, 9, 17, 8])
    sub = oracle.fused_proj(x, "channels_first", tokens=toks, **args)
    S = 9
    for i, t in enumerate(toks):
        bi, si = divmod(int(t), S)
        assert np.array_equal(sub.ff[i], full.ff[bi, si])
        for h in range(3):
            assert np.array_equal(sub.q[i, h], full.q[bi * 3 + h, si])
            assert np.array_equal(sub.k[i, h], full.k[bi * 3 + h, si])
            assert np.array_equal(sub.v[i, h], full.v[bi * 3 + h, si])


# --------------------------------------------------------------------------- split + head-major layout

def test_head_major_matches_pages_transpose_flatten():
    """[batch, tokens, heads, depth] -> transpose(1,2).flatten(end_dim=1) is the page's
    conversion to [batch*heads, tokens, depth]; computed here with torch (not the
    numpy reshape the oracle wrapper uses). Also pins q, k, v column order and
    that neither GELU nor RoPE touches v."""
    b_, S, C, H, hd, FF = 3, 5, 8, 2, 4, 4
    x, w, b = rng_inputs(31, (b_, S, C), C, FF + 3 * H * hd)
    res = oracle.fused_proj(x, "tokens_last", w, "cf", b, FF, "gelu", H, hd, rope=False)
    Y = torch.from_numpy(x.reshape(-1, C) @ w + b).reshape(b_, S, -1)
    for which, dst in enumerate([res.q, res.k, res.v]):
        sl = Y[..., FF + which * H * hd: FF + (which + 1) * H * hd].reshape(b_, S, H, hd)
        ref = sl.transpose(1, 2).flatten(end_dim=1).numpy()
        assert ref.shape == dst.shape
        assert np.allclose(dst, ref, rtol=0, atol=1e-12)


def test_fused_equals_separate_slice_projections():
    """The fused op equals separate projections with the W and b column slices,
    bitwise in float64 (no interaction between slices)."""
    x, w, b = rng_inputs(41, (2, 9, 16), 16, 8 + 3 * 2 * 4)
    FF, H, hd = 8, 2, 4
    fused = oracle.fused_proj(x, "tokens_last", w, "cf", b, FF, "gelu", H, hd, rope=True)
    ff_only = oracle.fused_proj(x, "tokens_last", w[:, :FF], "cf", b[:FF], FF, "gelu", 0, 0, rope=True)
    qkv_only = oracle.fused_proj(x, "tokens_last", w[:, FF:], "cf", b[FF:], 0, "none", H, hd, rope=True)
    assert np.array_equal(fused.ff, ff_only.ff)
    assert np.array_equal(fused.q, qkv_only.q)
    assert np.array_equal(fused.k, qkv_only.k)
    assert np.array_equal(fused.v, qkv_only.v)


# --------------------------------------------------------------------------- bias and GELU

def test_zero_weight_gives_activated_bias():
    """W = 0: ff = gelu(b), v = b, q/k = RoPE(b) at position 0 = b. Catches a missing
    bias, or a bias added after the activation."""
    C, FF, H, hd = 4, 6, 2, 4
    x = np.random.default_rng(1).standard_normal((1, 1, C))
    w = np.zeros((C, FF + 3 * H * hd))
    b = np.linspace(-2.0, 2.0, FF + 3 * H * hd)
    res = oracle.fused_proj(x, "tokens_last", w, "cf", b, FF, "gelu", H, hd, rope=True)
    from scipy.special import ndtr
    assert np.allclose(res.ff[0, 0], b[:FF] * ndtr(b[:FF]), rtol=0, atol=1e-15)
    assert np.array_equal(res.v[:, 0].reshape(-1), b[FF + 2 * H * hd:])
    assert np.array_equal(res.q[:, 0].reshape(-1), b[FF:FF + H * hd])  # position 0


@pytest.mark.parametrize("layout,x_shape", [("channels_first", (2, 0, 3, 4, 1)), ("tokens_last", (2, 6, 0))])
def test_no_channels_equals_one_zero_channel(layout, x_shape):
    """C = 0: the contraction is an empty sum, so y = b. The result must equal, bit for
    bit, a run with one channel whose x is zero (0 * w = 0 exactly), for any weight row;
    and v = b and an identity ff slice = b exactly."""
    FF, H, hd = 6, 2, 4
    F = FF + 3 * H * hd
    b = np.linspace(-2.0, 2.0, F)
    x0 = np.zeros(x_shape)
    one = list(x_shape)
    one[1 if layout == "channels_first" else 2] = 1
    x1 = np.zeros(one)
    w1 = np.random.default_rng(7).standard_normal((1, F))
    for act in ("none", "gelu", "relu2"):
        r0 = oracle.fused_proj(x0, layout, np.zeros((0, F)), "cf", b, FF, act, H, hd, rope=True, pos_offset=3)
        r1 = oracle.fused_proj(x1, layout, w1, "cf", b, FF, act, H, hd, rope=True, pos_offset=3)
        for a0, a1 in zip((r0.ff, r0.q, r0.k, r0.v), (r1.ff, r1.q, r1.k, r1.v)):
            assert np.array_equal(a0, a1)
        if act == "none":
            assert np.array_equal(r0.ff.reshape(-1, FF), np.broadcast_to(b[:FF], (r0.ff.size // FF, FF)))
        v = r0.v.reshape(2, H, -1, hd).transpose(0, 2, 1, 3).reshape(-1, H * hd)   # [b*S, H*hd]
        assert np.array_equal(v, np.broadcast_to(b[FF + 2 * H * hd:], v.shape))
    r_nb = oracle.fused_proj(x0, layout, np.zeros((F, 0)), "fc", None, FF, "gelu", H, hd, rope=True)
    assert all(np.count_nonzero(a) == 0 for a in (r_nb.ff, r_nb.q, r_nb.k, r_nb.v))


def test_activations_at_non_finite_values_match_torch():
    """The oracle's activations at NaN, +-inf and large values equal torch's float64 ones
    (exact GELU, tanh GELU, squared ReLU through torch.relu): NaN passes through every
    activation, GELU(+inf) = +inf, GELU(-inf) = NaN (y Phi(y) in IEEE arithmetic) and
    relu^2(-inf) = 0. One channel with weight 1, so each token's y is its own value."""
    import torch.nn.functional as F
    vals = np.array([np.nan, np.inf, -np.inf, -1e3, -1.5, 0.0, 2.5, 1e3])
    x = vals.reshape(1, -1, 1)
    tv = torch.from_numpy(vals)
    for act, ref in (("gelu", F.gelu(tv)), ("gelu_tanh", F.gelu(tv, approximate="tanh")),
                     ("relu2", torch.relu(tv) ** 2)):
        got = oracle.fused_proj(x, "tokens_last", np.ones((1, 1)), "cf", None, 1, act, 0, 0, rope=False).ff
        got, ref = got.reshape(-1), ref.numpy()
        assert np.array_equal(np.isnan(got), np.isnan(ref)), (act, got, ref)
        fin = ~np.isnan(ref)
        np.testing.assert_allclose(got[fin], ref[fin], rtol=1e-12, atol=0)


def _gelu_via_oracle(vals):
    """Run the oracle with W = I on the FF slice so that ff = gelu(x)."""
    n = len(vals)
    x = np.asarray(vals, dtype=np.float64).reshape(1, 1, n)
    w = np.eye(n)
    return oracle.fused_proj(x, "tokens_last", w, "cf", None, n, "gelu", 0, 0, rope=False).ff.reshape(-1)


def test_gelu_golden_values():
    rows = [l.split() for l in open(os.path.join(GOLDEN, "gelu_erf_values.txt")) if l.strip() and l[0] != "#"]
    ys = [float(r[0]) for r in rows]
    ref = [float(r[1]) for r in rows]
    got = _gelu_via_oracle(ys)
    assert np.allclose(got, ref, rtol=2e-15, atol=1e-300)


def test_gelu_identities_and_torch_exact_gelu():
    """gelu(y) - gelu(-y) = y; agreement with torch's exact GELU in float64.
    Catches the tanh approximation (off by up to ~5e-4)."""
    y = np.linspace(-6, 6, 97)
    g = _gelu_via_oracle(y)
    gm = _gelu_via_oracle(-y)
    assert np.allclose(g - gm, y, rtol=0, atol=4e-15)
    t = torch.nn.functional.gelu(torch.from_numpy(y), approximate="none").numpy()
    assert np.allclose(g, t, rtol=0, atol=1e-15)
    tanh = torch.nn.functional.gelu(torch.from_numpy(y), approximate="tanh").numpy()
    assert np.max(np.abs(g - tanh)) > 1e-4


def _act_via_oracle(vals, act):
    """Run the oracle with W = I on the FF slice so that ff = act(x)."""
    n = len(vals)
    x = np.asarray(vals, dtype=np.float64).reshape(1, 1, n)
    return oracle.fused_proj(x, "tokens_last", np.eye(n), "cf", None, n, act, 0, 0, rope=False).ff.reshape(-1)


def test_tanh_gelu_against_torch_tanh_gelu():
    """The tanh form of GELU (Hendrycks and Gimpel, 2016): torch's GELU with
    approximate='tanh' in float64 (a library routine), the odd-part identity
    g(y) - g(-y) = y, and a distance of 1e-4 .. 1e-3 from the exact-erf form. Catches a
    wrong constant (0.044715, sqrt(2/pi)), a missing cube, or the erf form in its place."""
    y = np.linspace(-8, 8, 161)
    g = _act_via_oracle(y, "gelu_tanh")
    gm = _act_via_oracle(-y, "gelu_tanh")
    assert np.allclose(g - gm, y, rtol=0, atol=4e-15)
    t = torch.nn.functional.gelu(torch.from_numpy(y), approximate="tanh").numpy()
    assert np.allclose(g, t, rtol=0, atol=2e-15)
    d = np.max(np.abs(g - _act_via_oracle(y, "gelu")))
    assert 1e-4 < d < 1e-3, d


def test_squared_relu_against_torch_relu():
    """Squared ReLU max(y, 0)^2 (named in the xformers PR discussion): zero for y <= 0,
    torch.relu(y) ** 2 in float64, and degree-2 homogeneity r(2y) = 4 r(y). Catches a
    missing square, |y| in place of max(y, 0), or a missing clamp."""
    y = np.linspace(-5, 5, 101)
    r = _act_via_oracle(y, "relu2")
    assert np.all(r[y <= 0] == 0.0)
    t = (torch.relu(torch.from_numpy(y)) ** 2).numpy()
    assert np.allclose(r, t, rtol=1e-15, atol=0)
    assert np.allclose(_act_via_oracle(2 * y, "relu2"), 4 * r, rtol=1e-15, atol=0)


def test_activation_applies_to_the_ff_slice_only():
    """The activation acts on the ff columns after the bias; q/k/v are untouched.
    Catches an activation on every column, or one applied before the bias."""
    x, w, b = rng_inputs(21, (2, 5, 12), 12, 8 + 3 * 8)
    for act in ("gelu_tanh", "relu2"):
        res = oracle.fused_proj(x, "tokens_last", w, "cf", b, 8, act, 2, 4, rope=False)
        plain = oracle.fused_proj(x, "tokens_last", w, "cf", b, 8, "none", 2, 4, rope=False)
        for a, c in ((res.q, plain.q), (res.k, plain.k), (res.v, plain.v)):
            assert np.array_equal(a, c)
        assert np.allclose(res.ff, _act_via_oracle(plain.ff.reshape(-1), act).reshape(plain.ff.shape),
                           rtol=0, atol=1e-15)


# --------------------------------------------------------------------------- grouped q/k/v (GQA)

def _head_major(a, nb, S, H, hd):
    """[nb*S, H*hd] token-major rows -> [nb*H, S, hd] (numpy reshape/transpose)."""
    return a.reshape(nb, S, H, hd).transpose(0, 2, 1, 3).reshape(nb * H, S, hd)


def test_grouped_order_column_formula():
    """The grouped q/k/v order (split_qkv in the nvFuser RoPE issue, the lit-gpt layout):
    each k/v group holds q_per_kv q heads, then one k head, then one v head, so element j of
    slot `slot` of group g sits in fused column ff + (g*(q_per_kv + 2) + slot)*hd + j. The
    expected buffers are filled element by element from that formula on the plain product
    x @ W. Catches swapped k/v slots and q heads numbered across groups."""
    B, T, C, H, G, hd = 2, 5, 12, 4, 2, 4
    qpk = H // G
    F = (H + 2 * G) * hd
    x, w, _ = rng_inputs(31, (B, T, C), C, F, bias=False)
    res = oracle.fused_proj(x, "tokens_last", w, "cf", None, 0, "none", H, hd, rope=False, n_kv_heads=G,
                            qkv_order="grouped")
    y = x.reshape(B, T, C) @ w                                          # [B, T, F]
    q = np.empty((B * H, T, hd))
    k = np.empty((B * G, T, hd))
    v = np.empty((B * G, T, hd))
    for b in range(B):
        for t in range(T):
            for g in range(G):
                for j in range(hd):
                    col = lambda slot: (g * (qpk + 2) + slot) * hd + j
                    for i in range(qpk):
                        q[b * H + g * qpk + i, t, j] = y[b, t, col(i)]
                    k[b * G + g, t, j] = y[b, t, col(qpk)]
                    v[b * G + g, t, j] = y[b, t, col(qpk + 1)]
    for got, ref in ((res.q, q), (res.k, k), (res.v, v)):
        assert got.shape == ref.shape
        assert np.allclose(got, ref, rtol=0, atol=1e-12)


def test_contiguous_gqa_slices():
    """Contiguous order with fewer k/v heads: q is the first H*hd columns, k and v the
    next two blocks of G*hd, each head-major. Catches k/v blocks sized by the q width."""
    B, T, C, H, G, hd = 2, 6, 10, 6, 3, 4
    F = 8 + (H + 2 * G) * hd
    x, w, b = rng_inputs(32, (B, T, C), C, F)
    res = oracle.fused_proj(x, "tokens_last", w, "cf", b, 8, "gelu", H, hd, rope=False, n_kv_heads=G)
    y = x.reshape(-1, C) @ w + b
    q0, k0 = 8, 8 + H * hd
    v0 = k0 + G * hd
    assert np.allclose(res.q, _head_major(y[:, q0:k0], B, T, H, hd), rtol=0, atol=1e-12)
    assert np.allclose(res.k, _head_major(y[:, k0:v0], B, T, G, hd), rtol=0, atol=1e-12)
    assert np.allclose(res.v, _head_major(y[:, v0:], B, T, G, hd), rtol=0, atol=1e-12)


def test_partial_rope_as_complex_rotation():
    """Partial rotary on q and k (rope_one_entry with rope_n_elem in the nvFuser RoPE
    issue): the pairs (i, i + R/2) of the first R elements of a head, read as the complex
    number z = y_i + 1j*y_{i+R/2}, are multiplied by e^{1j*phi_i} with
    phi_i = p * base^(-2i/R) (the angle convention shared with the GPU path); elements from
    R on pass through. Catches rotating the whole head, pairs taken across the head
    instead of across the rotated width, and the sign of the rotation."""
    B, T, C, H, G, hd, R = 1, 9, 8, 4, 2, 16, 8
    F = (H + 2 * G) * hd
    x, w, _ = rng_inputs(33, (B, T, C), C, F, bias=False)
    kw = dict(n_kv_heads=G, qkv_order="grouped")
    plain = oracle.fused_proj(x, "tokens_last", w, "cf", None, 0, "none", H, hd, rope=False, **kw)
    roped = oracle.fused_proj(x, "tokens_last", w, "cf", None, 0, "none", H, hd, rope=True, rope_dims=R, **kw)
    for got, pre in ((roped.q, plain.q), (roped.k, plain.k)):
        ref = pre.copy()
        for i in range(R // 2):
            phi = np.arange(T) * 10000.0 ** (-2.0 * i / R)                    # [T]
            z = (pre[..., i] + 1j * pre[..., i + R // 2]) * np.exp(1j * phi)[None, :]
            ref[..., i], ref[..., i + R // 2] = z.real, z.imag
        assert np.allclose(got, ref, rtol=0, atol=1e-12)
        assert np.array_equal(got[..., R:], pre[..., R:])
    assert np.array_equal(roped.v, plain.v)


def test_comparison_column_map_matches_oracle():
    """The parity bar's column map (oracle/compare.qkv_columns) picks, for every q/k/v
    element, the fused column the oracle writes there (both orders, fewer k/v heads)."""
    from oracle import compare as cmp
    B, T, C, H, G, hd = 2, 4, 6, 4, 2, 4
    for order in ("contiguous", "grouped"):
        F = 8 + (H + 2 * G) * hd
        x, w, _ = rng_inputs(35, (B, T, C), C, F, bias=False)
        res = oracle.fused_proj(x, "tokens_last", w, "cf", None, 8, "none", H, hd, rope=False, n_kv_heads=G,
                                qkv_order=order, tokens=np.arange(B * T))
        y = x.reshape(-1, C) @ w
        for got, cols in zip((res.q, res.k, res.v), cmp.qkv_columns(8, H, hd, G, order)):
            assert np.allclose(got, y[:, cols], rtol=0, atol=1e-12)


def test_full_width_rope_dims_equals_default():
    """rope_dims = head_dim is the full rotation (the default)."""
    x, w, b = rng_inputs(34, (2, 7, 8), 8, 3 * 2 * 8)
    a = oracle.fused_proj(x, "tokens_last", w, "cf", b, 0, "none", 2, 8, rope=True)
    c = oracle.fused_proj(x, "tokens_last", w, "cf", b, 0, "none", 2, 8, rope=True, rope_dims=8)
    for u, v in ((a.q, c.q), (a.k, c.k), (a.v, c.v)):
        assert np.array_equal(u, v)


# --------------------------------------------------------------------------- standalone split + RoPE

@pytest.mark.parametrize("order,kvh,rd", [("grouped", 2, 8), ("contiguous", 4, 0), ("grouped", 1, 4)])
def test_split_rope_equals_fused_projection_with_identity_weight(order, kvh, rd):
    """Split + RoPE of a projected tensor is the fused projection of that tensor with
    W = I: both layouts of the columns, fewer k/v heads, partial rotary, a position
    offset. Pins the standalone op to the pinned fused definition."""
    B, T, H, hd = 2, 6, 4, 16
    Fq = (H + 2 * kvh) * hd
    r = np.random.default_rng(41)
    y = r.standard_normal((B, T, Fq))
    q, k, v = oracle.split_rope(y, H, hd, n_kv_heads=kvh, qkv_order=order, rope=True, rope_dims=rd, pos_offset=3)
    ref = oracle.fused_proj(y, "tokens_last", np.eye(Fq), "cf", None, 0, "none", H, hd, rope=True, pos_offset=3,
                            n_kv_heads=kvh, qkv_order=order, rope_dims=rd)
    for a, c in ((q, ref.q), (k, ref.k), (v, ref.v)):
        assert a.shape == c.shape
        assert np.allclose(a, c, rtol=0, atol=1e-14)


def test_split_rope_transposed_key_and_plain_copy_of_v():
    """The transposed key is the [hd, T] transpose of each k head; v is a plain copy of
    its columns (no RoPE)."""
    B, T, H, G, hd = 1, 5, 4, 2, 8
    Fq = (H + 2 * G) * hd
    y = np.random.default_rng(42).standard_normal((B, T, Fq))
    args = dict(n_kv_heads=G, qkv_order="grouped", rope=True, rope_dims=4)
    q, k, v = oracle.split_rope(y, H, hd, **args)
    _, kt, _ = oracle.split_rope(y, H, hd, k_transposed=True, **args)
    assert np.array_equal(kt, k.transpose(0, 2, 1))
    vref = y.reshape(B, T, G, H // G + 2, hd)[:, :, :, H // G + 1].transpose(0, 2, 1, 3).reshape(B * G, T, hd)
    assert np.array_equal(v, vref)


# --------------------------------------------------------------------------- RoPE

def _rope_via_oracle(vec, p, base, which="q"):
    """Rotate one head vector at position p: W = I on the q (or k) slice, one token
    row placed at slab position p (tokens_last [1, p+1, hd], the last row used)."""
    hd = len(vec)
    S = p + 1
    x = np.zeros((1, S, hd))
    x[0, p] = vec
    w = np.zeros((hd, 3 * hd))
    col = 0 if which == "q" else hd
    w[:, col:col + hd] = np.eye(hd)
    res = oracle.fused_proj(x, "tokens_last", w, "cf", None, 0, "none", 1, hd, rope=True, rope_base=base)
    return (res.q if which == "q" else res.k)[0, p]


def _golden_rope_cases():
    out = []
    for line in open(os.path.join(GOLDEN, "rope_rotate_half_cases.txt")):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        lhs, rhs = line.split(":")
        hd, base, p, idx = lhs.split()
        terms = []
        for t in rhs.split():
            o, e = t.split("=")
            fn, ang = e[:-1].split("(")
            terms.append((int(o), fn, float(ang)))
        out.append((int(hd), float(base), int(p), int(idx), terms))
    return out


@pytest.mark.parametrize("case", _golden_rope_cases())
@pytest.mark.parametrize("which", ["q", "k"])
def test_rope_golden_unit_vectors(case, which):
    """A unit vector maps to one column of the rotate-half rotation, worked out by hand.
    Catches sign errors, interleaved (2i, 2i+1) pairing and a wrong frequency exponent."""
    hd, base, p, idx, terms = case
    v = np.zeros(hd)
    v[idx] = 1.0
    got = _rope_via_oracle(v, p, base, which)
    expect = np.zeros(hd)
    fns = {"cos": math.cos, "sin": math.sin, "-sin": lambda a: -math.sin(a)}
    for o, fn, ang in terms:
        expect[o] = fns[fn](ang)
    assert np.allclose(got, expect, rtol=0, atol=2e-12)


def test_rope_position_zero_identity_and_norm_preservation():
    """Position 0 leaves q/k unchanged exactly; each (i, i+hd/2) pair keeps its norm."""
    hd, H, C, S = 16, 3, 24, 40
    x, w, b = rng_inputs(51, (2, S, C), C, 3 * H * hd)
    r_on = oracle.fused_proj(x, "tokens_last", w, "cf", b, 0, "none", H, hd, rope=True)
    r_off = oracle.fused_proj(x, "tokens_last", w, "cf", b, 0, "none", H, hd, rope=False)
    # position 0 of EVERY slab (positions restart per slab)
    assert np.array_equal(r_on.q[:, 0], r_off.q[:, 0])
    assert np.array_equal(r_on.k[:, 0], r_off.k[:, 0])
    assert np.array_equal(r_on.v, r_off.v)
    half = hd // 2
    for a_on, a_off in [(r_on.q, r_off.q), (r_on.k, r_off.k)]:
        n_on = a_on[..., :half] ** 2 + a_on[..., half:] ** 2
        n_off = a_off[..., :half] ** 2 + a_off[..., half:] ** 2
        assert np.allclose(n_on, n_off, rtol=1e-13, atol=0)
        assert not np.allclose(a_on[:, 1:], a_off[:, 1:])


def test_rope_relative_position_and_pos_offset():
    """<R_p q, R_p' k> depends only on p - p' (rotations compose); pos_offset shifts
    the position of every token by the same amount."""
    hd, C, S = 8, 8, 12
    row = np.random.default_rng(61).standard_normal(C)
    x = np.tile(row, (1, S, 1))                    # identical token rows
    w = np.random.default_rng(62).standard_normal((C, 3 * hd))
    r = oracle.fused_proj(x, "tokens_last", w, "cf", None, 0, "none", 1, hd, rope=True)
    q, k = r.q[0], r.k[0]
    g = q @ k.T
    for d in range(-3, 4):
        vals = [g[i, i + d] for i in range(max(0, -d), min(S, S - d))]
        assert np.allclose(vals, vals[0], rtol=1e-12, atol=1e-12)
    r5 = oracle.fused_proj(x, "tokens_last", w, "cf", None, 0, "none", 1, hd, rope=True, pos_offset=5)
    assert np.allclose(r5.q[0, :S - 5], q[5:], rtol=0, atol=1e-13)
    assert np.allclose(r5.k[0, :S - 5], k[5:], rtol=0, atol=1e-13)


def test_oracle_rejects_bad_arguments():
    x = np.zeros((1, 4, 6))
    w = np.zeros((6, 10))
    with pytest.raises(ValueError):   # F != ff + 3*H*hd
        oracle.fused_proj(x, "tokens_last", w, "cf", None, 3, "none", 1, 2, rope=False)
    w2 = np.zeros((6, 1 + 9))
    with pytest.raises(ValueError):   # odd head_dim with RoPE
        oracle.fused_proj(x, "tokens_last", w2, "cf", None, 1, "none", 1, 3, rope=True)
    with pytest.raises(ValueError):   # token out of range
        oracle.fused_proj(x, "tokens_last", w, "cf", None, 4, "none", 1, 2, rope=False, tokens=np.array([4]))
