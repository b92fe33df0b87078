"""Pins of the float64 backward oracle (oracle.fused_proj_backward) to facts outside it
(CPU only).

The backward pass is the gradient of the forward definition, so its strongest pin is
the forward oracle itself: central finite differences of the scalar
L = <d_ff, ff> + <dq, q> + <dk, k> + <dv, v> with respect to every element of x, W
and the bias must equal the backward oracle's dx, dW and db. That catches a wrong
activation derivative, an inverse RoPE rotated the wrong way, a gradient scattered to
the wrong column, head or layout, and a missing bias in the recomputed pre-activation.
The three contractions are also pinned to numpy matmuls of the oracle's own dy, and dy
itself to the upstream gradients where the forward is a pure copy (no activation, no
RoPE).
"""
import math

import numpy as np
import pytest

import oracle


def _inputs(seed, layout, x_shape, C, F, w_layout, bias):
    r = np.random.default_rng(seed)
    x = r.standard_normal(x_shape)
    w = r.standard_normal((C, F)) / math.sqrt(C)
    if w_layout == "fc":
        w = np.ascontiguousarray(w.T)
    b = r.standard_normal(F) * 0.3 if bias else None
    return r, x, w, b


def _grads(r, nb, S, ff_dim, ff_layout, H, KVH, hd):
    d_ff = None
    if ff_dim > 0:
        d_ff = r.standard_normal((nb, ff_dim, S) if ff_layout == "channels_first" else (nb, S, ff_dim))
    dq = r.standard_normal((nb * H, S, hd)) if H else None
    dk = r.standard_normal((nb * KVH, S, hd)) if H else None
    dv = r.standard_normal((nb * KVH, S, hd)) if H else None
    return d_ff, dq, dk, dv


def _loss(x, w, b, layout, w_layout, kw, grads, ff_layout):
    res = oracle.fused_proj(x, layout, w, w_layout, b, **kw)
    d_ff, dq, dk, dv = grads
    total = 0.0
    if d_ff is not None:
        ff = res.ff
        if ff_layout == "channels_first":
            ff = ff.transpose(0, 2, 1)                 # [b, S, FF] -> [b, FF, S]
        total += float(np.sum(d_ff * ff))
    for g, o in ((dq, res.q), (dk, res.k), (dv, res.v)):
        if g is not None:
            total += float(np.sum(g * o))
    return total


CASES = [
    # name, layout, x_shape, w_layout, bias, ff_dim, act, H, KVH, hd, order, rope, rope_dims, pos, ff_layout
    ("cf_gelu_rope_offset", "channels_first", (2, 4, 3, 1), "cf", True, 4, "gelu", 2, 0, 4, "contiguous", True, 0,
     2, "tokens_last"),
    ("tl_fc_tanh_gqa_partial_ffcf", "tokens_last", (2, 3, 5), "fc", True, 6, "gelu_tanh", 4, 2, 4, "grouped", True,
     2, 0, "channels_first"),
    ("tl_relu2_mqa_nobias_norope", "tokens_last", (1, 4, 3), "cf", False, 4, "relu2", 2, 1, 2, "contiguous", False,
     0, 0, "tokens_last"),
    ("cf2d_none_grouped_rope", "channels_first", (2, 3, 2, 2), "fc", True, 2, "none", 2, 1, 4, "grouped", True, 0,
     5, "tokens_last"),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_backward_equals_finite_differences_of_the_forward(case):
    (name, layout, x_shape, w_layout, bias, ff_dim, act, H, kvh, hd, order, rope, rd, pos, ff_layout) = case
    C = x_shape[1] if layout == "channels_first" else x_shape[2]
    nb = x_shape[0]
    S = int(np.prod(x_shape[2:])) if layout == "channels_first" else x_shape[1]
    KVH = kvh if kvh > 0 else H
    F = ff_dim + (H + 2 * KVH) * hd
    r, x, w, b = _inputs(sum(map(ord, name)), layout, x_shape, C, F, w_layout, bias)
    grads = _grads(r, nb, S, ff_dim, ff_layout, H, KVH, hd)
    kw = dict(ff_dim=ff_dim, ff_act=act, n_heads=H, head_dim=hd, rope=rope, pos_offset=pos, n_kv_heads=kvh,
              qkv_order=order, rope_dims=rd, ff_layout=ff_layout)
    fwd_kw = {k: v for k, v in kw.items() if k != "ff_layout"}
    if act == "relu2":
        # keep every pre-activation away from the kink at 0
        y = oracle.fused_proj(x, layout, w, w_layout, b, ff_dim, "none", H, hd, False, n_kv_heads=kvh,
                              qkv_order=order).ff
        assert np.min(np.abs(y)) > 1e-3
    bw = oracle.fused_proj_backward(x, layout, w, w_layout, b, d_ff=grads[0], dq=grads[1], dk=grads[2],
                                    dv=grads[3], **kw)
    h = 1e-5

    def fd(arr, setter):
        g = np.empty(arr.size)
        flat = arr.reshape(-1)
        for i in range(arr.size):
            keep = flat[i]
            flat[i] = keep + h
            lp = setter()
            flat[i] = keep - h
            lm = setter()
            flat[i] = keep
            g[i] = (lp - lm) / (2 * h)
        return g.reshape(arr.shape)

    loss = lambda: _loss(x, w, b, layout, w_layout, fwd_kw, grads, ff_layout)
    np.testing.assert_allclose(bw.dx, fd(x, loss), rtol=0, atol=2e-7)
    np.testing.assert_allclose(bw.dw, fd(w, loss), rtol=0, atol=2e-7)
    if bias:
        np.testing.assert_allclose(bw.db, fd(b, loss), rtol=0, atol=2e-7)
    else:
        assert bw.db is None


def _gathered(x, layout):
    if layout == "channels_first":
        perm = (0,) + tuple(range(2, x.ndim)) + (1,)
        return x.transpose(perm).reshape(-1, x.shape[1])
    return x.reshape(-1, x.shape[2])


@pytest.mark.parametrize("layout,x_shape,w_layout", [("channels_first", (2, 6, 4, 2), "cf"),
                                                      ("tokens_last", (3, 5, 6), "fc")])
def test_contractions_equal_numpy_products_of_dy(layout, x_shape, w_layout):
    """Given the oracle's dy: dx = dy W^T, dW = X^T dy and db = column sums of dy, with
    numpy's matmul on the explicitly gathered X. Catches W read transposed, a dW over the
    wrong tokens, dx left in token-major order for a channels-first x."""
    C = x_shape[1] if layout == "channels_first" else x_shape[2]
    nb = x_shape[0]
    S = int(np.prod(x_shape[2:])) if layout == "channels_first" else x_shape[1]
    H, hd, ff_dim = 2, 4, 8
    F = ff_dim + 3 * H * hd
    r, x, w, b = _inputs(41, layout, x_shape, C, F, w_layout, True)
    grads = _grads(r, nb, S, ff_dim, "tokens_last", H, H, hd)
    bw = oracle.fused_proj_backward(x, layout, w, w_layout, b, ff_dim, "gelu", H, hd, True, *grads)
    w_cf = w if w_layout == "cf" else w.T
    X = _gathered(x, layout)
    dx_rows = bw.dy @ w_cf.T
    if layout == "channels_first":
        dx_ref = dx_rows.reshape(nb, S, C).transpose(0, 2, 1).reshape(x.shape)
    else:
        dx_ref = dx_rows.reshape(x.shape)
    np.testing.assert_allclose(bw.dx, dx_ref, rtol=1e-12, atol=1e-12)
    dw_cf = X.T @ bw.dy
    np.testing.assert_allclose(bw.dw, dw_cf if w_layout == "cf" else dw_cf.T, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(bw.db, bw.dy.sum(axis=0), rtol=1e-12, atol=1e-12)


def test_dy_without_activation_or_rope_is_the_upstream_gradient():
    """Where the forward only copies (no activation, no RoPE), dy holds the upstream
    gradients at their fused columns: ff column f, q head h element j at ff + h*hd + j, k
    and v after all q heads (contiguous order)."""
    nb, S, C, H, hd, ff_dim = 2, 3, 4, 2, 4, 4
    F = ff_dim + 3 * H * hd
    r, x, w, b = _inputs(43, "tokens_last", (nb, S, C), C, F, "cf", True)
    d_ff, dq, dk, dv = _grads(r, nb, S, ff_dim, "tokens_last", H, H, hd)
    bw = oracle.fused_proj_backward(x, "tokens_last", w, "cf", b, ff_dim, "none", H, hd, False, d_ff, dq, dk, dv)
    for bi in range(nb):
        for s in range(S):
            t = bi * S + s
            np.testing.assert_array_equal(bw.dy[t, :ff_dim], d_ff[bi, s])
            for which, g in enumerate((dq, dk, dv)):
                for h in range(H):
                    col = ff_dim + which * H * hd + h * hd
                    np.testing.assert_array_equal(bw.dy[t, col:col + hd], g[bi * H + h, s])


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_no_channels_equals_one_zero_channel(case):
    """C = 0: dx and dW are empty, and dy and db must equal, bit for bit, those of a run
    with one channel whose x is zero (the pre-activation is the bias in both)."""
    _, layout, x_shape, w_layout, bias, ff_dim, act, H, KVH, hd, order, rope, rd, pos, ff_layout = case
    KVH = KVH or H
    F = ff_dim + (H + 2 * KVH) * hd
    nb = x_shape[0]
    S = math.prod(x_shape[2:]) if layout == "channels_first" else x_shape[1]
    ci = 1 if layout == "channels_first" else 2
    shape0, shape1 = list(x_shape), list(x_shape)
    shape0[ci], shape1[ci] = 0, 1
    r = np.random.default_rng(51)
    b = r.standard_normal(F) * 0.3 if bias else None
    w1 = r.standard_normal((1, F)) if w_layout == "cf" else r.standard_normal((F, 1))
    w0 = np.zeros((0, F)) if w_layout == "cf" else np.zeros((F, 0))
    grads = _grads(r, nb, S, ff_dim, ff_layout, H, KVH, hd)
    kw = dict(rope_base=10000.0, pos_offset=pos, n_kv_heads=KVH, qkv_order=order, rope_dims=rd, ff_layout=ff_layout)
    b0 = oracle.fused_proj_backward(np.zeros(shape0), layout, w0, w_layout, b, ff_dim, act, H, hd, rope, *grads, **kw)
    b1 = oracle.fused_proj_backward(np.zeros(shape1), layout, w1, w_layout, b, ff_dim, act, H, hd, rope, *grads, **kw)
    assert b0.dx.size == 0 and b0.dw.size == 0
    assert np.count_nonzero(b1.dw) == 0
    np.testing.assert_array_equal(b0.dy, b1.dy)
    if bias:
        np.testing.assert_array_equal(b0.db, b1.db)
        np.testing.assert_allclose(b0.db, b0.dy.sum(axis=0), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("act,torch_act", [("gelu", "none"), ("gelu_tanh", "tanh"), ("relu2", None)])
def test_activation_derivatives_equal_torch_autograd(act, torch_act):
    """dy = d_ff * act'(y) with W = 0, so that y equals the bias, against torch's autograd of
    its own GELU (exact and tanh forms) and of relu(y)**2, in float64. GELU'(0) is 1/2."""
    import torch

    b_vals = np.array([0.0, 1.0, -1.0, 2.5, -3.25, 0.3])
    F = b_vals.size
    x = np.ones((1, 1, 2))
    w = np.zeros((2, F))
    d_ff = np.linspace(0.5, 2.0, F).reshape(1, 1, F)
    bw = oracle.fused_proj_backward(x, "tokens_last", w, "cf", b_vals, F, act, 0, 0, False, d_ff, None, None, None)
    y = torch.tensor(b_vals, dtype=torch.float64, requires_grad=True)
    out = torch.nn.functional.gelu(y, approximate=torch_act) if torch_act else torch.relu(y) ** 2
    (out * torch.from_numpy(d_ff[0, 0])).sum().backward()
    np.testing.assert_allclose(bw.dy[0], y.grad.numpy(), rtol=1e-14, atol=1e-15)
    if act == "gelu":
        assert bw.dy[0, 0] == 0.5 * d_ff[0, 0, 0]
