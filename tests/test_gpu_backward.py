"""GPU parity of the backward pass (fused_proj_backward through the C ABI) against the
float64 backward oracle, element by element.

Bar: each gradient element is one sum of products, and its error must stay within
8e-3 (bf16) or 1e-5 (fp32) of the Cauchy-Schwarz bound of that sum
(oracle/compare.py backward_scales, BACKWARD_REL): ||dy_t|| ||W_c|| for dx,
||x_c|| ||dy_f|| for dW, sqrt(M) ||dy_f|| for db, with dy the oracle's float64 gradient of
the fused output. dy is held in the storage type between the launches, which moves every
sum by at most 2^-8 of its bound for bf16, and the final rounding moves the result by 2^-8
of itself again; with few terms (3 tokens) both come close to their bound together.
Outputs start as NaN, so every element must have been written.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import compare as cmp
from ff_input_projection_amd import EALIAS, EALIGN, EINVAL, FusedProjError
from ff_input_projection_amd.workloads import WORKLOADS, make_grads, make_inputs, with_shape

from helpers import plan_for
from test_gpu_parity import SMALL

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _to_dev(t):
    return None if t is None else t.to(DEV)


def _token_rows(a, layout, nb, C, S):
    """dx (x's logical layout) as token-major rows [M, C]."""
    if layout == "channels_first":
        return a.reshape(nb, C, S).transpose(0, 2, 1).reshape(nb * S, C)
    return a.reshape(nb * S, C)


def run_backward(wl, inp=None, gr=None):
    inp = inp or make_inputs(wl)
    gr = gr or make_grads(wl)
    x, w, b = inp.x.to(DEV), inp.w.to(DEV), _to_dev(inp.bias)
    proj = plan_for(wl, x)
    outs = proj.alloc_grads(DEV)
    for t in outs:
        if t is not None:
            t.fill_(float("nan"))
    grads = proj.backward(x, w, b, _to_dev(gr.d_ff), _to_dev(gr.dq), _to_dev(gr.dk), _to_dev(gr.dv), out=outs)
    torch.cuda.synchronize()
    return proj, inp, gr, grads


def backward_verdict(wl, inp, gr, grads):
    ref = oracle.fused_proj_backward(inp.x64, wl.layout, inp.w64, wl.w_layout, inp.bias64, wl.ff_dim, wl.ff_act,
                                     wl.n_heads, wl.head_dim, wl.rope, gr.d_ff64, gr.dq64, gr.dk64, gr.dv64,
                                     rope_base=wl.rope_base, pos_offset=wl.pos_offset, n_kv_heads=wl.n_kv_heads,
                                     qkv_order=wl.qkv_order, rope_dims=wl.rope_dims, ff_layout=wl.ff_layout)
    rows, _ = cmp.token_rows(inp.x64, wl.layout, np.arange(wl.M, dtype=np.int64))
    w_cf = inp.w64 if wl.w_layout == "cf" else inp.w64.T
    sc = cmp.backward_scales(rows, w_cf, ref.dy)
    dx, dw, db = (None if t is None else t.double().cpu().numpy() for t in grads)
    got = [_token_rows(dx, wl.layout, wl.nb, wl.C, wl.S), dw if wl.w_layout == "cf" else dw.T]
    exp = [_token_rows(ref.dx, wl.layout, wl.nb, wl.C, wl.S), ref.dw if wl.w_layout == "cf" else ref.dw.T]
    scl = [sc.dx, sc.dw]
    if wl.has_bias:
        got.append(db)
        exp.append(ref.db)
        scl.append(sc.db)
    return cmp.compare_backward(got, exp, scl, wl.dtype)


def _check(wl, label):
    proj, inp, gr, grads = run_backward(wl)
    v = backward_verdict(wl, inp, gr, grads)
    print(f"[bwd parity] {label}: {v} ws={proj.workspace_bytes()}", flush=True)
    n = wl.M * wl.C + wl.C * wl.F + (wl.F if wl.has_bias else 0)
    assert v.ok and v.n == n, f"{label}: {v}"
    return v


@pytest.fixture(params=["auto", "general"])
def kernel_choice(request, monkeypatch):
    if request.param == "general":
        monkeypatch.setenv("FUSED_PROJ_KERNEL", "general")
    else:
        monkeypatch.delenv("FUSED_PROJ_KERNEL", raising=False)
    return request.param


FULL = ["tiny_f32", "walrus_bf16", "bert_ff_bf16", "bert_qkv_bf16", "decoder_qkv_rope_bf16", "smallk_qkv_bf16",
        "bert_ff_relu2_bf16", "gqa_rope8_bf16", "conv1x1_walrus_bf16"]


@pytest.mark.parametrize("name", FULL)
def test_backward_full_size_every_element(name):
    """Each workload at full size, every gradient element against the oracle."""
    wl = WORKLOADS[name]
    print(f"[case] backward full-size {name}", flush=True)
    _check(wl, name)


@pytest.mark.parametrize("wl", SMALL, ids=[w.name for w in SMALL])
def test_backward_small_ragged(wl, kernel_choice):
    """Small shapes with ragged token, channel and column tails, every layout, activation,
    grouping and rotary option, through both kernel choices for dx."""
    print(f"[case] backward small {wl.name} x={wl.x_shape} kernel={kernel_choice}", flush=True)
    _check(wl, wl.name)


SPLIT = [
    # few dW tiles (C 64, F 192): the token contraction is split into ranges; channels-first
    # with a slab length (40) that is not a multiple of the K step, [F,C] weight
    with_shape(WORKLOADS["walrus_bf16"], "bwd_split_cf_fc", x_shape=(6, 64, 5, 8, 1), ff_dim=64, n_heads=2,
               head_dim=32, w_layout="fc", seed=401),
    # token-major, [C,F], GQA grouped, partial rotary, no bias, 1000 tokens
    with_shape(WORKLOADS["gqa_rope8_bf16"], "bwd_split_tl_gqa", x_shape=(2, 500, 64), seed=402),
    # fp32, token-major, channels-first ff
    with_shape(WORKLOADS["tiny_f32"], "bwd_split_f32_ffcf", x_shape=(3, 48, 8, 6, 1), ff_dim=32, n_heads=2,
               head_dim=8, ff_layout="channels_first", seed=403),
]


@pytest.mark.parametrize("wl", SPLIT, ids=[w.name for w in SPLIT])
def test_backward_split_token_ranges(wl):
    _check(wl, wl.name)


DX_SPLIT = [
    # dx's large tiles one or two past a whole round: the last token tiles go through ranges
    # of the fused columns and a reduction. Token-major, 129 token tiles x 2 channel tiles
    # (the tail is the last tile row, 16 ranges); channels-first with 320-token slabs, 258
    # token tiles (the last one ragged) x 1 (the head keeps whole slabs: 255 tile rows; the
    # tail, 640 tokens in 11 ranges, is stored per slab)
    with_shape(WORKLOADS["bert_ff_bf16"], "bwd_dx_split_tl", x_shape=(3, 11008, 512), ff_dim=2048, seed=405),
    # ... with W stored [F, C] (the ranges then read W as [F, C] rows)
    with_shape(WORKLOADS["bert_ff_bf16"], "bwd_dx_split_tl_fc", x_shape=(3, 11008, 512), ff_dim=2048, w_layout="fc",
               seed=407),
    with_shape(WORKLOADS["walrus_bf16"], "bwd_dx_split_cf", x_shape=(206, 256, 320), ff_dim=1024, n_heads=2,
               head_dim=64, seed=406),
]


@pytest.mark.parametrize("wl", DX_SPLIT, ids=[w.name for w in DX_SPLIT])
def test_backward_dx_last_tiles_in_ranges(wl):
    _check(wl, wl.name)


DW_DIRECT = [
    # dW in one token range, stored straight into W's layout in bf16: [F, C] (a token-major
    # x, 4096 tokens, 256 dW tiles) and [C, F] with a channels-first x (224 dW tiles, RoPE
    # heads); the decoder's full-size case takes this path too
    with_shape(WORKLOADS["bert_ff_bf16"], "bwd_dw_direct_fc", x_shape=(2, 2048, 4096), ff_dim=4096, w_layout="fc",
               seed=408),
    with_shape(WORKLOADS["walrus_bf16"], "bwd_dw_direct_cf", x_shape=(4, 4096, 32, 32, 1), ff_dim=3072, n_heads=2,
               head_dim=64, seed=409),
]


@pytest.mark.parametrize("wl", DW_DIRECT, ids=[w.name for w in DW_DIRECT])
def test_backward_dw_stored_directly(wl):
    _check(wl, wl.name)


def test_backward_strided_channel_slice_view():
    """x as a channel slice of a wider tensor: the backward reads it in place; dx is dense."""
    wl = with_shape(WORKLOADS["walrus_bf16"], "bwd_view", x_shape=(2, 48, 8, 16, 1), ff_dim=64, n_heads=2,
                    head_dim=32, seed=404)
    inp = make_inputs(wl)
    gr = make_grads(wl)
    big = torch.zeros((2, 64, 8, 16, 1), dtype=torch.bfloat16)
    big[:, 8:56] = inp.x
    xv = big.to(DEV)[:, 8:56]
    proj = plan_for(wl, xv)
    grads = proj.backward(xv, inp.w.to(DEV), inp.bias.to(DEV), _to_dev(gr.d_ff), _to_dev(gr.dq), _to_dev(gr.dk),
                          _to_dev(gr.dv))
    torch.cuda.synchronize()
    v = backward_verdict(wl, inp, gr, grads)
    print(f"[bwd parity] channel-slice view: {v}", flush=True)
    assert v.ok


def test_backward_no_tokens_gives_zero_weight_gradients():
    wl = with_shape(WORKLOADS["walrus_bf16"], "bwd_empty", x_shape=(0, 64, 8, 8, 1), ff_dim=64, n_heads=2,
                    head_dim=32)
    x = torch.empty(wl.x_shape, dtype=torch.bfloat16, device=DEV)
    w = torch.randn((64, wl.F), device=DEV).to(torch.bfloat16)
    b = torch.randn((wl.F,), device=DEV).to(torch.bfloat16)
    proj = plan_for(wl, x)
    assert proj.workspace_bytes() == 0
    dx, dw, db = proj.alloc_grads(DEV)
    dw.fill_(float("nan"))
    db.fill_(float("nan"))
    ffs, qs, kvs = proj.out_shapes()
    e = lambda s: torch.empty(s, dtype=torch.bfloat16, device=DEV)
    proj.backward(x, w, b, e(ffs), e(qs), e(kvs), e(kvs), out=(dx, dw, db))
    torch.cuda.synchronize()
    assert torch.count_nonzero(dw).item() == 0 and torch.count_nonzero(db).item() == 0


NO_CHANNELS = [
    with_shape(WORKLOADS["walrus_bf16"], "bwd_c0_cf_gelu_rope", x_shape=(2, 0, 8, 8, 1), ff_dim=64, n_heads=2,
               head_dim=32),
    with_shape(WORKLOADS["bert_ff_relu2_bf16"], "bwd_c0_tl_relu2_fc", x_shape=(3, 40, 0), ff_dim=136,
               w_layout="fc"),
    with_shape(WORKLOADS["tiny_f32"], "bwd_c0_f32", x_shape=(1, 0, 8, 8, 1)),
]


@pytest.mark.parametrize("wl", NO_CHANNELS, ids=[w.name for w in NO_CHANNELS])
def test_backward_no_channels_gives_the_bias_gradient(wl, kernel_choice):
    """C = 0: dx and dW hold no elements; db is the sum over tokens of dy, whose ff part
    takes the activation's derivative at y = b and whose q/k part is rotated back."""
    assert wl.C == 0
    _check(wl, f"{wl.name} {kernel_choice}")


NON_FINITE = [
    with_shape(WORKLOADS["walrus_bf16"], "bwd_nonfinite_cf_gelu_rope", x_shape=(2, 64, 8, 8, 1), ff_dim=128,
               n_heads=2, head_dim=64),
    with_shape(WORKLOADS["bert_ff_relu2_bf16"], "bwd_nonfinite_tl_relu2_fc", x_shape=(2, 70, 64), ff_dim=256,
               w_layout="fc"),
    with_shape(WORKLOADS["tiny_f32"], "bwd_nonfinite_f32"),
]


@pytest.mark.parametrize("wl", NON_FINITE, ids=[w.name for w in NON_FINITE])
def test_backward_non_finite_inputs_give_the_oracles_non_finite_gradients(wl, kernel_choice):
    """NaN and infinities in x, in one W entry and in the upstream gradients: every element
    of dx, dW and db is NaN, +inf or -inf exactly where the backward oracle's is, and within
    the backward bar wherever the oracle and its bar are finite."""
    from ff_input_projection_amd.workloads import as_f64
    inp, gr = make_inputs(wl), make_grads(wl)
    x, w = inp.x.clone(), inp.w.clone()
    xv = x.view(wl.nb, wl.C, wl.S) if wl.layout == "channels_first" else x.view(wl.nb, wl.S, wl.C)
    for t, val in ((5, float("nan")), (9, float("inf")), (wl.M - 3, float("-inf"))):
        bi, sp = divmod(t, wl.S)
        if wl.layout == "channels_first":
            xv[bi, 3, sp] = val
        else:
            xv[bi, sp, 3] = val
    if wl.w_layout == "cf":
        w[5, 7] = float("nan")
    else:
        w[7, 5] = float("nan")
    inp.x, inp.w, inp.x64, inp.w64 = x, w, as_f64(x), as_f64(w)
    d_ff = gr.d_ff.clone()
    d_ff.view(-1)[40] = float("nan")
    d_ff.view(-1)[d_ff.numel() - 7] = float("inf")
    gr.d_ff, gr.d_ff64 = d_ff, as_f64(d_ff)
    if gr.dq is not None:
        dq = gr.dq.clone()
        dq.view(-1)[11] = float("-inf")
        gr.dq, gr.dq64 = dq, as_f64(dq)
    print(f"[case] backward non-finite {wl.name} kernel={kernel_choice}", flush=True)
    proj, inp, gr, grads = run_backward(wl, inp, gr)
    ref = oracle.fused_proj_backward(inp.x64, wl.layout, inp.w64, wl.w_layout, inp.bias64, wl.ff_dim, wl.ff_act,
                                     wl.n_heads, wl.head_dim, wl.rope, gr.d_ff64, gr.dq64, gr.dk64, gr.dv64,
                                     rope_base=wl.rope_base, pos_offset=wl.pos_offset, n_kv_heads=wl.n_kv_heads,
                                     qkv_order=wl.qkv_order, rope_dims=wl.rope_dims, ff_layout=wl.ff_layout)
    rows, _ = cmp.token_rows(inp.x64, wl.layout, np.arange(wl.M, dtype=np.int64))
    w_cf = inp.w64 if wl.w_layout == "cf" else inp.w64.T
    with np.errstate(invalid="ignore", over="ignore"):
        sc = cmp.backward_scales(rows, w_cf, ref.dy)
    dx, dw, db = (None if t is None else t.double().cpu().numpy() for t in grads)
    pairs = [("dx", _token_rows(dx, wl.layout, wl.nb, wl.C, wl.S), _token_rows(ref.dx, wl.layout, wl.nb, wl.C, wl.S),
              sc.dx),
             ("dW", dw if wl.w_layout == "cf" else dw.T, ref.dw if wl.w_layout == "cf" else ref.dw.T, sc.dw)]
    if wl.has_bias:
        pairs.append(("db", db, ref.db, sc.db))
    n_nonfinite = 0
    for name, g, r, scl in pairs:
        assert g.shape == r.shape == scl.shape, (name, g.shape, r.shape, scl.shape)
        for cls in (np.isnan, np.isposinf, np.isneginf):
            assert np.array_equal(cls(g), cls(r)), f"{wl.name} {kernel_choice} {name}: {cls.__name__} differs"
        n_nonfinite += int((~np.isfinite(r)).sum())
        ok = np.isfinite(r) & np.isfinite(scl)
        if ok.any():
            ratio = np.abs(g[ok] - r[ok]) / (cmp.BACKWARD_REL[wl.dtype] * scl[ok] + 1e-300)
            assert ratio.max() <= 1.0, f"{wl.name} {kernel_choice} {name}: {ratio.max()}"
    print(f"[bwd non-finite] {wl.name} {kernel_choice}: {n_nonfinite} non-finite gradients, classes equal",
          flush=True)
    assert n_nonfinite > 0


def test_backward_one_plan_on_two_streams_at_once():
    """The backward pass keeps its intermediates in the caller's workspace, so one plan may
    run it on two streams at once with two workspaces: 10 rounds on each stream without
    waiting, and each stream's gradients equal the eager ones of its own inputs, bit for bit."""
    wl = SPLIT[0]
    sets = [(make_inputs(wl), make_grads(wl)), (make_inputs(wl, seed=wl.seed + 55), make_grads(wl, seed=wl.seed + 55))]
    args = []
    for inp, gr in sets:
        args.append((inp.x.to(DEV), inp.w.to(DEV), inp.bias.to(DEV), *[_to_dev(t) for t in (gr.d_ff, gr.dq, gr.dk, gr.dv)]))
    proj = plan_for(wl, args[0][0])
    eager = [[t.clone() for t in proj.backward(*a)] for a in args]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [proj.alloc_grads(DEV) for _ in range(2)]
    wss = [torch.empty(proj.workspace_bytes(), dtype=torch.uint8, device=DEV) for _ in range(2)]
    for st in streams:
        st.wait_stream(torch.cuda.current_stream())
    for _ in range(10):
        for i in range(2):
            proj.backward(*args[i], out=outs[i], workspace=wss[i], stream=streams[i])
    for st in streams:
        torch.cuda.current_stream().wait_stream(st)
    torch.cuda.synchronize()
    for i in range(2):
        for e, g in zip(eager[i], outs[i]):
            assert torch.equal(e, g), f"stream {i}"


ONE_TOKEN = [
    # one token per sequence at a position offset: 16 sequences, GELU ff and RoPE heads
    with_shape(WORKLOADS["bert_qkv_bf16"], "bwd_one_token_gelu_rope", x_shape=(16, 1, 256), ff_dim=128,
               ff_act="gelu", n_heads=2, head_dim=64, rope=True, pos_offset=100, seed=431),
    # fp32, a single sequence of one token, grouped q/k/v with RoPE on 8 of 32
    with_shape(WORKLOADS["tiny_f32"], "bwd_one_token_f32_gqa", layout="tokens_last", x_shape=(1, 1, 64), ff_dim=32,
               n_heads=4, head_dim=32, n_kv_heads=2, qkv_order="grouped", rope_dims=8, pos_offset=7, seed=432),
]


@pytest.mark.parametrize("wl", ONE_TOKEN, ids=[w.name for w in ONE_TOKEN])
def test_backward_one_token_per_sequence(wl, kernel_choice):
    """S = 1 with a position offset: every gradient element against the oracle."""
    assert wl.S == 1
    _check(wl, f"{wl.name} {kernel_choice}")


def test_backward_deterministic_and_graph_replays():
    """Two eager calls give identical bits; a captured call replays to the same bits three
    times (the workspace and outputs are refilled with NaN between replays)."""
    wl = SPLIT[0]
    inp, gr = make_inputs(wl), make_grads(wl)
    x, w, b = inp.x.to(DEV), inp.w.to(DEV), inp.bias.to(DEV)
    ups = [_to_dev(t) for t in (gr.d_ff, gr.dq, gr.dk, gr.dv)]
    proj = plan_for(wl, x)
    e1 = [t.clone() for t in proj.backward(x, w, b, *ups)]
    e2 = proj.backward(x, w, b, *ups)
    torch.cuda.synchronize()
    for a, c in zip(e1, e2):
        assert torch.equal(a, c)
    outs = proj.alloc_grads(DEV)
    ws = torch.empty(proj.workspace_bytes(), dtype=torch.uint8, device=DEV)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            proj.backward(x, w, b, *ups, out=outs, workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    for rep in range(3):
        for t in outs:
            t.fill_(float("nan"))
        ws.fill_(255)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, c in zip(e1, outs):
            assert torch.equal(a, c), f"replay {rep}"


def test_backward_error_paths():
    wl = SPLIT[0]
    inp, gr = make_inputs(wl), make_grads(wl)
    x, w, b = inp.x.to(DEV), inp.w.to(DEV), inp.bias.to(DEV)
    d_ff, dq, dk, dv = (_to_dev(t) for t in (gr.d_ff, gr.dq, gr.dk, gr.dv))
    proj = plan_for(wl, x)
    dx, dw, db = proj.alloc_grads(DEV)
    nbytes = proj.workspace_bytes()
    ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    st = torch.cuda.current_stream().cuda_stream
    p = lambda t: t.data_ptr()
    args = [p(x), p(w), p(b), p(d_ff), p(dq), p(dk), p(dv), p(dx), p(dw), p(db), p(ws)]
    assert proj.backward_ptrs(*args, nbytes, st) == 0
    assert proj.backward_ptrs(*args, nbytes - 1, st) == EINVAL                   # short workspace
    bad = list(args)
    bad[6] = None
    assert proj.backward_ptrs(*bad, nbytes, st) == EINVAL                        # dv missing
    bad = list(args)
    bad[7] = p(dx) + 2
    assert proj.backward_ptrs(*bad, nbytes, st) == EALIGN
    bad = list(args)
    bad[8] = p(dx)
    assert proj.backward_ptrs(*bad, nbytes, st) == EALIAS                        # dw over dx
    bad = list(args)
    bad[10] = p(d_ff)
    assert proj.backward_ptrs(*bad, nbytes, st) == EALIAS                        # workspace over d_ff
    torch.cuda.synchronize()
    with pytest.raises(FusedProjError):
        proj.backward(x, w, b, d_ff, dq, dk, dv, out=(dx, dw, db), workspace=ws[:nbytes - 16])
