"""GPU parity of the standalone split + RoPE (split_rope.h) against the float64 oracle.

Bar: v and the elements RoPE leaves alone are copies, so they must equal the input
bit for bit; a rotated element o = y cos - y' sin (or y cos + y' sin) is computed in
fp32 from the bf16 inputs and rounded once, so |gpu - oracle| <= 2^-8 |o| + 1e-5 *
max|y| over the token's row (the table's fp32 rounding and the fp32 products)."""
import numpy as np
import pytest
import torch

import oracle
from ff_input_projection_amd import SplitRope, FusedProjError, EALIAS, EALIGN
from ff_input_projection_amd.workloads import SPLIT_ROPE_WORKLOADS, make_qkv

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

CASES = [
    # (batch, tokens, H, KVH, hd, order, rope_dims, k_transposed, pos_offset, seed)
    (2, 1024, 16, 4, 32, "grouped", 8, False, 0, 9),     # the page's workload
    (2, 1024, 16, 4, 32, "grouped", 8, True, 0, 9),      # ... with the key transposed
    (3, 37, 4, 4, 64, "contiguous", 0, False, 5, 10),    # plain multi-head, full rotation, ragged T
    (2, 48, 6, 2, 32, "contiguous", 16, True, 0, 11),    # grouped-query, contiguous, partial, K^T
    (1, 24, 8, 1, 16, "grouped", 0, False, 2, 12),       # multi-query, full rotation
    (2, 16, 4, 2, 24, "grouped", 6, False, 0, 13),       # rotated half (3) not a multiple of anything
    (2, 40, 4, 2, 128, "contiguous", 0, False, 3, 14),   # head size 128, full rotation
    (1, 64, 4, 4, 64, "grouped", 32, True, 0, 15),       # half the head rotated, K^T
    (16, 1, 32, 8, 128, "contiguous", 0, False, 4095, 16),   # decode step: one token per sequence at 4095
    (4, 1, 16, 4, 32, "grouped", 8, False, 1023, 17),        # decode step, grouped, partial rotation
]


def _run(batch, tokens, H, KVH, hd, order, rd, kt, off, seed):
    Fq = (H + 2 * KVH) * hd
    x, x64 = make_qkv(batch, tokens, Fq, seed)
    op = SplitRope(batch, tokens, H, hd, n_kv_heads=KVH, qkv_order=order, rope=True, rope_dims=rd,
                   pos_offset=off, k_transposed=kt)
    q, k, v = op(x.to(DEV))
    torch.cuda.synchronize()
    ref = oracle.split_rope(x64, H, hd, n_kv_heads=KVH, qkv_order=order, rope=True, rope_dims=rd, pos_offset=off,
                            k_transposed=kt)
    return x64, (q, k, v), ref


@pytest.mark.parametrize("case", CASES, ids=[f"b{c[0]}_T{c[1]}_H{c[2]}_KV{c[3]}_hd{c[4]}_{c[5]}_rd{c[6]}_kt{int(c[7])}"
                                            for c in CASES])
def test_split_rope_parity(case):
    print(f"[case] split_rope {case}", flush=True)
    batch, tokens, H, KVH, hd, order, rd, kt, off, seed = case
    x64, got, ref = _run(*case)
    rdim = rd if rd > 0 else hd
    rowmax = np.abs(x64).max(axis=2)                                   # [b, T]
    worst = 0.0
    for name, g, r in zip("qkv", got, ref):
        g = g.double().cpu().numpy()
        assert g.shape == r.shape, name
        if name == "v":
            assert np.array_equal(g, r), "v must be a copy"
            continue
        heads = H if name == "q" else KVH
        gm = g.transpose(0, 2, 1) if (name == "k" and kt) else g        # [b*heads, T, hd]
        rm = r.transpose(0, 2, 1) if (name == "k" and kt) else r
        assert np.array_equal(gm[..., rdim:], rm[..., rdim:]), f"{name}: unrotated elements must be copies"
        scale = np.repeat(rowmax, heads, axis=0).reshape(batch, heads, tokens).reshape(batch * heads, tokens, 1)
        tol = 2.0 ** -8 * np.abs(rm[..., :rdim]) + 1e-5 * scale
        ratio = np.abs(gm[..., :rdim] - rm[..., :rdim]) / tol
        worst = max(worst, float(ratio.max()))
    print(f"[parity] split_rope {case}: max err/tol {worst:.3g}", flush=True)
    assert worst <= 1.0


@pytest.mark.parametrize("kt", [False, True])
def test_split_rope_non_finite_values(kt):
    """NaN and infinities in the projected tensor: v and the unrotated elements copy them;
    a rotated element is NaN, +inf or -inf exactly where the oracle's is (its partner's
    NaN or infinity reaches it through the rotation), and finite elsewhere within the bar."""
    from ff_input_projection_amd.workloads import as_f64
    batch, tokens, H, KVH, hd, order, rd, off = 2, 40, 4, 2, 32, "grouped", 8, 3
    Fq = (H + 2 * KVH) * hd
    x, _ = make_qkv(batch, tokens, Fq, 21)
    xv = x.view(batch, tokens, Fq)
    for t, col, val in ((0, 0, float("nan")), (3, 5, float("inf")), (7, 2, float("-inf")), (11, 20, float("nan")),
                        (12, 40, float("inf")), (39, Fq - 1, float("nan"))):
        xv[t // tokens, t % tokens, col] = val
    x64 = as_f64(x)
    print(f"[case] split_rope non-finite kt={kt}", flush=True)
    op = SplitRope(batch, tokens, H, hd, n_kv_heads=KVH, qkv_order=order, rope=True, rope_dims=rd,
                   pos_offset=off, k_transposed=kt)
    got = op(x.to(DEV))
    torch.cuda.synchronize()
    ref = oracle.split_rope(x64, H, hd, n_kv_heads=KVH, qkv_order=order, rope=True, rope_dims=rd, pos_offset=off,
                            k_transposed=kt)
    n_nonfinite = 0
    for name, g, r in zip("qkv", got, ref):
        g = g.double().cpu().numpy()
        for cls in (np.isnan, np.isposinf, np.isneginf):
            assert np.array_equal(cls(g), cls(r)), f"{name}: {cls.__name__} differs"
        n_nonfinite += int((~np.isfinite(r)).sum())
        fin = np.isfinite(r)
        tol = 2.0 ** -8 * np.abs(r[fin]) + 1e-5 * np.abs(x64[np.isfinite(x64)]).max()
        assert (np.abs(g[fin] - r[fin]) <= tol).all(), name
    assert n_nonfinite == 9   # 8 in q (NaN or an infinity and its rotation partner), 1 in v


def test_split_rope_named_workloads_match_cases():
    for wl in SPLIT_ROPE_WORKLOADS.values():
        assert (wl.batch, wl.tokens, wl.n_heads, wl.n_kv_heads, wl.head_dim, wl.qkv_order, wl.rope_dims,
                wl.k_transposed, wl.pos_offset, wl.seed) in CASES


def test_split_rope_error_paths():
    op = SplitRope(1, 16, 4, 32, n_kv_heads=2, qkv_order="grouped", rope_dims=8)
    x, _ = make_qkv(1, 16, (4 + 4) * 32, 1)
    x = x.to(DEV)
    q, k, v = op.alloc_outputs(DEV)
    st = torch.cuda.current_stream().cuda_stream
    p = lambda t: t.data_ptr()
    assert op.run_ptrs(p(x), p(q), p(k), p(v), st) == 0
    assert op.run_ptrs(p(x), p(q) + 2, p(k), p(v), st) == EALIGN
    assert op.run_ptrs(p(x), p(q), p(q), p(v), st) == EALIAS
    assert op.run_ptrs(p(x), p(x), p(k), p(v), st) == EALIAS
    torch.cuda.synchronize()
    with pytest.raises(ValueError):
        op(x[:, :8])


def test_split_rope_hip_graph_replays_and_determinism():
    """split_rope_run allocates and synchronises nothing: captured into a HIP graph, every
    replay (with eager work and synchronisations between) equals the eager result, and
    two eager runs agree bit for bit."""
    op = SplitRope(2, 64, 8, 32, n_kv_heads=2, qkv_order="grouped", rope_dims=8, k_transposed=True)
    x, _ = make_qkv(2, 64, (8 + 4) * 32, 14)
    x = x.to(DEV)
    eager = [t.clone() for t in op(x)]
    again = op(x)
    torch.cuda.synchronize()
    for a, b in zip(eager, again):
        assert torch.equal(a, b)
    outs = op.alloc_outputs(DEV)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            op(x, out=outs)
    torch.cuda.current_stream().wait_stream(s)
    for rep in range(3):
        for t in outs:
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(eager, outs):
            assert torch.equal(a, b), f"replay {rep}"
