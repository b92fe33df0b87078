"""The allocation-free backward entry point (fused_proj_backward_noalloc) against the
workspace entry point (fused_proj_backward), through the C ABI, on two calls in a row,
the second with a smaller problem: both read and write the same kernels' results, so the
gradients must be identical bit for bit (which is within any parity bar). A problem whose
workspace exceeds the static scratch buffer is rejected with FUSED_PROJ_ESCRATCH."""
import pytest
import torch

from ff_input_projection_amd import ESCRATCH, FusedProjError
from ff_input_projection_amd.workloads import WORKLOADS, make_grads, make_inputs, with_shape

from helpers import plan_for

pytestmark = pytest.mark.gpu

DEV = "cuda:0"

CASES = [
    # larger first: channels-first, RoPE, GELU, split token ranges for dW (about 24 MB of scratch)
    with_shape(WORKLOADS["walrus_bf16"], "noalloc_cf_large", x_shape=(4, 256, 16, 16, 1), ff_dim=512, n_heads=4,
               head_dim=64, seed=501),
    # then smaller: token-major, [F,C] weight, grouped k/v heads, partial rotary, no bias
    with_shape(WORKLOADS["gqa_rope8_bf16"], "noalloc_tl_small", x_shape=(2, 200, 64), w_layout="fc", seed=502),
]


def _run(wl):
    inp, gr = make_inputs(wl), make_grads(wl)
    x, w = inp.x.to(DEV), inp.w.to(DEV)
    b = inp.bias.to(DEV) if inp.bias is not None else None
    ups = [None if t is None else t.to(DEV) for t in (gr.d_ff, gr.dq, gr.dk, gr.dv)]
    proj = plan_for(wl, x)
    print(f"[case] no-alloc backward {wl.name}: workspace {proj.workspace_bytes()} bytes", flush=True)
    ref = proj.backward(x, w, b, *ups)
    outs = proj.alloc_grads(DEV)
    for t in outs:
        if t is not None:
            t.fill_(float("nan"))
    got = proj.backward_noalloc(x, w, b, *ups, out=outs)
    torch.cuda.synchronize()
    for name, a, c in zip(("dx", "dw", "db"), ref, got):
        if a is None:
            assert c is None
            continue
        assert torch.isfinite(c).all().item(), name
        assert torch.equal(a, c), f"{wl.name}: {name} differs from the workspace entry point"


def test_noalloc_backward_equals_workspace_backward_twice():
    for wl in CASES:
        _run(wl)


def test_noalloc_backward_rejects_a_workspace_beyond_the_scratch():
    wl = WORKLOADS["walrus_bf16"]        # about 318 MB of workspace
    x = torch.empty(wl.x_shape, dtype=torch.bfloat16, device=DEV)
    proj = plan_for(wl, x)
    assert proj.workspace_bytes() > proj._lib.fused_proj_noalloc_scratch_bytes()
    w = torch.zeros((wl.C, wl.F), dtype=torch.bfloat16, device=DEV)
    b = torch.zeros((wl.F,), dtype=torch.bfloat16, device=DEV)
    ffs, qs, kvs = proj.out_shapes()
    e = lambda s: torch.zeros(s, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(FusedProjError) as ei:
        proj.backward_noalloc(x, w, b, e(ffs), e(qs), e(kvs), e(kvs))
    assert ei.value.code == ESCRATCH
