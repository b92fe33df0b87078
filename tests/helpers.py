"""Shared helpers for the parity tests: run the GPU path through the C ABI binding,
run the float64 oracle on the same stored inputs, compare per element."""
from __future__ import annotations

import numpy as np
import torch

import oracle
from oracle import compare as cmp
from ff_input_projection_amd import FusedProjection
from ff_input_projection_amd.workloads import Workload, make_inputs


def plan_for(wl: Workload, x: torch.Tensor) -> FusedProjection:
    return FusedProjection.for_tensor(
        x, wl.layout, w_layout=wl.w_layout, has_bias=wl.has_bias, ff_dim=wl.ff_dim, ff_act=wl.ff_act,
        n_heads=wl.n_heads, head_dim=wl.head_dim, rope=wl.rope, rope_base=wl.rope_base, pos_offset=wl.pos_offset,
        n_kv_heads=wl.n_kv_heads, qkv_order=wl.qkv_order, rope_dims=wl.rope_dims, ff_layout=wl.ff_layout)


def nan_outputs(proj: FusedProjection, device) -> tuple:
    """Output buffers filled with NaN, so that a finite value proves the kernel wrote it
    (torch.empty may hand back a block still holding an earlier run's correct results)."""
    outs = proj.alloc_outputs(device)
    for t in outs:
        if t is not None:
            t.fill_(float("nan"))
    return outs


def run_gpu(wl: Workload, inp, device="cuda:0", x_dev: torch.Tensor | None = None):
    x = x_dev if x_dev is not None else inp.x.to(device)
    w = inp.w.to(device)
    b = inp.bias.to(device) if inp.bias is not None else None
    proj = plan_for(wl, x)
    outs = proj(x, w, b, out=nan_outputs(proj, device))
    torch.cuda.synchronize()
    return proj, outs


def sample_tokens(wl: Workload, n: int = 256, seed: int = 0) -> np.ndarray:
    """Token sample: the ends, slab and 128-row tile boundaries, and random tokens."""
    M, S = wl.M, wl.S
    picks = {0, M - 1}
    for b in range(0, wl.nb, max(1, wl.nb // 4)):
        for d in (-1, 0, 1):
            picks.add(b * S + d)
    for t in range(127, M, max(128, (M // 16) // 128 * 128)):
        picks.update((t, t + 1))
    picks = {t for t in picks if 0 <= t < M}
    rng = np.random.default_rng(seed)
    extra = rng.choice(M, size=min(M, max(0, n - len(picks))), replace=False)
    return np.array(sorted(picks | set(int(t) for t in extra)), dtype=np.int64)


def gpu_rows(wl: Workload, outs, tokens: np.ndarray):
    """GPU outputs at the sampled tokens as float64: ff [n,FF], q/k/v [n,H,hd]."""
    ff, q, k, v = outs
    bi = torch.from_numpy(tokens // wl.S)
    s = torch.from_numpy(tokens % wl.S)
    res = []
    if ff is not None and wl.ff_layout == "channels_first":
        res.append(ff.view(wl.nb, wl.ff_dim, wl.S)[bi.to(ff.device), :, s.to(ff.device)].double().cpu().numpy())
    elif ff is not None:
        res.append(ff.view(wl.nb, wl.S, wl.ff_dim)[bi.to(ff.device), s.to(ff.device)].double().cpu().numpy())
    else:
        res.append(None)
    for t, heads in ((q, wl.n_heads), (k, wl.kvh), (v, wl.kvh)):
        if t is None:
            res.append(None)
            continue
        t4 = t.view(wl.nb, heads, wl.S, wl.head_dim)
        res.append(t4[bi.to(t.device), :, s.to(t.device)].double().cpu().numpy())
    return res


def oracle_rows(wl: Workload, inp, tokens: np.ndarray):
    r = oracle.fused_proj(inp.x64, wl.layout, inp.w64, wl.w_layout, inp.bias64, wl.ff_dim, wl.ff_act,
                          wl.n_heads, wl.head_dim, wl.rope, wl.rope_base, wl.pos_offset, tokens=tokens,
                          n_kv_heads=wl.n_kv_heads, qkv_order=wl.qkv_order, rope_dims=wl.rope_dims)
    return [r.ff, r.q, r.k, r.v]


def scales_for(wl: Workload, inp, tokens: np.ndarray, ref) -> cmp.Scales:
    """Per-element bar scales at the given tokens (ref: the oracle's rows there)."""
    rows, pos = cmp.token_rows(inp.x64, wl.layout, tokens)
    w_cf = inp.w64 if wl.w_layout == "cf" else inp.w64.T
    return cmp.scales(rows, pos, w_cf, inp.bias64, wl.ff_dim, wl.n_heads, wl.head_dim, wl.rope, wl.rope_base,
                      wl.pos_offset, ff_act=wl.ff_act, ff_ref=ref[0], n_kv_heads=wl.n_kv_heads,
                      qkv_order=wl.qkv_order, rope_dims=wl.rope_dims)


def verdict(wl: Workload, inp, outs, tokens: np.ndarray) -> cmp.Verdict:
    got = gpu_rows(wl, outs, tokens)
    ref = oracle_rows(wl, inp, tokens)
    sc = scales_for(wl, inp, tokens, ref)
    return cmp.compare(got, ref, [sc.ff, sc.q, sc.k, sc.v], wl.dtype)


def all_tokens(wl: Workload) -> np.ndarray:
    return np.arange(wl.M, dtype=np.int64)


__all__ = ["make_inputs", "plan_for", "nan_outputs", "run_gpu", "sample_tokens", "gpu_rows", "oracle_rows", "scales_for", "verdict",
           "all_tokens"]
