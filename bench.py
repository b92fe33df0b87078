#!/usr/bin/env python3
"""Benchmark of the fused input projection on one MI355X.

One step = one fused_proj_run over one batch: the token gather, the GEMM, bias,
GELU, the q/k/v split into head-major buffers and RoPE, all in one kernel
launch. Inputs are seeded synthetic tensors already resident in HBM; a ring of
input/output sets (>= 512 MB in total) keeps successive launches from hitting
the 256 MB Infinity Cache.

Prints ONE JSON line. `value` is the contraction's algorithmic TFLOP/s
(2*M*C*F per step) of the default workload, the Walrus-like bf16 block
(x [24,768,32,32,1] channels-first, W [768,5376], FF 3072 + Q/K/V 12x64, RoPE).
`roofline` prices the kernel against the dense bf16 MFMA peak (or HBM for a
memory-bound workload); `cpu_baseline` is the float64 oracle timed on this
host's cores over a bounded token sample, on which the GPU outputs are also
checked for parity.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fused projection TFLOP/s and GB/s on 1 MI355X, % of bf16 MFMA / HBM peak"
PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}   # dense MFMA, MI355X published
PEAK_HBM_GBS = 8000.0
CSRC = os.path.join(ROOT, "ff_input_projection_amd", "csrc")


def kernel_hash() -> str:
    """Hash of every kernel and C-ABI source: ties committed counter summaries to the code."""
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".hip", ".cpp", ".h")):
            with open(os.path.join(CSRC, name), "rb") as f:
                h.update(name.encode())
                h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(workload: str):
    """HBM bytes per launch from the committed counter summary, if it was taken on
    the current kernel sources; else None."""
    p = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        t = json.load(f)
    if t.get("kernel_hash") != kernel_hash():
        return None
    return t.get("bytes_per_launch")


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=300)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="walrus_bf16")
    ap.add_argument("--ring", type=int, default=0, help="input/output sets cycled through (0: auto, >=512 MB)")
    ap.add_argument("--graph", action="store_true", help="replay the timed steps from one HIP graph")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target oracle time for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB (5 times), to scale HBM counters")
    args = ap.parse_args()

    if args.calibrate_copy:
        import torch
        n = args.calibrate_copy << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 5}))
        return 0

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the fused projection is run and priced on a single MI355X "
              "(--gpus 1). Multi-GPU runs are not part of this benchmark.", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    from ff_input_projection_amd import FusedProjection
    from ff_input_projection_amd.workloads import SPLIT_ROPE_WORKLOADS, WORKLOADS, make_inputs

    if args.workload in SPLIT_ROPE_WORKLOADS:
        return bench_split_rope(args, SPLIT_ROPE_WORKLOADS[args.workload])
    wl = WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print(f"[bench] workload {wl.name}: {wl.description}", file=sys.stderr, flush=True)

    inp = make_inputs(wl)
    ring = args.ring or max(1, min(24, math.ceil(512e6 / wl.alg_bytes)))
    xs = [inp.x.to(dev) for _ in range(ring)]
    w = inp.w.to(dev)
    b = inp.bias.to(dev) if inp.bias is not None else None
    proj = FusedProjection.for_tensor(xs[0], wl.layout, w_layout=wl.w_layout, has_bias=wl.has_bias,
                                      ff_dim=wl.ff_dim, ff_act=wl.ff_act, n_heads=wl.n_heads,
                                      head_dim=wl.head_dim, rope=wl.rope, rope_base=wl.rope_base,
                                      pos_offset=wl.pos_offset, n_kv_heads=wl.n_kv_heads,
                                      qkv_order=wl.qkv_order, rope_dims=wl.rope_dims, ff_layout=wl.ff_layout)
    outs = [proj.alloc_outputs(dev) for _ in range(ring)]
    stream = torch.cuda.current_stream(dev)
    sh = stream.cuda_stream
    ptr = lambda t: None if t is None else t.data_ptr()
    calls = [(ptr(xs[i]), ptr(w), ptr(b), *[ptr(t) for t in outs[i]]) for i in range(ring)]

    def step(i):
        rc = proj.run_ptrs(*calls[i % ring], sh)
        if rc != 0:
            raise RuntimeError(f"fused_proj_run failed with status {rc}")

    print(f"[bench] plan: {proj.describe()} ring={ring}", file=sys.stderr, flush=True)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    graph = None
    if args.graph:
        s2 = torch.cuda.Stream(dev)
        s2.wait_stream(stream)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.stream(s2):
            with torch.cuda.graph(graph, stream=s2):
                cs = torch.cuda.current_stream(dev).cuda_stream
                for i in range(args.steps):
                    rc = proj.run_ptrs(*calls[i % ring], cs)
                    assert rc == 0
        stream.wait_stream(s2)
        graph.replay()
        torch.cuda.synchronize()

    # ---- timed region: exactly `steps` launches on `stream`, bracketed by HIP events
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    if graph is not None:
        graph.replay()
    else:
        for i in range(args.steps):
            step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = ev0.elapsed_time(ev1) / args.steps
    print(f"[bench] timed {args.steps} steps: {ms * 1e3:.2f} us/step (events), wall {wall * 1e6 / args.steps:.2f} us/step",
          file=sys.stderr, flush=True)

    tflops = wl.flops / (ms * 1e-3) / 1e12
    gbs = wl.alg_bytes / (ms * 1e-3) / 1e9
    mfma_frac = tflops / PEAK_TFLOPS[wl.dtype]
    hbm_frac = gbs / PEAK_HBM_GBS
    ridge = PEAK_TFLOPS[wl.dtype] * 1e12 / (PEAK_HBM_GBS * 1e9)
    hbm_bound = wl.flops / wl.alg_bytes < ridge
    traffic = load_traffic(wl.name)
    if hbm_bound:
        roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(hbm_frac, 4), "traffic": traffic}
    else:
        roof = {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_TFLOPS[wl.dtype], "unit": "TFLOP/s",
                "frac": round(mfma_frac, 4), "traffic": traffic}

    result = {
        "metric": METRIC, "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": wl.dtype,
        "data": "synthetic: seeded x ~ N(0,1), W ~ N(0,1/C), bias ~ N(0,0.02), rounded once to the storage type",
        "config": {"workload": wl.name, "x_shape": list(wl.x_shape), "layout": wl.layout, "C": wl.C, "F": wl.F,
                   "ff_dim": wl.ff_dim, "n_heads": wl.n_heads, "head_dim": wl.head_dim, "rope": wl.rope,
                   "n_kv_heads": wl.kvh, "qkv_order": wl.qkv_order, "rope_dims": wl.rd if wl.rope else 0,
                   "bias": wl.has_bias, "tokens": wl.M, "w_layout": wl.w_layout, "ring": ring,
                   "graph": bool(graph is not None)},
        "gb_per_s": round(gbs, 1), "hbm_frac": round(hbm_frac, 4), "mfma_frac": round(mfma_frac, 4),
        "roofline": roof,
        "kernel": proj.describe(), "kernel_hash": kernel_hash(),
    }

    # ---- CPU baseline (float64 oracle, bounded token sample) + parity on that sample
    if not args.no_cpu_baseline:
        import oracle
        from oracle import compare as cmp

        cores = len(os.sched_getaffinity(0))
        rng = np.random.default_rng(12345)
        per_tok_flops = 2.0 * wl.C * wl.F

        def run_oracle(tokens):
            t = time.perf_counter()
            r = oracle.fused_proj(inp.x64, wl.layout, inp.w64, wl.w_layout, inp.bias64, wl.ff_dim, wl.ff_act,
                                  wl.n_heads, wl.head_dim, wl.rope, wl.rope_base, wl.pos_offset, tokens=tokens,
                                  nthreads=cores, n_kv_heads=wl.n_kv_heads, qkv_order=wl.qkv_order,
                                  rope_dims=wl.rope_dims)
            return r, time.perf_counter() - t

        # calibrate on a probe large enough to amortise thread start-up, then size the sample
        probe = np.sort(rng.choice(wl.M, size=min(wl.M, max(64 * cores, 1)), replace=False)).astype(np.int64)
        _, tp = run_oracle(probe)
        per_tok = tp / len(probe)
        n = int(min(wl.M, max(len(probe), args.cpu_seconds / max(per_tok, 1e-9))))
        if n >= wl.M:
            # the whole workload fits the time budget: run all of it, repeated to fill it
            tokens = np.arange(wl.M, dtype=np.int64)
            reps = max(1, min(10, int(args.cpu_seconds / max(per_tok * wl.M, 1e-9))))
        else:
            tokens = np.sort(rng.choice(wl.M, size=n, replace=False)).astype(np.int64)
            reps = 1
        secs = 0.0
        for _ in range(reps):
            ref, s_ = run_oracle(tokens)
            secs += s_
        cpu_tflops = per_tok_flops * n * reps / secs / 1e12
        what = (f"all {wl.M} tokens x {reps} run(s)" if n >= wl.M
                else f"{n} of {wl.M} tokens (random, seed 12345)")
        result["cpu_baseline"] = {"value": round(cpu_tflops, 6), "unit": "TFLOP/s", "cores": cores,
                                  "kind": "oracle",
                                  "sample": f"{what}, all F={wl.F} columns, float64, {secs:.1f} s"}
        ff, q, k, v = outs[0]
        bi = torch.from_numpy(tokens // wl.S).to(dev)
        si = torch.from_numpy(tokens % wl.S).to(dev)
        if ff is None:
            got = [None]
        elif wl.ff_layout == "channels_first":
            got = [ff.view(wl.nb, wl.ff_dim, wl.S)[bi, :, si].double().cpu().numpy()]
        else:
            got = [ff.view(wl.nb, wl.S, wl.ff_dim)[bi, si].double().cpu().numpy()]
        for t, heads in ((q, wl.n_heads), (k, wl.kvh), (v, wl.kvh)):
            got.append(None if t is None else
                       t.view(wl.nb, heads, wl.S, wl.head_dim)[bi, :, si].double().cpu().numpy())
        rows, pos = cmp.token_rows(inp.x64, wl.layout, tokens)
        w_cf = inp.w64 if wl.w_layout == "cf" else inp.w64.T
        sc = cmp.scales(rows, pos, w_cf, inp.bias64, wl.ff_dim, wl.n_heads, wl.head_dim, wl.rope, wl.rope_base,
                        wl.pos_offset, ff_act=wl.ff_act, ff_ref=ref.ff, n_kv_heads=wl.n_kv_heads,
                        qkv_order=wl.qkv_order, rope_dims=wl.rope_dims)
        vd = cmp.compare(got, [ref.ff, ref.q, ref.k, ref.v], [sc.ff, sc.q, sc.k, sc.v], wl.dtype)
        result["parity"] = {"ok": vd.ok, "max_err_over_tol": round(vd.max_ratio, 5),
                            "tight_ratio": round(vd.max_tight_ratio, 5), "elements": vd.n}
        print(f"[bench] parity on the oracle sample: {vd}", file=sys.stderr, flush=True)

    print(json.dumps(result), flush=True)
    return 0


def bench_split_rope(args, wl) -> int:
    """The standalone split + RoPE (split_rope.h) on a seeded projected q/k/v tensor:
    memory-bound, priced against HBM bandwidth (input once + outputs once)."""
    import numpy as np
    import torch

    from ff_input_projection_amd import SplitRope
    from ff_input_projection_amd.workloads import make_qkv

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print(f"[bench] workload {wl.name}: {wl.description}", file=sys.stderr, flush=True)
    x, x64 = make_qkv(wl.batch, wl.tokens, wl.Fq, wl.seed)
    ring = args.ring or max(1, min(64, math.ceil(512e6 / wl.alg_bytes)))
    xs = [x.to(dev) for _ in range(ring)]
    op = SplitRope(wl.batch, wl.tokens, wl.n_heads, wl.head_dim, n_kv_heads=wl.n_kv_heads, qkv_order=wl.qkv_order,
                   rope=True, rope_dims=wl.rope_dims, pos_offset=wl.pos_offset, k_transposed=wl.k_transposed)
    outs = [op.alloc_outputs(dev) for _ in range(ring)]
    stream = torch.cuda.current_stream(dev)
    sh = stream.cuda_stream
    calls = [(xs[i].data_ptr(), *[t.data_ptr() for t in outs[i]]) for i in range(ring)]

    def step(i):
        rc = op.run_ptrs(*calls[i % ring], sh)
        if rc != 0:
            raise RuntimeError(f"split_rope_run failed with status {rc}")

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for i in range(args.steps):
        step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / args.steps
    gbs = wl.alg_bytes / (ms * 1e-3) / 1e9
    result = {
        "metric": METRIC, "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic: seeded qkv ~ N(0,1), rounded once to bf16",
        "config": {"workload": wl.name, "op": "split_rope", "batch": wl.batch, "tokens": wl.tokens,
                   "n_heads": wl.n_heads, "n_kv_heads": wl.n_kv_heads, "head_dim": wl.head_dim,
                   "qkv_order": wl.qkv_order, "rope_dims": wl.rope_dims, "k_transposed": wl.k_transposed,
                   "ring": ring},
        "gb_per_s": round(gbs, 1), "hbm_frac": round(gbs / PEAK_HBM_GBS, 4),
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None},
        "kernel": "split_rope_kernel", "kernel_hash": kernel_hash(),
    }
    if not args.no_cpu_baseline:
        import oracle

        t0 = time.perf_counter()
        reps = 0
        while True:
            ref = oracle.split_rope(x64, wl.n_heads, wl.head_dim, n_kv_heads=wl.n_kv_heads,
                                    qkv_order=wl.qkv_order, rope=True, rope_dims=wl.rope_dims,
                                    pos_offset=wl.pos_offset, k_transposed=wl.k_transposed)
            reps += 1
            secs = time.perf_counter() - t0
            if secs >= min(args.cpu_seconds, 10.0) or reps >= 50:
                break
        result["cpu_baseline"] = {"value": round(wl.alg_bytes * reps / secs / 1e9, 4), "unit": "GB/s", "cores": 1,
                                  "kind": "oracle",
                                  "sample": f"the whole tensor x {reps} run(s), float64, one thread, {secs:.1f} s"}
        q, k, v = (t.double().cpu().numpy() for t in outs[0])
        err = max(float(np.max(np.abs(g - r) / (2.0 ** -8 * np.abs(r) + 1e-5 * np.abs(x64).max())))
                  for g, r in zip((q, k, v), ref))
        result["parity"] = {"ok": err <= 1.0, "max_err_over_tol": round(err, 5)}
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
