#!/usr/bin/env python3
"""Benchmark of the fused input projection on one MI355X.

One step = one fused_proj_run over one batch: the token gather, the GEMM, bias,
GELU, the q/k/v split into head-major buffers and RoPE, all in one kernel
launch. Inputs are seeded synthetic tensors already resident in HBM; a ring of
input/output sets (>= 512 MB in total) keeps successive launches from hitting
the 256 MB Infinity Cache.

Prints ONE JSON line. `value` is the contraction's algorithmic TFLOP/s
(2*M*C*F per step) of the default workload, the Walrus-like bf16 block
(x [24,768,32,32,1] channels-first, W [768,5376], FF 3072 + Q/K/V 12x64, RoPE),
timed over exactly `steps` back-to-back launches bracketed by two HIP events
after a warm-up of at least `--min-warmup-s` seconds (whatever `--warmup` says:
the clocks take about a second to settle). A second pass over the same number of
launches, each between its own pair of events, gives the per-launch median, p10
and p90.

Also on the line:
  roofline      the dominant kernel against the dense bf16 MFMA peak (or HBM for a
                memory-bound workload), with the HBM bytes from the committed counter
                summary when it was taken on the current kernel sources;
  cpu_baseline  the float64 oracle timed on this host's cores;
  configs       every workload of the workload table (tiny fp32, Walrus, BERT FF and
                QKV, decoder, small-K), each timed the same way and checked against
                the oracle on every output element;
  cpu_1core     the oracle on one core for the tiny and small-K workloads;
  backward      fused_proj_backward (dy, dx, dW and db launches) timed per config, the
                headline's gradients checked against the float64 backward oracle;
  sclk_mhz      the graphics clock sampled while the headline kernel runs;
  mfma_ceiling  the bf16 rate the matrix cores sustain alone (an MFMA-only kernel on
                pseudo-random operands, clock sampled), and frac_of_mfma_ceiling beside
                roofline.frac for the headline and every MFMA-bound configuration;
  context       the pages' own figures for the pathology this op removes.
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
# the workload table's configurations, in its order (3 is the BERT FF + QKV pair)
CONFIG_WORKLOADS = ["tiny_f32", "walrus_bf16", "bert_ff_bf16", "bert_qkv_bf16", "decoder_qkv_rope_bf16",
                    "smallk_qkv_bf16"]
ONE_CORE_WORKLOADS = ["tiny_f32", "smallk_qkv_bf16"]
# the variants beside the table: grouped-query heads with 8-column RoPE, the 1x1x1
# convolution's channels-first output, squared ReLU, and the Walrus width 1408 (timed and
# checked the same way, reported under "variants")
VARIANT_WORKLOADS = ["gqa_rope8_bf16", "conv1x1_walrus_bf16", "bert_ff_relu2_bf16", "walrus_c1408_bf16"]
# The Walrus PR's own measurements (L40S, before its fix), restated: the figures this
# op exists to remove. Context only, not a target.
CONTEXT = {
    "source": "Walrus PR 'Make fused_ff_qkv contiguous' (profiles in its comments, NVIDIA L40S, torch 2.5.1)",
    "forward_before_s": "about 6-7 s per bf16 forward of the batch-4 Walrus processor before the fix",
    "bmm_share_of_device_time": 0.857,
    "gemv_calls_per_projection": 24576,
    "speedup_from_contiguous_input": "about 6x",
}


# the MFMA-only calibration kernel runs in none of the profiled launches
HASH_EXCLUDED = {"mfma_ceiling.hip"}


def kernel_hash() -> str:
    """Hash of every kernel and C-ABI source: ties committed counter summaries to the code."""
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".hip", ".cpp", ".h")) and name not in HASH_EXCLUDED:
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


def pct(vals, q):
    s = sorted(vals)
    if not s:
        return None
    i = min(len(s) - 1, max(0, int(round(q / 100.0 * (len(s) - 1)))))
    return s[i]


def time_launches(launch, steps: int, warmup: int, min_warmup_s: float, stream, per_launch: bool = True):
    """Warm up for at least `warmup` launches and `min_warmup_s` seconds, then time
    exactly `steps` launches between two HIP events on `stream` (the stream the kernel
    runs on); then, when per_launch, the same number again with an event pair around
    each launch. launch(i) enqueues launch i. Returns a dict of microsecond figures."""
    import torch

    t0 = time.perf_counter()
    n = 0
    while n < warmup or time.perf_counter() - t0 < min_warmup_s:
        for _ in range(16):
            launch(n)
            n += 1
        torch.cuda.synchronize()
    warm_s = time.perf_counter() - t0

    # ---- timed region: exactly `steps` launches, bracketed by two events
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    w0 = time.perf_counter()
    ev0.record(stream)
    for i in range(steps):
        launch(n + i)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    mean_us = ev0.elapsed_time(ev1) * 1e3 / max(steps, 1)
    res = {"mean_us": mean_us, "wall_us_per_step": wall * 1e6 / max(steps, 1), "warmup_launches": n,
           "warmup_s": round(warm_s, 3)}
    if per_launch:
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        evs[0].record(stream)
        for i in range(steps):
            launch(n + steps + i)
            evs[i + 1].record(stream)
        torch.cuda.synchronize()
        per = [evs[i].elapsed_time(evs[i + 1]) * 1e3 for i in range(steps)]
        res.update({"median_us": pct(per, 50), "p10_us": pct(per, 10), "p90_us": pct(per, 90),
                    "min_us": min(per), "max_us": max(per), "per_launch_n": steps})
    return res


def sample_sclk(launch, kernel_us: float, seconds: float = 0.4):
    """Graphics clock (MHz) sampled through amdsmi while `launch` keeps the GPU busy
    (about 20 ms of launches queued per 10 ms sample interval); None when the clock
    cannot be read here."""
    import torch

    try:
        import amdsmi
    except Exception:
        return None
    try:
        amdsmi.amdsmi_init()
    except Exception:
        return None
    try:
        props = torch.cuda.get_device_properties(torch.cuda.current_device())
        want = (int(getattr(props, "pci_domain_id", 0)), int(getattr(props, "pci_bus_id", -1)))
        handle = None
        for h in amdsmi.amdsmi_get_processor_handles():
            bdf = amdsmi.amdsmi_get_gpu_device_bdf(h)          # "dddd:bb:dd.f"
            dom, bus = bdf.split(":")[0], bdf.split(":")[1]
            if (int(dom, 16), int(bus, 16)) == want:
                handle = h
                break
        if handle is None:
            return None
        samples = []
        chunk = max(1, int(20e-3 / max(kernel_us * 1e-6, 1e-7)))
        t0 = time.perf_counter()
        i = 0
        while time.perf_counter() - t0 < seconds:
            for _ in range(chunk):
                launch(i)
                i += 1
            info = amdsmi.amdsmi_get_clock_info(handle, amdsmi.AmdSmiClkType.GFX)
            samples.append(int(info["clk"]))
            time.sleep(0.01)
        torch.cuda.synchronize()
        if not samples:
            return None
        return {"median": pct(samples, 50), "min": min(samples), "max": max(samples), "n": len(samples),
                "source": "amdsmi_get_clock_info(GFX) during back-to-back launches"}
    except Exception as e:   # measurement aid only: never fail the bench on it
        return {"error": str(e)[:200]}
    finally:
        try:
            amdsmi.amdsmi_shut_down()
        except Exception:
            pass


def measure_mfma_ceiling(dev, min_warmup_s: float, iterations: int = 2000, steps: int = 20):
    """The bf16 rate the matrix cores sustain on their own on this GPU: launches of a kernel
    that issues only v_mfma_f32_32x32x16_bf16 (one wave per SIMD on every CU, 8 independent
    accumulators, pseudo-random operands rotated between instructions;
    fused_proj_mfma_ceiling), timed like the projection, with the clock sampled while they
    run. The published peak assumes the top clock; this is what the power limit leaves."""
    import torch

    import ff_input_projection_amd as fpa

    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    sink = torch.empty(cus * 256, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    flops = fpa.mfma_ceiling_launch(iterations, sink, stream)

    def launch(i):
        fpa.mfma_ceiling_launch(iterations, sink, stream, seed=12345 + i)

    t = time_launches(launch, steps, 4, min_warmup_s, stream)
    sclk = sample_sclk(launch, t["mean_us"])
    torch.cuda.synchronize()
    return {"tflop_per_s": round(flops / (t["mean_us"] * 1e-6) / 1e12, 1),
            "tflop_per_s_median": round(flops / (t["median_us"] * 1e-6) / 1e12, 1),
            "us_per_launch": round(t["mean_us"], 1), "sclk_mhz": sclk.get("median") if sclk else None,
            "kernel": f"fused_proj_mfma_ceiling: v_mfma_f32_32x32x16_bf16 only, {cus} CUs x 4 waves x "
                      f"{iterations * 16} MFMAs, pseudo-random bf16 operands"}


def measure_stream_ceiling(dev, read_bytes, write_bytes, row_elems, dtype, steps, min_warmup_s):
    """A plain streaming kernel over the same bytes as a memory-bound launch, timed the same
    way: a row gather (torch.index_select) writing rows of row_elems elements from a buffer
    of read_bytes (read once from HBM; rows it reads again come from the caches). The
    ceiling an HBM-bound kernel of this size reaches in this harness."""
    import torch

    es = 2 if dtype == "bf16" else 4
    out_rows = max(1, int(write_bytes) // (row_elems * es))
    in_rows = max(1, round(read_bytes / (row_elems * es)))
    ring = max(1, min(24, math.ceil(512e6 / (read_bytes + write_bytes))))
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    srcs = [torch.randn(in_rows, row_elems, device=dev).to(dt) for _ in range(ring)]
    dsts = [torch.empty(out_rows, row_elems, dtype=dt, device=dev) for _ in range(ring)]
    idx = torch.arange(out_rows, device=dev) % in_rows
    stream = torch.cuda.current_stream(dev)

    def launch(i):
        torch.index_select(srcs[i % ring], 0, idx, out=dsts[i % ring])

    t = time_launches(launch, steps, 10, min_warmup_s, stream)
    moved = (in_rows + out_rows) * row_elems * es
    return {"kernel": "torch.index_select row gather", "read_bytes": in_rows * row_elems * es,
            "write_bytes": out_rows * row_elems * es, "us_mean": round(t["mean_us"], 2),
            "us_median": round(t["median_us"], 2), "gb_per_s": round(moved / (t["mean_us"] * 1e-6) / 1e9, 1)}


def make_plan(wl, x):
    from ff_input_projection_amd import FusedProjection

    return FusedProjection.for_tensor(x, wl.layout, w_layout=wl.w_layout, has_bias=wl.has_bias,
                                      ff_dim=wl.ff_dim, ff_act=wl.ff_act, n_heads=wl.n_heads,
                                      head_dim=wl.head_dim, rope=wl.rope, rope_base=wl.rope_base,
                                      pos_offset=wl.pos_offset, n_kv_heads=wl.n_kv_heads,
                                      qkv_order=wl.qkv_order, rope_dims=wl.rope_dims, ff_layout=wl.ff_layout)


def gpu_outputs_to_host(wl, outs):
    """The outputs of one launch, as CPU tensors in their storage type."""
    return [None if t is None else t.cpu() for t in outs]


def host_rows(wl, outs, tokens):
    """Outputs (CPU tensors) as float64 token-major rows: ff [n, FF], q/k/v [n, heads, hd]."""
    import torch

    ff, q, k, v = outs
    bi = torch.from_numpy(tokens // wl.S)
    si = torch.from_numpy(tokens % wl.S)
    if ff is None:
        got = [None]
    elif wl.ff_layout == "channels_first":
        got = [ff.view(wl.nb, wl.ff_dim, wl.S)[bi, :, si].double().numpy()]
    else:
        got = [ff.view(wl.nb, wl.S, wl.ff_dim)[bi, si].double().numpy()]
    for t, heads in ((q, wl.n_heads), (k, wl.kvh), (v, wl.kvh)):
        got.append(None if t is None else t.view(wl.nb, heads, wl.S, wl.head_dim)[bi, :, si].double().numpy())
    return got


def run_oracle(wl, inp, tokens, threads):
    import oracle

    t = time.perf_counter()
    r = oracle.fused_proj(inp.x64, wl.layout, inp.w64, wl.w_layout, inp.bias64, wl.ff_dim, wl.ff_act,
                          wl.n_heads, wl.head_dim, wl.rope, wl.rope_base, wl.pos_offset, tokens=tokens,
                          nthreads=threads, n_kv_heads=wl.n_kv_heads, qkv_order=wl.qkv_order,
                          rope_dims=wl.rope_dims)
    return r, time.perf_counter() - t


def parity(wl, inp, host_outs, tokens, ref):
    """Per-element comparison of the GPU outputs with the oracle's at `tokens`."""
    from oracle import compare as cmp

    got = host_rows(wl, host_outs, tokens)
    rows, pos = cmp.token_rows(inp.x64, wl.layout, tokens)
    w_cf = inp.w64 if wl.w_layout == "cf" else inp.w64.T
    sc = cmp.scales(rows, pos, w_cf, inp.bias64, wl.ff_dim, wl.n_heads, wl.head_dim, wl.rope, wl.rope_base,
                    wl.pos_offset, ff_act=wl.ff_act, ff_ref=ref.ff, n_kv_heads=wl.n_kv_heads,
                    qkv_order=wl.qkv_order, rope_dims=wl.rope_dims)
    vd = cmp.compare(got, [ref.ff, ref.q, ref.k, ref.v], [sc.ff, sc.q, sc.k, sc.v], wl.dtype)
    return {"ok": vd.ok, "max_err_over_tol": round(vd.max_ratio, 5), "tight_ratio": round(vd.max_tight_ratio, 5),
            "elements": vd.n, "all_elements": vd.n == wl.M * wl.F}


def roofline_of(wl, us):
    tflops = wl.flops / (us * 1e-6) / 1e12
    gbs = wl.alg_bytes / (us * 1e-6) / 1e9
    ridge = PEAK_TFLOPS[wl.dtype] * 1e12 / (PEAK_HBM_GBS * 1e9)
    if wl.flops / wl.alg_bytes < ridge:
        return tflops, gbs, {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                             "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": load_traffic(wl.name)}
    return tflops, gbs, {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_TFLOPS[wl.dtype],
                         "unit": "TFLOP/s", "frac": round(tflops / PEAK_TFLOPS[wl.dtype], 4),
                         "traffic": load_traffic(wl.name)}


def measure_workload(wl, dev, steps, warmup, min_warmup_s, ring_arg=0, graph=False, want_sclk=False):
    """Time one workload on the GPU. Returns (timing dict, plan description, host copy of
    one launch's outputs, inputs, sclk)."""
    import torch

    from ff_input_projection_amd.workloads import make_inputs

    inp = make_inputs(wl)
    ring = ring_arg or max(1, min(24, math.ceil(512e6 / wl.alg_bytes)))
    xs = [inp.x.to(dev) for _ in range(ring)]
    w = inp.w.to(dev)
    b = inp.bias.to(dev) if inp.bias is not None else None
    proj = make_plan(wl, xs[0])
    outs = [proj.alloc_outputs(dev) for _ in range(ring)]
    stream = torch.cuda.current_stream(dev)
    sh = stream.cuda_stream
    ptr = lambda t: None if t is None else t.data_ptr()
    calls = [(ptr(xs[i]), ptr(w), ptr(b), *[ptr(t) for t in outs[i]]) for i in range(ring)]

    def launch(i):
        rc = proj.run_ptrs(*calls[i % ring], sh)
        if rc != 0:
            raise RuntimeError(f"fused_proj_run failed with status {rc}")

    desc = proj.describe()
    print(f"[bench] {wl.name}: {desc} ring={ring}", file=sys.stderr, flush=True)
    if graph:
        # the timed launches replayed from one HIP graph (launch overhead excluded): warm
        # up eagerly, then time one replay of `steps` launches between two events
        s2 = torch.cuda.Stream(dev)
        s2.wait_stream(stream)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(s2):
            with torch.cuda.graph(g, stream=s2):
                cs = torch.cuda.current_stream(dev).cuda_stream
                for i in range(steps):
                    assert proj.run_ptrs(*calls[i % ring], cs) == 0
        stream.wait_stream(s2)
        torch.cuda.synchronize()
        t = time_launches(launch, 0, warmup, min_warmup_s, stream, per_launch=False)
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record(stream)
        g.replay()
        ev1.record(stream)
        torch.cuda.synchronize()
        t["mean_us"] = ev0.elapsed_time(ev1) * 1e3 / steps
    else:
        t = time_launches(launch, steps, warmup, min_warmup_s, stream)
    sclk = sample_sclk(launch, t["mean_us"]) if want_sclk else None
    torch.cuda.synchronize()
    host = gpu_outputs_to_host(wl, outs[0])
    t["ring"] = ring
    del xs, outs, w, b
    proj.close()
    torch.cuda.empty_cache()
    return t, desc, host, inp, sclk


def backward_flops(wl) -> float:
    """Algorithmic flops of the backward pass: dx = dy W^T and dW = X^T dy (2 M C F each),
    plus the ff columns' forward product recomputed where an activation is differentiated."""
    f = 4.0 * wl.M * wl.C * wl.F
    if wl.ff_dim > 0 and wl.ff_act != "none":
        f += 2.0 * wl.M * wl.C * wl.ff_dim
    return f


def measure_backward(wl, dev, steps, min_warmup_s, check: bool):
    """Time fused_proj_backward (all of its launches) on one workload; optionally check
    every gradient element against the float64 backward oracle."""
    import numpy as np
    import torch

    from ff_input_projection_amd.workloads import make_grads, make_inputs

    inp, gr = make_inputs(wl), make_grads(wl)
    x, w = inp.x.to(dev), inp.w.to(dev)
    b = inp.bias.to(dev) if inp.bias is not None else None
    ups = [None if t is None else t.to(dev) for t in (gr.d_ff, gr.dq, gr.dk, gr.dv)]
    proj = make_plan(wl, x)
    outs = proj.alloc_grads(dev)
    nbytes = proj.workspace_bytes()
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    sh = stream.cuda_stream
    ptr = lambda t: None if t is None else t.data_ptr()
    args = [ptr(x), ptr(w), ptr(b), *[ptr(t) for t in ups], *[ptr(t) for t in outs], ptr(ws)]

    def launch(i):
        rc = proj.backward_ptrs(*args, nbytes, sh)
        if rc != 0:
            raise RuntimeError(f"fused_proj_backward failed with status {rc}")

    t = time_launches(launch, steps, 3, min_warmup_s, stream)
    flops = backward_flops(wl)
    entry = {"workload": wl.name, "us_mean": round(t["mean_us"], 2), "us_median": round(t["median_us"], 2),
             "us_p10": round(t["p10_us"], 2), "us_p90": round(t["p90_us"], 2), "launches": steps,
             "gflop": round(flops / 1e9, 2), "tflop_per_s": round(flops / (t["mean_us"] * 1e-6) / 1e12, 2),
             "frac": round(flops / (t["mean_us"] * 1e-6) / 1e12 / PEAK_TFLOPS[wl.dtype], 4),
             "workspace_bytes": nbytes}
    if check:
        import oracle
        from oracle import compare as cmp

        torch.cuda.synchronize()
        ref = oracle.fused_proj_backward(inp.x64, wl.layout, inp.w64, wl.w_layout, inp.bias64, wl.ff_dim,
                                         wl.ff_act, wl.n_heads, wl.head_dim, wl.rope, gr.d_ff64, gr.dq64, gr.dk64,
                                         gr.dv64, rope_base=wl.rope_base, pos_offset=wl.pos_offset,
                                         n_kv_heads=wl.n_kv_heads, qkv_order=wl.qkv_order, rope_dims=wl.rope_dims,
                                         ff_layout=wl.ff_layout)
        rows, _ = cmp.token_rows(inp.x64, wl.layout, np.arange(wl.M, dtype=np.int64))
        w_cf = inp.w64 if wl.w_layout == "cf" else inp.w64.T
        sc = cmp.backward_scales(rows, w_cf, ref.dy)

        def token_rows(a):
            if wl.layout == "channels_first":
                return a.reshape(wl.nb, wl.C, wl.S).transpose(0, 2, 1).reshape(wl.M, wl.C)
            return a.reshape(wl.M, wl.C)

        dx, dw, db = (None if t_ is None else t_.double().cpu().numpy() for t_ in outs)
        got = [token_rows(dx), dw if wl.w_layout == "cf" else dw.T]
        exp = [token_rows(ref.dx), ref.dw if wl.w_layout == "cf" else ref.dw.T]
        scl = [sc.dx, sc.dw]
        if wl.has_bias:
            got.append(db)
            exp.append(ref.db)
            scl.append(sc.db)
        vd = cmp.compare_backward(got, exp, scl, wl.dtype)
        entry["parity"] = {"ok": vd.ok, "max_err_over_tol": round(vd.max_ratio, 5), "elements": vd.n}
    del x, w, b, ups, outs, ws
    proj.close()
    torch.cuda.empty_cache()
    return entry


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=300)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--min-warmup-s", type=float, default=1.5,
                    help="warm up for at least this long whatever --warmup is (clock ramp)")
    ap.add_argument("--workload", default="walrus_bf16")
    ap.add_argument("--ring", type=int, default=0, help="input/output sets cycled through (0: auto, >=512 MB)")
    ap.add_argument("--graph", action="store_true", help="replay the timed steps from one HIP graph")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="target oracle time for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle (timing and parity)")
    ap.add_argument("--no-configs", action="store_true", help="time only --workload (no per-config array)")
    ap.add_argument("--config-steps", type=int, default=200, help="timed launches per config (x5 for small-K)")
    ap.add_argument("--no-backward", action="store_true", help="skip timing the backward pass")
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

    from ff_input_projection_amd.workloads import SPLIT_ROPE_WORKLOADS, WORKLOADS

    if args.workload in SPLIT_ROPE_WORKLOADS:
        return bench_split_rope(args, SPLIT_ROPE_WORKLOADS[args.workload])
    wl = WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print(f"[bench] workload {wl.name}: {wl.description}", file=sys.stderr, flush=True)

    t, desc, host, inp, sclk = measure_workload(wl, dev, args.steps, args.warmup, args.min_warmup_s, args.ring,
                                                args.graph, want_sclk=not args.graph)
    us = t["mean_us"]
    ms = us * 1e-3
    print(f"[bench] timed {args.steps} steps: {us:.2f} us/step (events), median {t.get('median_us', 0):.2f}, "
          f"wall {t['wall_us_per_step']:.2f} us/step", file=sys.stderr, flush=True)
    tflops, gbs, roof = roofline_of(wl, us)
    result = {
        "metric": METRIC, "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": wl.dtype,
        "data": "synthetic: seeded x ~ N(0,1), W ~ N(0,1/C), bias ~ N(0,0.02), rounded once to the storage type",
        "config": {"workload": wl.name, "x_shape": list(wl.x_shape), "layout": wl.layout, "C": wl.C, "F": wl.F,
                   "ff_dim": wl.ff_dim, "n_heads": wl.n_heads, "head_dim": wl.head_dim, "rope": wl.rope,
                   "n_kv_heads": wl.kvh, "qkv_order": wl.qkv_order, "rope_dims": wl.rd if wl.rope else 0,
                   "bias": wl.has_bias, "tokens": wl.M, "w_layout": wl.w_layout, "ring": t["ring"],
                   "graph": bool(args.graph)},
        "gb_per_s": round(gbs, 1), "hbm_frac": round(gbs / PEAK_HBM_GBS, 4),
        "mfma_frac": round(tflops / PEAK_TFLOPS[wl.dtype], 4),
        "roofline": roof,
        "launch_us": {k: (round(v, 2) if isinstance(v, float) else v) for k, v in t.items()},
        "sclk_mhz": sclk,
        "kernel": desc, "kernel_hash": kernel_hash(),
        "context": CONTEXT,
    }
    # the matrix cores' own sustained rate, beside the published peak (bf16 workloads)
    mfma_ceiling = None
    if wl.dtype == "bf16" and not args.graph:
        mfma_ceiling = measure_mfma_ceiling(dev, min(args.min_warmup_s, 1.0))
        result["mfma_ceiling"] = mfma_ceiling
        result["frac_of_mfma_ceiling"] = round(tflops / mfma_ceiling["tflop_per_s"], 4)
        print(f"[bench] sustained MFMA rate: {mfma_ceiling}", file=sys.stderr, flush=True)

    # ---- every configuration of the workload table, timed the same way (GPU first;
    # the oracle checks follow on the CPU)
    measured = {wl.name: (t, desc, host, inp)}
    ceiling = None
    if not args.no_configs:
        for name in CONFIG_WORKLOADS + VARIANT_WORKLOADS:
            if name in measured:
                continue
            cw = WORKLOADS[name]
            steps = args.config_steps * (5 if name in ("smallk_qkv_bf16", "gqa_rope8_bf16") else 1)
            ct, cdesc, chost, cinp, _ = measure_workload(cw, dev, steps, 10, min(args.min_warmup_s, 1.0))
            measured[name] = (ct, cdesc, chost, cinp)
            if name == "smallk_qkv_bf16":
                out_b = cw.M * cw.F * cw.elem_bytes
                ceiling = measure_stream_ceiling(dev, int(cw.alg_bytes - out_b), out_b, cw.F, cw.dtype, steps,
                                                 min(args.min_warmup_s, 1.0))
                print(f"[bench] stream ceiling for {name}: {ceiling}", file=sys.stderr, flush=True)
            print(f"[bench] {name}: mean {ct['mean_us']:.2f} us, median {ct['median_us']:.2f} "
                  f"(p10 {ct['p10_us']:.2f}, p90 {ct['p90_us']:.2f})", file=sys.stderr, flush=True)

    # ---- the backward pass of every configuration (its own launches; the headline's
    # gradients checked against the oracle on every element)
    if not args.no_backward:
        bwd = []
        for name in (CONFIG_WORKLOADS if not args.no_configs else [wl.name]):
            e = measure_backward(WORKLOADS[name], dev, 50, min(args.min_warmup_s, 0.5),
                                 check=(name == wl.name and not args.no_cpu_baseline))
            print(f"[bench] backward {name}: {e}", file=sys.stderr, flush=True)
            bwd.append(e)
        result["backward"] = bwd

    # ---- the oracle: CPU baseline on the headline workload, then every output element of
    # every measured workload against it
    cores = len(os.sched_getaffinity(0))
    refs = {}
    if not args.no_cpu_baseline:
        import oracle

        tokens = np.arange(wl.M, dtype=np.int64)
        ref, secs = run_oracle(wl, inp, tokens, cores)
        reps = 1
        while secs < args.cpu_seconds and reps < 10:
            _, s_ = run_oracle(wl, inp, tokens, cores)
            secs += s_
            reps += 1
        refs[wl.name] = ref
        result["cpu_baseline"] = {"value": round(wl.flops * reps / secs / 1e12, 6), "unit": "TFLOP/s",
                                  "cores": cores, "kind": "oracle",
                                  "sample": f"all {wl.M} tokens x {reps} run(s), all F={wl.F} columns, float64, "
                                            f"{secs:.1f} s on {cores} threads"}
        result["parity"] = parity(wl, inp, host, tokens, ref)
        print(f"[bench] parity {wl.name}: {result['parity']}", file=sys.stderr, flush=True)

        one_core = []
        for name in ONE_CORE_WORKLOADS:
            cw = WORKLOADS[name]
            cinp = measured[name][3] if name in measured else None
            if cinp is None:
                continue
            _, s1 = run_oracle(cw, cinp, np.arange(cw.M, dtype=np.int64), 1)
            one_core.append({"workload": name, "seconds": round(s1, 4), "gflop_per_s": round(cw.flops / s1 / 1e9, 3),
                             "tokens": cw.M, "cores": 1})
        result["cpu_1core"] = one_core

    configs, variants = [], []
    for name in (CONFIG_WORKLOADS + VARIANT_WORKLOADS if not args.no_configs else [wl.name]):
        if name not in measured:
            continue
        ct, cdesc, chost, cinp = measured[name]
        cw = WORKLOADS[name]
        c_tflops, c_gbs, c_roof = roofline_of(cw, ct["mean_us"])
        entry = {"workload": name, "tokens": cw.M, "C": cw.C, "F": cw.F, "dtype": cw.dtype,
                 "us_mean": round(ct["mean_us"], 2), "us_median": round(ct["median_us"], 2),
                 "us_p10": round(ct["p10_us"], 2), "us_p90": round(ct["p90_us"], 2), "launches": ct["per_launch_n"],
                 "tflop_per_s": round(c_tflops, 2), "gb_per_s": round(c_gbs, 1), "bound": c_roof["bound"],
                 "frac": c_roof["frac"], "frac_at_median": round(roofline_of(cw, ct["median_us"])[2]["frac"], 4),
                 "kernel": cdesc}
        if mfma_ceiling is not None and cw.dtype == "bf16" and c_roof["bound"] == "mfma":
            entry["frac_of_mfma_ceiling"] = round(c_tflops / mfma_ceiling["tflop_per_s"], 4)
        if name == "smallk_qkv_bf16" and ceiling is not None:
            # the same bytes through a plain streaming kernel in this harness
            entry["stream_ceiling"] = ceiling
            entry["frac_of_stream_ceiling"] = round(ceiling["us_mean"] / ct["mean_us"], 4)
        if not args.no_cpu_baseline:
            if name == wl.name:
                entry["parity"] = result["parity"]
            else:
                tokens = np.arange(cw.M, dtype=np.int64)
                ref, s_ = run_oracle(cw, cinp, tokens, cores)
                entry["parity"] = parity(cw, cinp, chost, tokens, ref)
                entry["oracle_s"] = round(s_, 2)
                del ref
            print(f"[bench] parity {name}: {entry['parity']}", file=sys.stderr, flush=True)
        (variants if name in VARIANT_WORKLOADS else configs).append(entry)
    result["configs"] = configs
    if variants:
        result["variants"] = variants

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

    def launch(i):
        rc = op.run_ptrs(*calls[i % ring], sh)
        if rc != 0:
            raise RuntimeError(f"split_rope_run failed with status {rc}")

    t = time_launches(launch, args.steps, args.warmup, args.min_warmup_s, stream)
    us = t["mean_us"]
    gbs = wl.alg_bytes / (us * 1e-6) / 1e9
    result = {
        "metric": METRIC, "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(us * 1e-3, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic: seeded qkv ~ N(0,1), rounded once to bf16",
        "config": {"workload": wl.name, "op": "split_rope", "batch": wl.batch, "tokens": wl.tokens,
                   "n_heads": wl.n_heads, "n_kv_heads": wl.n_kv_heads, "head_dim": wl.head_dim,
                   "qkv_order": wl.qkv_order, "rope_dims": wl.rope_dims, "k_transposed": wl.k_transposed,
                   "ring": ring},
        "gb_per_s": round(gbs, 1), "hbm_frac": round(gbs / PEAK_HBM_GBS, 4),
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None},
        "launch_us": {k: (round(v, 2) if isinstance(v, float) else v) for k, v in t.items()},
        "kernel": "split_rope_kernel", "kernel_hash": kernel_hash(),
    }
    # the same bytes through a plain streaming kernel in this harness
    qkv_b = 2 * wl.batch * wl.tokens * wl.Fq
    ceiling = measure_stream_ceiling(dev, qkv_b, qkv_b, wl.Fq, "bf16", args.steps, min(args.min_warmup_s, 1.0))
    result["stream_ceiling"] = ceiling
    result["frac_of_stream_ceiling"] = round(ceiling["us_mean"] / us, 4)
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
        q, k, v = (t_.double().cpu().numpy() for t_ in outs[0])
        err = max(float(np.max(np.abs(g - r) / (2.0 ** -8 * np.abs(r) + 1e-5 * np.abs(x64).max())))
                  for g, r in zip((q, k, v), ref))
        result["parity"] = {"ok": err <= 1.0, "max_err_over_tol": round(err, 5)}
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
