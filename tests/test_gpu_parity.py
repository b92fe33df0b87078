"""GPU parity: the HIP path through the C ABI against the float64 oracle, per element.

Bar (stated for the fused projection): |gpu - oracle| <= 4e-3 * (||x_t|| ||w_col|| + |b|)
for bf16 and 1e-5 * the same scale for fp32, with the RoPE-effective column for q/k
(see oracle/compare.py). Every named workload is checked at full size on every
token; small shapes that span several tiles with ragged tails too; forced-kernel
cases on sampled tokens (ends, slab and tile boundaries, random).
"""
import numpy as np
import pytest
import torch

from ff_input_projection_amd import FusedProjError, EALIAS, EALIGN, EINVAL
from ff_input_projection_amd.workloads import WORKLOADS, make_inputs, with_shape

from oracle import compare as cmp

from helpers import all_tokens, gpu_rows, nan_outputs, oracle_rows, plan_for, run_gpu, sample_tokens, scales_for, verdict

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _check(wl, inp, outs, tokens, label):
    v = verdict(wl, inp, outs, tokens)
    print(f"[parity] {label}: {v}", flush=True)
    assert v.ok, f"{label}: {v}"
    assert v.max_tight_ratio <= 1.0, f"{label} (tight bar): {v}"
    return v


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_workload_full_size_every_token(name, monkeypatch):
    """Every named workload at full size, every output element compared with the oracle
    (run once on all host cores), through the default kernel choice and through the
    general kernel. Outputs start as NaN, so every element must have been written."""
    wl = WORKLOADS[name]
    inp = make_inputs(wl)
    tokens = all_tokens(wl)
    print(f"[case] full-size {name}: oracle on {wl.M} tokens", flush=True)
    ref = oracle_rows(wl, inp, tokens)
    sc = scales_for(wl, inp, tokens, ref)
    for choice in ("auto", "general"):
        if choice == "general":
            monkeypatch.setenv("FUSED_PROJ_KERNEL", "general")
        else:
            monkeypatch.delenv("FUSED_PROJ_KERNEL", raising=False)
        print(f"[case] full-size {name} kernel={choice}", flush=True)
        proj, outs = run_gpu(wl, inp, DEV)
        print(f"[plan] {proj.describe()}", flush=True)
        v = cmp.compare(gpu_rows(wl, outs, tokens), ref, [sc.ff, sc.q, sc.k, sc.v], wl.dtype)
        print(f"[parity] {name} {choice}: {v}", flush=True)
        assert v.ok and v.n == wl.M * wl.F, f"{name} {choice}: {v}"
        assert v.max_tight_ratio <= 1.0, f"{name} {choice} (tight bar): {v}"
        del outs, proj
        torch.cuda.empty_cache()


SMALL = [
    # channels-first, RoPE, GELU, ragged M (120 tokens), K tail (72), 3 column tiles with a ragged last one
    with_shape(WORKLOADS["walrus_bf16"], "cf_rope_ragged", x_shape=(3, 72, 5, 8, 1), ff_dim=64, n_heads=3,
               head_dim=32, seed=101),
    # token-major, [F,C] weight, RoPE hd 16, ragged everything
    with_shape(WORKLOADS["bert_qkv_bf16"], "tl_fc_rope", x_shape=(2, 77, 80), ff_dim=48, ff_act="gelu",
               n_heads=2, head_dim=16, rope=True, w_layout="fc", seed=102),
    # channels-first, [F,C] weight, no bias, hd 128, pos_offset
    with_shape(WORKLOADS["walrus_bf16"], "cf_fc_hd128_offset", x_shape=(2, 136, 6, 20), ff_dim=128,
               n_heads=2, head_dim=128, has_bias=False, w_layout="fc", pos_offset=7, seed=103),
    # token-major, [C,F] weight, ff only, K = 8 (one chunk), 9 tokens
    with_shape(WORKLOADS["bert_ff_bf16"], "tl_tiny_k", x_shape=(1, 9, 8), ff_dim=24, seed=104),
    # several M tiles, hd 64 without RoPE, 3 heads (192 columns per slice)
    with_shape(WORKLOADS["smallk_qkv_bf16"], "cf_smallk_multitile", x_shape=(2, 64, 16, 24), n_heads=3,
               seed=105),
    # K = 40 (one full 32-wide K step and a ragged one), channels-first, RoPE hd 64, ragged F tile
    with_shape(WORKLOADS["walrus_bf16"], "cf_ktail_hd64", x_shape=(2, 40, 4, 24, 1), ff_dim=64, n_heads=3,
               head_dim=64, seed=108),
    # token-major [F,C] weight, RoPE hd 32, two M tiles + tail, bias, no GELU
    with_shape(WORKLOADS["bert_qkv_bf16"], "tl_fc_hd32", x_shape=(3, 100, 96), ff_dim=32, n_heads=4,
               head_dim=32, rope=True, w_layout="fc", seed=109),
    # the fast kernel's small tiles: 256 tokens (two whole 128-token tiles), K = 72 (two
    # whole K steps, a ragged one and a padding one), F = 448 (a ragged last 128-column
    # tile), RoPE hd 64, GELU
    with_shape(WORKLOADS["walrus_bf16"], "cf_small_tiles_rope", x_shape=(2, 72, 8, 16, 1), ff_dim=64,
               n_heads=2, head_dim=64, seed=110),
    # small tiles whose waves straddle slabs (48 and 80 tokens per slab): the per-token
    # store offsets take the general path
    with_shape(WORKLOADS["walrus_bf16"], "cf_small_tiles_straddle", x_shape=(8, 64, 6, 8, 1), ff_dim=64,
               n_heads=2, head_dim=64, seed=111),
    with_shape(WORKLOADS["bert_qkv_bf16"], "tl_small_tiles_straddle", x_shape=(8, 80, 64), ff_dim=0, n_heads=3,
               head_dim=64, rope=True, w_layout="fc", seed=112),
    # small tiles with one K step (K = 24: the load pipeline is deeper than the K loop), with
    # K = 160 (five whole steps: one pass of the five-stage loop, no partial steps) and with
    # K = 224 (seven whole steps: a pass and a remainder of two)
    with_shape(WORKLOADS["walrus_bf16"], "cf_small_tiles_one_kstep", x_shape=(2, 24, 8, 16, 1), ff_dim=64,
               n_heads=2, head_dim=64, seed=113),
    with_shape(WORKLOADS["bert_qkv_bf16"], "tl_small_tiles_k160", x_shape=(2, 128, 160), ff_dim=0, n_heads=2,
               head_dim=64, seed=114),
    with_shape(WORKLOADS["smallk_qkv_bf16"], "cf_small_tiles_k224", x_shape=(2, 224, 8, 16), n_heads=2,
               seed=115),
    # the other ff activations (general kernel): tanh GELU with RoPE on a token-major x, and
    # squared ReLU on a shape the fast kernel's small tiles would take with exact GELU
    with_shape(WORKLOADS["bert_ff_bf16"], "tl_gelu_tanh_rope", x_shape=(2, 70, 96), ff_dim=64,
               ff_act="gelu_tanh", n_heads=2, head_dim=32, rope=True, seed=117),
    with_shape(WORKLOADS["walrus_bf16"], "cf_relu2", x_shape=(2, 72, 8, 16, 1), ff_dim=128, ff_act="relu2",
               n_heads=2, head_dim=64, seed=118),
    with_shape(WORKLOADS["tiny_f32"], "f32_tl_gelu_tanh", layout="tokens_last", x_shape=(2, 40, 48), ff_dim=32,
               ff_act="gelu_tanh", n_heads=2, head_dim=8, seed=119),
    with_shape(WORKLOADS["tiny_f32"], "f32_cf_relu2", x_shape=(1, 40, 8, 8, 1), ff_dim=64, ff_act="relu2",
               n_heads=2, head_dim=8, seed=120),
    # fewer k/v heads than q heads, both column orders, partial rotary (by default the fast
    # kernel takes the bf16 ones rotating 8 columns or whole heads, the general kernel
    # rotary width 16 and fp32)
    with_shape(WORKLOADS["gqa_rope8_bf16"], "tl_gqa_grouped_rope8", x_shape=(2, 77, 64), seed=122),
    with_shape(WORKLOADS["bert_qkv_bf16"], "tl_gqa_contiguous_rope16", x_shape=(2, 90, 96), ff_dim=64,
               ff_act="gelu", n_heads=6, head_dim=32, n_kv_heads=2, rope=True, rope_dims=16, seed=123),
    with_shape(WORKLOADS["walrus_bf16"], "cf_mqa_grouped_fullrope", x_shape=(2, 64, 8, 8, 1), ff_dim=64,
               n_heads=4, head_dim=64, n_kv_heads=1, qkv_order="grouped", seed=124),
    with_shape(WORKLOADS["tiny_f32"], "f32_gqa_grouped_rope4", layout="tokens_last", x_shape=(2, 30, 32), ff_dim=0,
               n_heads=4, head_dim=8, n_kv_heads=2, qkv_order="grouped", rope_dims=4, has_bias=True, seed=125),
    # channels-first ff output (the 1x1x1-convolution layout; general kernel): with q/k/v
    # and RoPE on a channels-first x, GELU on a token-major x, and fp32
    with_shape(WORKLOADS["walrus_bf16"], "cf_ff_channels_first", x_shape=(2, 64, 8, 16, 1), ff_dim=128,
               n_heads=2, head_dim=32, ff_layout="channels_first", seed=126),
    with_shape(WORKLOADS["bert_ff_bf16"], "tl_ff_channels_first", x_shape=(3, 40, 96), ff_dim=136,
               ff_layout="channels_first", seed=127),
    with_shape(WORKLOADS["tiny_f32"], "f32_cf_ff_channels_first", x_shape=(1, 32, 6, 6, 1), ff_dim=64,
               ff_layout="channels_first", seed=128),
    # fp32, token-major, [F,C], RoPE hd 8, GELU
    with_shape(WORKLOADS["tiny_f32"], "f32_tl_fc", layout="tokens_last", x_shape=(3, 50, 36), ff_dim=16,
               n_heads=3, head_dim=8, w_layout="fc", seed=106),
    # fp32, channels-first, several tiles
    with_shape(WORKLOADS["tiny_f32"], "f32_cf_multitile", x_shape=(2, 68, 10, 16, 1), ff_dim=136,
               n_heads=5, head_dim=8, seed=107),
]


@pytest.fixture(params=["auto", "general"])
def kernel_choice(request, monkeypatch):
    """Run a case through the default kernel choice and through the general kernel."""
    if request.param == "general":
        monkeypatch.setenv("FUSED_PROJ_KERNEL", "general")
    else:
        monkeypatch.delenv("FUSED_PROJ_KERNEL", raising=False)
    return request.param


@pytest.mark.parametrize("wl", SMALL, ids=[w.name for w in SMALL])
def test_small_ragged_all_tokens(wl, kernel_choice):
    print(f"[case] small {wl.name} x={wl.x_shape} kernel={kernel_choice}", flush=True)
    inp = make_inputs(wl)
    proj, outs = run_gpu(wl, inp, DEV)
    print(f"[plan] {proj.describe()}", flush=True)
    _check(wl, inp, outs, all_tokens(wl), wl.name)


def test_fast_kernel_on_padded_or_ragged_tiling(monkeypatch):
    """The small-K workload (padded K steps, a ragged column tile, fewer large tiles than
    CUs) forced onto the fast kernel, which takes its small tiles there. This shape once
    faulted the GPU: the cause, missing wait states before the inline-asm loads, is fixed
    and pinned on the CPU by test_isa_hazards.py."""
    monkeypatch.setenv("FUSED_PROJ_KERNEL", "fast")
    wl = WORKLOADS["smallk_qkv_bf16"]
    inp = make_inputs(wl)
    _, outs = run_gpu(wl, inp, DEV)
    _check(wl, inp, outs, sample_tokens(wl, 384, seed=1), wl.name)


FAST_VARIANTS = [
    # tanh GELU and squared ReLU on the fast kernel's small and large tiles
    # (these epilogues are compiled without RoPE: heads without it)
    with_shape(WORKLOADS["walrus_bf16"], "fast_gelu_tanh_small", x_shape=(2, 64, 8, 16, 1), ff_dim=64,
               ff_act="gelu_tanh", n_heads=2, head_dim=64, rope=False, seed=121),
    with_shape(WORKLOADS["walrus_bf16"], "fast_relu2_small", x_shape=(2, 64, 8, 16, 1), ff_dim=64,
               ff_act="relu2", n_heads=2, head_dim=64, rope=False, seed=134),
    with_shape(WORKLOADS["bert_ff_bf16"], "fast_gelu_tanh_large", x_shape=(16, 512, 256), ff_dim=2048,
               ff_act="gelu_tanh", seed=135),
    with_shape(WORKLOADS["bert_ff_bf16"], "fast_relu2_large_ragged_m", x_shape=(2, 8150, 256), ff_dim=1536,
               ff_act="relu2", n_heads=4, head_dim=64, seed=136),
    # channels-first ff output (ff_dim a multiple of 128, no RoPE) on small tiles with a
    # ragged token tile and slabs of 120 tokens, and on large tiles with q/k/v heads
    with_shape(WORKLOADS["walrus_bf16"], "fast_ffcf_small_ragged", x_shape=(3, 128, 10, 12, 1), ff_dim=256,
               n_heads=2, head_dim=64, rope=False, ff_layout="channels_first", seed=137),
    with_shape(WORKLOADS["walrus_bf16"], "fast_ffcf_large_heads", x_shape=(16, 256, 32, 32, 1), ff_dim=1024,
               n_heads=4, head_dim=64, rope=False, ff_layout="channels_first", seed=138),
    with_shape(WORKLOADS["bert_ff_bf16"], "fast_ffcf_tokens_last_gelu", x_shape=(8, 1000, 128), ff_dim=512,
               ff_layout="channels_first", seed=139),
    # fewer k/v heads and grouped columns: RoPE on the first 8 columns of each head on large
    # tiles with a GELU ff slice; 8-column heads rotated whole (k/v contiguous, ragged tokens);
    # whole-head RoPE with 4 k/v heads, contiguous, on large tiles with a [F,C] weight
    with_shape(WORKLOADS["gqa_rope8_bf16"], "fast_rope8_large_grouped_ff", x_shape=(4, 2048, 256), ff_dim=1024,
               ff_act="gelu", n_heads=16, head_dim=64, n_kv_heads=4, rope_dims=8, has_bias=True, seed=140),
    with_shape(WORKLOADS["gqa_rope8_bf16"], "fast_rope8_hd8_contiguous", x_shape=(2, 150, 64), n_heads=4,
               head_dim=8, n_kv_heads=2, qkv_order="contiguous", rope_dims=0, seed=141),
    with_shape(WORKLOADS["bert_qkv_bf16"], "fast_gqa_fullrope_large_fc", x_shape=(16, 1024, 256), ff_dim=0,
               n_heads=16, head_dim=64, n_kv_heads=4, rope=True, w_layout="fc", pos_offset=3, seed=142),
]


@pytest.mark.parametrize("wl", FAST_VARIANTS, ids=[w.name for w in FAST_VARIANTS])
def test_fast_kernel_activation_and_ff_layout_variants(wl):
    """tanh GELU, squared ReLU, the channels-first ff output and the grouped-query layouts on
    the fast kernel (planned by default), every output element against the oracle; outputs
    start as NaN."""
    print(f"[case] fast variant {wl.name} x={wl.x_shape}", flush=True)
    inp = make_inputs(wl)
    proj, outs = run_gpu(wl, inp, DEV)
    desc = proj.describe()
    print(f"[plan] {desc}", flush=True)
    assert "fused_proj_fast_kernel" in desc, desc
    _check(wl, inp, outs, all_tokens(wl), wl.name)


RAGGED_M = [
    # token counts that are not whole tiles, forced onto the fast kernel: large tiles
    # (16300 tokens, 640 tiles of 256 x 256, RoPE, GELU, token-major) and small tiles
    # (8144 tokens of the small-K shape, channels-first, slabs of 4072 tokens)
    with_shape(WORKLOADS["bert_qkv_bf16"], "tl_large_tiles_ragged_m", x_shape=(2, 8150, 256), ff_dim=1024,
               ff_act="gelu", n_heads=8, head_dim=64, rope=True, seed=129),
    with_shape(WORKLOADS["smallk_qkv_bf16"], "cf_small_tiles_ragged_m", x_shape=(2, 320, 4072), seed=130),
]


RAGGED_M += [
    # large tiles with C not a multiple of 128 (partial and zero-padding K steps): the
    # small-K shape at batch 8 (32768 tokens, C 320, 512 tiles), a token-major C 72 and a
    # channels-first C 200 with RoPE and GELU
    with_shape(WORKLOADS["smallk_qkv_bf16"], "cf_large_tiles_c320", x_shape=(8, 320, 64, 64), seed=131),
    with_shape(WORKLOADS["bert_qkv_bf16"], "tl_large_tiles_c72", x_shape=(4, 4000, 72), ff_dim=1024, ff_act="gelu",
               n_heads=4, head_dim=64, seed=132),
    with_shape(WORKLOADS["walrus_bf16"], "cf_large_tiles_c200", x_shape=(12, 200, 32, 32, 1), ff_dim=512,
               n_heads=8, head_dim=64, seed=133),
]


@pytest.mark.parametrize("wl", RAGGED_M, ids=[w.name for w in RAGGED_M])
def test_fast_kernel_ragged_token_count(wl, monkeypatch):
    """The fast kernel on token counts that are not whole tiles: tokens past M read token
    0 and are not stored. Sampled tokens include the last ones and the slab boundary."""
    monkeypatch.setenv("FUSED_PROJ_KERNEL", "fast")
    print(f"[case] fast kernel, ragged M: {wl.name} x={wl.x_shape} M={wl.M}", flush=True)
    inp = make_inputs(wl)
    proj, outs = run_gpu(wl, inp, DEV)
    desc = proj.describe()
    print(f"[plan] {desc}", flush=True)
    assert "fused_proj_fast_kernel" in desc, desc
    tokens = np.unique(np.concatenate([sample_tokens(wl, 384, seed=3), np.arange(wl.M - 300, wl.M)]))
    _check(wl, inp, outs, tokens, wl.name)
    for t in outs:
        if t is not None:
            assert torch.isfinite(t).all().item()


LARGE_FC = [
    # [F,C] weights (nn.Linear layout) on the large tiles, both x layouts: 8192 tokens,
    # C = 256, F = 1024 + 3 * 512 = 2560 (320 tiles of 256 x 256), RoPE hd 64, GELU
    with_shape(WORKLOADS["bert_qkv_bf16"], "tl_fc_large_tiles", x_shape=(16, 512, 256), ff_dim=1024,
               ff_act="gelu", n_heads=8, head_dim=64, rope=True, w_layout="fc", pos_offset=3, seed=113),
    with_shape(WORKLOADS["walrus_bf16"], "cf_fc_large_tiles", x_shape=(8, 256, 32, 32, 1), ff_dim=1024,
               n_heads=8, head_dim=64, w_layout="fc", seed=114),
]


LARGE_FC += [
    # large tiles with a ragged last column tile: F = 1152 + 3 * 256 = 1920 (7.5 column
    # tiles of 256), 16384 tokens (64 x 8 = 512 tiles), RoPE hd 64, GELU, [C,F] weight
    with_shape(WORKLOADS["walrus_bf16"], "cf_large_tiles_ragged_f", x_shape=(16, 256, 32, 32, 1), ff_dim=1152,
               n_heads=4, head_dim=64, seed=116),
]


@pytest.mark.parametrize("wl", LARGE_FC, ids=[w.name for w in LARGE_FC])
def test_large_tiles_with_fc_weights(wl):
    """The fast kernel's large-tile instantiations that read W as [F,C] (K-contiguous
    rows), which none of the named workloads uses, and a ragged last column tile."""
    print(f"[case] large tiles, [F,C] weight: {wl.name} x={wl.x_shape}", flush=True)
    inp = make_inputs(wl)
    proj, outs = run_gpu(wl, inp, DEV)
    desc = proj.describe()
    print(f"[plan] {desc}", flush=True)
    assert "fused_proj_fast_kernel" in desc and "tile=256x256" in desc, desc
    _check(wl, inp, outs, sample_tokens(wl, 384, seed=2), wl.name)


TAIL = [
    # (CUs planned for, shape): with few CUs these small shapes walk the large tiles
    # persistently with a part-filled last round, which the split moves to small tiles.
    # token-major, RoPE hd 64, GELU ff, bias: 4 token rows x 5 column tiles on 16 CUs
    (16, with_shape(WORKLOADS["bert_qkv_bf16"], "tail_tl_rope_gelu", x_shape=(8, 128, 192), ff_dim=512,
                    ff_act="gelu", n_heads=4, head_dim=64, rope=True, seed=151)),
    # channels-first x, grouped query heads with RoPE on 8 columns, no ff: 9 tiles on 8 CUs
    (8, with_shape(WORKLOADS["gqa_rope8_bf16"], "tail_cf_gqa_rope8", layout="channels_first",
                   x_shape=(6, 256, 16, 16, 1), ff_dim=0, n_heads=8, head_dim=64, n_kv_heads=2, rope_dims=8,
                   seed=152)),
    # channels-first x and ff output, [F,C] weight, slabs of 64 tokens: 9 tiles on 8 CUs
    (8, with_shape(WORKLOADS["walrus_bf16"], "tail_cf_ffcf_fc", x_shape=(10, 128, 8, 8, 1), ff_dim=256,
                   n_heads=2, head_dim=64, rope=False, w_layout="fc", ff_layout="channels_first", seed=153)),
    # squared ReLU, slabs of 150 tokens (the head ends inside a large tile row): 10 tiles on 8 CUs
    (8, with_shape(WORKLOADS["bert_ff_bf16"], "tail_tl_relu2_ragged_s", x_shape=(8, 150, 96), ff_dim=320,
                   ff_act="relu2", n_heads=1, head_dim=64, seed=154)),
]


@pytest.mark.parametrize("cus,wl", TAIL, ids=[w.name for _, w in TAIL])
def test_large_tiles_with_small_tile_tail(cus, wl, monkeypatch):
    """The large tiles' last round moved to a second launch on small tiles (whole slabs
    from the split token on, every pointer advanced by it): planned for a few CUs and
    forced, every output element against the oracle; outputs start as NaN."""
    monkeypatch.setenv("FUSED_PROJ_CUS", str(cus))
    monkeypatch.setenv("FUSED_PROJ_TAIL", "1")
    print(f"[case] small-tile tail {wl.name} x={wl.x_shape} cus={cus}", flush=True)
    inp = make_inputs(wl)
    proj, outs = run_gpu(wl, inp, DEV)
    desc = proj.describe()
    print(f"[plan] {desc}", flush=True)
    assert "tile=256x256" in desc and " tail=" in desc, desc
    _check(wl, inp, outs, all_tokens(wl), wl.name)
    for t in outs:
        if t is not None:
            assert torch.isfinite(t).all().item()


def test_strided_views_channel_slice_and_row_stride(kernel_choice):
    """x as a view: a channel slice of a wider channels-first tensor, and a token-major
    view whose row stride exceeds C. No copy is made; results match the oracle."""
    wl = with_shape(WORKLOADS["walrus_bf16"], "cf_view", x_shape=(2, 48, 8, 16, 1), ff_dim=64, n_heads=2,
                    head_dim=32, seed=201)
    inp = make_inputs(wl)
    big = torch.zeros((2, 64, 8, 16, 1), dtype=torch.bfloat16)
    big[:, 8:56] = inp.x
    xv = big.to(DEV)[:, 8:56]
    assert not xv.is_contiguous()
    _, outs = run_gpu(wl, inp, DEV, x_dev=xv)
    _check(wl, inp, outs, all_tokens(wl), "channel-slice view")

    wl2 = with_shape(WORKLOADS["bert_qkv_bf16"], "tl_view", x_shape=(3, 40, 64), n_heads=2, head_dim=32,
                     seed=202)
    inp2 = make_inputs(wl2)
    wide = torch.zeros((3, 40, 96), dtype=torch.bfloat16)
    wide[:, :, :64] = inp2.x
    xv2 = wide.to(DEV)[:, :, :64]
    _, outs2 = run_gpu(wl2, inp2, DEV, x_dev=xv2)
    _check(wl2, inp2, outs2, all_tokens(wl2), "row-stride view")


def test_x_span_beyond_4gib_takes_the_general_kernel():
    """A token-major x whose span reaches past 4 GiB: 65536 tokens of 256 channels with a
    row stride of 33024 elements (4.33 GB). That is beyond the fast kernel's 32-bit
    offsets, so the plan takes the general kernel, whose offsets are 64-bit. Every output
    element against the oracle; outputs start as NaN."""
    wl = with_shape(WORKLOADS["bert_qkv_bf16"], "tl_span_4gib", x_shape=(1, 65536, 256), ff_dim=128,
                    ff_act="gelu", n_heads=2, head_dim=64, rope=True, seed=203)
    stride = 33024
    assert ((wl.M - 1) * stride + wl.C) * 2 >= 1 << 32
    print(f"[case] x span past 4 GiB: {wl.name} x={wl.x_shape} row stride {stride}", flush=True)
    inp = make_inputs(wl)
    big = torch.empty((1, wl.M, stride), dtype=torch.bfloat16, device=DEV)
    big[:, :, :wl.C] = inp.x.to(DEV)
    proj, outs = run_gpu(wl, inp, DEV, x_dev=big[:, :, :wl.C])
    desc = proj.describe()
    print(f"[plan] {desc}", flush=True)
    assert "fused_proj_tile_kernel" in desc, desc
    _check(wl, inp, outs, all_tokens(wl), wl.name)
    for t in outs:
        if t is not None:
            assert torch.isfinite(t).all().item()
    del big, outs, proj
    torch.cuda.empty_cache()


def test_layout_invariance_on_gpu(kernel_choice):
    """Channels-first input and its channels-last copy give the same outputs."""
    wl = with_shape(WORKLOADS["walrus_bf16"], "inv", x_shape=(2, 64, 8, 16, 1), ff_dim=64, n_heads=2,
                    head_dim=32, seed=301)
    inp = make_inputs(wl)
    _, o1 = run_gpu(wl, inp, DEV)
    xl = inp.x.permute(0, 2, 3, 4, 1).reshape(2, 128, 64).contiguous()
    wl2 = with_shape(wl, "inv_tl", layout="tokens_last", x_shape=(2, 128, 64))
    _, o2 = run_gpu(wl2, inp, DEV, x_dev=xl.to(DEV))
    for a, b in zip(o1, o2):
        if a is not None:
            assert torch.equal(a, b)


def test_determinism_bitwise():
    wl = WORKLOADS["bert_qkv_bf16"]
    inp = make_inputs(wl)
    x, w, b = inp.x.to(DEV), inp.w.to(DEV), inp.bias.to(DEV)
    proj = plan_for(wl, x)
    o1 = [t.clone() for t in proj(x, w, b) if t is not None]
    o2 = [t for t in proj(x, w, b) if t is not None]
    torch.cuda.synchronize()
    for a, c in zip(o1, o2):
        assert torch.equal(a, c)


GUARDED = [SMALL[0], LARGE_FC[-1], RAGGED_M[0]]


@pytest.mark.parametrize("wl", GUARDED, ids=[w.name for w in GUARDED])
def test_canary_guard_bands_untouched(wl):
    """Outputs live inside larger NaN-filled buffers: every output element is written,
    nothing outside is. Cases: a small ragged shape, a large-tile shape with a ragged last
    column tile, and a large-tile shape with a ragged last token tile."""
    inp = make_inputs(wl)
    x, w, b = inp.x.to(DEV), inp.w.to(DEV), inp.bias.to(DEV)
    proj = plan_for(wl, x)
    print(f"[case] guard bands {wl.name}: {proj.describe()}", flush=True)
    ffs, qs, kvs = proj.out_shapes()
    guard = 4096
    bufs, outs = [], []
    for s in (ffs, qs, kvs, kvs):
        if s is None:
            bufs.append(None)
            outs.append(None)
            continue
        n = int(np.prod(s))
        buf = torch.full((n + 2 * guard,), float("nan"), dtype=torch.bfloat16, device=DEV)
        bufs.append(buf)
        outs.append(buf[guard:guard + n].view(s))
    proj(x, w, b, out=outs)
    torch.cuda.synchronize()
    for buf, o in zip(bufs, outs):
        if buf is None:
            continue
        assert torch.isfinite(o).all().item()
        assert torch.isnan(buf[:guard]).all().item() and torch.isnan(buf[-guard:]).all().item()


def test_empty_batch_is_a_noop():
    wl = with_shape(WORKLOADS["walrus_bf16"], "empty", x_shape=(0, 64, 8, 8, 1), ff_dim=64, n_heads=2,
                    head_dim=32)
    x = torch.empty(wl.x_shape, dtype=torch.bfloat16, device=DEV)
    w = torch.empty((64, wl.F), dtype=torch.bfloat16, device=DEV)
    b = torch.empty((wl.F,), dtype=torch.bfloat16, device=DEV)
    proj = plan_for(wl, x)
    ff, q, k, v = proj(x, w, b)
    torch.cuda.synchronize()
    assert ff.numel() == 0 and q.numel() == 0


NO_CHANNELS = [
    # channels-first, exact GELU, RoPE over heads of 32, bias: ff = gelu(b), q/k = RoPE(b)
    with_shape(WORKLOADS["walrus_bf16"], "c0_cf_gelu_rope", x_shape=(2, 0, 8, 8, 1), ff_dim=64, n_heads=2,
               head_dim=32),
    # fp32, channels-first, 224 columns (two column tiles, the last ragged)
    with_shape(WORKLOADS["tiny_f32"], "c0_f32", x_shape=(1, 0, 8, 8, 1)),
    # token-major, squared ReLU on a ragged ff slice of 136, three slabs of 40 tokens
    with_shape(WORKLOADS["bert_ff_relu2_bf16"], "c0_tl_relu2", x_shape=(3, 40, 0), ff_dim=136),
    # grouped q/k/v with RoPE on 8 of 32, no bias: every output is zero
    with_shape(WORKLOADS["gqa_rope8_bf16"], "c0_gqa_no_bias", x_shape=(2, 40, 0)),
    # channels-first ff output
    with_shape(WORKLOADS["conv1x1_walrus_bf16"], "c0_ff_channels_first", x_shape=(2, 0, 4, 4, 1), ff_dim=256),
]


@pytest.mark.parametrize("choice", ["auto", "general", "fast"])
@pytest.mark.parametrize("wl", NO_CHANNELS, ids=[w.name for w in NO_CHANNELS])
def test_no_channels_outputs_the_bias(wl, choice, monkeypatch):
    """C = 0: the contraction is empty, so every output is the bias through the activation
    or RoPE (zero without a bias). x and W hold no elements; every output element is
    compared with the oracle. The fast kernel runs one K step read from its zero block."""
    if choice == "auto":
        monkeypatch.delenv("FUSED_PROJ_KERNEL", raising=False)
    else:
        monkeypatch.setenv("FUSED_PROJ_KERNEL", choice)
    inp = make_inputs(wl)
    assert wl.C == 0 and inp.x.numel() == 0 and inp.w.numel() == 0
    print(f"[case] no channels {wl.name} kernel={choice}", flush=True)
    proj, outs = run_gpu(wl, inp, DEV)
    print(f"[plan] {proj.describe()}", flush=True)
    v = _check(wl, inp, outs, all_tokens(wl), f"{wl.name} {choice}")
    assert v.n == wl.M * wl.F


DECODE = [
    # one new token per sequence (a decode step): 16 sequences at position 4095 of the
    # decoder's 4096-token context, RoPE over heads of 128, no bias (96 column tiles)
    with_shape(WORKLOADS["decoder_qkv_rope_bf16"], "decode_16_at_4095", x_shape=(16, 1, 4096), pos_offset=4095),
    # a single sequence, grouped q/k/v with RoPE on 8 of 32, at position 1023
    with_shape(WORKLOADS["gqa_rope8_bf16"], "decode_gqa_1_at_1023", x_shape=(1, 1, 512), pos_offset=1023),
    # fp32, token-major, exact GELU and RoPE over heads of 8, 3 sequences at position 77
    with_shape(WORKLOADS["tiny_f32"], "decode_f32_3_at_77", layout="tokens_last", x_shape=(3, 1, 32),
               pos_offset=77),
]


@pytest.mark.parametrize("choice", ["auto", "general"])
@pytest.mark.parametrize("wl", DECODE, ids=[w.name for w in DECODE])
def test_decode_step_one_token_per_sequence(wl, choice, monkeypatch):
    """S = 1 with a position offset: every sequence's token sits at the offset, so RoPE
    rotates all of them by the same angles; each output element against the oracle."""
    if choice == "general":
        monkeypatch.setenv("FUSED_PROJ_KERNEL", "general")
    else:
        monkeypatch.delenv("FUSED_PROJ_KERNEL", raising=False)
    assert wl.S == 1 and wl.pos_offset > 0
    inp = make_inputs(wl)
    print(f"[case] decode step {wl.name} kernel={choice}", flush=True)
    proj, outs = run_gpu(wl, inp, DEV)
    print(f"[plan] {proj.describe()}", flush=True)
    v = _check(wl, inp, outs, all_tokens(wl), f"{wl.name} {choice}")
    assert v.n == wl.M * wl.F


NON_FINITE = [
    # channels-first, exact GELU, RoPE over heads of 64, bias, 4 column tiles
    with_shape(WORKLOADS["walrus_bf16"], "nonfinite_cf_gelu_rope", x_shape=(2, 64, 8, 8, 1), ff_dim=128,
               n_heads=2, head_dim=64),
    # token-major, squared ReLU, [F, C] weight, ragged tokens
    with_shape(WORKLOADS["bert_ff_relu2_bf16"], "nonfinite_tl_relu2_fc", x_shape=(2, 70, 64), ff_dim=256,
               w_layout="fc"),
    # token-major, tanh GELU
    with_shape(WORKLOADS["bert_ff_bf16"], "nonfinite_tl_tanh", x_shape=(2, 70, 64), ff_dim=256, ff_act="gelu_tanh"),
    # grouped q/k/v with RoPE on 8 of 32, no bias
    with_shape(WORKLOADS["gqa_rope8_bf16"], "nonfinite_gqa_rope8", x_shape=(1, 100, 64)),
    # fp32, channels-first, exact GELU and RoPE over heads of 8
    with_shape(WORKLOADS["tiny_f32"], "nonfinite_f32"),
    # large tiles (planned for 8 CUs: 8 tiles of 256 x 256), exact GELU and RoPE
    with_shape(WORKLOADS["walrus_bf16"], "nonfinite_large_cf_gelu_rope", x_shape=(4, 64, 16, 16, 1), ff_dim=128,
               n_heads=2, head_dim=64),
    # large tiles, squared ReLU, token-major
    with_shape(WORKLOADS["bert_ff_relu2_bf16"], "nonfinite_large_tl_relu2", x_shape=(2, 512, 64), ff_dim=512),
]


def _plant_non_finite(wl, inp):
    """NaN, +inf and -inf in x (token 0 among them: rows past the last token read it), a NaN
    in one weight entry, and (with a bias) +inf and -inf on two ff columns and NaN on a q
    column, whose RoPE partner then turns NaN as well."""
    from ff_input_projection_amd.workloads import as_f64
    x, w = inp.x.clone(), inp.w.clone()
    xv = x.view(wl.nb, wl.C, wl.S) if wl.layout == "channels_first" else x.view(wl.nb, wl.S, wl.C)
    for t, val in ((0, float("nan")), (5, float("nan")), (9, float("inf")), (wl.M - 3, float("-inf"))):
        bi, sp = divmod(t, wl.S)
        if wl.layout == "channels_first":
            xv[bi, 3, sp] = val
        else:
            xv[bi, sp, 3] = val
    col_w = wl.ff_dim + 3 if wl.n_heads else 7
    if wl.w_layout == "cf":
        w[5, col_w] = float("nan")
    else:
        w[col_w, 5] = float("nan")
    inp.x, inp.w, inp.x64, inp.w64 = x, w, as_f64(x), as_f64(w)
    if wl.has_bias:
        b = inp.bias.clone()
        if wl.ff_dim >= 3:
            b[1], b[2] = float("inf"), float("-inf")
        if wl.n_heads:
            b[wl.ff_dim + 1] = float("nan")
        inp.bias, inp.bias64 = b, as_f64(b)
    return inp


@pytest.mark.parametrize("choice", ["auto", "general"])
@pytest.mark.parametrize("wl", NON_FINITE, ids=[w.name for w in NON_FINITE])
def test_non_finite_inputs_give_the_oracles_non_finite_outputs(wl, choice, monkeypatch):
    """NaN and infinities in x, W and the bias: every output element is NaN, +inf or -inf
    exactly where the oracle's is (NaN through every activation, GELU(+inf) = +inf,
    GELU(-inf) = NaN, relu^2(-inf) = 0), and within the bar wherever the oracle and its
    bar are finite. Nothing is hidden, and nothing leaks into other tokens or columns."""
    if choice == "general":
        monkeypatch.setenv("FUSED_PROJ_KERNEL", "general")
    else:
        monkeypatch.delenv("FUSED_PROJ_KERNEL", raising=False)
    if "_large_" in wl.name:
        monkeypatch.setenv("FUSED_PROJ_CUS", "8")
    inp = _plant_non_finite(wl, make_inputs(wl))
    print(f"[case] non-finite inputs {wl.name} kernel={choice}", flush=True)
    proj, outs = run_gpu(wl, inp, DEV)
    print(f"[plan] {proj.describe()}", flush=True)
    if "_large_" in wl.name and choice == "auto":
        assert "tile=256x256" in proj.describe(), proj.describe()
    tokens = all_tokens(wl)
    got = gpu_rows(wl, outs, tokens)
    ref = oracle_rows(wl, inp, tokens)
    with np.errstate(invalid="ignore", over="ignore"):
        sc = scales_for(wl, inp, tokens, ref)
    n_nonfinite = 0
    for name, g, r, scl in zip(("ff", "q", "k", "v"), got, ref, (sc.ff, sc.q, sc.k, sc.v)):
        if r is None:
            continue
        g, r = np.asarray(g, np.float64).reshape(r.shape), np.asarray(r)
        for cls in (np.isnan, np.isposinf, np.isneginf):
            assert np.array_equal(cls(g), cls(r)), f"{wl.name} {choice} {name}: {cls.__name__} differs"
        n_nonfinite += int((~np.isfinite(r)).sum())
        scl = np.asarray(scl).reshape(r.shape)
        ok = np.isfinite(r) & np.isfinite(scl)
        with np.errstate(invalid="ignore"):
            ratio = np.abs(g[ok] - r[ok]) / (cmp.REL[wl.dtype] * scl[ok] + 1e-300)
        assert ratio.size and ratio.max() <= 1.0, f"{wl.name} {choice} {name}: {ratio.max()}"
    print(f"[non-finite] {wl.name} {choice}: {n_nonfinite} non-finite outputs, classes equal", flush=True)
    assert n_nonfinite > 0


def test_run_error_paths():
    wl = SMALL[0]
    inp = make_inputs(wl)
    x, w, b = inp.x.to(DEV), inp.w.to(DEV), inp.bias.to(DEV)
    proj = plan_for(wl, x)
    ff, q, k, v = proj.alloc_outputs(DEV)
    st = torch.cuda.current_stream().cuda_stream
    p = lambda t: t.data_ptr()
    assert proj.run_ptrs(p(x), p(w), p(b), p(ff), p(q), p(k), p(v), st) == 0
    assert proj.run_ptrs(p(x), p(w), p(b), p(ff), p(q), p(k), None, st) == EINVAL
    assert proj.run_ptrs(p(x), p(w), None, p(ff), p(q), p(k), p(v), st) == EINVAL    # bias required
    assert proj.run_ptrs(p(x), p(w), p(b), p(ff) + 2, p(q), p(k), p(v), st) == EALIGN
    assert proj.run_ptrs(p(x), p(w), p(b), p(ff), p(q), p(q), p(v), st) == EALIAS    # q == k
    assert proj.run_ptrs(p(x), p(w), p(b), p(x), p(q), p(k), p(v), st) == EALIAS     # ff over x
    torch.cuda.synchronize()
    with pytest.raises(FusedProjError):
        proj(x, w, b, out=(ff, q, q, v))


@pytest.mark.parametrize("wl", [SMALL[0], SMALL[1]], ids=[SMALL[0].name, SMALL[1].name])
def test_one_plan_on_two_streams_at_once(wl):
    """A plan holds only read-only tables (RoPE cos/sin, column descriptors), so launches of
    one plan on two streams may run at the same time: 20 rounds, each launching on both
    streams without waiting, and each stream's outputs equal the eager result of its own
    inputs, bit for bit."""
    inp_a, inp_b = make_inputs(wl), make_inputs(wl, seed=wl.seed + 77)
    dev = lambda inp: (inp.x.to(DEV), inp.w.to(DEV), None if inp.bias is None else inp.bias.to(DEV))
    a, b = dev(inp_a), dev(inp_b)
    proj = plan_for(wl, a[0])
    eager = [[t.clone() for t in proj(*args) if t is not None] for args in (a, b)]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [[proj.alloc_outputs(DEV) for _ in range(2)] for _ in range(2)]   # [stream][buffer set]
    for st in streams:
        st.wait_stream(torch.cuda.current_stream())
    for rnd in range(20):
        for i, (st, args) in enumerate(zip(streams, (a, b))):
            proj(*args, out=outs[i][rnd % 2], stream=st)
    for st in streams:
        torch.cuda.current_stream().wait_stream(st)
    torch.cuda.synchronize()
    for i in range(2):
        for j in range(2):
            got = [t for t in outs[i][j] if t is not None]
            for e, g in zip(eager[i], got):
                assert torch.equal(e, g), f"stream {i} buffer set {j}"


def test_hip_graph_capture_replays_match_eager():
    """fused_proj_run allocates and synchronises nothing, so it can be captured;
    every replay must equal the eager result."""
    wl = SMALL[1]
    inp = make_inputs(wl)
    x, w, b = inp.x.to(DEV), inp.w.to(DEV), inp.bias.to(DEV)
    proj = plan_for(wl, x)
    eager = [t.clone() for t in proj(x, w, b) if t is not None]
    outs = proj.alloc_outputs(DEV)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            proj(x, w, b, out=outs)
    torch.cuda.current_stream().wait_stream(s)
    for rep in range(3):
        for t in outs:
            if t is not None:
                t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, c in zip(eager, [t for t in outs if t is not None]):
            assert torch.equal(a, c), f"replay {rep}"
