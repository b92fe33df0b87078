"""GPU parity on seeded random shapes: each case draws a valid combination of storage
type, x and W layouts, sizes (ragged against every tile), heads, k/v grouping and column
order, rotary width, activation, ff layout, bias and position offset, and checks every
token against the float64 oracle, through the default kernel choice and the general
kernel. The draws are fixed by the seed, so a failure names a reproducible shape."""
import numpy as np
import pytest

from ff_input_projection_amd.workloads import WORKLOADS, make_inputs, with_shape

from helpers import all_tokens, run_gpu, verdict

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
N_CASES = 24


def draw(seed: int):
    r = np.random.default_rng(1000 + seed)
    dtype = "f32" if r.random() < 0.25 else "bf16"
    V = 8 if dtype == "bf16" else 4
    hd = int(r.choice([8, 16, 32, 64, 128] if dtype == "bf16" else [4, 8, 16, 32]))
    hd = max(hd, V)
    H = int(r.integers(1, 5))
    kvh = int(r.choice([d for d in range(1, H + 1) if H % d == 0]))
    order = "grouped" if r.random() < 0.4 else "contiguous"
    rope = bool(r.random() < 0.7)
    rd = 0
    if rope and r.random() < 0.4:
        rd = int(r.choice([k for k in range(2, hd + 1, 2)]))
    ff_dim = hd * int(r.integers(0, 4))
    if ff_dim == 0 and r.random() < 0.3:
        H, kvh = 0, 0
        ff_dim = V * int(r.integers(1, 40))
    act = str(r.choice(["none", "gelu", "gelu_tanh", "relu2"])) if ff_dim > 0 else "none"
    C = V * int(r.integers(1, 33))
    nb = int(r.integers(1, 4))
    layout = "channels_first" if r.random() < 0.5 else "tokens_last"
    if layout == "channels_first":
        S = V * int(r.integers(1, 80))
        x_shape = (nb, C, S)
    else:
        S = int(r.integers(1, 700))
        x_shape = (nb, S, C)
    ff_layout = "channels_first" if (ff_dim > 0 and S % V == 0 and r.random() < 0.3) else "tokens_last"
    base = WORKLOADS["tiny_f32" if dtype == "f32" else "walrus_bf16"]
    return with_shape(base, f"random_{seed}", layout=layout, x_shape=x_shape, ff_dim=ff_dim, ff_act=act,
                      n_heads=H, head_dim=hd if H > 0 else 0, has_bias=bool(r.random() < 0.7),
                      rope=rope and H > 0, w_layout="fc" if r.random() < 0.4 else "cf",
                      pos_offset=int(r.integers(0, 50)) if r.random() < 0.3 else 0,
                      n_kv_heads=kvh if H > 0 else 0, qkv_order=order if H > 0 else "contiguous",
                      rope_dims=rd if (rope and H > 0) else 0, ff_layout=ff_layout, seed=2000 + seed)


@pytest.fixture(params=["auto", "general"])
def kernel_choice(request, monkeypatch):
    if request.param == "general":
        monkeypatch.setenv("FUSED_PROJ_KERNEL", "general")
    else:
        monkeypatch.delenv("FUSED_PROJ_KERNEL", raising=False)
    return request.param


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_shape_parity(seed, kernel_choice):
    wl = draw(seed)
    print(f"[case] random {seed} kernel={kernel_choice}: {wl}", flush=True)
    inp = make_inputs(wl)
    proj, outs = run_gpu(wl, inp, DEV)
    print(f"[plan] {proj.describe()}", flush=True)
    v = verdict(wl, inp, outs, all_tokens(wl))
    print(f"[parity] random {seed}: {v}", flush=True)
    assert v.ok, f"random {seed}: {v}"
    if wl.dtype == "bf16":
        assert v.max_tight_ratio <= 1.0, f"random {seed} (tight bar): {v}"


N_FAST = 12


def draw_fast(seed: int):
    """A random shape inside the fast kernel's envelope (bf16, q/k/v contiguous with as many
    k/v heads as q heads, full RoPE with a head size of 32, 64 or 128 or none, exact GELU or
    none, token-major ff), ragged in tokens and columns; every third draw is large enough
    for the 256 x 256 tiles (then C is a multiple of 128)."""
    r = np.random.default_rng(3000 + seed)
    hd = int(r.choice([32, 64, 128]))
    H = int(r.integers(0, 5))
    rope = bool(H > 0 and r.random() < 0.7)
    ff_dim = hd * int(r.integers(0 if H > 0 else 1, 9))
    large = seed % 3 == 0
    if large:
        C = 128 * int(r.integers(1, 4))
        M_target = int(r.integers(6000, 12000))
        F_min = 256 * 256 * 256 // M_target + 256
        while ff_dim + 3 * H * hd < F_min:
            ff_dim += hd
    else:
        C = 8 * int(r.integers(1, 65))
        M_target = int(r.integers(1, 3000))
    nb = int(r.integers(1, 4))
    layout = "channels_first" if r.random() < 0.5 else "tokens_last"
    if layout == "channels_first":
        S = max(8, (M_target // nb) // 8 * 8)
        x_shape = (nb, C, S)
    else:
        S = max(1, M_target // nb)
        x_shape = (nb, S, C)
    return with_shape(WORKLOADS["walrus_bf16"], f"random_fast_{seed}", layout=layout, x_shape=x_shape,
                      ff_dim=ff_dim, ff_act=str(r.choice(["none", "gelu"])) if ff_dim > 0 else "none",
                      n_heads=H, head_dim=hd if H > 0 else 0, has_bias=bool(r.random() < 0.7), rope=rope,
                      w_layout="fc" if r.random() < 0.4 else "cf",
                      pos_offset=int(r.integers(0, 50)) if r.random() < 0.3 else 0, seed=4000 + seed)


@pytest.mark.parametrize("seed", range(N_FAST))
def test_random_shape_parity_fast_kernel(seed):
    from helpers import sample_tokens
    wl = draw_fast(seed)
    print(f"[case] random fast {seed}: {wl}", flush=True)
    inp = make_inputs(wl)
    proj, outs = run_gpu(wl, inp, DEV)
    desc = proj.describe()
    print(f"[plan] {desc}", flush=True)
    assert "fused_proj_fast_kernel" in desc, desc
    tokens = all_tokens(wl) if wl.M <= 3000 else np.unique(
        np.concatenate([sample_tokens(wl, 384, seed=seed), np.arange(max(0, wl.M - 200), wl.M)]))
    v = verdict(wl, inp, outs, tokens)
    print(f"[parity] random fast {seed}: {v}", flush=True)
    assert v.ok and v.max_tight_ratio <= 1.0, f"random fast {seed}: {v}"


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_shape_backward(seed):
    """The same draws through the backward pass (default kernel choice): every element of
    dx, dW and db against the float64 backward oracle."""
    from test_gpu_backward import _check

    wl = draw(seed)
    print(f"[case] random backward {seed}: {wl}", flush=True)
    _check(wl, f"random backward {seed}")
