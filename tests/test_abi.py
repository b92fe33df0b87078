"""C ABI checks that need no GPU: the library loads, exports every function the
header declares, and the host-only descriptor check returns the documented codes."""
import ctypes
import os
import re
import subprocess

import pytest

import ff_input_projection_amd as fpa
from ff_input_projection_amd import Desc, make_desc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in ("fused_proj.h", "split_rope.h", "fused_proj_calibrate.h")]


def declared_functions():
    names = set()
    for header in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(header).read(), flags=re.S)
        names.update(re.findall(r"\b((?:fused_proj|split_rope)_[a-z_]+)\s*\(", text))
    return sorted(names)


def test_library_exports_every_declared_symbol():
    lib = fpa.load_library()
    decl = declared_functions()
    assert set(decl) == set(fpa.EXPORTED_SYMBOLS), decl
    for name in decl:
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", fpa.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T ((?:fused_proj|split_rope)_\w+)", out))
    assert set(decl) <= exported


def test_header_compiles_as_plain_c():
    src = ('#include "fused_proj.h"\n#include "split_rope.h"\n'
           'int main(void){ fused_proj_desc d; split_rope_desc e; (void)d; (void)e; return 0; }\n')
    r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
                        "-x", "c", "-", "-fsyntax-only"], input=src, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_desc_struct_layout_matches_c():
    src = ('#include <stdio.h>\n#include <stddef.h>\n#include "fused_proj.h"\n'
           'int main(void){printf("%zu %zu %zu %zu\\n", sizeof(fused_proj_desc), '
           'offsetof(fused_proj_desc, rope_base), offsetof(fused_proj_desc, x_stride_spatial), '
           'offsetof(fused_proj_desc, pos_offset)); return 0;}\n')
    exe = os.path.join("/tmp", f"fp_desc_layout_{os.getpid()}")
    r = subprocess.run(["gcc", "-std=c99", "-I", os.path.join(ROOT, "include"), "-x", "c", "-", "-o", exe],
                       input=src, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    vals = list(map(int, subprocess.run([exe], capture_output=True, text=True).stdout.split()))
    os.remove(exe)
    assert vals == [ctypes.sizeof(Desc), Desc.rope_base.offset, Desc.x_stride_spatial.offset,
                    Desc.pos_offset.offset]


def test_split_rope_desc_layout_matches_c():
    src = ('#include <stdio.h>\n#include <stddef.h>\n#include "split_rope.h"\n'
           'int main(void){printf("%zu %zu %zu %zu\\n", sizeof(split_rope_desc), '
           'offsetof(split_rope_desc, rope_base), offsetof(split_rope_desc, rope_dims), '
           'offsetof(split_rope_desc, k_transposed)); return 0;}\n')
    exe = os.path.join("/tmp", f"sr_desc_layout_{os.getpid()}")
    r = subprocess.run(["gcc", "-std=c99", "-I", os.path.join(ROOT, "include"), "-x", "c", "-", "-o", exe],
                       input=src, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    vals = list(map(int, subprocess.run([exe], capture_output=True, text=True).stdout.split()))
    os.remove(exe)
    D = fpa.SplitRopeDesc
    assert vals == [ctypes.sizeof(D), D.rope_base.offset, D.rope_dims.offset, D.k_transposed.offset]


@pytest.mark.parametrize("kw,code", [
    (dict(), fpa.OK),
    (dict(k_transposed=True), fpa.OK),
    (dict(n_kv_heads=5), fpa.EINVAL),        # does not divide 16
    (dict(rope_dims=9), fpa.EINVAL),         # odd rotated width
    (dict(rope_dims=64), fpa.EINVAL),        # wider than the head
    (dict(rope_base=0.0), fpa.EINVAL),
    (dict(qkv_order="contiguous", n_kv_heads=16), fpa.OK),
])
def test_split_rope_validate(kw, code):
    base = dict(n_kv_heads=4, qkv_order="grouped", rope_dims=8)
    base.update(kw)
    d = fpa.make_split_rope_desc(2, 1024, 16, 32, **base)
    assert fpa.validate_split_rope(d) == code


def test_split_rope_validate_unsupported():
    d = fpa.make_split_rope_desc(2, 1024, 16, 12)            # head size not a multiple of 8
    assert fpa.validate_split_rope(d) == fpa.EUNSUPPORTED
    d = fpa.make_split_rope_desc(2, 1020, 16, 32, k_transposed=True)   # T not a multiple of 8
    assert fpa.validate_split_rope(d) == fpa.EUNSUPPORTED
    d = fpa.make_split_rope_desc(2, 1024, 16, 32, dtype=__import__("torch").float32)
    assert fpa.validate_split_rope(d) == fpa.EUNSUPPORTED


def walrus_desc(**kw):
    import torch
    shape = (24, 768, 32, 32, 1)
    strides = (768 * 1024, 1024, 32, 1, 1)
    base = dict(w_layout="cf", has_bias=True, ff_dim=3072, ff_act="gelu", n_heads=12, head_dim=64, rope=True)
    base.update(kw)
    return make_desc(shape, strides, "channels_first", torch.bfloat16, **base)


def test_validate_accepts_all_benchmark_workloads():
    import torch
    from ff_input_projection_amd.workloads import WORKLOADS
    for wl in WORKLOADS.values():
        t = torch.empty(wl.x_shape, dtype=torch.bfloat16 if wl.dtype == "bf16" else torch.float32, device="meta")
        d = make_desc(t.shape, t.stride(), wl.layout, t.dtype, w_layout=wl.w_layout, has_bias=wl.has_bias,
                      ff_dim=wl.ff_dim, ff_act=wl.ff_act, n_heads=wl.n_heads, head_dim=wl.head_dim, rope=wl.rope)
        assert fpa.validate(d) == fpa.OK, wl.name


def test_validate_accepts_every_activation():
    for act in ("none", "gelu", "gelu_tanh", "relu2"):
        d = walrus_desc(ff_act=act)
        assert fpa.validate(d) == fpa.OK, act


@pytest.mark.parametrize("mutate,code", [
    (lambda d: setattr(d, "dtype", 7), fpa.EINVAL),
    (lambda d: setattr(d, "x_layout", 5), fpa.EINVAL),
    (lambda d: setattr(d, "w_layout", 2), fpa.EINVAL),
    (lambda d: setattr(d, "ff_act", 9), fpa.EINVAL),
    (lambda d: setattr(d, "n_kv_heads", 5), fpa.EINVAL),     # does not divide 12 q heads
    (lambda d: setattr(d, "n_kv_heads", -1), fpa.EINVAL),
    (lambda d: setattr(d, "qkv_order", 2), fpa.EINVAL),
    (lambda d: setattr(d, "rope_dims", 7), fpa.EINVAL),      # odd rotated width
    (lambda d: setattr(d, "rope_dims", 128), fpa.EINVAL),    # wider than the 64-element head
    (lambda d: setattr(d, "ff_layout", 2), fpa.EINVAL),
    (lambda d: setattr(d, "batch", -1), fpa.EINVAL),
    (lambda d: setattr(d, "n_spatial", 4), fpa.EINVAL),
    (lambda d: setattr(d, "head_dim", 0), fpa.EINVAL),             # heads without width
    (lambda d: (setattr(d, "ff_dim", 0), setattr(d, "n_heads", 0), setattr(d, "head_dim", 0)), fpa.EINVAL),
    (lambda d: setattr(d, "rope_base", 0.0), fpa.EINVAL),
    (lambda d: setattr(d, "pos_offset", -3), fpa.EINVAL),
    (lambda d: setattr(d, "x_stride_channel", -1024), fpa.EINVAL),
    (lambda d: setattr(d, "channels", 764), fpa.EUNSUPPORTED),      # C not a multiple of 8 (bf16)
    (lambda d: setattr(d, "ff_dim", 3076), fpa.EUNSUPPORTED),       # ff not a multiple of 8
    (lambda d: setattr(d, "ff_dim", 3104), fpa.EUNSUPPORTED),       # ff not a multiple of hd (RoPE)
    (lambda d: setattr(d, "head_dim", 24), fpa.EUNSUPPORTED),       # hd/2 not a multiple of 8
    (lambda d: setattr(d, "head_dim", 96), fpa.EUNSUPPORTED),       # a 128-wide tile cannot hold whole heads
    (lambda d: d.x_stride_spatial.__setitem__(0, 33), fpa.EUNSUPPORTED),  # spatial dims do not flatten
    (lambda d: setattr(d, "x_stride_channel", 1020), fpa.EUNSUPPORTED),   # misaligned channel stride
    (lambda d: setattr(d, "batch", 1 << 22), fpa.EUNSUPPORTED),     # more than 2^31 tokens
])
def test_validate_error_codes(mutate, code):
    d = walrus_desc()
    assert fpa.validate(d) == fpa.OK
    mutate(d)
    assert fpa.validate(d) == code


def test_validate_accepts_edge_shapes():
    import torch
    # odd head_dim is fine without RoPE only if it is a multiple of 8; hd=24 without RoPE is supported
    d = walrus_desc(rope=False, head_dim=24, ff_dim=3072)
    assert fpa.validate(d) == fpa.OK
    # empty batch: a valid no-op
    d = walrus_desc()
    d.batch = 0
    assert fpa.validate(d) == fpa.OK
    # fp32 allows 4-wide vectors: hd 8 with RoPE
    d = make_desc((1, 32, 8, 8, 1), (2048, 64, 8, 1, 1), "channels_first", torch.float32, has_bias=True,
                  ff_dim=128, ff_act="gelu", n_heads=4, head_dim=8, rope=True)
    assert fpa.validate(d) == fpa.OK
    # token-major with a row stride larger than C (a channel slice of a wider tensor)
    d = make_desc((2, 100, 64), (100 * 96, 96, 1), "tokens_last", torch.bfloat16, ff_dim=64)
    assert fpa.validate(d) == fpa.OK


@pytest.mark.parametrize("shape,strides,layout", [
    ((2, 0, 8, 8, 1), (0, 0, 0, 0, 0), "channels_first"),    # an empty array's strides
    ((2, 0, 8, 8, 1), (64, 64, 8, 1, 1), "channels_first"),
    ((3, 40, 0), (0, 0, 0), "tokens_last"),
    ((0, 64, 8, 8, 1), (0, 0, 0, 0, 0), "channels_first"),   # no tokens
])
def test_validate_ignores_the_strides_of_an_empty_x(shape, strides, layout):
    """x is read only when it holds elements (C > 0 and b*S > 0); an empty x passes with
    whatever non-negative strides it reports, while a non-empty x with all-zero strides is
    refused and a negative stride is malformed either way."""
    import torch
    kw = dict(has_bias=True, ff_dim=64, ff_act="gelu", n_heads=2, head_dim=32, rope=True)
    assert fpa.validate(make_desc(shape, strides, layout, torch.bfloat16, **kw)) == fpa.OK
    if not any(strides):
        full = tuple(8 if n == 0 else n for n in shape)
        assert fpa.validate(make_desc(full, strides, layout, torch.bfloat16, **kw)) == fpa.EUNSUPPORTED
    neg = (-1,) + tuple(strides[1:])
    assert fpa.validate(make_desc(shape, neg, layout, torch.bfloat16, **kw)) == fpa.EINVAL


def test_null_handles_and_strerror():
    lib = fpa.load_library()
    assert lib.fused_proj_validate(None) == fpa.EINVAL
    assert lib.fused_proj_destroy(None) == fpa.OK
    assert lib.fused_proj_run(None, None, None, None, None, None, None, None, None) == fpa.EINVAL
    assert lib.fused_proj_create(ctypes.byref(walrus_desc()), None) == fpa.EINVAL
    buf = ctypes.create_string_buffer(16)
    assert lib.fused_proj_describe(None, buf, 16) == fpa.EINVAL
    for code in (0, -1, -2, -3, -4):
        assert len(fpa.strerror(code)) > 3
    assert "unknown" in fpa.strerror(42)


def test_mfma_ceiling_rejects_bad_arguments():
    """The calibration call checks its arguments before touching a device."""
    import ctypes

    lib = fpa.load_library()
    sink = (ctypes.c_float * 16)()
    flops = ctypes.c_double(-1.0)
    # no iterations, no flop counter, no sink
    assert lib.fused_proj_mfma_ceiling(0, 1, ctypes.cast(sink, ctypes.c_void_p), 64, None, ctypes.byref(flops)) == \
        fpa.EINVAL
    assert lib.fused_proj_mfma_ceiling(10, 1, ctypes.cast(sink, ctypes.c_void_p), 64, None, None) == fpa.EINVAL
    assert lib.fused_proj_mfma_ceiling(10, 1, None, 64, None, ctypes.byref(flops)) == fpa.EINVAL
    assert flops.value == -1.0


def test_product_path_fails_loudly_without_the_library_and_never_imports_the_oracle():
    """With the HIP library absent, planning raises (there is no CPU fallback); importing
    the package and planning bring in nothing from oracle/. Run in a fresh interpreter."""
    import subprocess
    import sys
    code = r"""
import sys
import ff_input_projection_amd as fpa
fpa.LIB_PATH = "/nonexistent/libfused_proj.so"
fpa._lib = None
import torch
try:
    fpa.FusedProjection((1, 8, 8), (64, 8, 1), "tokens_last", torch.bfloat16, ff_dim=8)
except RuntimeError as e:
    assert "no CPU fallback" in str(e), e
else:
    raise SystemExit("planning without the library did not raise")
try:
    fpa.SplitRope(1, 8, 1, 8)
except RuntimeError as e:
    assert "no CPU fallback" in str(e), e
else:
    raise SystemExit("split+RoPE without the library did not raise")
assert not any(m == "oracle" or m.startswith("oracle.") for m in sys.modules), "the package imported the oracle"
print("ok")
"""
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, "-c", code], cwd=root, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stdout + r.stderr
