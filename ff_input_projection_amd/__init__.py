"""MI355X (gfx950) fused input projection.

Python binding over the C ABI in ``include/fused_proj.h`` (``libfused_proj.so``,
built in-tree by ``ff_input_projection_amd.build``). It only marshals
arguments: every step of the projection runs in the HIP kernels. PyTorch is used
for device memory (output allocation) and for the current HIP stream.

The op (Walrus PR "Make fused_ff_qkv contiguous"; xformers PR "Fused linear:
small FW cleanup and much better perfs"): gather token rows of a
channels-first [b,c,h,w,d] or token-major [b,s,c] activation without a copy,
y = x W + b as one GEMM, GELU on the ff slice, q/k/v split into head-major
[b*H, S, hd] buffers, rotate-half RoPE on q and k.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = ["FusedProjection", "FusedProjError", "SplitRope", "load_library", "LIB_PATH", "EXPORTED_SYMBOLS", "Desc",
           "SplitRopeDesc"]

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libfused_proj.so")

EXPORTED_SYMBOLS = ["fused_proj_validate", "fused_proj_create", "fused_proj_run", "fused_proj_destroy",
                    "fused_proj_strerror", "fused_proj_describe", "fused_proj_backward_workspace_size",
                    "fused_proj_backward", "fused_proj_backward_noalloc", "fused_proj_noalloc_scratch_bytes",
                    "split_rope_validate", "split_rope_create", "split_rope_run", "split_rope_destroy",
                    "fused_proj_mfma_ceiling"]

OK, EINVAL, EUNSUPPORTED, EALIGN, EALIAS, EHIP, ESCRATCH = 0, -1, -2, -3, -4, -5, -6
BF16, F32 = 0, 1
X_CHANNELS_FIRST, X_TOKENS_LAST = 0, 1
W_CF, W_FC = 0, 1
ACT_NONE, ACT_GELU_ERF, ACT_GELU_TANH, ACT_RELU_SQUARED = 0, 1, 2, 3
QKV_CONTIGUOUS, QKV_GROUPED = 0, 1


class Desc(ctypes.Structure):
    """Mirror of ``fused_proj_desc``."""
    _fields_ = [
        ("dtype", ctypes.c_int32), ("x_layout", ctypes.c_int32),
        ("batch", ctypes.c_int64), ("channels", ctypes.c_int64),
        ("n_spatial", ctypes.c_int32), ("spatial", ctypes.c_int64 * 3),
        ("x_stride_batch", ctypes.c_int64), ("x_stride_channel", ctypes.c_int64),
        ("x_stride_spatial", ctypes.c_int64 * 3),
        ("w_layout", ctypes.c_int32), ("has_bias", ctypes.c_int32),
        ("ff_dim", ctypes.c_int64), ("ff_act", ctypes.c_int32),
        ("n_heads", ctypes.c_int64), ("head_dim", ctypes.c_int64),
        ("rope", ctypes.c_int32), ("rope_base", ctypes.c_double), ("pos_offset", ctypes.c_int64),
        ("n_kv_heads", ctypes.c_int64), ("qkv_order", ctypes.c_int32), ("rope_dims", ctypes.c_int64),
        ("ff_layout", ctypes.c_int32),
    ]


class SplitRopeDesc(ctypes.Structure):
    """Mirror of ``split_rope_desc``."""
    _fields_ = [
        ("dtype", ctypes.c_int32), ("batch", ctypes.c_int64), ("tokens", ctypes.c_int64),
        ("n_heads", ctypes.c_int64), ("n_kv_heads", ctypes.c_int64), ("head_dim", ctypes.c_int64),
        ("qkv_order", ctypes.c_int32), ("rope", ctypes.c_int32), ("rope_dims", ctypes.c_int64),
        ("rope_base", ctypes.c_double), ("pos_offset", ctypes.c_int64), ("k_transposed", ctypes.c_int32),
    ]


class FusedProjError(RuntimeError):
    def __init__(self, code: int, what: str):
        self.code = code
        super().__init__(f"{what}: {strerror(code)} (code {code})")


_lib = None


def load_library():
    """Load libfused_proj.so; raises if it has not been built (no fallback path exists)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m ff_input_projection_amd.build` "
                           "(there is no CPU fallback)")
    lib = ctypes.CDLL(LIB_PATH)
    _check_single_hip_runtime()
    vp = ctypes.c_void_p
    lib.fused_proj_validate.argtypes = [ctypes.POINTER(Desc)]
    lib.fused_proj_validate.restype = ctypes.c_int
    lib.fused_proj_create.argtypes = [ctypes.POINTER(Desc), ctypes.POINTER(vp)]
    lib.fused_proj_create.restype = ctypes.c_int
    lib.fused_proj_run.argtypes = [vp] * 9
    lib.fused_proj_run.restype = ctypes.c_int
    lib.fused_proj_destroy.argtypes = [vp]
    lib.fused_proj_destroy.restype = ctypes.c_int
    lib.fused_proj_strerror.argtypes = [ctypes.c_int]
    lib.fused_proj_strerror.restype = ctypes.c_char_p
    lib.fused_proj_describe.argtypes = [vp, ctypes.c_char_p, ctypes.c_size_t]
    lib.fused_proj_describe.restype = ctypes.c_int
    lib.fused_proj_backward_workspace_size.argtypes = [vp, ctypes.POINTER(ctypes.c_size_t)]
    lib.fused_proj_backward_workspace_size.restype = ctypes.c_int
    lib.fused_proj_backward.argtypes = [vp] * 12 + [ctypes.c_size_t, vp]
    lib.fused_proj_backward.restype = ctypes.c_int
    lib.fused_proj_backward_noalloc.argtypes = [vp] * 12
    lib.fused_proj_backward_noalloc.restype = ctypes.c_int
    lib.fused_proj_noalloc_scratch_bytes.argtypes = []
    lib.fused_proj_noalloc_scratch_bytes.restype = ctypes.c_size_t
    lib.split_rope_validate.argtypes = [ctypes.POINTER(SplitRopeDesc)]
    lib.split_rope_validate.restype = ctypes.c_int
    lib.split_rope_create.argtypes = [ctypes.POINTER(SplitRopeDesc), ctypes.POINTER(vp)]
    lib.split_rope_create.restype = ctypes.c_int
    lib.split_rope_run.argtypes = [vp] * 6
    lib.split_rope_run.restype = ctypes.c_int
    lib.split_rope_destroy.argtypes = [vp]
    lib.split_rope_destroy.restype = ctypes.c_int
    lib.fused_proj_mfma_ceiling.argtypes = [ctypes.c_int, ctypes.c_uint, vp, ctypes.c_size_t, vp,
                                            ctypes.POINTER(ctypes.c_double)]
    lib.fused_proj_mfma_ceiling.restype = ctypes.c_int
    _lib = lib
    return lib


def _check_single_hip_runtime():
    # torch ships its own libamdhip64 (same SONAME). torch is imported before the
    # library is opened, so the loader binds the library to torch's runtime: one
    # runtime owns the streams and the memory both sides use. Two mapped copies
    # would mean two runtimes, whose handles must never be mixed.
    try:
        with open("/proc/self/maps") as f:
            paths = {l.split()[-1] for l in f if "libamdhip64" in l}
    except OSError:
        return
    real = {os.path.realpath(p) for p in paths}
    if len(real) > 1:
        raise RuntimeError(f"two HIP runtimes are loaded ({sorted(real)}); import torch before "
                           "ff_input_projection_amd")


def strerror(code: int) -> str:
    return load_library().fused_proj_strerror(code).decode()


def mfma_ceiling_launch(iterations: int, sink: torch.Tensor, stream=None, seed: int = 12345) -> float:
    """Enqueues one launch of the MFMA-only calibration kernel (fused_proj_mfma_ceiling)
    on `stream` (default: the current stream of sink's device); returns its flop count.
    sink: a float32 device tensor of at least CUs * 256 elements."""
    lib = load_library()
    if stream is None:
        stream = torch.cuda.current_stream(sink.device)
    flops = ctypes.c_double(0.0)
    rc = lib.fused_proj_mfma_ceiling(int(iterations), int(seed) & 0xFFFFFFFF, ctypes.c_void_p(sink.data_ptr()),
                                     sink.numel() * sink.element_size(), ctypes.c_void_p(stream.cuda_stream),
                                     ctypes.byref(flops))
    if rc != OK:
        raise FusedProjError(rc, "fused_proj_mfma_ceiling")
    return flops.value


_DTYPES = {torch.bfloat16: BF16, torch.float32: F32}


def make_desc(x_shape, x_strides, layout: str, dtype: torch.dtype, *, w_layout: str = "cf",
              has_bias: bool = False, ff_dim: int = 0, ff_act: str = "none", n_heads: int = 0,
              head_dim: int = 0, rope: bool = False, rope_base: float = 10000.0, pos_offset: int = 0,
              n_kv_heads: int = 0, qkv_order: str = "contiguous", rope_dims: int = 0,
              ff_layout: str = "tokens_last") -> Desc:
    """Descriptor from an activation's shape and element strides.
    layout "channels_first": x [b, c, spatial...] (1-3 spatial dims);
    layout "tokens_last": x [b, s, c]."""
    d = Desc()
    d.dtype = _DTYPES[dtype]
    if layout == "channels_first":
        d.x_layout = X_CHANNELS_FIRST
        sp, sps = x_shape[2:], x_strides[2:]
        d.batch, d.channels = x_shape[0], x_shape[1]
        d.x_stride_batch, d.x_stride_channel = x_strides[0], x_strides[1]
    elif layout == "tokens_last":
        d.x_layout = X_TOKENS_LAST
        sp, sps = x_shape[1:2], x_strides[1:2]
        d.batch, d.channels = x_shape[0], x_shape[2]
        d.x_stride_batch, d.x_stride_channel = x_strides[0], x_strides[2]
    else:
        raise ValueError(f"unknown layout {layout!r}")
    d.n_spatial = len(sp)
    for i, (n, st) in enumerate(zip(sp, sps)):
        d.spatial[i] = n
        d.x_stride_spatial[i] = st
    d.w_layout = {"cf": W_CF, "fc": W_FC}[w_layout]
    d.has_bias = int(bool(has_bias))
    d.ff_dim = ff_dim
    d.ff_act = {"none": ACT_NONE, "gelu": ACT_GELU_ERF, "gelu_tanh": ACT_GELU_TANH, "relu2": ACT_RELU_SQUARED}[ff_act]
    d.n_heads, d.head_dim = n_heads, head_dim
    d.rope, d.rope_base, d.pos_offset = int(bool(rope)), float(rope_base), pos_offset
    d.n_kv_heads = n_kv_heads
    d.qkv_order = {"contiguous": QKV_CONTIGUOUS, "grouped": QKV_GROUPED}[qkv_order]
    d.rope_dims = rope_dims
    d.ff_layout = {"tokens_last": 0, "channels_first": 1}[ff_layout]
    return d


def validate(desc: Desc) -> int:
    return load_library().fused_proj_validate(ctypes.byref(desc))


class FusedProjection:
    """One planned fused projection (owns the plan and its RoPE table).

    Call with device tensors ``x`` (shape/strides/dtype as planned), ``w``
    ([C,F] or [F,C]) and optional ``bias`` [F]; returns ``(ff, q, k, v)`` with
    ``None`` for empty slices. Outputs may be passed in; missing ones are
    allocated with ``torch.empty`` on x's device. The launch goes to torch's
    current stream (or ``stream``) and is asynchronous.
    """

    def __init__(self, x_shape, x_strides, layout: str, dtype: torch.dtype, **kw):
        self._lib = load_library()
        self.desc = make_desc(tuple(x_shape), tuple(x_strides), layout, dtype, **kw)
        self.x_shape, self.x_strides, self.layout, self.dtype = tuple(x_shape), tuple(x_strides), layout, dtype
        self.w_layout = kw.get("w_layout", "cf")
        d = self.desc
        self.S = 1
        for i in range(d.n_spatial):
            self.S *= d.spatial[i]
        self.B, self.C = d.batch, d.channels
        self.H, self.hd, self.ff_dim = d.n_heads, d.head_dim, d.ff_dim
        self.KVH = d.n_kv_heads if d.n_kv_heads > 0 else d.n_heads
        self.ff_channels_first = d.ff_layout == 1
        self.F = d.ff_dim + (d.n_heads + 2 * self.KVH) * d.head_dim
        self.has_bias = bool(d.has_bias)
        h = ctypes.c_void_p()
        rc = self._lib.fused_proj_create(ctypes.byref(self.desc), ctypes.byref(h))
        if rc != OK:
            raise FusedProjError(rc, "fused_proj_create")
        self._h = h

    @classmethod
    def for_tensor(cls, x: torch.Tensor, layout: str, **kw) -> "FusedProjection":
        return cls(x.shape, x.stride(), layout, x.dtype, **kw)

    def describe(self) -> str:
        buf = ctypes.create_string_buffer(512)
        self._lib.fused_proj_describe(self._h, buf, 512)
        return buf.value.decode()

    def out_shapes(self):
        """(ff, q, kv) shapes: ff [b, S, ff_dim] (or [b, ff_dim, S]), q [b*H, S, hd], k and v
        [b*KVH, S, hd]."""
        ff = None
        if self.ff_dim > 0:
            ff = (self.B, self.ff_dim, self.S) if self.ff_channels_first else (self.B, self.S, self.ff_dim)
        q = (self.B * self.H, self.S, self.hd) if self.H * self.hd > 0 else None
        kv = (self.B * self.KVH, self.S, self.hd) if self.H * self.hd > 0 else None
        return ff, q, kv

    def alloc_outputs(self, device):
        ffs, qs, kvs = self.out_shapes()
        mk = lambda s: None if s is None else torch.empty(s, dtype=self.dtype, device=device)
        return mk(ffs), mk(qs), mk(kvs), mk(kvs)

    def __call__(self, x: torch.Tensor, w: torch.Tensor, bias: torch.Tensor | None = None,
                 out=None, stream: torch.cuda.Stream | None = None):
        if tuple(x.shape) != self.x_shape or tuple(x.stride()) != self.x_strides:
            raise ValueError(f"x has shape {tuple(x.shape)} strides {tuple(x.stride())}; "
                             f"planned for {self.x_shape} / {self.x_strides}")
        for name, t in (("x", x), ("w", w), ("bias", bias)):
            if t is not None and (t.dtype != self.dtype or not t.is_cuda):
                raise TypeError(f"{name} must be a {self.dtype} GPU tensor")
        wshape = (self.C, self.F) if self.w_layout == "cf" else (self.F, self.C)
        if tuple(w.shape) != wshape or not w.is_contiguous():
            raise ValueError(f"w must be contiguous {wshape}")
        if self.has_bias:
            if bias is None or tuple(bias.shape) != (self.F,) or not bias.is_contiguous():
                raise ValueError(f"bias must be a contiguous [{self.F}] tensor")
        ff, q, k, v = out if out is not None else self.alloc_outputs(x.device)
        ffs, qs, kvs = self.out_shapes()
        for t, s in ((ff, ffs), (q, qs), (k, kvs), (v, kvs)):
            if s is not None and (t is None or tuple(t.shape) != s or not t.is_contiguous()
                                  or t.dtype != self.dtype):
                raise ValueError(f"output must be a contiguous {s} {self.dtype} tensor")
        st = stream if stream is not None else torch.cuda.current_stream(x.device)
        p = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
        rc = self._lib.fused_proj_run(self._h, p(x), p(w), p(bias) if self.has_bias else None,
                                      p(ff), p(q), p(k), p(v), ctypes.c_void_p(st.cuda_stream))
        if rc != OK:
            raise FusedProjError(rc, "fused_proj_run")
        return ff, q, k, v

    def run_ptrs(self, x, w, bias, ff, q, k, v, stream_handle: int) -> int:
        """Raw call with integer device addresses (for timing loops); returns the status."""
        c = lambda a: None if a is None else ctypes.c_void_p(a)
        return self._lib.fused_proj_run(self._h, c(x), c(w), c(bias), c(ff), c(q), c(k), c(v),
                                        ctypes.c_void_p(stream_handle))

    # ---------------------------------------------------------------- backward pass
    def workspace_bytes(self) -> int:
        """Device workspace the backward pass needs (fused_proj_backward_workspace_size)."""
        n = ctypes.c_size_t()
        rc = self._lib.fused_proj_backward_workspace_size(self._h, ctypes.byref(n))
        if rc != OK:
            raise FusedProjError(rc, "fused_proj_backward_workspace_size")
        return int(n.value)

    def grad_shapes(self):
        """(dx, dw, db) shapes: dx dense in x's logical shape, dw in W's layout, db [F]."""
        if self.layout == "channels_first":
            dx = (self.B, self.C) + tuple(self.desc.spatial[i] for i in range(self.desc.n_spatial))
        else:
            dx = (self.B, self.S, self.C)
        dw = (self.C, self.F) if self.w_layout == "cf" else (self.F, self.C)
        return dx, dw, ((self.F,) if self.has_bias else None)

    def alloc_grads(self, device):
        mk = lambda s: None if s is None else torch.empty(s, dtype=self.dtype, device=device)
        return tuple(mk(s) for s in self.grad_shapes())

    def backward(self, x: torch.Tensor, w: torch.Tensor, bias: torch.Tensor | None, d_ff=None, dq=None,
                 dk=None, dv=None, out=None, workspace: torch.Tensor | None = None,
                 stream: torch.cuda.Stream | None = None):
        """Gradients (dx, dw, db) of x, W and the bias for upstream gradients shaped like the
        outputs (None for empty slices). Outputs may be passed in; the workspace (uint8
        device tensor of at least workspace_bytes()) is allocated when not given."""
        ffs, qs, kvs = self.out_shapes()
        for name, t, shp in (("d_ff", d_ff, ffs), ("dq", dq, qs), ("dk", dk, kvs), ("dv", dv, kvs)):
            if shp is None:
                continue
            if t is None or tuple(t.shape) != shp or not t.is_contiguous() or t.dtype != self.dtype:
                raise ValueError(f"{name} must be a contiguous {shp} {self.dtype} tensor")
        dx, dw, db = out if out is not None else self.alloc_grads(x.device)
        for t, shp in zip((dx, dw, db), self.grad_shapes()):
            if shp is not None and (t is None or tuple(t.shape) != shp or not t.is_contiguous()
                                    or t.dtype != self.dtype):
                raise ValueError(f"gradient output must be a contiguous {shp} {self.dtype} tensor")
        need = self.workspace_bytes()
        if workspace is None and need > 0:
            workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
        st = stream if stream is not None else torch.cuda.current_stream(x.device)
        p = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
        wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
        rc = self._lib.fused_proj_backward(self._h, p(x), p(w), p(bias) if self.has_bias else None, p(d_ff),
                                           p(dq), p(dk), p(dv), p(dx), p(dw), p(db) if self.has_bias else None,
                                           p(workspace), ctypes.c_size_t(wsb), ctypes.c_void_p(st.cuda_stream))
        if rc != OK:
            raise FusedProjError(rc, "fused_proj_backward")
        return dx, dw, db

    def backward_noalloc(self, x: torch.Tensor, w: torch.Tensor, bias: torch.Tensor | None, d_ff=None, dq=None,
                         dk=None, dv=None, out=None, stream: torch.cuda.Stream | None = None):
        """The backward pass through fused_proj_backward_noalloc: the library's static scratch
        buffer serves as the workspace (nothing is allocated when `out` is given). Calls on
        one GPU share that buffer and must not overlap."""
        ffs, qs, kvs = self.out_shapes()
        for name, t, shp in (("d_ff", d_ff, ffs), ("dq", dq, qs), ("dk", dk, kvs), ("dv", dv, kvs)):
            if shp is not None and (t is None or tuple(t.shape) != shp or not t.is_contiguous()
                                    or t.dtype != self.dtype):
                raise ValueError(f"{name} must be a contiguous {shp} {self.dtype} tensor")
        dx, dw, db = out if out is not None else self.alloc_grads(x.device)
        for t, shp in zip((dx, dw, db), self.grad_shapes()):
            if shp is not None and (t is None or tuple(t.shape) != shp or not t.is_contiguous()
                                    or t.dtype != self.dtype):
                raise ValueError(f"gradient output must be a contiguous {shp} {self.dtype} tensor")
        st = stream if stream is not None else torch.cuda.current_stream(x.device)
        p = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
        rc = self._lib.fused_proj_backward_noalloc(self._h, p(x), p(w), p(bias) if self.has_bias else None,
                                                   p(d_ff), p(dq), p(dk), p(dv), p(dx), p(dw),
                                                   p(db) if self.has_bias else None, ctypes.c_void_p(st.cuda_stream))
        if rc != OK:
            raise FusedProjError(rc, "fused_proj_backward_noalloc")
        return dx, dw, db

    def backward_ptrs(self, x, w, bias, d_ff, dq, dk, dv, dx, dw, db, workspace, workspace_bytes: int,
                      stream_handle: int) -> int:
        """Raw backward call with integer device addresses (for timing loops); returns the status."""
        c = lambda a: None if a is None else ctypes.c_void_p(a)
        return self._lib.fused_proj_backward(self._h, c(x), c(w), c(bias), c(d_ff), c(dq), c(dk), c(dv), c(dx),
                                             c(dw), c(db), c(workspace), ctypes.c_size_t(workspace_bytes),
                                             ctypes.c_void_p(stream_handle))

    def close(self):
        if getattr(self, "_h", None) is not None and self._h.value:
            self._lib.fused_proj_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def make_split_rope_desc(batch: int, tokens: int, n_heads: int, head_dim: int, *, n_kv_heads: int = 0,
                         qkv_order: str = "contiguous", rope: bool = True, rope_dims: int = 0,
                         rope_base: float = 10000.0, pos_offset: int = 0, k_transposed: bool = False,
                         dtype: torch.dtype = torch.bfloat16) -> SplitRopeDesc:
    d = SplitRopeDesc()
    d.dtype = _DTYPES[dtype]
    d.batch, d.tokens, d.n_heads, d.n_kv_heads, d.head_dim = batch, tokens, n_heads, n_kv_heads, head_dim
    d.qkv_order = {"contiguous": QKV_CONTIGUOUS, "grouped": QKV_GROUPED}[qkv_order]
    d.rope, d.rope_dims, d.rope_base, d.pos_offset = int(bool(rope)), rope_dims, float(rope_base), pos_offset
    d.k_transposed = int(bool(k_transposed))
    return d


def validate_split_rope(desc: SplitRopeDesc) -> int:
    return load_library().split_rope_validate(ctypes.byref(desc))


class SplitRope:
    """One planned standalone split + RoPE (owns its cos/sin table; see split_rope.h).

    Call with a contiguous bf16 GPU tensor ``qkv`` [b, T, (H + 2*KVH)*hd]; returns
    ``(q, k, v)``: q [b*H, T, hd], k [b*KVH, T, hd] (or [b*KVH, hd, T] when
    k_transposed), v [b*KVH, T, hd]. Outputs may be passed in; the launch goes to
    torch's current stream (or ``stream``) and is asynchronous.
    """

    def __init__(self, batch: int, tokens: int, n_heads: int, head_dim: int, **kw):
        self._lib = load_library()
        self.desc = make_split_rope_desc(batch, tokens, n_heads, head_dim, **kw)
        self.B, self.T, self.H, self.hd = batch, tokens, n_heads, head_dim
        self.KVH = self.desc.n_kv_heads if self.desc.n_kv_heads > 0 else n_heads
        self.k_transposed = bool(self.desc.k_transposed)
        h = ctypes.c_void_p()
        rc = self._lib.split_rope_create(ctypes.byref(self.desc), ctypes.byref(h))
        if rc != OK:
            raise FusedProjError(rc, "split_rope_create")
        self._h = h

    def shapes(self):
        q = (self.B * self.H, self.T, self.hd)
        kv = (self.B * self.KVH, self.T, self.hd)
        k = (self.B * self.KVH, self.hd, self.T) if self.k_transposed else kv
        return (self.B, self.T, (self.H + 2 * self.KVH) * self.hd), q, k, kv

    def alloc_outputs(self, device):
        _, qs, ks, vs = self.shapes()
        return tuple(torch.empty(s, dtype=torch.bfloat16, device=device) for s in (qs, ks, vs))

    def __call__(self, qkv: torch.Tensor, out=None, stream: torch.cuda.Stream | None = None):
        ins, qs, ks, vs = self.shapes()
        if tuple(qkv.shape) != ins or not qkv.is_contiguous() or qkv.dtype != torch.bfloat16 or not qkv.is_cuda:
            raise ValueError(f"qkv must be a contiguous bf16 GPU tensor of shape {ins}")
        q, k, v = out if out is not None else self.alloc_outputs(qkv.device)
        for t, s in ((q, qs), (k, ks), (v, vs)):
            if tuple(t.shape) != s or not t.is_contiguous() or t.dtype != torch.bfloat16:
                raise ValueError(f"output must be a contiguous bf16 tensor of shape {s}")
        st = stream if stream is not None else torch.cuda.current_stream(qkv.device)
        p = lambda t: ctypes.c_void_p(t.data_ptr())
        rc = self._lib.split_rope_run(self._h, p(qkv), p(q), p(k), p(v), ctypes.c_void_p(st.cuda_stream))
        if rc != OK:
            raise FusedProjError(rc, "split_rope_run")
        return q, k, v

    def run_ptrs(self, qkv, q, k, v, stream_handle: int) -> int:
        c = lambda a: None if a is None else ctypes.c_void_p(a)
        return self._lib.split_rope_run(self._h, c(qkv), c(q), c(k), c(v), ctypes.c_void_p(stream_handle))

    def close(self):
        if getattr(self, "_h", None) is not None and self._h.value:
            self._lib.split_rope_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
