"""Thin ctypes binding over libnpa.so (the C ABI declared in include/npa.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI.  PyTorch supplies device memory and the current
stream.  If the library is missing or fails to load, every call raises --
there is no fallback.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
from ctypes import POINTER, c_float, c_int32, c_int64, c_void_p
from typing import Optional, Sequence, Tuple

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libnpa.so")

NPA_OK = 0
NPA_ERR_INVALID_ARG = -1
NPA_ERR_SHAPE = -2
NPA_ERR_UNSUPPORTED = -3
NPA_ERR_HIP = -4
NPA_F32, NPA_BF16 = 0, 1
NPA_MODE_STRIPS, NPA_MODE_WINDOW = 0, 1

# Every symbol include/npa.h declares.
EXPORTED = ("npa_attn_fwd", "npa_plan", "npa_useful_flops", "npa_sg_blend", "npa_asg_blend", "npa_last_error")


class Layout(ctypes.Structure):
    _fields_ = [
        ("batch", c_int32), ("heads", c_int32), ("head_dim", c_int32),
        ("map_h", c_int32), ("map_w", c_int32),
        ("stride_b", c_int64), ("stride_n", c_int64), ("stride_h", c_int64),
        ("dtype", c_int32), ("scale", c_float),
    ]


class Halo(ctypes.Structure):
    _fields_ = [
        ("mode", c_int32), ("num_strips", c_int32), ("p", c_float), ("halo_rows", c_int32),
        ("tile_h", c_int32), ("tile_w", c_int32), ("halo_h", c_int32), ("halo_w", c_int32),
        ("text_tokens", c_int32),
    ]


class Segment(ctypes.Structure):
    _fields_ = [("src", c_int32), ("start", c_int32), ("row_len", c_int32), ("rows", c_int32), ("pitch", c_int32)]


class TileDesc(ctypes.Structure):
    _fields_ = [("queries", Segment), ("n_segments", c_int32), ("keys", Segment * 3)]


class NpaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"npa status {status}: {msg}")
        self.status = status


_lib = None


def load(build_if_missing: bool = True):
    """Load libnpa.so (building it in-tree first only if no library exists)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        if not build_if_missing:
            raise RuntimeError(f"{LIB_PATH} is missing; build it with partial_context_patch_amd.build")
        from . import build as _build

        _build.build()
    lib = ctypes.CDLL(LIB_PATH)
    lib.npa_attn_fwd.restype = c_int32
    lib.npa_attn_fwd.argtypes = [c_void_p] * 5 + [POINTER(Layout), POINTER(Halo), c_void_p, c_void_p]
    lib.npa_plan.restype = c_int32
    lib.npa_plan.argtypes = [POINTER(Layout), POINTER(Halo), POINTER(TileDesc), c_int32, POINTER(c_int32), POINTER(c_int64)]
    lib.npa_useful_flops.restype = c_int64
    lib.npa_useful_flops.argtypes = [POINTER(Layout), POINTER(Halo)]
    lib.npa_sg_blend.restype = c_int32
    lib.npa_sg_blend.argtypes = [c_void_p, c_void_p, c_void_p, c_int32, c_int32, c_int32, c_int32, c_float, c_float, c_void_p]
    lib.npa_asg_blend.restype = c_int32
    lib.npa_asg_blend.argtypes = [c_void_p, c_void_p, c_void_p, c_void_p, c_int64, c_float, c_void_p]
    lib.npa_last_error.restype = ctypes.c_char_p
    lib.npa_last_error.argtypes = []
    _lib = lib
    return lib


def _check(status: int):
    if status != NPA_OK:
        raise NpaError(status, load().npa_last_error().decode())


def make_halo(*, strips: Optional[int] = None, p: Optional[float] = None, halo_rows: Optional[int] = None,
              tile: Optional[Tuple[int, int]] = None, halo: Optional[Tuple[int, int]] = None,
              text_tokens: int = 0) -> Halo:
    """strips=n with p or halo_rows (partially conditioned strips), or
    tile=(th, tw) with halo=(eh, ew) (neighbourhood windows), optionally with
    text_tokens global tokens stored before the map's tokens."""
    h = Halo()
    h.text_tokens = int(text_tokens)
    if strips is not None:
        if tile is not None:
            raise ValueError("give either strips or tile, not both")
        h.mode = NPA_MODE_STRIPS
        h.num_strips = int(strips)
        h.p = float(p) if p is not None else 0.0
        h.halo_rows = int(halo_rows) if halo_rows is not None else -1
        if p is None and halo_rows is None:
            raise ValueError("strips need p or halo_rows")
    elif tile is not None:
        h.mode = NPA_MODE_WINDOW
        h.tile_h, h.tile_w = (int(x) for x in tile)
        eh, ew = halo if halo is not None else (0, 0)
        h.halo_h, h.halo_w = int(eh), int(ew)
    else:
        raise ValueError("give strips=... or tile=...")
    return h


def make_layout(batch: int, heads: int, head_dim: int, map_h: int, map_w: int, *, dtype: str = "bf16",
                strides: Optional[Sequence[int]] = None, scale: Optional[float] = None) -> Layout:
    L = Layout()
    L.batch, L.heads, L.head_dim, L.map_h, L.map_w = batch, heads, head_dim, map_h, map_w
    if strides is None:
        strides = (map_h * map_w * heads * head_dim, heads * head_dim, head_dim)
    L.stride_b, L.stride_n, L.stride_h = (int(s) for s in strides)
    L.dtype = {"bf16": NPA_BF16, "f32": NPA_F32}[dtype]
    L.scale = float(scale) if scale is not None else 0.0
    return L


def plan(layout: Layout, halo: Halo):
    """Host-only planner: (list of tile dicts, attended pairs per (batch, head))."""
    lib = load()
    n = c_int32()
    pairs = c_int64()
    _check(lib.npa_plan(ctypes.byref(layout), ctypes.byref(halo), None, 0, ctypes.byref(n), ctypes.byref(pairs)))
    arr = (TileDesc * max(1, n.value))()
    _check(lib.npa_plan(ctypes.byref(layout), ctypes.byref(halo), arr, n.value, ctypes.byref(n), ctypes.byref(pairs)))

    def seg(s):
        return dict(src=s.src, start=s.start, row_len=s.row_len, rows=s.rows, pitch=s.pitch)

    tiles = [dict(queries=seg(t.queries), keys=[seg(t.keys[i]) for i in range(t.n_segments)]) for t in arr[: n.value]]
    return tiles, pairs.value


def useful_flops(layout: Layout, halo: Halo) -> int:
    v = load().npa_useful_flops(ctypes.byref(layout), ctypes.byref(halo))
    if v < 0:
        _check(NPA_ERR_INVALID_ARG)
    return v


def _stream_ptr(device) -> int:
    import torch

    return torch.cuda.current_stream(device).cuda_stream


def _on(device):
    """Make `device` current for the call (the library launches on the current
    device); a no-op context when it already is, which is the common case."""
    import torch

    if device.index is None or device.index == torch.cuda.current_device():
        return contextlib.nullcontext()
    return torch.cuda.device(device)


def attn_fwd(q, k, v, k_stale=None, v_stale=None, *, map_hw: Tuple[int, int], strips: Optional[int] = None,
             p: Optional[float] = None, halo_rows: Optional[int] = None, tile: Optional[Tuple[int, int]] = None,
             halo: Optional[Tuple[int, int]] = None, text_tokens: int = 0, scale: Optional[float] = None, out=None):
    """Partial attention over device tensors [batch, tokens, heads, head_dim].

    All tensors share one dtype (bfloat16 or float32), one device and one set of
    strides, with head_dim contiguous; tokens = text_tokens + map_h * map_w
    (text tokens first).  Returns `out` (allocated if None).
    """
    import torch

    lib = load()
    if q.dim() != 4:
        raise ValueError("q must be [batch, tokens, heads, head_dim]")
    B, N, Hh, d = q.shape
    H, W = map_hw
    if text_tokens + H * W != N:
        raise ValueError(f"{text_tokens} text tokens and a {H}x{W} map do not match {N} tokens")
    dt = {torch.bfloat16: "bf16", torch.float32: "f32"}.get(q.dtype)
    if dt is None:
        raise TypeError("q must be bfloat16 or float32")
    if out is None:
        out = torch.empty_strided(q.shape, q.stride(), dtype=q.dtype, device=q.device)
    ts = [t for t in (q, k, v, k_stale, v_stale, out) if t is not None]
    for t in ts:
        if not t.is_cuda or t.device != q.device:
            raise ValueError("all tensors must live on q's GPU")
        if t.dtype != q.dtype or tuple(t.shape) != tuple(q.shape):
            raise ValueError("all tensors must share q's dtype and shape")
        if t.stride() != q.stride() or t.stride(-1) != 1:
            raise ValueError("all tensors must share q's strides with head_dim contiguous")
    L = make_layout(B, Hh, d, H, W, dtype=dt, strides=q.stride()[:3], scale=scale)
    h = make_halo(strips=strips, p=p, halo_rows=halo_rows, tile=tile, halo=halo, text_tokens=text_tokens)
    ptr = lambda t: None if t is None else t.data_ptr()
    # the library launches on the current device, on that device's current stream
    with _on(q.device):
        _check(lib.npa_attn_fwd(ptr(q), ptr(k), ptr(v), ptr(k_stale), ptr(v_stale), ctypes.byref(L),
                                ctypes.byref(h), ptr(out), _stream_ptr(q.device)))
    return out


def sg_blend(x, ref, w_t: float, sigma: float, out=None):
    """out = x + w_t * (G_sigma*ref - G_sigma*x) on fp32 [n, c, h, w] device tensors."""
    import torch

    lib = load()
    if x.dim() != 4 or x.shape != ref.shape:
        raise ValueError("x and ref must be [n, c, h, w] of one shape")
    if out is None:
        out = torch.empty_like(x)
    for t in (x, ref, out):
        if t.dtype != torch.float32 or not t.is_contiguous() or not t.is_cuda or t.device != x.device:
            raise ValueError("x, ref, out must be contiguous fp32 tensors on one GPU")
    if out.shape != x.shape:
        raise ValueError("out must have x's shape")
    n, c, h, w = x.shape
    with _on(x.device):
        _check(lib.npa_sg_blend(x.data_ptr(), ref.data_ptr(), out.data_ptr(), n, c, h, w, float(w_t), float(sigma),
                                _stream_ptr(x.device)))
    return out


def asg_blend(eps, eps_ref_prev, mask, w_t: float, out=None):
    """out = eps + w_t * mask * (eps_ref_prev - eps), element-wise on fp32 device tensors."""
    import torch

    lib = load()
    if out is None:
        out = torch.empty_like(eps)
    for t in (eps, eps_ref_prev, mask, out):
        if (t.dtype != torch.float32 or not t.is_contiguous() or not t.is_cuda or t.shape != eps.shape
                or t.device != eps.device):
            raise ValueError("eps, eps_ref_prev, mask, out must be contiguous fp32 tensors of one shape on one GPU")
    with _on(eps.device):
        _check(lib.npa_asg_blend(eps.data_ptr(), eps_ref_prev.data_ptr(), mask.data_ptr(), out.data_ptr(),
                                 eps.numel(), float(w_t), _stream_ptr(eps.device)))
    return out
