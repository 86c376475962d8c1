"""Python binding of the attn_jvp C-ABI library (fused attention JVP, gfx950).

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libattn_jvp.so``.  The library must have been built
(``python -m attention_jvp_amd.build`` or ``__graft_entry__.build()``);
importing this package does not load it, the first call does, and a missing
library raises instead of falling back to anything else.

Functions named like the C entry points take raw device pointers (ints) and
return the C status; ``fwd`` is the torch-facing convenience that allocates
the outputs with ``torch.empty`` and passes the current HIP stream.
"""

import ctypes
import os

__all__ = [
    "ATTN_JVP_BF16", "ATTN_JVP_FP32", "AttnJvpError", "Layout", "Mask", "Shape",
    "attn_jvp_check", "attn_jvp_check_ex", "attn_jvp_fwd", "attn_jvp_fwd_ex",
    "attn_jvp_fwd_strided", "attn_jvp_status_string", "attn_jvp_tile_shape",
    "attn_jvp_tile_shape_ex", "attn_jvp_visible_tiles", "attn_jvp_fwd_partial",
    "attn_jvp_merge", "attn_jvp_splitkv_plan", "attn_jvp_fwd_splitkv", "exported_symbols",
    "fwd", "fwd_partial", "fwd_splitkv", "merge", "library_path", "load",
    "BwdLayout", "attn_jvp_bwd", "attn_jvp_bwd_check", "attn_jvp_bwd_visible_tiles", "bwd",
    "attn_jvp_fwd_splitkv_noalloc", "NOALLOC_SCRATCH_BYTES", "attn_jvp_fwd_geometry",
]

NOALLOC_SCRATCH_BYTES = 64 << 20

ATTN_JVP_BF16 = 0
ATTN_JVP_FP32 = 1
ATTN_JVP_MASK_FRAME_WINDOW = 1

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libattn_jvp.so"


class AttnJvpError(RuntimeError):
    def __init__(self, status, what=""):
        self.status = status
        super().__init__(f"{what}: attn_jvp status {status} ({attn_jvp_status_string(status)})")


class Mask(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "kind", "frames", "tokens_per_frame", "chunk_frames", "radius_chunks",
        "anchor_first", "anchor_last", "anchor_queries_see_all")]

    @classmethod
    def frame_window(cls, frames, tokens_per_frame, chunk_frames, radius_chunks,
                     anchor_first=1, anchor_last=1, anchor_queries_see_all=0):
        return cls(ATTN_JVP_MASK_FRAME_WINDOW, frames, tokens_per_frame,
                   chunk_frames, radius_chunks, int(anchor_first), int(anchor_last),
                   int(anchor_queries_see_all))


class Layout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64 * 3) for n in ("q", "k", "v", "dq", "dk", "dv", "o", "dout")]


class BwdLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64 * 3) for n in ("q", "k", "v", "o", "go", "gq", "gk", "gv")]


class Shape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "batch", "heads", "seqlen_q", "seqlen_kv", "head_dim_qk", "head_dim_v")]


_lib = None

EXPORTS = ("attn_jvp_fwd", "attn_jvp_fwd_strided", "attn_jvp_fwd_ex", "attn_jvp_check",
           "attn_jvp_check_ex", "attn_jvp_tile_shape", "attn_jvp_tile_shape_ex",
           "attn_jvp_visible_tiles", "attn_jvp_fwd_partial", "attn_jvp_merge",
           "attn_jvp_splitkv_plan", "attn_jvp_fwd_splitkv", "attn_jvp_bwd",
           "attn_jvp_bwd_check", "attn_jvp_bwd_visible_tiles", "attn_jvp_status_string",
           "attn_jvp_build_id", "attn_jvp_fwd_splitkv_noalloc", "attn_jvp_fwd_geometry")


def library_path():
    return os.path.join(_HERE, _LIB_NAME)


def load():
    """Load the built library (once) and declare its signatures."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run `python -m attention_jvp_amd.build`")
    lib = ctypes.CDLL(path)
    # refuse a library built from other sources than the ones beside it
    from .build import source_digest
    lib.attn_jvp_build_id.argtypes = []
    lib.attn_jvp_build_id.restype = ctypes.c_char_p
    built, now = lib.attn_jvp_build_id().decode(), source_digest()
    if built != now:
        raise ImportError(f"{path} was built from other sources (build id {built[:12]}, "
                          f"sources {now[:12]}); rebuild with `python -m attention_jvp_amd.build`")
    vp, i32, f32, i64p = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.POINTER(ctypes.c_int64)
    ptrs10 = [vp] * 6 + [vp, vp, vp, vp]
    lib.attn_jvp_fwd.argtypes = ptrs10 + [i32, i32, i32, i32, f32, i32, ctypes.POINTER(Mask), vp]
    lib.attn_jvp_fwd.restype = i32
    lib.attn_jvp_fwd_strided.argtypes = ptrs10 + [i32, i32, i32, i32, f32, i32,
                                                  ctypes.POINTER(Layout), ctypes.POINTER(Mask), vp]
    lib.attn_jvp_fwd_strided.restype = i32
    lib.attn_jvp_check.argtypes = ptrs10 + [i32, i32, i32, i32, i32,
                                            ctypes.POINTER(Layout), ctypes.POINTER(Mask)]
    lib.attn_jvp_check.restype = i32
    lib.attn_jvp_fwd_ex.argtypes = ptrs10 + [ctypes.POINTER(Shape), f32, i32,
                                             ctypes.POINTER(Layout), ctypes.POINTER(Mask), vp]
    lib.attn_jvp_fwd_ex.restype = i32
    lib.attn_jvp_check_ex.argtypes = ptrs10 + [ctypes.POINTER(Shape), i32,
                                               ctypes.POINTER(Layout), ctypes.POINTER(Mask)]
    lib.attn_jvp_check_ex.restype = i32
    lib.attn_jvp_tile_shape_ex.argtypes = [i32, i32, i32, ctypes.POINTER(i32), ctypes.POINTER(i32)]
    lib.attn_jvp_tile_shape_ex.restype = i32
    lib.attn_jvp_fwd_geometry.argtypes = [ctypes.POINTER(Shape), i32, ctypes.POINTER(Mask),
                                          ctypes.POINTER(i32), ctypes.POINTER(i32)]
    lib.attn_jvp_fwd_geometry.restype = i32
    lib.attn_jvp_fwd_partial.argtypes = ptrs10 + [ctypes.POINTER(Shape), f32, i32,
                                                  ctypes.POINTER(Layout), vp]
    lib.attn_jvp_fwd_partial.restype = i32
    lib.attn_jvp_merge.argtypes = [i32] + [vp] * 8 + [i32] * 5 + [i64p, vp]
    lib.attn_jvp_merge.restype = i32
    sz = ctypes.c_size_t
    lib.attn_jvp_splitkv_plan.argtypes = [ctypes.POINTER(Shape), i32, ctypes.POINTER(Mask),
                                          ctypes.POINTER(i32), ctypes.POINTER(sz)]
    lib.attn_jvp_splitkv_plan.restype = i32
    lib.attn_jvp_fwd_splitkv.argtypes = ptrs10 + [ctypes.POINTER(Shape), f32, i32,
                                                  ctypes.POINTER(Layout), ctypes.POINTER(Mask),
                                                  i32, vp, sz, vp]
    lib.attn_jvp_fwd_splitkv.restype = i32
    lib.attn_jvp_fwd_splitkv_noalloc.argtypes = ptrs10 + [ctypes.POINTER(Shape), f32, i32,
                                                          ctypes.POINTER(Layout),
                                                          ctypes.POINTER(Mask), i32, vp]
    lib.attn_jvp_fwd_splitkv_noalloc.restype = i32
    lib.attn_jvp_bwd.argtypes = [vp] * 10 + [ctypes.POINTER(Shape), f32, i32,
                                             ctypes.POINTER(BwdLayout), ctypes.POINTER(Mask), vp]
    lib.attn_jvp_bwd.restype = i32
    lib.attn_jvp_bwd_check.argtypes = [vp] * 10 + [ctypes.POINTER(Shape), i32,
                                                   ctypes.POINTER(BwdLayout),
                                                   ctypes.POINTER(Mask)]
    lib.attn_jvp_bwd_check.restype = i32
    lib.attn_jvp_tile_shape.argtypes = [i32, i32, ctypes.POINTER(i32), ctypes.POINTER(i32)]
    lib.attn_jvp_tile_shape.restype = i32
    lib.attn_jvp_visible_tiles.argtypes = [i32, i32, i32, ctypes.POINTER(Mask), i64p]
    lib.attn_jvp_visible_tiles.restype = i32
    lib.attn_jvp_bwd_visible_tiles.argtypes = [i32, i32, i32, i32, ctypes.POINTER(Mask), i64p]
    lib.attn_jvp_bwd_visible_tiles.restype = i32
    lib.attn_jvp_status_string.argtypes = [i32]
    lib.attn_jvp_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def exported_symbols():
    """Names of the C entry points the loaded library resolves."""
    lib = load()
    return [n for n in EXPORTS if hasattr(lib, n)]


def _mask_ptr(mask):
    if mask is None:
        return None
    if isinstance(mask, dict):
        mask = Mask.frame_window(**mask)
    return ctypes.pointer(mask)


# ---- C entry points, same names, raw pointers -----------------------------

def attn_jvp_fwd(Q, K, V, dQ, dK, dV, O, dO, LSE, dLSE, B, H, N, d, scale, dtype,
                 mask=None, stream=None):
    return load().attn_jvp_fwd(Q, K, V, dQ, dK, dV, O, dO, LSE, dLSE, B, H, N, d,
                               scale, dtype, _mask_ptr(mask), stream)


def attn_jvp_fwd_strided(Q, K, V, dQ, dK, dV, O, dO, LSE, dLSE, B, H, N, d, scale,
                         dtype, layout, mask=None, stream=None):
    return load().attn_jvp_fwd_strided(Q, K, V, dQ, dK, dV, O, dO, LSE, dLSE, B, H, N,
                                       d, scale, dtype, ctypes.byref(layout),
                                       _mask_ptr(mask), stream)


def attn_jvp_check(Q, K, V, dQ, dK, dV, O, dO, LSE, dLSE, B, H, N, d, dtype, layout,
                   mask=None):
    lay = None if layout is None else ctypes.byref(layout)
    return load().attn_jvp_check(Q, K, V, dQ, dK, dV, O, dO, LSE, dLSE, B, H, N, d,
                                 dtype, lay, _mask_ptr(mask))


def attn_jvp_fwd_ex(Q, K, V, dQ, dK, dV, O, dO, LSE, dLSE, shape, scale, dtype,
                    layout=None, mask=None, stream=None):
    lay = None if layout is None else ctypes.byref(layout)
    return load().attn_jvp_fwd_ex(Q, K, V, dQ, dK, dV, O, dO, LSE, dLSE, ctypes.byref(shape),
                                  scale, dtype, lay, _mask_ptr(mask), stream)


def attn_jvp_check_ex(Q, K, V, dQ, dK, dV, O, dO, LSE, dLSE, shape, dtype, layout=None,
                      mask=None):
    lay = None if layout is None else ctypes.byref(layout)
    return load().attn_jvp_check_ex(Q, K, V, dQ, dK, dV, O, dO, LSE, dLSE,
                                    ctypes.byref(shape), dtype, lay, _mask_ptr(mask))


def attn_jvp_fwd_partial(Q, K, V, dQ, dK, dV, O, dO, LSE, dLSE, shape, scale, dtype,
                         layout=None, stream=None):
    lay = None if layout is None else ctypes.byref(layout)
    return load().attn_jvp_fwd_partial(Q, K, V, dQ, dK, dV, O, dO, LSE, dLSE,
                                       ctypes.byref(shape), scale, dtype, lay, stream)


def attn_jvp_merge(num_parts, O_parts, dO_parts, LSE_parts, dLSE_parts, O, dO, LSE, dLSE,
                   B, H, Lq, d_v, dtype, o_strides=None, stream=None):
    st = None if o_strides is None else (ctypes.c_int64 * 3)(*o_strides)
    return load().attn_jvp_merge(num_parts, O_parts, dO_parts, LSE_parts, dLSE_parts, O, dO,
                                 LSE, dLSE, B, H, Lq, d_v, dtype, st, stream)


def attn_jvp_splitkv_plan(shape, dtype, mask=None, num_splits=0):
    """(num_splits used, workspace bytes) for a split-KV call."""
    ns, ws = ctypes.c_int(num_splits), ctypes.c_size_t()
    st = load().attn_jvp_splitkv_plan(ctypes.byref(shape), dtype, _mask_ptr(mask),
                                      ctypes.byref(ns), ctypes.byref(ws))
    if st != 0:
        raise AttnJvpError(st, "attn_jvp_splitkv_plan")
    return ns.value, ws.value


def attn_jvp_fwd_splitkv(Q, K, V, dQ, dK, dV, O, dO, LSE, dLSE, shape, scale, dtype, layout,
                         mask, num_splits, workspace, workspace_bytes, stream=None):
    lay = None if layout is None else ctypes.byref(layout)
    return load().attn_jvp_fwd_splitkv(Q, K, V, dQ, dK, dV, O, dO, LSE, dLSE,
                                       ctypes.byref(shape), scale, dtype, lay, _mask_ptr(mask),
                                       num_splits, workspace, workspace_bytes, stream)


def attn_jvp_fwd_splitkv_noalloc(Q, K, V, dQ, dK, dV, O, dO, LSE, dLSE, shape, scale, dtype,
                                 layout, mask, num_splits, stream=None):
    lay = None if layout is None else ctypes.byref(layout)
    return load().attn_jvp_fwd_splitkv_noalloc(Q, K, V, dQ, dK, dV, O, dO, LSE, dLSE,
                                               ctypes.byref(shape), scale, dtype, lay,
                                               _mask_ptr(mask), num_splits, stream)


def attn_jvp_bwd(Q, K, V, O, gO, LSE, gQ, gK, gV, delta, shape, scale, dtype, layout=None,
                 mask=None, stream=None):
    lay = None if layout is None else ctypes.byref(layout)
    return load().attn_jvp_bwd(Q, K, V, O, gO, LSE, gQ, gK, gV, delta, ctypes.byref(shape),
                               scale, dtype, lay, _mask_ptr(mask), stream)


def attn_jvp_bwd_check(Q, K, V, O, gO, LSE, gQ, gK, gV, delta, shape, dtype, layout=None,
                       mask=None):
    lay = None if layout is None else ctypes.byref(layout)
    return load().attn_jvp_bwd_check(Q, K, V, O, gO, LSE, gQ, gK, gV, delta,
                                     ctypes.byref(shape), dtype, lay, _mask_ptr(mask))


def attn_jvp_tile_shape_ex(dtype, d_qk, d_v):
    bm, bn = ctypes.c_int(), ctypes.c_int()
    st = load().attn_jvp_tile_shape_ex(dtype, d_qk, d_v, ctypes.byref(bm), ctypes.byref(bn))
    if st != 0:
        raise AttnJvpError(st, "attn_jvp_tile_shape_ex")
    return bm.value, bn.value


def attn_jvp_fwd_geometry(B, H, Lq, Lkv, d_qk, d_v, dtype, mask=None):
    """(block_m, block_n) that attn_jvp_fwd_ex launches for this call."""
    bm, bn = ctypes.c_int(), ctypes.c_int()
    shape = Shape(B, H, Lq, Lkv, d_qk, d_v)
    st = load().attn_jvp_fwd_geometry(ctypes.byref(shape), dtype, _mask_ptr(mask),
                                      ctypes.byref(bm), ctypes.byref(bn))
    if st != 0:
        raise AttnJvpError(st, "attn_jvp_fwd_geometry")
    return bm.value, bn.value


def attn_jvp_tile_shape(dtype, d):
    bm, bn = ctypes.c_int(), ctypes.c_int()
    st = load().attn_jvp_tile_shape(dtype, d, ctypes.byref(bm), ctypes.byref(bn))
    if st != 0:
        raise AttnJvpError(st, "attn_jvp_tile_shape")
    return bm.value, bn.value


def attn_jvp_visible_tiles(N, dtype, d, mask=None):
    bm, _ = attn_jvp_tile_shape(dtype, d)
    out = (ctypes.c_int64 * ((N + bm - 1) // bm))()
    st = load().attn_jvp_visible_tiles(N, dtype, d, _mask_ptr(mask), out)
    if st != 0:
        raise AttnJvpError(st, "attn_jvp_visible_tiles")
    return list(out)


def attn_jvp_bwd_visible_tiles(N, block_rows, tile_rows, keys, mask=None):
    out = (ctypes.c_int64 * ((N + block_rows - 1) // block_rows))()
    st = load().attn_jvp_bwd_visible_tiles(N, block_rows, tile_rows, int(bool(keys)),
                                           _mask_ptr(mask), out)
    if st != 0:
        raise AttnJvpError(st, "attn_jvp_bwd_visible_tiles")
    return list(out)


def attn_jvp_status_string(status):
    return load().attn_jvp_status_string(status).decode()


# ---- torch convenience ----------------------------------------------------
#
# Every tensor the caller hands over (inputs, ``out=`` tensors, the saved lse,
# a workspace) is checked here for shape, dtype, device and, where the C side
# assumes it, contiguity, before any pointer reaches the library: the C entry
# points see raw addresses only and cannot detect a short or misplaced buffer.

def _torch_dtypes():
    import torch
    return {torch.bfloat16: ATTN_JVP_BF16, torch.float32: ATTN_JVP_FP32}


def _strides3(t):
    s = t.stride()
    if s[3] != 1:
        raise ValueError("the last (head) dimension must be contiguous")
    return (s[0], s[1], s[2])


def layout_of(q, k, v, dq, dk, dv, o, do):
    lay = Layout()
    for name, t in zip(("q", "k", "v", "dq", "dk", "dv", "o", "dout"),
                       (q, k, v, dq, dk, dv, o, do)):
        getattr(lay, name)[:] = _strides3(t)
    return lay


def _require_gpu(t, what):
    if not t.is_cuda:
        raise ValueError(f"{what} must be on a GPU device, got {t.device}")


def check_tensor(t, name, shape, dtype, device, contiguous=False):
    """Raise ValueError unless ``t`` is a tensor of this shape, dtype and
    device (and contiguous when asked)."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a tensor, got {type(t).__name__}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def check_qkv(q, k, v, dq, dk, dv):
    """(dtype code, Shape) of a JVP call's inputs; raises on any mismatch of
    shape, dtype or device between them."""
    dtypes = _torch_dtypes()
    if q.dtype not in dtypes:
        raise TypeError(f"unsupported dtype {q.dtype}")
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be 4-d [B, H, L, d]")
    B, H, Lq, dqk = q.shape
    Lkv, dv_ = k.shape[2], v.shape[3]
    if tuple(k.shape) != (B, H, Lkv, dqk) or tuple(v.shape) != (B, H, Lkv, dv_):
        raise ValueError("shapes must be q [B,H,Lq,d_qk], k [B,H,Lkv,d_qk], v [B,H,Lkv,d_v]")
    for t, ref in ((dq, q), (dk, k), (dv, v)):
        if t.shape != ref.shape:
            raise ValueError("each tangent must have its primal's shape")
    for t in (k, v, dq, dk, dv):
        if t.dtype != q.dtype or t.device != q.device:
            raise ValueError("q, k, v, dq, dk, dv must share dtype and device")
    return dtypes[q.dtype], Shape(B, H, Lq, Lkv, dqk, dv_)


def check_fwd_out(out, q, shape, out_dtype=None):
    """Validate ``out = (o, do, lse, dlse)`` of a JVP call: o, do [B, H, Lq,
    d_v] in ``out_dtype`` (q's dtype by default) with a contiguous head dim,
    lse, dlse contiguous float32 [B, H, Lq], all on q's device."""
    import torch
    if len(out) != 4:
        raise ValueError("out must be (o, do, lse, dlse)")
    o, do, lse, dlse = out
    B, H, Lq, dv_ = shape.batch, shape.heads, shape.seqlen_q, shape.head_dim_v
    dt = q.dtype if out_dtype is None else out_dtype
    for name, t in (("o", o), ("do", do)):
        check_tensor(t, name, (B, H, Lq, dv_), dt, q.device)
        _strides3(t)
    for name, t in (("lse", lse), ("dlse", dlse)):
        check_tensor(t, name, (B, H, Lq), torch.float32, q.device, contiguous=True)
    return o, do, lse, dlse


def _alloc_fwd_out(q, shape, dtype):
    import torch
    B, H, Lq, dv_ = shape.batch, shape.heads, shape.seqlen_q, shape.head_dim_v
    o = torch.empty((B, H, Lq, dv_), device=q.device, dtype=dtype)
    do = torch.empty_like(o)
    lse = torch.empty((B, H, Lq), device=q.device, dtype=torch.float32)
    dlse = torch.empty_like(lse)
    return o, do, lse, dlse


def fwd(q, k, v, dq, dk, dv, scale=None, mask=None, out=None):
    """(o, do, lse, dlse) for GPU tensors q [B, H, Lq, d_qk], k [B, H, Lkv,
    d_qk], v [B, H, Lkv, d_v] (bf16 or float32).

    Tangents must have their primal's shape and strides.  ``mask`` is None or
    a frame-window dict/Mask (self-attention, Lq == Lkv).  Outputs o, do
    [B, H, Lq, d_v] and lse, dlse [B, H, Lq] are allocated contiguous unless
    ``out = (o, do, lse, dlse)`` is given.  Runs on the current stream.
    """
    import torch
    dt, shape = check_qkv(q, k, v, dq, dk, dv)
    _require_gpu(q, "q")
    o, do, lse, dlse = (_alloc_fwd_out(q, shape, q.dtype) if out is None
                        else check_fwd_out(out, q, shape))
    lay = layout_of(q, k, v, dq, dk, dv, o, do)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    st = attn_jvp_fwd_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), dq.data_ptr(),
                         dk.data_ptr(), dv.data_ptr(), o.data_ptr(), do.data_ptr(),
                         lse.data_ptr(), dlse.data_ptr(), shape,
                         0.0 if scale is None else float(scale), dt, lay, mask, stream)
    if st != 0:
        raise AttnJvpError(st, "attn_jvp_fwd_ex")
    return o, do, lse, dlse


def fwd_partial(q, k, v, dq, dk, dv, scale=None):
    """float32 partials (o, do, lse, dlse) of the keys given (see
    attn_jvp_fwd_partial): o, do [B, H, Lq, d_v], lse, dlse [B, H, Lq]."""
    import torch
    dt, shape = check_qkv(q, k, v, dq, dk, dv)
    _require_gpu(q, "q")
    o, do, lse, dlse = _alloc_fwd_out(q, shape, torch.float32)
    lay = layout_of(q, k, v, dq, dk, dv, q, dq)     # o / dout strides are ignored
    st = attn_jvp_fwd_partial(q.data_ptr(), k.data_ptr(), v.data_ptr(), dq.data_ptr(),
                              dk.data_ptr(), dv.data_ptr(), o.data_ptr(), do.data_ptr(),
                              lse.data_ptr(), dlse.data_ptr(), shape,
                              0.0 if scale is None else float(scale), dt, lay,
                              torch.cuda.current_stream(q.device).cuda_stream)
    if st != 0:
        raise AttnJvpError(st, "attn_jvp_fwd_partial")
    return o, do, lse, dlse


def check_merge(o_parts, do_parts, lse_parts, dlse_parts, dtype, out=None):
    """Validate a merge call; returns (P, Shape, out tensors or None)."""
    import torch
    if dtype not in _torch_dtypes():
        raise TypeError(f"unsupported output dtype {dtype}")
    if o_parts.dim() != 5:
        raise ValueError("o_parts must be [P, B, H, Lq, d_v]")
    P, B, H, Lq, dv_ = o_parts.shape
    dev = o_parts.device
    check_tensor(o_parts, "o_parts", (P, B, H, Lq, dv_), torch.float32, dev, contiguous=True)
    check_tensor(do_parts, "do_parts", (P, B, H, Lq, dv_), torch.float32, dev, contiguous=True)
    check_tensor(lse_parts, "lse_parts", (P, B, H, Lq), torch.float32, dev, contiguous=True)
    check_tensor(dlse_parts, "dlse_parts", (P, B, H, Lq), torch.float32, dev, contiguous=True)
    shape = Shape(B, H, Lq, Lq, dv_, dv_)
    if out is not None:
        out = check_fwd_out(out, o_parts, shape, out_dtype=dtype)
    return P, shape, out


def merge(o_parts, do_parts, lse_parts, dlse_parts, dtype, out=None):
    """Merge float32 partials stacked on a leading parts axis (o_parts, do_parts
    [P, B, H, Lq, d_v], lse_parts, dlse_parts [P, B, H, Lq], contiguous) into
    (o, do, lse, dlse) with o, do in ``dtype`` (torch.bfloat16/float32)."""
    import torch
    P, shape, out = check_merge(o_parts, do_parts, lse_parts, dlse_parts, dtype, out)
    _require_gpu(o_parts, "o_parts")
    o, do, lse, dlse = _alloc_fwd_out(o_parts, shape, dtype) if out is None else out
    B, H, Lq, dv_ = shape.batch, shape.heads, shape.seqlen_q, shape.head_dim_v
    st = attn_jvp_merge(P, o_parts.data_ptr(), do_parts.data_ptr(), lse_parts.data_ptr(),
                        dlse_parts.data_ptr(), o.data_ptr(), do.data_ptr(), lse.data_ptr(),
                        dlse.data_ptr(), B, H, Lq, dv_, _torch_dtypes()[dtype], _strides3(o),
                        torch.cuda.current_stream(o_parts.device).cuda_stream)
    if st != 0:
        raise AttnJvpError(st, "attn_jvp_merge")
    return o, do, lse, dlse


def check_workspace(workspace, need, device):
    """A caller's split-KV workspace: a contiguous tensor on ``device`` of at
    least ``need`` bytes."""
    import torch
    if not isinstance(workspace, torch.Tensor):
        raise ValueError("workspace must be a tensor")
    if workspace.device != device:
        raise ValueError(f"workspace must be on {device}, got {workspace.device}")
    if not workspace.is_contiguous():
        raise ValueError("workspace must be contiguous")
    nbytes = workspace.numel() * workspace.element_size()
    if nbytes < need:
        raise ValueError(f"workspace holds {nbytes} bytes, the plan needs {need}")
    return nbytes


def fwd_splitkv(q, k, v, dq, dk, dv, scale=None, mask=None, num_splits=0, workspace=None,
                out=None):
    """``fwd`` with key splits and a merge (attn_jvp_fwd_splitkv).  The
    workspace (a GPU tensor of at least the plan's size, on q's device) is
    allocated with torch.empty when not given.  Returns (o, do, lse, dlse,
    splits)."""
    import torch
    dt, shape = check_qkv(q, k, v, dq, dk, dv)
    o, do, lse, dlse = (_alloc_fwd_out(q, shape, q.dtype) if out is None
                        else check_fwd_out(out, q, shape))
    _require_gpu(q, "q")
    ns, need = attn_jvp_splitkv_plan(shape, dt, mask, num_splits)
    if workspace is None and need:
        workspace = torch.empty(need, device=q.device, dtype=torch.uint8)
    wp, wb = 0, 0
    if workspace is not None:
        wb = check_workspace(workspace, need, q.device)
        wp = workspace.data_ptr()
    lay = layout_of(q, k, v, dq, dk, dv, o, do)
    st = attn_jvp_fwd_splitkv(q.data_ptr(), k.data_ptr(), v.data_ptr(), dq.data_ptr(),
                              dk.data_ptr(), dv.data_ptr(), o.data_ptr(), do.data_ptr(),
                              lse.data_ptr(), dlse.data_ptr(), shape,
                              0.0 if scale is None else float(scale), dt, lay, mask, ns,
                              wp or None, wb, torch.cuda.current_stream(q.device).cuda_stream)
    if st != 0:
        raise AttnJvpError(st, "attn_jvp_fwd_splitkv")
    return o, do, lse, dlse, ns


def check_bwd_args(q, k, v, o, go, lse, out=None):
    """(dtype code, Shape, out tensors or None) of a backward call; raises on
    any mismatch of shape, dtype or device, a non-contiguous lse or out
    tensors of the wrong shape, dtype or device."""
    import torch
    dtypes = _torch_dtypes()
    if q.dtype not in dtypes:
        raise TypeError(f"unsupported dtype {q.dtype}")
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be 4-d [B, H, L, d]")
    B, H, Lq, d = q.shape
    Lkv, dv_ = k.shape[2], v.shape[3]
    if tuple(k.shape) != (B, H, Lkv, d) or tuple(v.shape) != (B, H, Lkv, dv_) \
            or tuple(o.shape) != (B, H, Lq, dv_) or tuple(go.shape) != (B, H, Lq, dv_):
        raise ValueError("shapes must be q [B,H,Lq,d], k, v [B,H,Lkv,d], o, go [B,H,Lq,d]")
    for t in (k, v, o, go):
        if t.dtype != q.dtype or t.device != q.device:
            raise ValueError("q, k, v, o, go must share dtype and device")
    check_tensor(lse, "lse", (B, H, Lq), torch.float32, q.device, contiguous=True)
    if out is not None:
        if len(out) != 4:
            raise ValueError("out must be (gq, gk, gv, delta)")
        gq, gk, gv, delta = out
        check_tensor(gq, "gq", q.shape, q.dtype, q.device)
        check_tensor(gk, "gk", k.shape, q.dtype, q.device)
        check_tensor(gv, "gv", v.shape, q.dtype, q.device)
        check_tensor(delta, "delta", (B, H, Lq), torch.float32, q.device, contiguous=True)
        for t in (gq, gk, gv):
            _strides3(t)
    return dtypes[q.dtype], Shape(B, H, Lq, Lkv, d, dv_), out


def bwd(q, k, v, o, go, lse, scale=None, mask=None, out=None):
    """Primal gradients (gq, gk, gv, delta) of a loss with dL/dO = go, for
    q [B, H, Lq, d], k, v [B, H, Lkv, d], o, go [B, H, Lq, d] (bf16 or
    float32) and the forward's lse [B, H, Lq] (float32).  delta is
    rowsum(go * o).  ``mask`` (as for ``fwd``) gives the gradients of the
    masked attention; o and lse must come from the forward with the same
    mask.  Outputs are allocated contiguous unless ``out = (gq, gk, gv,
    delta)`` is given.  Runs on the current stream."""
    import torch
    dt, shape, out = check_bwd_args(q, k, v, o, go, lse, out)
    _require_gpu(q, "q")
    if out is None:
        gq, gk, gv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        delta = torch.empty((shape.batch, shape.heads, shape.seqlen_q), device=q.device,
                            dtype=torch.float32)
    else:
        gq, gk, gv, delta = out
    lay = BwdLayout()
    for name, t in zip(("q", "k", "v", "o", "go", "gq", "gk", "gv"), (q, k, v, o, go, gq, gk, gv)):
        getattr(lay, name)[:] = _strides3(t)
    st = attn_jvp_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), go.data_ptr(),
                      lse.data_ptr(), gq.data_ptr(), gk.data_ptr(), gv.data_ptr(),
                      delta.data_ptr(), shape, 0.0 if scale is None else float(scale),
                      dt, lay, mask, torch.cuda.current_stream(q.device).cuda_stream)
    if st != 0:
        raise AttnJvpError(st, "attn_jvp_bwd")
    return gq, gk, gv, delta
