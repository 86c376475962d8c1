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
]

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
           "attn_jvp_bwd_check", "attn_jvp_bwd_visible_tiles", "attn_jvp_status_string")


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


def fwd(q, k, v, dq, dk, dv, scale=None, mask=None, out=None):
    """(o, do, lse, dlse) for CUDA tensors q [B, H, Lq, d_qk], k [B, H, Lkv,
    d_qk], v [B, H, Lkv, d_v] (bf16 or float32).

    Tangents must have their primal's shape and strides.  ``mask`` is None or
    a frame-window dict/Mask (self-attention, Lq == Lkv).  Outputs o, do
    [B, H, Lq, d_v] and lse, dlse [B, H, Lq] are allocated contiguous unless
    ``out = (o, do, lse, dlse)`` is given.  Runs on the current stream.
    """
    import torch
    dtypes = {torch.bfloat16: ATTN_JVP_BF16, torch.float32: ATTN_JVP_FP32}
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
    if out is None:
        o = torch.empty((B, H, Lq, dv_), device=q.device, dtype=q.dtype)
        do = torch.empty_like(o)
        lse = torch.empty((B, H, Lq), device=q.device, dtype=torch.float32)
        dlse = torch.empty_like(lse)
    else:
        o, do, lse, dlse = out
    lay = layout_of(q, k, v, dq, dk, dv, o, do)
    shape = Shape(B, H, Lq, Lkv, dqk, dv_)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    st = attn_jvp_fwd_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), dq.data_ptr(),
                         dk.data_ptr(), dv.data_ptr(), o.data_ptr(), do.data_ptr(),
                         lse.data_ptr(), dlse.data_ptr(), shape,
                         0.0 if scale is None else float(scale), dtypes[q.dtype],
                         lay, mask, stream)
    if st != 0:
        raise AttnJvpError(st, "attn_jvp_fwd_ex")
    return o, do, lse, dlse


def _check_qkv(q, k, v, dq, dk, dv):
    import torch
    dtypes = {torch.bfloat16: ATTN_JVP_BF16, torch.float32: ATTN_JVP_FP32}
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


def fwd_partial(q, k, v, dq, dk, dv, scale=None):
    """float32 partials (o, do, lse, dlse) of the keys given (see
    attn_jvp_fwd_partial): o, do [B, H, Lq, d_v], lse, dlse [B, H, Lq]."""
    import torch
    dt, shape = _check_qkv(q, k, v, dq, dk, dv)
    B, H, Lq, dv_ = shape.batch, shape.heads, shape.seqlen_q, shape.head_dim_v
    o = torch.empty((B, H, Lq, dv_), device=q.device, dtype=torch.float32)
    do = torch.empty_like(o)
    lse = torch.empty((B, H, Lq), device=q.device, dtype=torch.float32)
    dlse = torch.empty_like(lse)
    lay = layout_of(q, k, v, dq, dk, dv, q, dq)     # o / dout strides are ignored
    st = attn_jvp_fwd_partial(q.data_ptr(), k.data_ptr(), v.data_ptr(), dq.data_ptr(),
                              dk.data_ptr(), dv.data_ptr(), o.data_ptr(), do.data_ptr(),
                              lse.data_ptr(), dlse.data_ptr(), shape,
                              0.0 if scale is None else float(scale), dt, lay,
                              torch.cuda.current_stream(q.device).cuda_stream)
    if st != 0:
        raise AttnJvpError(st, "attn_jvp_fwd_partial")
    return o, do, lse, dlse


def merge(o_parts, do_parts, lse_parts, dlse_parts, dtype, out=None):
    """Merge float32 partials stacked on a leading parts axis (o_parts, do_parts
    [P, B, H, Lq, d_v], lse_parts, dlse_parts [P, B, H, Lq], contiguous) into
    (o, do, lse, dlse) with o, do in ``dtype`` (torch.bfloat16/float32)."""
    import torch
    P, B, H, Lq, dv_ = o_parts.shape
    for t in (o_parts, do_parts, lse_parts, dlse_parts):
        if t.dtype != torch.float32 or not t.is_contiguous():
            raise ValueError("partials must be contiguous float32")
    if tuple(do_parts.shape) != tuple(o_parts.shape) or tuple(lse_parts.shape) != (P, B, H, Lq) \
            or tuple(dlse_parts.shape) != (P, B, H, Lq):
        raise ValueError("inconsistent partial shapes")
    dt = {torch.bfloat16: ATTN_JVP_BF16, torch.float32: ATTN_JVP_FP32}[dtype]
    if out is None:
        o = torch.empty((B, H, Lq, dv_), device=o_parts.device, dtype=dtype)
        do = torch.empty_like(o)
        lse = torch.empty((B, H, Lq), device=o_parts.device, dtype=torch.float32)
        dlse = torch.empty_like(lse)
    else:
        o, do, lse, dlse = out
    st = attn_jvp_merge(P, o_parts.data_ptr(), do_parts.data_ptr(), lse_parts.data_ptr(),
                        dlse_parts.data_ptr(), o.data_ptr(), do.data_ptr(), lse.data_ptr(),
                        dlse.data_ptr(), B, H, Lq, dv_, dt, _strides3(o),
                        torch.cuda.current_stream(o_parts.device).cuda_stream)
    if st != 0:
        raise AttnJvpError(st, "attn_jvp_merge")
    return o, do, lse, dlse


def fwd_splitkv(q, k, v, dq, dk, dv, scale=None, mask=None, num_splits=0, workspace=None,
                out=None):
    """``fwd`` with key splits and a merge (attn_jvp_fwd_splitkv).  The
    workspace (a CUDA uint8 tensor of at least the plan's size) is allocated
    with torch.empty when not given.  Returns (o, do, lse, dlse, splits)."""
    import torch
    dt, shape = _check_qkv(q, k, v, dq, dk, dv)
    ns, need = attn_jvp_splitkv_plan(shape, dt, mask, num_splits)
    B, H, Lq, dv_ = shape.batch, shape.heads, shape.seqlen_q, shape.head_dim_v
    if out is None:
        o = torch.empty((B, H, Lq, dv_), device=q.device, dtype=q.dtype)
        do = torch.empty_like(o)
        lse = torch.empty((B, H, Lq), device=q.device, dtype=torch.float32)
        dlse = torch.empty_like(lse)
    else:
        o, do, lse, dlse = out
    if workspace is None and need:
        workspace = torch.empty(need, device=q.device, dtype=torch.uint8)
    wp = 0 if workspace is None else workspace.data_ptr()
    wb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    lay = layout_of(q, k, v, dq, dk, dv, o, do)
    st = attn_jvp_fwd_splitkv(q.data_ptr(), k.data_ptr(), v.data_ptr(), dq.data_ptr(),
                              dk.data_ptr(), dv.data_ptr(), o.data_ptr(), do.data_ptr(),
                              lse.data_ptr(), dlse.data_ptr(), shape,
                              0.0 if scale is None else float(scale), dt, lay, mask, ns,
                              wp or None, wb, torch.cuda.current_stream(q.device).cuda_stream)
    if st != 0:
        raise AttnJvpError(st, "attn_jvp_fwd_splitkv")
    return o, do, lse, dlse, ns


def bwd(q, k, v, o, go, lse, scale=None, mask=None, out=None):
    """Primal gradients (gq, gk, gv, delta) of a loss with dL/dO = go, for
    q [B, H, Lq, d], k, v [B, H, Lkv, d], o, go [B, H, Lq, d] (bf16 or
    float32) and the forward's lse [B, H, Lq] (float32).  delta is
    rowsum(go * o).  ``mask`` (as for ``fwd``) gives the gradients of the
    masked attention; o and lse must come from the forward with the same
    mask.  Outputs are allocated contiguous unless ``out = (gq, gk, gv,
    delta)`` is given.  Runs on the current stream."""
    import torch
    dtypes = {torch.bfloat16: ATTN_JVP_BF16, torch.float32: ATTN_JVP_FP32}
    if q.dtype not in dtypes:
        raise TypeError(f"unsupported dtype {q.dtype}")
    B, H, Lq, d = q.shape
    Lkv = k.shape[2]
    if tuple(k.shape) != (B, H, Lkv, d) or tuple(v.shape) != (B, H, Lkv, v.shape[3]) \
            or tuple(o.shape) != (B, H, Lq, v.shape[3]) or go.shape != o.shape:
        raise ValueError("shapes must be q [B,H,Lq,d], k, v [B,H,Lkv,d], o, go [B,H,Lq,d]")
    if tuple(lse.shape) != (B, H, Lq) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be contiguous float32 [B, H, Lq]")
    for t in (k, v, o, go):
        if t.dtype != q.dtype or t.device != q.device:
            raise ValueError("q, k, v, o, go must share dtype and device")
    if out is None:
        gq, gk, gv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        delta = torch.empty((B, H, Lq), device=q.device, dtype=torch.float32)
    else:
        gq, gk, gv, delta = out
    lay = BwdLayout()
    for name, t in zip(("q", "k", "v", "o", "go", "gq", "gk", "gv"), (q, k, v, o, go, gq, gk, gv)):
        getattr(lay, name)[:] = _strides3(t)
    shape = Shape(B, H, Lq, Lkv, d, v.shape[3])
    st = attn_jvp_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), go.data_ptr(),
                      lse.data_ptr(), gq.data_ptr(), gk.data_ptr(), gv.data_ptr(),
                      delta.data_ptr(), shape, 0.0 if scale is None else float(scale),
                      dtypes[q.dtype], lay, mask, torch.cuda.current_stream(q.device).cuda_stream)
    if st != 0:
        raise AttnJvpError(st, "attn_jvp_bwd")
    return gq, gk, gv, delta
