"""GPU parity: the HIP path (through the C-ABI) against the float64 oracle.

Bounds (tests/tolerances.py): the contract (normwise max|gpu - ref| /
max|ref| <= 1e-5 for O and 1e-4 for dO with float32 inputs, 2e-2 with
bfloat16), a tighter regression ceiling from the path's error model, and an
absolute bound in nats on LSE.  Small
shapes are compared element by element on every row; the full-size workloads
on a deterministic row sample, in the launch configuration the benchmark
times.
"""

import ctypes
import math

import numpy as np
import pytest
import torch

import attention_jvp_amd as aj
from oracle import FrameWindow, attention_jvp, attention_jvp_rows
from synth import WORKLOADS, Workload, make_inputs, sample_rows, to_float64
from tolerances import compare_bwd, compare_fwd, say

pytestmark = pytest.mark.gpu

NAMES = ("q", "k", "v", "dq", "dk", "dv")
_say = say


def _dev(x):
    return {n: x[n].cuda() for n in NAMES}


def _run(x, mask=None, scale=None):
    g = _dev(x)
    out = aj.fwd(*(g[n] for n in NAMES), scale=scale, mask=mask)
    torch.cuda.synchronize()
    return out


def _compare(gpu, ref, dtype, what, **kw):
    return compare_fwd(gpu, ref, dtype, what, **kw)


def _full_check(w, mask=None, scale=None, seed=None, **kw):
    x = make_inputs(w, seed=seed)
    mask = x["mask"] if mask is None else mask
    out = _run(x, mask=mask, scale=scale)
    gpu = [to_float64(t) for t in out]
    vis = None if mask is None else FrameWindow(**{k: bool(v) if k.startswith("anchor") else v
                                                   for k, v in mask.items()})
    ref = attention_jvp(*(to_float64(x[n]) for n in NAMES), scale=scale, visible=vis)
    return _compare(gpu, ref, w.dtype, f"{w.name} B{w.B} H{w.H} N{w.N} d{w.d}", **kw)


# ---- small shapes: every row, several tiles, ragged tails -----------------

SMALL = [
    ("fp32", 1, 2, 128, 64), ("fp32", 1, 1, 1, 64), ("fp32", 2, 1, 77, 64),
    ("fp32", 1, 1, 300, 64),
    ("bf16", 1, 2, 256, 128), ("bf16", 1, 1, 1, 128), ("bf16", 1, 1, 63, 128),
    ("bf16", 1, 1, 65, 128), ("bf16", 2, 2, 129, 128), ("bf16", 1, 2, 333, 128),
    ("bf16", 1, 1, 1, 64), ("bf16", 2, 2, 200, 64), ("bf16", 1, 3, 517, 64),
]


@pytest.mark.parametrize("dtype,B,H,N,d", SMALL)
def test_small_shapes_every_row(dtype, B, H, N, d):
    _say(f"small {dtype} B{B} H{H} N{N} d{d}")
    w = Workload("small", B, H, N, d, dtype, 77 + N + d, tangent_scale=0.1)
    _full_check(w)


def test_tiny_fp32_workload():
    _full_check(WORKLOADS["tiny_fp32"])


def test_custom_scale():
    w = Workload("scale", 1, 2, 190, 128, "bf16", 5, tangent_scale=0.3)
    _full_check(w, scale=0.05)


def test_small_trigflow_and_rms_recipe():
    w = Workload("trig", 1, 2, 300, 128, "bf16", 6, rms_qk=True, tangents="trigflow")
    _full_check(w)


def test_large_logits_bf16():
    # scores of magnitude up to ~100: the running max and rescaling matter;
    # float32 scores that large carry absolute rounding errors about 30x
    # those of unit-size scores, so LSE gets a 1e-3 nat bound here
    w = Workload("big", 1, 2, 400, 64, "bf16", 8, tangent_scale=0.1)
    _full_check(w, scale=4.0, lse_abs=1e-3)


@pytest.mark.parametrize("dtype,d", [("bf16", 16), ("bf16", 32), ("bf16", 64), ("bf16", 128),
                                     ("bf16", 256), ("fp32", 16), ("fp32", 64)])
@pytest.mark.parametrize("rising", [True, False])
def test_logits_ramp_along_keys(dtype, d, rising):
    # q_0 = 4 and k_0 a ramp over the keys from -8 to 8 (or back): the row
    # maxima grow through the whole walk (the reference moves every few
    # tiles) or peak in the first tile (it never moves again); 700 keys are
    # several tiles and a ragged tail.  Scores reach |S| ~ 60, where their
    # float32 rounding (relative 2^-24 of each product sum) moves P by up to
    # ~1e-5: float32 O is held to the contract there, not the unit-score
    # ceiling
    N = 700
    _say(f"ramp {dtype} d{d} {'rising' if rising else 'falling'}")
    w = Workload("ramp", 1, 2, N, d, dtype, 40 + d, tangent_scale=0.1)
    x = make_inputs(w)
    ramp = torch.linspace(-8.0, 8.0, N) if rising else torch.linspace(8.0, -8.0, N)
    x["q"][..., 0] = 4.0
    x["k"][..., 0] = ramp.to(x["k"].dtype)
    out = _run(x, scale=1.0)
    gpu = [to_float64(t) for t in out]
    ref = attention_jvp(*(to_float64(x[n]) for n in NAMES), scale=1.0)
    _compare(gpu, ref, dtype, f"ramp {dtype} d{d} rising={rising}",
             lse_abs=1e-3 if dtype == "bf16" else 1e-4,
             ceiling={"O": 1e-5} if dtype == "fp32" else None)


@pytest.mark.parametrize("F,T,C,R,first,last,see_all,dtype,d", [
    (7, 37, 2, 1, 1, 1, 0, "bf16", 128),
    (9, 64, 3, 0, 1, 0, 0, "bf16", 64),
    (6, 50, 2, 0, 0, 1, 1, "bf16", 128),
    (11, 40, 1, 1, 1, 1, 0, "fp32", 64),
    (5, 100, 5, 0, 0, 0, 0, "bf16", 128),
])
def test_frame_window_mask_every_row(F, T, C, R, first, last, see_all, dtype, d):
    N = F * T
    _say(f"mask F{F} T{T} C{C} R{R} a{first}{last}{see_all} {dtype} d{d}")
    mask = dict(frames=F, tokens_per_frame=T, chunk_frames=C, radius_chunks=R,
                anchor_first=first, anchor_last=last, anchor_queries_see_all=see_all)
    w = Workload("mask", 1, 2, N, d, dtype, 900 + N, tangent_scale=0.1)
    _full_check(w, mask=mask)


@pytest.mark.parametrize("B,H,N", [(8, 6, 1000), (5, 8, 1200), (8, 6, 1024)])
def test_small_geometry_every_row(B, H, N):
    # bf16 d = 64 grids that take 64-row blocks and 32-key tiles (ragged
    # last blocks for N = 1000 and 1200)
    assert aj.attn_jvp_fwd_geometry(B, H, N, N, 64, 64, 0) == (64, 32)
    _say(f"small geometry B{B} H{H} N{N}")
    w = Workload("small-geometry", B, H, N, 64, "bf16", 500 + N, tangent_scale=0.1)
    _full_check(w)


def test_small_geometry_strided_views():
    B, H, N, d = 8, 6, 1000, 64
    assert aj.attn_jvp_fwd_geometry(B, H, N, N, d, d, 0) == (64, 32)
    w = Workload("small-bshd", B, H, N, d, "bf16", 12, tangent_scale=0.1)
    x = make_inputs(w)
    g = {n: x[n].transpose(1, 2).contiguous().cuda().transpose(1, 2) for n in NAMES}
    out = aj.fwd(*(g[n] for n in NAMES))
    torch.cuda.synchronize()
    ref = attention_jvp(*(to_float64(x[n]) for n in NAMES))
    _compare([to_float64(t) for t in out], ref, "bf16", "small-geometry bshd")


def test_strided_bshd_views():
    # tensors stored [B, N, H, d] and passed as [B, H, N, d] views
    B, H, N, d = 2, 3, 150, 128
    w = Workload("bshd", B, H, N, d, "bf16", 11, tangent_scale=0.1)
    x = make_inputs(w)
    g = {n: x[n].transpose(1, 2).contiguous().cuda().transpose(1, 2) for n in NAMES}
    assert g["q"].stride() == (N * H * d, d, H * d, 1)
    out = aj.fwd(*(g[n] for n in NAMES))
    torch.cuda.synchronize()
    ref = attention_jvp(*(to_float64(x[n]) for n in NAMES))
    _compare([to_float64(t) for t in out], ref, "bf16", "bshd")


def _far_batch_view(t, sb):
    # a [B, H, N, d] view whose batch stride sb is beyond 2^31 elements:
    # 64-bit element offsets in every address of the path
    B, H, N, d = t.shape
    base = torch.empty(sb * (B - 1) + H * N * d, device="cuda", dtype=t.dtype)
    v = base.as_strided((B, H, N, d), (sb, N * d, d, 1))
    v.copy_(t.cuda())
    return v


def test_batch_stride_beyond_2_31_elements():
    sb = (1 << 31) + (1 << 20)
    w = Workload("far", 2, 1, 256, 128, "bf16", 14, tangent_scale=0.1)
    x = make_inputs(w)
    g = {n: _far_batch_view(x[n], sb) for n in NAMES}
    o = _far_batch_view(torch.zeros_like(x["q"]), sb)
    do = _far_batch_view(torch.zeros_like(x["q"]), sb)
    lse = torch.empty((2, 1, 256), device="cuda")
    dlse = torch.empty_like(lse)
    aj.fwd(*(g[n] for n in NAMES), out=(o, do, lse, dlse))
    torch.cuda.synchronize()
    ref = attention_jvp(*(to_float64(x[n]) for n in NAMES))
    _compare([to_float64(t) for t in (o, do, lse, dlse)], ref, "bf16", "far batch stride")
    # the primal backward on the same far views
    from oracle import attention_backward
    gcpu = torch.from_numpy(np.random.default_rng(15).standard_normal((2, 1, 256, 128))).bfloat16()
    go = _far_batch_view(gcpu, sb)
    outs = (_far_batch_view(torch.zeros_like(x["q"]), sb), _far_batch_view(torch.zeros_like(x["k"]), sb),
            _far_batch_view(torch.zeros_like(x["v"]), sb), torch.empty((2, 1, 256), device="cuda"))
    gq, gk, gv, _ = aj.bwd(g["q"], g["k"], g["v"], o, go, lse, out=outs)
    torch.cuda.synchronize()
    refb = attention_backward(to_float64(x["q"]), to_float64(x["k"]), to_float64(x["v"]),
                              to_float64(gcpu))
    compare_bwd([to_float64(t) for t in (gq, gk, gv)], refb, "bf16", "far batch stride backward")
    del g, o, do, go, outs
    torch.cuda.empty_cache()


def test_contiguous_entry_point_raw_pointers():
    w = Workload("raw", 1, 2, 200, 64, "bf16", 12, tangent_scale=0.1)
    x = make_inputs(w)
    g = _dev(x)
    o = torch.empty_like(g["q"])
    do = torch.empty_like(o)
    lse = torch.empty((1, 2, 200), device="cuda", dtype=torch.float32)
    dlse = torch.empty_like(lse)
    st = aj.attn_jvp_fwd(*(g[n].data_ptr() for n in NAMES), o.data_ptr(), do.data_ptr(),
                         lse.data_ptr(), dlse.data_ptr(), 1, 2, 200, 64, 0.0,
                         aj.ATTN_JVP_BF16, None, torch.cuda.current_stream().cuda_stream)
    assert st == 0
    torch.cuda.synchronize()
    ref = attention_jvp(*(to_float64(x[n]) for n in NAMES))
    _compare([to_float64(t) for t in (o, do, lse, dlse)], ref, "bf16", "raw")


def test_errors_launch_nothing():
    w = Workload("err", 1, 1, 64, 128, "bf16", 13)
    g = _dev(make_inputs(w))
    # a tangent whose row stride differs from its primal's: rejected by the C side
    wide = torch.zeros((1, 1, 64, 136), device="cuda", dtype=torch.bfloat16)
    wide[..., :128] = g["dq"]
    with pytest.raises(aj.AttnJvpError) as e:
        aj.fwd(g["q"], g["k"], g["v"], wide[..., :128], g["dk"], g["dv"])
    assert e.value.status == -3
    # a non-contiguous head dimension cannot be described to the C side
    with pytest.raises(ValueError):
        aj.fwd(g["q"], g["k"], g["v"], g["dq"].transpose(2, 3).contiguous().transpose(2, 3),
               g["dk"], g["dv"])
    bad = {n: g[n][..., :96].contiguous() for n in NAMES}
    with pytest.raises(aj.AttnJvpError) as e:
        aj.fwd(*(bad[n] for n in NAMES))
    assert e.value.status == -2


def test_bitwise_deterministic():
    w = Workload("det", 2, 4, 1000, 128, "bf16", 14, tangent_scale=0.1)
    g = _dev(make_inputs(w))
    a = aj.fwd(*(g[n] for n in NAMES))
    b = aj.fwd(*(g[n] for n in NAMES))
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_nan_in_one_query_row_stays_in_that_row():
    w = Workload("nan", 1, 2, 300, 128, "bf16", 15, tangent_scale=0.1)
    x = make_inputs(w)
    x["q"][0, 1, 137, 5] = float("nan")
    o, do, lse, dlse = _run(x)
    bad = torch.isnan(o).any(-1) | torch.isnan(do).any(-1) | torch.isnan(lse) | torch.isnan(dlse)
    expect = torch.zeros_like(bad)
    expect[0, 1, 137] = True
    assert torch.equal(bad.cpu(), expect.cpu())


@pytest.mark.parametrize("tensor", ["k", "dk"])
def test_nan_in_one_key_reaches_exactly_the_rows_that_see_it(tensor):
    # under the frame window a key in a middle frame is seen by the queries
    # of its chunk and the neighbouring ones only: those rows turn NaN, every
    # other row (and every other head) matches the oracle, which hides the
    # key from them before any arithmetic
    F, T = 9, 37
    mask = dict(frames=F, tokens_per_frame=T, chunk_frames=2, radius_chunks=1,
                anchor_first=1, anchor_last=1, anchor_queries_see_all=0)
    w = Workload("nan-key", 1, 2, F * T, 128, "bf16", 17, tangent_scale=0.1)
    x = make_inputs(w)
    x[tensor][0, 1, 4 * T + 5, 7] = float("nan")
    gpu = [to_float64(t) for t in _run(x, mask=mask)]
    vis = FrameWindow(**{k: bool(v) if k.startswith("anchor") else v for k, v in mask.items()})
    ref = attention_jvp(*(to_float64(x[n]) for n in NAMES), visible=vis)

    def nan_rows(out):
        o, do, lse, dlse = out
        return np.isnan(o).any(-1) | np.isnan(do).any(-1) | np.isnan(lse) | np.isnan(dlse)

    bad, bad_ref = nan_rows(gpu), nan_rows(ref)
    assert np.array_equal(bad, bad_ref)
    assert bad_ref[0, 1].any() and not bad_ref[0, 1].all() and not bad_ref[0, 0].any()
    keep = [np.where(bad_ref[..., None] if a.ndim == 4 else bad_ref, 0.0, a) for a in gpu]
    keep_ref = [np.where(bad_ref[..., None] if a.ndim == 4 else bad_ref, 0.0, a) for a in ref]
    _compare(keep, keep_ref, "bf16", f"NaN in one key of {tensor}")


@pytest.mark.parametrize("dtype,d,F,T", [("bf16", 128, 7, 150), ("bf16", 64, 5, 333),
                                         ("fp32", 64, 3, 100)])
def test_all_visible_window_equals_dense_bitwise(dtype, d, F, T):
    # a frame window whose chunk spans every frame hides nothing: the masked
    # kernel instance walks the same key tiles in the same order (one range,
    # no element masks but the key tail's) and must give the dense
    # instance's outputs bit for bit
    mask = dict(frames=F, tokens_per_frame=T, chunk_frames=F, radius_chunks=0,
                anchor_first=1, anchor_last=1, anchor_queries_see_all=0)
    w = Workload("allvis", 2, 3, F * T, d, dtype, 18 + d + F, tangent_scale=0.1)
    _say(f"all-visible window {dtype} d{d} N{F * T}")
    x = make_inputs(w)
    dense, masked = _run(x), _run(x, mask=mask)
    for a, b in zip(dense, masked):
        assert torch.equal(a, b)


def test_zero_score_tangent_matches_output_with_dv_bitwise():
    # dQ = dK = 0: the tangent accumulator sums exactly the products the
    # output accumulator sums when V is replaced by dV
    w = WORKLOADS["image_dit_4096"]
    small = Workload("zst", 1, 4, w.N, w.d, "bf16", 16)
    x = make_inputs(small)
    g = _dev(x)
    z = torch.zeros_like(g["q"])
    o, do, lse, dlse = aj.fwd(g["q"], g["k"], g["v"], z, z, g["dv"])
    o2, _, _, _ = aj.fwd(g["q"], g["k"], g["dv"], z, z, g["dv"])
    torch.cuda.synchronize()
    assert torch.equal(do, o2)
    assert torch.all(dlse == 0)


# ---- full-size workloads, sampled rows --------------------------------------

def _sampled_check(name, every):
    w = WORKLOADS[name]
    _say(f"workload {name}: generating inputs")
    x = make_inputs(w)
    _say(f"workload {name}: running GPU")
    out = _run(x, mask=x["mask"])
    m = x["mask"]
    rows = sample_rows(w.N, every=every, tokens_per_frame=m["tokens_per_frame"] if m else None)
    idx = torch.from_numpy(rows).cuda()
    gpu = [to_float64(t.index_select(2, idx)) for t in out]
    vis = None if m is None else FrameWindow(**{k: bool(v) if k.startswith("anchor") else v
                                                for k, v in m.items()})
    _say(f"workload {name}: oracle on {len(rows)} rows x {w.B * w.H} heads")
    # float32 holds every bf16 value exactly; the oracle widens to float64
    ref = attention_jvp_rows(*(x[n].float().numpy() for n in NAMES), rows, visible=vis)
    return _compare(gpu, ref, w.dtype, f"{name} ({len(rows)} rows/head)")


def test_workload_image_dit_4096():
    _sampled_check("image_dit_4096", every=32)


def test_workload_t2i_prefix_4352():
    _sampled_check("t2i_prefix_4352", every=32)


def test_workload_video_dit_32760():
    _sampled_check("video_dit_32760", every=256)


def test_workload_long_video_65520():
    _sampled_check("long_video_65520", every=512)
