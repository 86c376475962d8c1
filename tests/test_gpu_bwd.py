"""GPU parity for the primal backward (attn_jvp_bwd): dQ, dK, dV of a loss
with upstream gradient G = dL/dO, from the row log-sum-exp the forward
stored.  Reference: the float64 oracle backward (every element).  Bounds
(tests/tolerances.py): normwise max|gpu - ref| / max|ref| of each output
within the contract (2e-2 bf16, 1e-4 float32) and the regression ceiling.
Only where the exact dQ and dK are zero (a single key) are their errors
measured against max|dV_ref| instead, the test asserting that the exact
values are zero.  D = rowsum(G . O) is checked against the same O the
kernel read.
"""

import numpy as np
import pytest
import torch

import attention_jvp_amd as aj
from oracle import FrameWindow, attention_backward, attention_jvp
from synth import Workload, make_inputs, to_float64
from tolerances import compare_bwd, normwise, say

pytestmark = pytest.mark.gpu

NAMES = ("q", "k", "v", "dq", "dk", "dv")
_say = say


def _grad_input(w, seed):
    g = np.random.default_rng(seed).standard_normal((w.B, w.H, w.N, w.dv))
    return torch.from_numpy(g).to({"bf16": torch.bfloat16, "fp32": torch.float32}[w.dtype])


def _check(w, scale=None, from_oracle=False, what=""):
    x = make_inputs(w)
    q, k, v = (x[n].cuda() for n in ("q", "k", "v"))
    g_cpu = _grad_input(w, w.seed + 1)
    go = g_cpu.cuda()
    if from_oracle:
        # the backward alone: O and LSE from the float64 definition
        o64, _, lse64, _ = attention_jvp(*(to_float64(x[n]) for n in NAMES), scale=scale)
        o = torch.from_numpy(o64).to(q.dtype).cuda()
        lse = torch.from_numpy(lse64).float().cuda()
    else:
        o, _, lse, _ = aj.fwd(*(x[n].cuda() for n in NAMES), scale=scale)
    gq, gk, gv, delta = aj.bwd(q, k, v, o, go, lse, scale=scale)
    torch.cuda.synchronize()
    ref = attention_backward(to_float64(x["q"]), to_float64(x["k"]), to_float64(x["v"]),
                             to_float64(g_cpu), scale=scale)
    errs = compare_bwd([to_float64(t) for t in (gq, gk, gv)], ref, w.dtype, what,
                       zero_dq_dk=(w.Nkv == 1))
    d_ref = (to_float64(g_cpu) * to_float64(o)).sum(-1)
    errs["D"] = normwise(to_float64(delta), d_ref)
    assert errs["D"] <= 1e-5, f"{what}: D error {errs['D']:.3e}"
    _say(what, " ".join(f"{k}={v:.2e}" for k, v in errs.items()))


@pytest.mark.parametrize("dtype,d", [("bf16", 16), ("bf16", 32), ("bf16", 64), ("bf16", 128),
                                     ("bf16", 256), ("fp32", 16), ("fp32", 32), ("fp32", 64)])
@pytest.mark.parametrize("Nq,Nkv", [(200, 200), (77, 300), (300, 45)])
def test_backward_matches_oracle(dtype, d, Nq, Nkv):
    w = Workload("bwd", 1, 2, Nq, d, dtype, 9000 + d + Nq + 3 * Nkv, tangent_scale=0.1,
                 n_kv=Nkv)
    _say(f"bwd {dtype} d{d} Lq{Nq} Lkv{Nkv}")
    _check(w, what=f"bwd {dtype} d{d} Lq{Nq} Lkv{Nkv}")


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("fp32", 32)])
@pytest.mark.parametrize("Nq,Nkv", [(1, 1), (1, 300), (300, 1)])
def test_backward_single_row_or_key(dtype, d, Nq, Nkv):
    w = Workload("bwd1", 1, 2, Nq, d, dtype, 9050 + d + Nq + Nkv, tangent_scale=0.1, n_kv=Nkv)
    _say(f"bwd {dtype} d{d} Lq{Nq} Lkv{Nkv}")
    _check(w, what=f"bwd {dtype} d{d} Lq{Nq} Lkv{Nkv}")


def test_backward_alone_on_oracle_forward():
    w = Workload("bwdo", 2, 2, 333, 128, "bf16", 9100, tangent_scale=0.1, n_kv=257)
    _check(w, from_oracle=True, what="bwd from oracle O, LSE")


def test_backward_custom_scale_and_rms_inputs():
    w = Workload("bwds", 1, 3, 400, 64, "bf16", 9200, rms_qk=True, tangent_scale=0.1)
    _check(w, scale=0.3, what="bwd scale 0.3")


def test_backward_image_dit_shape_sampled():
    # the image-DiT shape at full size: compare a few heads every element
    w = Workload("bwdi", 1, 2, 4096, 128, "bf16", 9300, rms_qk=True, tangent_scale=0.1)
    _check(w, what="bwd 1x2x4096x128")


@pytest.mark.parametrize("dtype,d,Nq,Nkv", [("bf16", 128, 150, 333), ("bf16", 64, 97, 70),
                                           ("fp32", 32, 130, 40)])
def test_backward_rows_without_keys(dtype, d, Nq, Nkv):
    # a forward whose rows 0, 5, 6 and the last see no key stores LSE = -inf
    # and O = 0 there; the backward must give those rows P = 0 (dQ row 0, no
    # contribution to dK, dV) and the other rows their unmasked gradients
    w = Workload("bwdz", 1, 2, Nq, d, dtype, 9600 + d + Nq, tangent_scale=0.1, n_kv=Nkv)
    x = make_inputs(w)
    empty = np.array([0, 5, 6, Nq - 1])
    vis = lambda qi, ki: ~np.isin(qi, empty)[:, None] & np.ones((1, len(ki)), dtype=bool)
    o64, _, lse64, _ = attention_jvp(*(to_float64(x[n]) for n in NAMES), visible=vis)
    assert np.isneginf(lse64[:, :, empty]).all() and np.isfinite(lse64[:, :, 1]).all()
    q, k, v = (x[n].cuda() for n in ("q", "k", "v"))
    o = torch.from_numpy(o64).to(q.dtype).cuda()
    lse = torch.from_numpy(lse64).float().cuda()
    g_cpu = _grad_input(w, w.seed + 1)
    gq, gk, gv, delta = aj.bwd(q, k, v, o, g_cpu.cuda(), lse)
    torch.cuda.synchronize()
    ref = attention_backward(to_float64(x["q"]), to_float64(x["k"]), to_float64(x["v"]),
                             to_float64(g_cpu), visible=vis)
    errs = compare_bwd([to_float64(t) for t in (gq, gk, gv)], ref, dtype,
                       f"bwd rows without keys {dtype} d{d}")
    assert np.all(to_float64(gq)[:, :, empty] == 0.0)
    _say(f"bwd rows without keys {dtype} d{d}", " ".join(f"{k}={v:.2e}" for k, v in errs.items()))


@pytest.mark.parametrize("Nkv", [4096, 4001])
def test_backward_image_dit_heads_sampled(Nkv):
    # 2 x 24 heads x 4096 queries at d = 128: the dK/dV launch takes 128 keys
    # per workgroup (at least 512 workgroups); 4001 keys leave a last block of
    # 33 (one full wave of 32, one key in the next).  Every element of three
    # heads against the oracle.
    w = Workload("bwdI", 2, 24, 4096, 128, "bf16", 9320 + Nkv, rms_qk=True, tangent_scale=0.1,
                 n_kv=Nkv)
    x = make_inputs(w)
    q, k, v = (x[n].cuda() for n in ("q", "k", "v"))
    o, _, lse, _ = aj.fwd(*(x[n].cuda() for n in NAMES))
    g_cpu = _grad_input(w, w.seed + 1)
    gq, gk, gv, _ = aj.bwd(q, k, v, o, g_cpu.cuda(), lse)
    torch.cuda.synchronize()
    for b, h in ((0, 0), (1, 23), (1, 7)):
        sl = lambda t: to_float64(t[b:b + 1, h:h + 1])
        ref = attention_backward(sl(x["q"]), sl(x["k"]), sl(x["v"]), sl(g_cpu))
        what = f"bwd 2x24x4096x{Nkv} head ({b},{h})"
        errs = compare_bwd([sl(t.cpu()) for t in (gq, gk, gv)], ref, "bf16", what)
        _say(what, " ".join(f"{k}={v:.2e}" for k, v in errs.items()))


def test_backward_rows_without_keys_many_heads():
    # rows with LSE = -inf (no visible key) in a launch wide enough for 128
    # keys per dK/dV workgroup: they add nothing to dK, dV
    Nq, Nkv = 150, 333
    w = Workload("bwdZ", 2, 256, Nq, 128, "bf16", 9650, tangent_scale=0.1, n_kv=Nkv)
    x = make_inputs(w)
    empty = np.array([0, 5, 6, 64, 127, Nq - 1])
    vis = lambda qi, ki: ~np.isin(qi, empty)[:, None] & np.ones((1, len(ki)), dtype=bool)
    o64, _, lse64, _ = attention_jvp(*(to_float64(x[n]) for n in NAMES), visible=vis)
    q, k, v = (x[n].cuda() for n in ("q", "k", "v"))
    o = torch.from_numpy(o64).to(q.dtype).cuda()
    lse = torch.from_numpy(lse64).float().cuda()
    g_cpu = _grad_input(w, w.seed + 1)
    gq, gk, gv, _ = aj.bwd(q, k, v, o, g_cpu.cuda(), lse)
    torch.cuda.synchronize()
    ref = attention_backward(to_float64(x["q"]), to_float64(x["k"]), to_float64(x["v"]),
                             to_float64(g_cpu), visible=vis)
    errs = compare_bwd([to_float64(t) for t in (gq, gk, gv)], ref, "bf16",
                       "bwd rows without keys, 2x256 heads")
    assert np.all(to_float64(gq)[:, :, empty] == 0.0)
    _say("bwd rows without keys, 2x256 heads", " ".join(f"{k}={v:.2e}" for k, v in errs.items()))


def test_backward_strided_bshd_views():
    # inputs and outputs stored [B, N, H, d] and passed as [B, H, N, d] views
    B, H, Nq, Nkv, d = 2, 3, 170, 230, 64
    w = Workload("bwdv", B, H, Nq, d, "bf16", 9700, tangent_scale=0.1, n_kv=Nkv)
    x = make_inputs(w)
    bshd = lambda t: t.transpose(1, 2).contiguous().cuda().transpose(1, 2)
    q, k, v = (bshd(x[n]) for n in ("q", "k", "v"))
    assert q.stride() == (Nq * H * d, d, H * d, 1)
    o, _, lse, _ = aj.fwd(*(bshd(x[n]) for n in NAMES))
    o = bshd(o.cpu())
    g_cpu = _grad_input(w, 77)
    go = bshd(g_cpu)
    out = (bshd(torch.zeros_like(x["q"])), bshd(torch.zeros_like(x["k"])),
           bshd(torch.zeros_like(x["v"])), torch.empty((B, H, Nq), device="cuda"))
    gq, gk, gv, delta = aj.bwd(q, k, v, o, go, lse, out=out)
    torch.cuda.synchronize()
    assert gq.stride() == q.stride() and gk.stride() == k.stride()
    ref = attention_backward(to_float64(x["q"]), to_float64(x["k"]), to_float64(x["v"]),
                             to_float64(g_cpu))
    errs = compare_bwd([to_float64(t) for t in (gq, gk, gv)], ref, "bf16", "bwd bshd")
    _say("bwd bshd", " ".join(f"{k}={v:.2e}" for k, v in errs.items()))


@pytest.mark.parametrize("F,T,C,R,first,last,see_all,dtype,d", [
    (7, 37, 2, 1, 1, 1, 0, "bf16", 128),
    (9, 64, 3, 0, 1, 0, 0, "bf16", 64),
    (6, 50, 2, 0, 0, 1, 1, "bf16", 128),
    (12, 30, 2, 0, 1, 1, 1, "bf16", 64),     # anchor query frames far from the window
    (11, 40, 1, 1, 1, 1, 0, "fp32", 64),
    (5, 100, 5, 0, 0, 0, 0, "bf16", 128),
    (8, 33, 3, 1, 0, 0, 1, "bf16", 256),
])
def test_backward_frame_window(F, T, C, R, first, last, see_all, dtype, d):
    # masked forward (O, LSE) then the masked backward, against the oracle's
    # backward of the masked attention
    N = F * T
    what = f"bwd mask F{F} T{T} C{C} R{R} a{first}{last}{see_all} {dtype} d{d}"
    _say(what)
    mask = dict(frames=F, tokens_per_frame=T, chunk_frames=C, radius_chunks=R,
                anchor_first=first, anchor_last=last, anchor_queries_see_all=see_all)
    vis = FrameWindow(frames=F, tokens_per_frame=T, chunk_frames=C, radius_chunks=R,
                      anchor_first=bool(first), anchor_last=bool(last),
                      anchor_queries_see_all=bool(see_all))
    w = Workload("bwdm", 1, 2, N, d, dtype, 9800 + N + d, tangent_scale=0.1)
    x = make_inputs(w)
    q, k, v = (x[n].cuda() for n in ("q", "k", "v"))
    o, _, lse, _ = aj.fwd(*(x[n].cuda() for n in NAMES), mask=mask)
    g_cpu = _grad_input(w, w.seed + 1)
    gq, gk, gv, delta = aj.bwd(q, k, v, o, g_cpu.cuda(), lse, mask=mask)
    torch.cuda.synchronize()
    ref = attention_backward(to_float64(x["q"]), to_float64(x["k"]), to_float64(x["v"]),
                             to_float64(g_cpu), visible=vis)
    errs = compare_bwd([to_float64(t) for t in (gq, gk, gv)], ref, dtype, what)
    _say(what, " ".join(f"{k}={v:.2e}" for k, v in errs.items()))


@pytest.mark.parametrize("d,Nq,Nkv", [(128, 300, 70), (64, 70, 300)])
def test_backward_two_row_blocks_per_wave(d, Nq, Nkv):
    # enough heads that a launch gives each wave two 16-row blocks (bf16;
    # d = 128: the dQ launch, d = 64: the dK/dV launch; at least 512
    # workgroups of 256 rows): oracle parity, and one head equals the same
    # head run alone (one block per wave)
    w = Workload("bwd2r", 2, 256, Nq, d, "bf16", 9900 + d, tangent_scale=0.1, n_kv=Nkv)
    _check(w, what=f"bwd two row blocks d{d}")
    x = make_inputs(w)
    q, k, v = (x[n].cuda() for n in ("q", "k", "v"))
    o, _, lse, _ = aj.fwd(*(x[n].cuda() for n in NAMES))
    go = _grad_input(w, 31).cuda()
    full = aj.bwd(q, k, v, o, go, lse)
    b, h = 1, 77
    one = aj.bwd(*(t[b:b + 1, h:h + 1].contiguous() for t in (q, k, v, o, go, lse)))
    torch.cuda.synchronize()
    for a, c in zip(full, one):
        assert torch.equal(a[b:b + 1, h:h + 1], c)


@pytest.mark.parametrize("d", [128, 64])
def test_backward_two_row_blocks_frame_window(d):
    mask = dict(frames=10, tokens_per_frame=30, chunk_frames=2, radius_chunks=1,
                anchor_first=1, anchor_last=1, anchor_queries_see_all=0)
    vis = FrameWindow(frames=10, tokens_per_frame=30, chunk_frames=2, radius_chunks=1)
    w = Workload("bwd2m", 2, 256, 300, d, "bf16", 9950 + d, tangent_scale=0.1)
    x = make_inputs(w)
    q, k, v = (x[n].cuda() for n in ("q", "k", "v"))
    o, _, lse, _ = aj.fwd(*(x[n].cuda() for n in NAMES), mask=mask)
    g_cpu = _grad_input(w, w.seed + 1)
    gq, gk, gv, _ = aj.bwd(q, k, v, o, g_cpu.cuda(), lse, mask=mask)
    torch.cuda.synchronize()
    ref = attention_backward(to_float64(x["q"]), to_float64(x["k"]), to_float64(x["v"]),
                             to_float64(g_cpu), visible=vis)
    compare_bwd([to_float64(t) for t in (gq, gk, gv)], ref, "bf16", f"two row blocks d{d}, mask")


def test_backward_deterministic():
    w = Workload("bwdd", 1, 2, 500, 128, "bf16", 9400, tangent_scale=0.1, n_kv=700)
    x = make_inputs(w)
    q, k, v = (x[n].cuda() for n in ("q", "k", "v"))
    o, _, lse, _ = aj.fwd(*(x[n].cuda() for n in NAMES))
    go = _grad_input(w, 5).cuda()
    a = aj.bwd(q, k, v, o, go, lse)
    b = aj.bwd(q, k, v, o, go, lse)
    torch.cuda.synchronize()
    for s, t in zip(a, b):
        assert torch.equal(s, t)


@pytest.mark.parametrize("dtype,d,F,T", [("bf16", 128, 7, 150), ("bf16", 64, 5, 333),
                                         ("fp32", 32, 3, 100)])
def test_backward_all_visible_window_equals_dense_bitwise(dtype, d, F, T):
    # a frame window that hides nothing: both masked launches walk every
    # streamed tile in the dense order with no element masks, so the
    # gradients equal the dense launches' bit for bit
    mask = dict(frames=F, tokens_per_frame=T, chunk_frames=F, radius_chunks=0,
                anchor_first=1, anchor_last=1, anchor_queries_see_all=0)
    w = Workload("bwdallvis", 2, 3, F * T, d, dtype, 9600 + d + F, tangent_scale=0.1)
    _say(f"bwd all-visible window {dtype} d{d} N{F * T}")
    x = make_inputs(w)
    q, k, v = (x[n].cuda() for n in ("q", "k", "v"))
    o, _, lse, _ = aj.fwd(*(x[n].cuda() for n in NAMES))
    go = _grad_input(w, 7).cuda()
    dense = aj.bwd(q, k, v, o, go, lse)
    masked = aj.bwd(q, k, v, o, go, lse, mask=mask)
    torch.cuda.synchronize()
    for s, t in zip(dense, masked):
        assert torch.equal(s, t)


def test_backward_errors_launch_nothing():
    w = Workload("bwde", 1, 1, 64, 64, "bf16", 9500, n_kv=64, d_v=32)
    x = make_inputs(w)
    q, k, v = (x[n].cuda() for n in ("q", "k", "v"))
    o = torch.zeros((1, 1, 64, 32), device="cuda", dtype=torch.bfloat16)
    lse = torch.zeros((1, 1, 64), device="cuda", dtype=torch.float32)
    with pytest.raises(aj.AttnJvpError) as e:      # d_qk != d_v: not built, as on the pages
        aj.bwd(q, k, v, o, o.clone(), lse)
    assert e.value.status == -2
