"""GPU parity for the general shapes of the op contract: Lq != Lkv
(cross-attention) and d_qk != d_v, head dims 16, 32, 64, 128, 256 (bf16) and
16, 32, 64 (float32), through attn_jvp_fwd_ex.  Every output row is compared
with the float64 oracle under the bounds of tests/tolerances.py.
"""

import numpy as np
import pytest
import torch

import attention_jvp_amd as aj
from oracle import FrameWindow, attention_jvp
from synth import Workload, make_inputs, to_float64
from tolerances import compare_fwd, say

pytestmark = pytest.mark.gpu

NAMES = ("q", "k", "v", "dq", "dk", "dv")
BF16_DIMS = (16, 32, 64, 128, 256)
FP32_DIMS = (16, 32, 64)


_say = say


def _check(w, mask=None, scale=None, what=""):
    x = make_inputs(w)
    g = {n: x[n].cuda() for n in NAMES}
    out = aj.fwd(*(g[n] for n in NAMES), scale=scale, mask=mask)
    torch.cuda.synchronize()
    assert out[0].shape == (w.B, w.H, w.N, w.dv) and out[2].shape == (w.B, w.H, w.N)
    gpu = [to_float64(t) for t in out]
    vis = None if mask is None else FrameWindow(**{k: bool(v) if k.startswith("anchor") else v
                                                   for k, v in mask.items()})
    ref = attention_jvp(*(to_float64(x[n]) for n in NAMES), scale=scale, visible=vis)
    compare_fwd(gpu, ref, w.dtype, what)


@pytest.mark.parametrize("dqk", BF16_DIMS)
@pytest.mark.parametrize("dv", BF16_DIMS)
def test_bf16_head_dims_cross_attention(dqk, dv):
    # Lq spans two query blocks with a tail; Lkv several key tiles with a tail
    w = Workload("x", 1, 2, 150, dqk, "bf16", 3000 + dqk + 7 * dv, tangent_scale=0.1,
                 n_kv=201, d_v=dv)
    _say(f"bf16 dqk{dqk} dv{dv} Lq{w.N} Lkv{w.Nkv}")
    _check(w, what=f"bf16 dqk{dqk} dv{dv}")


@pytest.mark.parametrize("dqk", FP32_DIMS)
@pytest.mark.parametrize("dv", FP32_DIMS)
def test_fp32_head_dims_cross_attention(dqk, dv):
    w = Workload("x", 1, 2, 90, dqk, "fp32", 4000 + dqk + 7 * dv, tangent_scale=0.1,
                 n_kv=133, d_v=dv)
    _say(f"fp32 dqk{dqk} dv{dv} Lq{w.N} Lkv{w.Nkv}")
    _check(w, what=f"fp32 dqk{dqk} dv{dv}")


@pytest.mark.parametrize("dtype,d", [("bf16", 16), ("bf16", 32), ("bf16", 256),
                                     ("fp32", 16), ("fp32", 32)])
def test_frame_window_mask_other_head_dims(dtype, d):
    mask = dict(frames=7, tokens_per_frame=37, chunk_frames=2, radius_chunks=1,
                anchor_first=1, anchor_last=1, anchor_queries_see_all=0)
    w = Workload("m", 1, 2, 259, d, dtype, 5000 + d, tangent_scale=0.1)
    _say(f"mask {dtype} d{d}")
    _check(w, mask=mask, what=f"mask {dtype} d{d}")


@pytest.mark.parametrize("Nq,Nkv", [(1, 300), (300, 1), (1, 1), (129, 64), (64, 65)])
def test_edge_lengths(Nq, Nkv):
    w = Workload("e", 2, 1, Nq, 64, "bf16", 6000 + Nq + Nkv, tangent_scale=0.1,
                 n_kv=Nkv, d_v=128)
    _say(f"edge Lq{Nq} Lkv{Nkv}")
    _check(w, what=f"edge Lq{Nq} Lkv{Nkv}")


def test_text_cross_attention_shape():
    # image tokens attending to a short text sequence (DiT cross-attention)
    w = Workload("text", 1, 4, 4096, 128, "bf16", 7000, tangent_scale=0.1, n_kv=300)
    _say("text cross-attention Lq4096 Lkv300")
    _check(w, what="text Lq4096 Lkv300")


@pytest.mark.parametrize("B,H,Nq,Nkv,d", [(2, 23, 4000, 500, 128), (4, 16, 4352, 333, 64)])
def test_cross_attention_many_blocks(B, H, Nq, Nkv, d):
    # short key walks (8 and 6 tiles) over more query blocks than CUs: 1,472
    # blocks, a ragged last query block and a ragged key tail; every row
    # against the oracle, and one head alone (a launch of 32 or 23 blocks)
    # gives the same outputs bitwise
    w = Workload("xblocks", B, H, Nq, d, "bf16", 7300 + d, tangent_scale=0.1, n_kv=Nkv)
    _say(f"cross-attention B{B} H{H} Lq{Nq} Lkv{Nkv} d{d}")
    _check(w, what=f"cross Lq{Nq} Lkv{Nkv} d{d}")
    x = make_inputs(w)
    g = {n: x[n].cuda() for n in NAMES}
    full = aj.fwd(*(g[n] for n in NAMES))
    b, h = B - 1, H // 2
    one = aj.fwd(*(g[n][b:b + 1, h:h + 1].contiguous() for n in NAMES))
    torch.cuda.synchronize()
    for a, c in zip(full, one):
        assert torch.equal(a[b:b + 1, h:h + 1], c)


@pytest.mark.parametrize("B,H,Nq,Nkv,d", [(2, 23, 4000, 500, 128), (1, 3, 333, 333, 128),
                                           (2, 2, 200, 230, 64)])
def test_row_stores_into_strided_outputs(B, H, Nq, Nkv, d):
    # inputs and outputs stored [B, N, H, d] and passed as [B, H, N, d] views
    # (rows H * d apart): the epilogue's whole-row stores follow the output
    # strides and skip the rows past Lq; bitwise the same as contiguous
    # tensors (many blocks and few, ragged last query block)
    w = Workload("rows", B, H, Nq, d, "bf16", 7400 + d + Nq, tangent_scale=0.1, n_kv=Nkv)
    x = make_inputs(w)
    flat = aj.fwd(*(x[n].cuda() for n in NAMES))
    g = {n: x[n].transpose(1, 2).contiguous().cuda().transpose(1, 2) for n in NAMES}
    o = torch.full((B, Nq, H, d), float("nan"), device="cuda", dtype=torch.bfloat16).transpose(1, 2)
    do = torch.full_like(o, float("nan"))
    lse = torch.empty((B, H, Nq), device="cuda")
    dlse = torch.empty_like(lse)
    aj.fwd(*(g[n] for n in NAMES), out=(o, do, lse, dlse))
    torch.cuda.synchronize()
    for a, c in zip(flat, (o, do, lse, dlse)):
        assert torch.equal(a, c)


def test_custom_scale_unequal_dims():
    w = Workload("s", 1, 2, 100, 32, "bf16", 7100, tangent_scale=0.3, n_kv=250, d_v=256)
    _check(w, scale=0.5, what="scale dqk32 dv256")


def test_binding_rejects_inconsistent_shapes():
    w = Workload("r", 1, 1, 64, 64, "bf16", 7200, n_kv=80, d_v=32)
    g = {n: t.cuda() for n, t in make_inputs(w).items() if n in NAMES}
    with pytest.raises(ValueError):      # K and V with different Lkv
        aj.fwd(g["q"], g["k"][:, :, :70], g["v"], g["dq"], g["dk"][:, :, :70], g["dv"])
    with pytest.raises(ValueError):      # a tangent with another shape
        aj.fwd(g["q"], g["k"], g["v"], g["dq"], g["dk"], g["dv"][..., :16])
    # a frame window needs Lq == Lkv
    mask = dict(frames=2, tokens_per_frame=32, chunk_frames=1, radius_chunks=0)
    with pytest.raises(aj.AttnJvpError) as e:
        aj.fwd(*(g[n] for n in NAMES), mask=mask)
    assert e.value.status in (-2, -4)
