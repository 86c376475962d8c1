"""GPU parity for key splits: attn_jvp_fwd_splitkv (split workgroups + merge
kernel), attn_jvp_fwd_partial over key ranges merged with attn_jvp_merge
(the ring-style building block), and the merge kernel alone on the oracle's
own partials.  References: the float64 oracle's full result (every row) and
its merge of partials.
"""

import numpy as np
import pytest
import torch

import attention_jvp_amd as aj
from oracle import FrameWindow, attention_jvp, merge_partials
from synth import Workload, make_inputs, to_float64
from tolerances import compare_fwd, say

pytestmark = pytest.mark.gpu

NAMES = ("q", "k", "v", "dq", "dk", "dv")
_say = say


def _compare(gpu, ref, dtype, what, ceiling=None):
    compare_fwd(gpu, ref, dtype, what, ceiling=ceiling)


def _vis(mask):
    return None if mask is None else FrameWindow(
        **{k: bool(v) if k.startswith("anchor") else v for k, v in mask.items()})


@pytest.mark.parametrize("dtype,B,H,Lq,Lkv,d,dv,splits", [
    ("bf16", 1, 2, 100, 3000, 128, 128, 2),
    ("bf16", 1, 2, 100, 3000, 128, 128, 5),
    ("bf16", 1, 2, 100, 3000, 128, 128, 0),
    ("bf16", 2, 1, 37, 2100, 64, 64, 7),
    ("bf16", 1, 1, 130, 1000, 256, 64, 3),
    ("bf16", 1, 2, 64, 300, 128, 128, 64),      # more splits than key tiles
    ("bf16", 2, 3, 1, 3000, 128, 128, 0),       # one query row
    ("bf16", 1, 2, 50, 1, 64, 64, 4),           # one key, more splits than tiles
    ("fp32", 1, 2, 64, 1500, 64, 32, 4),
])
def test_splitkv_matches_oracle(dtype, B, H, Lq, Lkv, d, dv, splits):
    _say(f"splitkv {dtype} B{B} H{H} Lq{Lq} Lkv{Lkv} d{d}/{dv} splits{splits}")
    w = Workload("sk", B, H, Lq, d, dtype, 8000 + Lq + Lkv + splits, tangent_scale=0.1,
                 n_kv=Lkv, d_v=dv)
    x = make_inputs(w)
    g = [x[n].cuda() for n in NAMES]
    o, do, lse, dlse, ns = aj.fwd_splitkv(*g, num_splits=splits)
    torch.cuda.synchronize()
    assert ns >= 1 and (splits == 0 or ns == splits)
    ref = attention_jvp(*(to_float64(x[n]) for n in NAMES))
    _compare([to_float64(t) for t in (o, do, lse, dlse)], ref, dtype, f"splitkv ns{ns}")


def test_splitkv_frame_window():
    # splits of a masked walk: some splits hold no key a row can see
    mask = dict(frames=10, tokens_per_frame=60, chunk_frames=2, radius_chunks=0,
                anchor_first=1, anchor_last=1, anchor_queries_see_all=0)
    w = Workload("skm", 1, 2, 600, 128, "bf16", 8100, tangent_scale=0.1)
    x = make_inputs(w)
    g = [x[n].cuda() for n in NAMES]
    for splits in (3, 6):
        o, do, lse, dlse, ns = aj.fwd_splitkv(*g, mask=mask, num_splits=splits)
        torch.cuda.synchronize()
        ref = attention_jvp(*(to_float64(x[n]) for n in NAMES), visible=_vis(mask))
        _compare([to_float64(t) for t in (o, do, lse, dlse)], ref, "bf16", f"splitkv mask ns{ns}")


def test_splitkv_strided_views():
    # inputs and outputs stored [B, N, H, d] and passed as [B, H, N, d] views
    B, H, Lq, Lkv, d = 1, 3, 90, 2500, 128
    w = Workload("skv", B, H, Lq, d, "bf16", 8600, tangent_scale=0.1, n_kv=Lkv)
    x = make_inputs(w)
    bshd = lambda t: t.transpose(1, 2).contiguous().cuda().transpose(1, 2)
    g = [bshd(x[n]) for n in NAMES]
    o = bshd(torch.zeros((B, H, Lq, d), dtype=torch.bfloat16))
    do = bshd(torch.zeros((B, H, Lq, d), dtype=torch.bfloat16))
    lse = torch.empty((B, H, Lq), device="cuda")
    dlse = torch.empty_like(lse)
    _, _, _, _, ns = aj.fwd_splitkv(*g, num_splits=5, out=(o, do, lse, dlse))
    torch.cuda.synchronize()
    assert ns == 5 and o.stride() == (Lq * H * d, d, H * d, 1)
    ref = attention_jvp(*(to_float64(x[n]) for n in NAMES))
    _compare([to_float64(t) for t in (o, do, lse, dlse)], ref, "bf16", "splitkv bshd")


def test_one_split_is_fwd_ex_bitwise():
    w = Workload("sk1", 1, 2, 200, 128, "bf16", 8200, tangent_scale=0.1, n_kv=700)
    x = make_inputs(w)
    g = [x[n].cuda() for n in NAMES]
    a = aj.fwd(*g)
    b = aj.fwd_splitkv(*g, num_splits=1)[:4]
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_splitkv_deterministic():
    w = Workload("skd", 1, 2, 64, 128, "bf16", 8300, tangent_scale=0.1, n_kv=2000)
    x = make_inputs(w)
    g = [x[n].cuda() for n in NAMES]
    a = aj.fwd_splitkv(*g, num_splits=6)[:4]
    b = aj.fwd_splitkv(*g, num_splits=6)[:4]
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_partials_over_key_ranges_then_merge(dtype):
    # ring-style: each call sees one key range (views into K, V, dK, dV)
    w = Workload("ring", 2, 2, 150, 64, dtype, 8400, tangent_scale=0.1, n_kv=1000, d_v=32)
    x = make_inputs(w)
    g = {n: x[n].cuda() for n in NAMES}
    cuts = [0, 256, 264, 700, 1000]
    parts = []
    for a, b in zip(cuts[:-1], cuts[1:]):
        sl = slice(a, b)
        parts.append(aj.fwd_partial(g["q"], g["k"][:, :, sl], g["v"][:, :, sl], g["dq"],
                                    g["dk"][:, :, sl], g["dv"][:, :, sl]))
    stack = [torch.stack([p[i] for p in parts]).contiguous() for i in range(4)]
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    out = aj.merge(*stack, tdt)
    torch.cuda.synchronize()
    ref = attention_jvp(*(to_float64(x[n]) for n in NAMES))
    _compare([to_float64(t) for t in out], ref, dtype, f"ring {dtype}")
    # each partial on its own is the attention JVP over its key range
    a, b = cuts[1], cuts[2]
    sub = attention_jvp(to_float64(x["q"]), to_float64(x["k"][:, :, a:b]),
                        to_float64(x["v"][:, :, a:b]), to_float64(x["dq"]),
                        to_float64(x["dk"][:, :, a:b]), to_float64(x["dv"][:, :, a:b]))
    _compare([to_float64(t) for t in parts[1]], sub, dtype, f"partial {dtype}")


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_merge_kernel_on_oracle_partials(out_dtype):
    # the merge alone, fed the oracle's float64 partials rounded to float32
    # (one part empty for some rows, some rows empty in every part)
    rng = np.random.default_rng(21)
    B, H, N, d, dv = 1, 3, 96, 16, 64
    q, k, v = (rng.standard_normal((B, H, N, d)), rng.standard_normal((B, H, N, d)),
               rng.standard_normal((B, H, N, dv)))
    dq, dk, dvv = (0.1 * rng.standard_normal(t.shape) for t in (q, k, v))
    win = FrameWindow(frames=8, tokens_per_frame=12, chunk_frames=2, radius_chunks=0,
                      anchor_first=False, anchor_last=False)
    cuts = [48, 72, 96]       # keys 48..95 only: query chunk 0 sees none of them
    parts = []
    for a, b in zip(cuts[:-1], cuts[1:]):
        vis = (lambda a_: (lambda qi, ki: win(qi, ki + a_)))(a)
        parts.append(attention_jvp(q, k[:, :, a:b], v[:, :, a:b], dq, dk[:, :, a:b],
                                   dvv[:, :, a:b], visible=vis))
    ref = merge_partials(parts)
    stack = [torch.from_numpy(np.stack([p[i] for p in parts])).float().contiguous().cuda()
             for i in range(4)]
    out = aj.merge(*stack, out_dtype)
    torch.cuda.synchronize()
    got = [to_float64(t) for t in out]
    assert np.isneginf(ref[2]).any()
    # float32 partials in, one rounding of the result: 2e-6 in float32, the
    # bfloat16 output rounding u = 2^-8 otherwise
    c = 2e-6 if out_dtype == torch.float32 else 2.0 ** -8
    _compare(got, ref, "fp32" if out_dtype == torch.float32 else "bf16", f"merge {out_dtype}",
             ceiling={"O": c, "dO": c, "dLSE": 2e-6})


def test_splitkv_errors_launch_nothing():
    w = Workload("ske", 1, 1, 64, 128, "bf16", 8500, n_kv=2000)
    x = make_inputs(w)
    g = [x[n].cuda() for n in NAMES]
    shape = aj.Shape(1, 1, 64, 2000, 128, 128)
    ns, need = aj.attn_jvp_splitkv_plan(shape, aj.ATTN_JVP_BF16, None, 4)
    assert ns == 4 and need > 0
    small = torch.empty(need - 256, device="cuda", dtype=torch.uint8)
    # the binding refuses a short workspace before the call ...
    with pytest.raises(ValueError):
        aj.fwd_splitkv(*g, num_splits=4, workspace=small)
    # ... and so does the C entry point
    o = torch.empty((1, 1, 64, 128), device="cuda", dtype=torch.bfloat16)
    do = torch.empty_like(o)
    lse = torch.empty((1, 1, 64), device="cuda")
    dlse = torch.empty_like(lse)
    lay = aj.layout_of(*g, o, do)
    st = aj.attn_jvp_fwd_splitkv(*(t.data_ptr() for t in g), o.data_ptr(), do.data_ptr(),
                                 lse.data_ptr(), dlse.data_ptr(), shape, 0.0, aj.ATTN_JVP_BF16,
                                 lay, None, 4, small.data_ptr(), need - 256,
                                 torch.cuda.current_stream().cuda_stream)
    assert st == -1
    # a workspace that overlaps an input
    with pytest.raises(aj.AttnJvpError) as e:
        big = torch.empty(need + 2 * 2000 * 128 * 2, device="cuda", dtype=torch.uint8)
        kk = big[:2000 * 128 * 2].view(torch.bfloat16).view(1, 1, 2000, 128)
        kk.copy_(g[1])
        aj.fwd_splitkv(g[0], kk, g[2], g[3], g[4], g[5], num_splits=4, workspace=big)
    assert e.value.status == -3
