"""GPU: the entry points captured into a HIP graph (torch.cuda.CUDAGraph)
and replayed.  Every launch of the path is a plain kernel launch on the
caller's stream with no allocation, memset or host synchronisation inside,
so a captured call must replay to the eager result bit for bit.  Each graph
is replayed several times with eager work in between (the outputs refilled
with NaN, another eager call of the library on other inputs, a
synchronisation), and every replay is compared with the eager outputs.
"""

import pytest
import torch

import attention_jvp_amd as aj
from synth import Workload, make_inputs
from tolerances import say

pytestmark = pytest.mark.gpu

NAMES = ("q", "k", "v", "dq", "dk", "dv")
REPLAYS = 3
MASK = dict(frames=10, tokens_per_frame=60, chunk_frames=2, radius_chunks=1,
            anchor_first=1, anchor_last=1, anchor_queries_see_all=0)


def _inputs(name, B, H, N, d, dtype, seed, n_kv=None):
    w = Workload(name, B, H, N, d, dtype, seed, tangent_scale=0.1, n_kv=n_kv)
    x = make_inputs(w)
    return w, [x[n].cuda() for n in NAMES]


def _fwd_outs(w, like):
    o = torch.empty((w.B, w.H, w.N, w.dv), device="cuda", dtype=like.dtype)
    lse = torch.empty((w.B, w.H, w.N), device="cuda", dtype=torch.float32)
    return o, torch.empty_like(o), lse, torch.empty_like(lse)


def _check_replays(run, outs, between):
    """Eager result of run(), then REPLAYS replays of its captured graph,
    each after `between()` and with the outputs refilled with NaN."""
    run()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]
    # warm-up on a side stream, as torch asks before capture
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    torch.cuda.synchronize()
    for i in range(REPLAYS):
        for t in outs:
            t.fill_(float("nan"))
        between()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip(outs, ref):
            assert torch.equal(a, b), f"replay {i}"
    del graph


def _other_call():
    # eager work of the same library on other inputs and shapes
    w, g = _inputs("graph-other", 1, 3, 333, 64, "bf16", 9901)
    aj.fwd(*g)


@pytest.mark.parametrize("dtype,d,mask", [("bf16", 128, None), ("bf16", 64, None),
                                          ("bf16", 128, MASK), ("fp32", 64, None)])
def test_fwd_graph_replays(dtype, d, mask):
    say(f"graph fwd {dtype} d{d} mask {mask is not None}")
    w, g = _inputs("graph-fwd", 2, 3, 600, d, dtype, 9900 + d)
    outs = _fwd_outs(w, g[0])
    _check_replays(lambda: aj.fwd(*g, mask=mask, out=outs), outs, _other_call)


def test_fwd_splitkv_graph_replays():
    # split workgroups, then the merge kernel, with a caller workspace
    say("graph fwd_splitkv")
    w, g = _inputs("graph-sk", 1, 2, 100, 128, "bf16", 9910, n_kv=3000)
    outs = _fwd_outs(w, g[0])
    dt = aj.ATTN_JVP_BF16
    ns, need = aj.attn_jvp_splitkv_plan(aj.Shape(w.B, w.H, w.N, w.Nkv, w.d, w.dv), dt, None, 5)
    ws = torch.empty(need, device="cuda", dtype=torch.uint8)
    _check_replays(lambda: aj.fwd_splitkv(*g, num_splits=ns, workspace=ws, out=outs), outs,
                   _other_call)


def test_noalloc_splitkv_graph_replays():
    # the static-scratch entry point; the eager split-KV call between the
    # replays rewrites the same scratch
    say("graph fwd_splitkv_noalloc")
    w, g = _inputs("graph-na", 1, 2, 100, 128, "bf16", 9920, n_kv=2500)
    outs = _fwd_outs(w, g[0])
    dt = aj.ATTN_JVP_BF16
    shape = aj.Shape(w.B, w.H, w.N, w.Nkv, w.d, w.dv)
    lay = aj.layout_of(*g, *outs[:2])

    def run():
        st = aj.attn_jvp_fwd_splitkv_noalloc(*(t.data_ptr() for t in g),
                                             *(t.data_ptr() for t in outs), shape, 0.0, dt,
                                             lay, None, 4,
                                             torch.cuda.current_stream().cuda_stream)
        assert st == 0

    w2, g2 = _inputs("graph-na2", 1, 1, 64, 64, "bf16", 9921, n_kv=1500)

    def between():
        _other_call()
        aj.fwd_splitkv(*g2, num_splits=3)

    _check_replays(run, outs, between)


@pytest.mark.parametrize("mask", [None, MASK])
def test_bwd_graph_replays(mask):
    say(f"graph bwd mask {mask is not None}")
    w, g = _inputs("graph-bwd", 2, 3, 600, 128, "bf16", 9930)
    o, do, lse, dlse = aj.fwd(*g, mask=mask)
    go = torch.randn(o.shape, generator=torch.Generator().manual_seed(9931)).to(o.dtype).cuda()
    grads = (torch.empty_like(g[0]), torch.empty_like(g[1]), torch.empty_like(g[2]),
             torch.empty_like(lse))
    _check_replays(lambda: aj.bwd(g[0], g[1], g[2], o, go, lse, mask=mask, out=grads), grads,
                   _other_call)
