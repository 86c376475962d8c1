"""GPU: the allocation-free split-KV entry point (attn_jvp_fwd_splitkv_noalloc,
partials in the library's static device scratch) against the entry point it
varies (attn_jvp_fwd_splitkv with a caller workspace) and the float64
oracle.  Two calls in a row, the second on a smaller input, must each equal
the workspace path bitwise (same kernels, same split count) and the oracle
under the bounds of tests/tolerances.py; a split count whose partials exceed
the scratch is refused with ATTN_JVP_ENOSCRATCH and launches nothing, and the
plan's own choice shrinks to the splits that fit.
"""

import numpy as np
import pytest
import torch

import attention_jvp_amd as aj
from oracle import FrameWindow, attention_jvp, attention_jvp_rows
from synth import Workload, make_inputs, to_float64
from tolerances import compare_fwd, say

pytestmark = pytest.mark.gpu

NAMES = ("q", "k", "v", "dq", "dk", "dv")
ENOSCRATCH = -6


def _outs(w, dtype):
    o = torch.full((w.B, w.H, w.N, w.dv), 7.0, device="cuda", dtype=dtype)
    lse = torch.full((w.B, w.H, w.N), 7.0, device="cuda")
    return o, o.clone(), lse, lse.clone()


def _noalloc(g, outs, w, mask, num_splits):
    dt = aj.ATTN_JVP_BF16 if w.dtype == "bf16" else aj.ATTN_JVP_FP32
    shape = aj.Shape(w.B, w.H, w.N, w.Nkv, w.d, w.dv)
    lay = aj.layout_of(*g, *outs[:2])
    return aj.attn_jvp_fwd_splitkv_noalloc(*(t.data_ptr() for t in g),
                                           *(t.data_ptr() for t in outs), shape, 0.0, dt, lay,
                                           mask, num_splits,
                                           torch.cuda.current_stream().cuda_stream)


def _vis(mask):
    return None if mask is None else FrameWindow(
        **{k: bool(v) if k.startswith("anchor") else v for k, v in mask.items()})


@pytest.mark.parametrize("first,second", [
    # (workload, mask, splits): the second call is smaller than the first
    ((Workload("na1", 2, 3, 200, 128, "bf16", 8800, tangent_scale=0.1, n_kv=3000), None, 5),
     (Workload("na2", 1, 2, 64, 64, "bf16", 8801, tangent_scale=0.1, n_kv=1000), None, 3)),
    ((Workload("na3", 1, 2, 600, 128, "bf16", 8802, tangent_scale=0.1),
      dict(frames=10, tokens_per_frame=60, chunk_frames=2, radius_chunks=0, anchor_first=1,
           anchor_last=1, anchor_queries_see_all=0), 4),
     (Workload("na4", 1, 1, 90, 64, "fp32", 8803, tangent_scale=0.1, n_kv=700, d_v=32),
      None, 0)),
])
def test_noalloc_equals_workspace_path_twice(first, second):
    for w, mask, splits in (first, second):
        say(f"noalloc {w.name} B{w.B} H{w.H} Lq{w.N} Lkv{w.Nkv} {w.dtype} splits {splits}")
        x = make_inputs(w)
        g = [x[n].cuda() for n in NAMES]
        tdt = g[0].dtype
        outs = _outs(w, tdt)
        st = _noalloc(g, outs, w, mask, splits)
        assert st == 0, aj.attn_jvp_status_string(st)
        ref_outs = aj.fwd_splitkv(*g, mask=mask, num_splits=splits)
        torch.cuda.synchronize()
        assert ref_outs[4] > 1 or splits == 0
        for a, b in zip(outs, ref_outs[:4]):
            assert torch.equal(a, b)
        ref = attention_jvp(*(to_float64(x[n]) for n in NAMES), visible=_vis(mask))
        compare_fwd([to_float64(t) for t in outs], ref, w.dtype, f"noalloc {w.name}")


def test_noalloc_scratch_limit():
    # 16 heads x 128 queries x 32 splits of d_v = 128 partials: 65,536 rows of
    # 1,032 bytes, just over the 64 MiB scratch
    w = Workload("nal", 1, 16, 128, 128, "bf16", 8810, tangent_scale=0.1, n_kv=65536)
    shape = aj.Shape(w.B, w.H, w.N, w.Nkv, w.d, w.dv)
    ns32, need32 = aj.attn_jvp_splitkv_plan(shape, aj.ATTN_JVP_BF16, None, 32)
    assert need32 > aj.NOALLOC_SCRATCH_BYTES
    x = make_inputs(w)
    g = [x[n].cuda() for n in NAMES]
    outs = _outs(w, torch.bfloat16)
    assert _noalloc(g, outs, w, None, 32) == ENOSCRATCH
    torch.cuda.synchronize()
    assert all(torch.all(t == 7.0) for t in outs)          # nothing was launched
    # the plan's own choice, shrunk to the splits that fit
    ns, need = aj.attn_jvp_splitkv_plan(shape, aj.ATTN_JVP_BF16, None, 0)
    while ns > 1 and aj.attn_jvp_splitkv_plan(shape, aj.ATTN_JVP_BF16, None, ns)[1] > \
            aj.NOALLOC_SCRATCH_BYTES:
        ns -= 1
    assert ns > 1
    assert _noalloc(g, outs, w, None, 0) == 0
    ref_outs = aj.fwd_splitkv(*g, num_splits=ns)
    torch.cuda.synchronize()
    for a, b in zip(outs, ref_outs[:4]):
        assert torch.equal(a, b)
    rows = np.array([0, 1, 63, 64, 127])
    idx = torch.from_numpy(rows).cuda()
    got = [to_float64(t.index_select(2, idx)) for t in outs]
    ref = attention_jvp_rows(*(x[n].float().numpy() for n in NAMES), rows)
    compare_fwd(got, ref, "bf16", f"noalloc shrunk to {ns} splits")
