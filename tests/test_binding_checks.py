"""CPU: the Python binding rejects caller tensors the C side cannot check
(wrong shape, dtype, device or contiguity of out= tensors, the saved lse,
the split-KV workspace, host tensors), before any pointer reaches the
library.  No GPU and no library call is needed: every case raises first.
"""

import pytest
import torch

import attention_jvp_amd as aj

B, H, LQ, LKV, DQK, DV = 1, 2, 33, 40, 64, 32


def _inputs(dtype=torch.bfloat16):
    q = torch.zeros((B, H, LQ, DQK), dtype=dtype)
    k = torch.zeros((B, H, LKV, DQK), dtype=dtype)
    v = torch.zeros((B, H, LKV, DV), dtype=dtype)
    return q, k, v, q.clone(), k.clone(), v.clone()


def _good_out(dtype=torch.bfloat16):
    o = torch.empty((B, H, LQ, DV), dtype=dtype)
    lse = torch.empty((B, H, LQ), dtype=torch.float32)
    return [o, o.clone(), lse, lse.clone()]


def test_good_out_passes_the_checks():
    x = _inputs()
    dt, shape = aj.check_qkv(*x)
    assert dt == aj.ATTN_JVP_BF16 and (shape.seqlen_q, shape.head_dim_v) == (LQ, DV)
    aj.check_fwd_out(_good_out(), x[0], shape)


@pytest.mark.parametrize("slot,bad", [
    (0, lambda t: t[:, :, :-1]),                        # o one row short
    (1, lambda t: t.float()),                           # do in float32 next to bf16 inputs
    (2, lambda t: torch.empty((B, H, LQ - 1))),         # lse one row short
    (3, lambda t: torch.empty((B, H, 2 * LQ))[..., ::2]),   # dlse not contiguous
    (2, lambda t: t.double()),                          # lse not float32
    (0, lambda t: torch.empty((B, H, LQ, DV), dtype=torch.bfloat16, device="meta")),
    (0, lambda t: torch.empty((B, H, DV, LQ), dtype=torch.bfloat16).transpose(2, 3)),
])
def test_fwd_out_rejected(slot, bad):
    x = _inputs()
    out = _good_out()
    out[slot] = bad(out[slot])
    _, shape = aj.check_qkv(*x)
    with pytest.raises(ValueError):
        aj.check_fwd_out(out, x[0], shape)
    with pytest.raises(ValueError):
        aj.fwd(*x, out=tuple(out))


def test_host_tensors_rejected_before_the_library():
    x = _inputs()
    with pytest.raises(ValueError, match="GPU"):
        aj.fwd(*x)
    with pytest.raises(ValueError, match="GPU"):
        aj.fwd_splitkv(*x)
    with pytest.raises(ValueError, match="GPU"):
        aj.fwd_partial(*x)


def test_inputs_must_agree():
    q, k, v, dq, dk, dv = _inputs()
    with pytest.raises(ValueError):
        aj.check_qkv(q, k, v, dq.float(), dk, dv)
    with pytest.raises(ValueError):
        aj.check_qkv(q, k, v[:, :, :-1], dq, dk, dv[:, :, :-1])
    with pytest.raises(ValueError):
        aj.check_qkv(q, k, v, dq[:, :, :-1], dk, dv)


def _bwd_args():
    q = torch.zeros((B, H, LQ, DQK), dtype=torch.bfloat16)
    k = torch.zeros((B, H, LKV, DQK), dtype=torch.bfloat16)
    v = torch.zeros((B, H, LKV, DQK), dtype=torch.bfloat16)
    o = torch.zeros((B, H, LQ, DQK), dtype=torch.bfloat16)
    lse = torch.zeros((B, H, LQ), dtype=torch.float32)
    return q, k, v, o, o.clone(), lse


def test_bwd_checks():
    q, k, v, o, go, lse = _bwd_args()
    aj.check_bwd_args(q, k, v, o, go, lse)
    with pytest.raises(ValueError):                     # lse short
        aj.check_bwd_args(q, k, v, o, go, lse[:, :, :-1])
    with pytest.raises(ValueError):                     # lse strided
        aj.check_bwd_args(q, k, v, o, go, torch.zeros((B, H, 2 * LQ))[..., ::2])
    with pytest.raises(ValueError):                     # lse on another device
        aj.check_bwd_args(q, k, v, o, go, lse.to("meta"))
    good = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v),
            torch.empty((B, H, LQ), dtype=torch.float32))
    aj.check_bwd_args(q, k, v, o, go, lse, good)
    for slot, bad in ((0, good[0][:, :, :-1]), (1, good[1].float()), (2, good[2].to("meta")),
                      (3, torch.empty((B, H, 2 * LQ))[..., ::2])):
        out = list(good)
        out[slot] = bad
        with pytest.raises(ValueError):
            aj.check_bwd_args(q, k, v, o, go, lse, tuple(out))
        with pytest.raises(ValueError):
            aj.bwd(q, k, v, o, go, lse, out=tuple(out))
    with pytest.raises(ValueError, match="GPU"):
        aj.bwd(q, k, v, o, go, lse)


def test_merge_checks():
    P = 3
    op = torch.zeros((P, B, H, LQ, DV))
    lp = torch.zeros((P, B, H, LQ))
    aj.check_merge(op, op.clone(), lp, lp.clone(), torch.bfloat16)
    with pytest.raises(ValueError):
        aj.check_merge(op, op.transpose(3, 4).contiguous().transpose(3, 4)[..., :DV], lp, lp,
                       torch.bfloat16)
    with pytest.raises(ValueError):
        aj.check_merge(op, op, lp[:2], lp, torch.bfloat16)
    with pytest.raises(ValueError):
        aj.check_merge(op, op, lp, lp.double(), torch.bfloat16)
    out = _good_out(torch.float32)
    with pytest.raises(ValueError):                     # out dtype is not the requested one
        aj.check_merge(op, op, lp, lp, torch.bfloat16, out)
    aj.check_merge(op, op, lp, lp, torch.float32, out)
    with pytest.raises(ValueError, match="GPU"):
        aj.merge(op, op, lp, lp, torch.float32)


def test_workspace_checks():
    dev = torch.device("cpu")
    ws = torch.empty(1024, dtype=torch.uint8)
    assert aj.check_workspace(ws, 1000, dev) == 1024
    with pytest.raises(ValueError):
        aj.check_workspace(ws, 1025, dev)
    with pytest.raises(ValueError):
        aj.check_workspace(ws.to("meta"), 10, dev)
    with pytest.raises(ValueError):
        aj.check_workspace(torch.empty((64, 64), dtype=torch.uint8).t(), 10, dev)
