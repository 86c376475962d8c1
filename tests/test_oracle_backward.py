"""Pins for the oracle's primal backward: torch autograd of a plain float64
attention (a library routine), central differences of sum(G ⊙ O), and
closed forms."""

import numpy as np
import pytest
import torch

from oracle import FrameWindow, attention_backward, attention_jvp


def _rand(rng, B, H, N, d, Nk=None, dv=None):
    Nk = N if Nk is None else Nk
    dv = d if dv is None else dv
    return (rng.standard_normal((B, H, N, d)), rng.standard_normal((B, H, Nk, d)),
            rng.standard_normal((B, H, Nk, dv)), rng.standard_normal((B, H, N, dv)))


@pytest.mark.parametrize("B,H,N,Nk,d,dv,scale", [
    (1, 1, 1, 1, 4, 4, None), (2, 2, 9, 9, 8, 8, None), (1, 2, 17, 5, 16, 16, 0.3),
    (1, 1, 6, 30, 4, 12, None),
])
def test_matches_torch_autograd(B, H, N, Nk, d, dv, scale):
    rng = np.random.default_rng(31)
    q, k, v, g = _rand(rng, B, H, N, d, Nk, dv)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    s = d ** -0.5 if scale is None else scale
    o = torch.softmax(tq @ tk.transpose(-1, -2) * s, -1) @ tv
    o.backward(torch.from_numpy(g))
    dq, dk, dv_ = attention_backward(q, k, v, g, scale=scale)
    np.testing.assert_allclose(dq, tq.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dv_, tv.grad.numpy(), atol=1e-12)


def test_matches_central_differences_of_the_loss():
    # L = sum(G ⊙ O(q, k, v)); dL/dx along a random direction
    rng = np.random.default_rng(32)
    q, k, v, g = _rand(rng, 1, 2, 7, 5, Nk=11)
    dq, dk, dv = attention_backward(q, k, v, g)

    def loss(q_, k_, v_):
        zero = np.zeros_like
        o = attention_jvp(q_, k_, v_, zero(q_), zero(k_), zero(v_))[0]
        return float((g * o).sum())

    for x, grad, idx in ((q, dq, 0), (k, dk, 1), (v, dv, 2)):
        t = rng.standard_normal(x.shape)
        h = 1e-5
        args_p = [q, k, v]
        args_m = [q, k, v]
        args_p[idx] = x + h * t
        args_m[idx] = x - h * t
        fd = (loss(*args_p) - loss(*args_m)) / (2 * h)
        assert abs(fd - float((grad * t).sum())) < 1e-7 * max(1.0, abs(fd))


def test_masked_matches_torch_autograd():
    rng = np.random.default_rng(33)
    w = FrameWindow(frames=6, tokens_per_frame=3, chunk_frames=2, radius_chunks=0,
                    anchor_first=True, anchor_last=False)
    q, k, v, g = _rand(rng, 1, 2, 18, 6)
    vis = torch.from_numpy(w(np.arange(18), np.arange(18)))
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    sc = (tq @ tk.transpose(-1, -2) * 6 ** -0.5).masked_fill(~vis, -np.inf)
    (torch.softmax(sc, -1) @ tv).backward(torch.from_numpy(g))
    dq, dk, dv = attention_backward(q, k, v, g, visible=w)
    for a, b in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        np.testing.assert_allclose(a, b.numpy(), atol=1e-12)


def test_single_key_and_uniform_scores():
    rng = np.random.default_rng(34)
    # one key: P = 1, so dV = sum_i G_i and dS = 0 (dQ = dK = 0)
    q, k, v, g = _rand(rng, 1, 1, 5, 4, Nk=1)
    dq, dk, dv = attention_backward(q, k, v, g)
    np.testing.assert_allclose(dv[0, 0, 0], g[0, 0].sum(axis=0), atol=1e-13)
    assert np.abs(dq).max() < 1e-14 and np.abs(dk).max() < 1e-14
    # q = 0: P uniform over keys, so dV_j = (1/Nk) sum_i G_i for every key
    q, k, v, g = _rand(rng, 1, 1, 4, 3, Nk=6)
    q[:] = 0
    _, _, dv = attention_backward(q, k, v, g)
    np.testing.assert_allclose(dv[0, 0], np.broadcast_to(g[0, 0].sum(0) / 6, (6, 3)), atol=1e-13)
