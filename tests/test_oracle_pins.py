"""Pins for the oracle's attention and attention-JVP definition.

Each check ties the oracle to something other than itself: a library routine
(torch's float64 CPU scaled_dot_product_attention, logsumexp and
torch.func.jvp), central finite differences, closed forms and invariants that
the pages' chain rule implies, and the pages' own streaming recurrence.
"""

import numpy as np
import pytest
import torch

from oracle import (FrameWindow, attention_jvp, attention_jvp_rows,
                    attention_jvp_streaming, merge_partials)


def _rand(rng, B, H, N, d, Nk=None, dv=None, scale_t=1.0):
    Nk = N if Nk is None else Nk
    dv = d if dv is None else dv
    q = rng.standard_normal((B, H, N, d))
    k = rng.standard_normal((B, H, Nk, d))
    v = rng.standard_normal((B, H, Nk, dv))
    dq = rng.standard_normal((B, H, N, d)) * scale_t
    dk = rng.standard_normal((B, H, Nk, d)) * scale_t
    dv_ = rng.standard_normal((B, H, Nk, dv)) * scale_t
    return q, k, v, dq, dk, dv_


def _t(x):
    return torch.from_numpy(np.ascontiguousarray(x))


SHAPES = [(1, 1, 1, 1, 1), (1, 2, 3, 4, 5), (2, 1, 17, 8, 17), (1, 2, 64, 64, 40)]


@pytest.mark.parametrize("B,H,N,d,Nk", SHAPES)
def test_forward_matches_torch_sdpa(B, H, N, d, Nk):
    rng = np.random.default_rng(1)
    q, k, v, dq, dk, dv = _rand(rng, B, H, N, d, Nk)
    o, _, lse, _ = attention_jvp(q, k, v, dq, dk, dv)
    ref = torch.nn.functional.scaled_dot_product_attention(_t(q), _t(k), _t(v))
    np.testing.assert_allclose(o, ref.numpy(), rtol=0, atol=1e-12)
    s = _t(q) @ _t(k).transpose(-1, -2) * d ** -0.5
    np.testing.assert_allclose(lse, torch.logsumexp(s, -1).numpy(), rtol=0, atol=1e-12)


@pytest.mark.parametrize("N,Nk,d,dv", [(9, 23, 16, 48), (40, 7, 32, 8), (1, 5, 4, 1)])
def test_forward_unequal_shapes_matches_torch_sdpa(N, Nk, d, dv):
    # cross-attention shapes: Lq != Lkv and d_v != d_qk (the pages' op contract)
    rng = np.random.default_rng(11)
    q, k, v, dq, dk, dv_ = _rand(rng, 2, 2, N, d, Nk=Nk, dv=dv)
    o, _, lse, _ = attention_jvp(q, k, v, dq, dk, dv_)
    assert o.shape == (2, 2, N, dv) and lse.shape == (2, 2, N)
    ref = torch.nn.functional.scaled_dot_product_attention(_t(q), _t(k), _t(v))
    np.testing.assert_allclose(o, ref.numpy(), rtol=0, atol=1e-12)
    s = _t(q) @ _t(k).transpose(-1, -2) * d ** -0.5
    np.testing.assert_allclose(lse, torch.logsumexp(s, -1).numpy(), rtol=0, atol=1e-12)


def test_forward_custom_scale_and_mask_matches_sdpa():
    rng = np.random.default_rng(2)
    q, k, v, dq, dk, dv = _rand(rng, 1, 2, 21, 6)
    w = FrameWindow(frames=7, tokens_per_frame=3, chunk_frames=2, radius_chunks=0,
                    anchor_first=True, anchor_last=False)
    vis = w(np.arange(21), np.arange(21))
    o, _, lse, _ = attention_jvp(q, k, v, dq, dk, dv, scale=0.37, visible=w)
    ref = torch.nn.functional.scaled_dot_product_attention(
        _t(q), _t(k), _t(v), attn_mask=torch.from_numpy(vis), scale=0.37)
    np.testing.assert_allclose(o, ref.numpy(), rtol=0, atol=1e-12)
    s = (_t(q) @ _t(k).transpose(-1, -2) * 0.37).masked_fill(~torch.from_numpy(vis), -np.inf)
    np.testing.assert_allclose(lse, torch.logsumexp(s, -1).numpy(), rtol=0, atol=1e-12)


def test_single_key_closed_form():
    # one key: P = 1, so O = V, LSE = s q.k, dO = dV, dLSE = s (dq.k + q.dk)
    rng = np.random.default_rng(3)
    q, k, v, dq, dk, dv = _rand(rng, 2, 3, 5, 7, Nk=1)
    s = 0.3
    o, do, lse, dlse = attention_jvp(q, k, v, dq, dk, dv, scale=s)
    np.testing.assert_allclose(o, np.broadcast_to(v, o.shape), atol=1e-14)
    np.testing.assert_allclose(do, np.broadcast_to(dv, do.shape), atol=1e-14)
    np.testing.assert_allclose(lse, s * (q @ k.transpose(0, 1, 3, 2))[..., 0], atol=1e-13)
    ref = s * (dq @ k.transpose(0, 1, 3, 2) + q @ dk.transpose(0, 1, 3, 2))[..., 0]
    np.testing.assert_allclose(dlse, ref, atol=1e-13)


def _fd(fun, x, t, h):
    def cd(hh):
        plus = fun(*[a + hh * b for a, b in zip(x, t)])
        minus = fun(*[a - hh * b for a, b in zip(x, t)])
        return [(p - m) / (2 * hh) for p, m in zip(plus, minus)]
    d1, d2 = cd(h), cd(h / 2)
    return [(4 * b - a) / 3 for a, b in zip(d1, d2)]      # Richardson


@pytest.mark.parametrize("N,d,Nk", [(1, 1, 1), (2, 4, 2), (3, 4, 3), (17, 64, 17), (5, 1, 9)])
def test_tangents_match_central_differences(N, d, Nk):
    rng = np.random.default_rng(10 + N + d)
    q, k, v, dq, dk, dv = _rand(rng, 1, 2, N, d, Nk)
    _, do, _, dlse = attention_jvp(q, k, v, dq, dk, dv)

    def fwd(q_, k_, v_):
        o_, _, lse_, _ = attention_jvp(q_, k_, v_, q_, k_, v_)
        return o_, lse_

    fd_o, fd_lse = _fd(fwd, (q, k, v), (dq, dk, dv), 1e-3)
    scale = max(1.0, np.abs(fd_o).max())
    np.testing.assert_allclose(do, fd_o, rtol=0, atol=1e-8 * scale)
    np.testing.assert_allclose(dlse, fd_lse, rtol=0, atol=1e-8 * max(1.0, np.abs(fd_lse).max()))


def test_tangents_match_central_differences_masked():
    rng = np.random.default_rng(11)
    w = FrameWindow(frames=5, tokens_per_frame=4, chunk_frames=2, radius_chunks=0,
                    anchor_first=False, anchor_last=True)
    q, k, v, dq, dk, dv = _rand(rng, 1, 1, 20, 8)
    _, do, _, dlse = attention_jvp(q, k, v, dq, dk, dv, visible=w)

    def fwd(q_, k_, v_):
        o_, _, lse_, _ = attention_jvp(q_, k_, v_, q_, k_, v_, visible=w)
        return o_, lse_

    fd_o, fd_lse = _fd(fwd, (q, k, v), (dq, dk, dv), 1e-3)
    np.testing.assert_allclose(do, fd_o, rtol=0, atol=1e-8)
    np.testing.assert_allclose(dlse, fd_lse, rtol=0, atol=1e-8)


def test_matches_torch_func_jvp():
    rng = np.random.default_rng(4)
    q, k, v, dq, dk, dv = _rand(rng, 2, 2, 33, 16, Nk=29, dv=12)
    s = 16 ** -0.5

    def f(q_, k_, v_):
        sc = q_ @ k_.transpose(-1, -2) * s
        return torch.softmax(sc, -1) @ v_, torch.logsumexp(sc, -1)

    (o_t, lse_t), (do_t, dlse_t) = torch.func.jvp(
        f, (_t(q), _t(k), _t(v)), (_t(dq), _t(dk), _t(dv)))
    o, do, lse, dlse = attention_jvp(q, k, v, dq, dk, dv)
    np.testing.assert_allclose(o, o_t.numpy(), atol=1e-12)
    np.testing.assert_allclose(lse, lse_t.numpy(), atol=1e-12)
    np.testing.assert_allclose(do, do_t.numpy(), atol=1e-12)
    np.testing.assert_allclose(dlse, dlse_t.numpy(), atol=1e-12)


def test_zero_score_tangent_gives_p_times_dv():
    # dQ = dK = 0 => t_s = 0 => dO = P dV exactly and dLSE = 0
    rng = np.random.default_rng(5)
    q, k, v, dq, dk, dv = _rand(rng, 1, 3, 40, 8)
    z = np.zeros_like(q)
    _, do, _, dlse = attention_jvp(q, k, v, z, np.zeros_like(k), dv)
    o_dv, _, _, _ = attention_jvp(q, k, dv, z, np.zeros_like(k), dv)
    np.testing.assert_allclose(do, o_dv, rtol=0, atol=1e-13)
    assert np.all(dlse == 0)


def test_value_tangent_equal_to_value_gives_output():
    rng = np.random.default_rng(6)
    q, k, v, _, _, _ = _rand(rng, 1, 2, 30, 8)
    o, do, _, _ = attention_jvp(q, k, v, np.zeros_like(q), np.zeros_like(k), v)
    np.testing.assert_allclose(do, o, rtol=0, atol=1e-13)


def test_linear_in_tangents():
    rng = np.random.default_rng(7)
    q, k, v, dq1, dk1, dv1 = _rand(rng, 1, 2, 25, 8)
    _, _, _, dq2, dk2, dv2 = _rand(rng, 1, 2, 25, 8)
    a, b = 0.7, -1.9
    _, do1, _, dl1 = attention_jvp(q, k, v, dq1, dk1, dv1)
    _, do2, _, dl2 = attention_jvp(q, k, v, dq2, dk2, dv2)
    _, do12, _, dl12 = attention_jvp(q, k, v, a * dq1 + b * dq2, a * dk1 + b * dk2,
                                     a * dv1 + b * dv2)
    np.testing.assert_allclose(do12, a * do1 + b * do2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(dl12, a * dl1 + b * dl2, rtol=0, atol=1e-12)


def test_row_constant_score_tangent_is_absorbed_by_softmax():
    # dQ = 0, every dK_j = c: t_s is constant along each row, the softmax
    # ignores it, so dO = P dV and dLSE = s q.c
    rng = np.random.default_rng(8)
    q, k, v, _, _, dv = _rand(rng, 1, 2, 19, 8, Nk=23)
    c = rng.standard_normal(8)
    dk = np.broadcast_to(c, k.shape).copy()
    s = 0.25
    _, do, _, dlse = attention_jvp(q, k, v, np.zeros_like(q), dk, dv, scale=s)
    o_dv, _, _, _ = attention_jvp(q, k, dv, q, k, dv, scale=s)
    np.testing.assert_allclose(do, o_dv, rtol=0, atol=1e-12)
    np.testing.assert_allclose(dlse, s * (q @ c), rtol=0, atol=1e-12)


@pytest.mark.parametrize("block", [1, 7, 16, 64, 128])
def test_streaming_recurrence_matches_dense(block):
    rng = np.random.default_rng(9)
    q, k, v, dq, dk, dv = _rand(rng, 1, 2, 37, 16, Nk=100)
    dense = attention_jvp(q, k, v, dq, dk, dv)
    stream = attention_jvp_streaming(q, k, v, dq, dk, dv, block)
    for a, b in zip(dense, stream):
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)


def test_streaming_recurrence_matches_dense_masked():
    rng = np.random.default_rng(12)
    w = FrameWindow(frames=7, tokens_per_frame=5, chunk_frames=2, radius_chunks=1)
    q, k, v, dq, dk, dv = _rand(rng, 1, 1, 35, 8)
    dense = attention_jvp(q, k, v, dq, dk, dv, visible=w)
    stream = attention_jvp_streaming(q, k, v, dq, dk, dv, 4, visible=w)
    for a, b in zip(dense, stream):
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)


def test_split_kv_merge_identity():
    # results over two disjoint key sets merge into the full result computed
    # directly from the definition
    rng = np.random.default_rng(13)
    q, k, v, dq, dk, dv = _rand(rng, 1, 2, 11, 8, Nk=30)
    full = attention_jvp(q, k, v, dq, dk, dv)
    sl = [slice(0, 13), slice(13, 30)]
    parts = [attention_jvp(q, k[:, :, s], v[:, :, s], dq, dk[:, :, s], dv[:, :, s]) for s in sl]
    for a, b in zip(full, merge_partials(parts)):
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)


def test_merge_with_empty_parts_and_empty_rows():
    # a frame window split into key ranges: some rows see no key of a range
    # (LSE_k = -inf there); rows of a query frame cut off from every key
    # (a window with no anchors over a key subset) stay empty after the merge
    rng = np.random.default_rng(17)
    N = 24
    q, k, v, dq, dk, dv = _rand(rng, 1, 2, N, 6, dv=5)
    w = FrameWindow(frames=8, tokens_per_frame=3, chunk_frames=2, radius_chunks=0,
                    anchor_first=True, anchor_last=False)
    full = attention_jvp(q, k, v, dq, dk, dv, visible=w)
    cuts = [0, 5, 6, 17, 24]
    parts = []
    for a, b in zip(cuts[:-1], cuts[1:]):
        vis = (lambda a_: (lambda qi, ki: w(qi, ki + a_)))(a)
        parts.append(attention_jvp(q, k[:, :, a:b], v[:, :, a:b], dq, dk[:, :, a:b],
                                   dv[:, :, a:b], visible=vis))
    assert any(np.isneginf(p[2]).any() for p in parts)
    merged = merge_partials(parts)
    for a, b in zip(full, merged):
        np.testing.assert_array_equal(np.isfinite(a), np.isfinite(b))
        fin = np.isfinite(a)
        np.testing.assert_allclose(a[fin], b[fin], rtol=0, atol=1e-12)
    # keys 12..23 only: query frames 0..1 (chunk 0) see nothing there
    sub = attention_jvp(q, k[:, :, 12:], v[:, :, 12:], dq, dk[:, :, 12:], dv[:, :, 12:],
                        visible=lambda qi, ki: w(qi, ki + 12))
    o, do, lse, dlse = merge_partials([sub, sub])
    rows = np.arange(6)
    assert np.isneginf(lse[:, :, rows]).all()
    assert (o[:, :, rows] == 0).all() and (do[:, :, rows] == 0).all()
    assert (dlse[:, :, rows] == 0).all()


def test_invisible_keys_do_not_matter():
    rng = np.random.default_rng(14)
    w = FrameWindow(frames=6, tokens_per_frame=3, chunk_frames=2, radius_chunks=0,
                    anchor_first=False, anchor_last=False)
    q, k, v, dq, dk, dv = _rand(rng, 1, 1, 18, 4)
    base = attention_jvp(q, k, v, dq, dk, dv, visible=w)
    # rows of frames 0..1 (chunk 0) cannot see keys of frames 2..5
    k2, v2, dk2, dv2 = (x.copy() for x in (k, v, dk, dv))
    for x in (k2, v2, dk2, dv2):
        x[:, :, 6:] = rng.standard_normal(x[:, :, 6:].shape) * 100
    pert = attention_jvp(q, k2, v2, dq, dk2, dv2, visible=w)
    for a, b in zip(base, pert):
        np.testing.assert_array_equal(a[:, :, :6], b[:, :, :6])


def test_row_subset_equals_full_rows():
    rng = np.random.default_rng(15)
    q, k, v, dq, dk, dv = _rand(rng, 2, 2, 50, 8)
    rows = np.array([0, 3, 17, 49])
    full = attention_jvp(q, k, v, dq, dk, dv)
    sub = attention_jvp_rows(q, k, v, dq, dk, dv, rows, row_chunk=3)
    for a, b in zip(full, sub):
        np.testing.assert_allclose(a[:, :, rows], b, rtol=0, atol=1e-14)


def test_row_with_no_visible_key_convention():
    rng = np.random.default_rng(16)
    q, k, v, dq, dk, dv = _rand(rng, 1, 1, 4, 3)

    def vis(qi, ki):
        m = np.ones((len(qi), len(ki)), bool)
        m[np.asarray(qi) == 2] = False
        return m

    o, do, lse, dlse = attention_jvp(q, k, v, dq, dk, dv, visible=vis)
    assert np.all(o[0, 0, 2] == 0) and np.all(do[0, 0, 2] == 0)
    assert lse[0, 0, 2] == -np.inf and dlse[0, 0, 2] == 0
    assert np.all(np.isfinite(o[0, 0, [0, 1, 3]]))
