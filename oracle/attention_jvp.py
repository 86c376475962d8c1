"""Dense float64 definition of attention and its forward-mode derivative.

TEST INFRASTRUCTURE (the oracle): never imported by the library.

Page "带分数正则的一致性蒸馏" (gitcode.csdn.net), section 注意力:

* 普通注意力的实现: the scores are Q Kᵀ times the scale (default 1/sqrt(d_qk)),
  masked entries get -inf, a softmax over the key axis gives P, and the output
  is P V.
* The prose after it: with tangents t_q, t_k, t_v the score tangent is
  t_s = t_q Kᵀ + Q t_kᵀ; the softmax Jacobian gives
  t_p = P ⊙ t_s - (P t_sᵀ) P; the output tangent is t_o = P t_v + t_p V.
  The 前向 kernel applies the same scale to t_s as to the scores.
* 前向 kernel epilogue: the per-row value it stores is the natural-log
  log-sum-exp of the scaled scores.

The row tangent of the log-sum-exp is not stored by the pages' kernel; it is
the derivative of logsumexp along t_s, i.e. the softmax-weighted mean of t_s,
which is exactly the quantity P t_sᵀ in the chain rule above.

Nothing here is blocked, fused or reordered: every query row sees every key.
Rows are processed in chunks only to bound memory.
"""

import numpy as np

__all__ = ["attention_jvp", "attention_jvp_rows", "default_scale"]


def default_scale(d):
    """1/sqrt(d_qk): the kernel's default when no scale is given (前向)."""
    return float(d) ** -0.5


def _rows(q, k, v, dq, dk, dv, scale, visible):
    """Outputs for a block of query rows of one (batch, head).

    q, dq: [R, d]; k, dk: [N, d]; v, dv: [N, dv]; visible: [R, N] bool or None.
    Returns O [R, dv], dO [R, dv], LSE [R], dLSE [R] in float64.
    """
    s = scale * (q @ k.T)                                  # scores
    ts = scale * (dq @ k.T + q @ dk.T)                     # score tangent t_s
    if visible is not None:
        s = np.where(visible, s, -np.inf)
        ts = np.where(visible, ts, 0.0)

    m = s.max(axis=1)
    empty = ~np.isfinite(m)                                # row with no visible key
    m_safe = np.where(empty, 0.0, m)
    e = np.exp(s - m_safe[:, None])
    l = e.sum(axis=1)
    l_safe = np.where(empty, 1.0, l)
    p = e / l_safe[:, None]                                # softmax P

    o = p @ v                                              # O = P V
    lse = np.where(empty, -np.inf, m_safe + np.log(l_safe))

    mu = (p * ts).sum(axis=1)                              # P t_sᵀ, per row
    tp = p * ts - mu[:, None] * p                          # t_p
    do = p @ dv + tp @ v                                   # t_o = P t_v + t_p V
    dlse = mu                                              # d/d(eps) logsumexp
    return o, do, lse, dlse


def _as64(x):
    return np.asarray(x, dtype=np.float64)


def attention_jvp(q, k, v, dq, dk, dv, scale=None, visible=None, row_chunk=256):
    """O, dO, LSE, dLSE for tensors laid out [B, H, N, d].

    q, dq: [B, H, Nq, d]; k, dk: [B, H, Nk, d]; v, dv: [B, H, Nk, dv].
    scale: float or None (None -> 1/sqrt(d)).
    visible: None (every key visible) or a callable ``visible(qi, ki)`` that
      returns a bool matrix [len(qi), len(ki)] for integer index vectors.
    Returns float64 arrays O [B,H,Nq,dv], dO [B,H,Nq,dv], LSE [B,H,Nq],
    dLSE [B,H,Nq].  A query row that sees no key gets O = dO = 0,
    LSE = -inf, dLSE = 0.
    """
    q, k, v, dq, dk, dv = map(_as64, (q, k, v, dq, dk, dv))
    nq = q.shape[2]
    return attention_jvp_rows(q, k, v, dq, dk, dv, np.arange(nq), scale,
                              visible, row_chunk)


def attention_jvp_rows(q, k, v, dq, dk, dv, rows, scale=None, visible=None,
                       row_chunk=256):
    """Same as ``attention_jvp`` restricted to the query rows ``rows``.

    ``rows`` is an integer vector (the same rows for every batch and head).
    Returns O, dO [B, H, len(rows), dv] and LSE, dLSE [B, H, len(rows)].
    The inputs may be any float dtype; every row is converted to float64
    before use.
    """
    rows = np.asarray(rows, dtype=np.int64)
    B, H, _, d = q.shape
    nk = k.shape[2]
    dvd = v.shape[3]
    if scale is None:
        scale = default_scale(d)
    R = rows.shape[0]
    o = np.zeros((B, H, R, dvd))
    do = np.zeros((B, H, R, dvd))
    lse = np.zeros((B, H, R))
    dlse = np.zeros((B, H, R))
    kidx = np.arange(nk)
    for b in range(B):
        for h in range(H):
            kb, dkb = _as64(k[b, h]), _as64(dk[b, h])
            vb, dvb = _as64(v[b, h]), _as64(dv[b, h])
            for c0 in range(0, R, row_chunk):
                rr = rows[c0:c0 + row_chunk]
                vis = None if visible is None else visible(rr, kidx)
                res = _rows(_as64(q[b, h][rr]), kb, vb, _as64(dq[b, h][rr]),
                            dkb, dvb, scale, vis)
                sl = slice(c0, c0 + rr.shape[0])
                o[b, h, sl], do[b, h, sl], lse[b, h, sl], dlse[b, h, sl] = res
    return o, do, lse, dlse
