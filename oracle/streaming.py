"""The pages' streaming (online-softmax) recurrence for attention and its JVP.

TEST INFRASTRUCTURE (the oracle): never imported by the library.

Page "带分数正则的一致性蒸馏" (gitcode.csdn.net), section 注意力, the two
paragraphs that stream K/V in blocks of length l.  Per query row the state is
a running max m (start -inf), a running exponential sum s (start 0), the
tangent sum r (start 0) and three vectors O, A, B (start 0).  For each key
block i:

  S_i = Q K_iᵀ,  t_si = t_q K_iᵀ + Q t_kiᵀ          (both times the scale)
  m_hat = max(m, max_j S_ij),  P_i = exp(S_i - m_hat)
  s <- exp(m - m_hat) s + sum_j P_ij
  O <- exp(m - m_hat) O + P_i V_i
  A <- exp(m - m_hat) A + P_i t_vi
  H_i = P_i ⊙ t_si
  r <- exp(m - m_hat) r + sum_j H_ij
  B <- exp(m - m_hat) B + H_i V_i
  m <- m_hat

and at the end O <- O / s and t_o = (A + B - r O) / s, with O already divided.
The pages' kernel stores the row log-sum-exp m + log s; r / s is the row
tangent of that log-sum-exp.

This is a second, independent statement of the same mathematics as
``attention_jvp``; the tests require the two to agree to rounding for any
block length.  It runs in float64 with no low-precision casts.
"""

import numpy as np

__all__ = ["attention_jvp_streaming"]


def attention_jvp_streaming(q, k, v, dq, dk, dv, block, scale=None,
                            visible=None):
    """Streaming form over key blocks of length ``block`` for [B,H,N,d] input.

    ``visible`` as in ``attention_jvp`` (callable or None).  Rows that see no
    key at all are not supported here (their m stays -inf).
    Returns O, dO [B,H,Nq,dv] and LSE, dLSE [B,H,Nq] in float64.
    """
    q, k, v, dq, dk, dv = (np.asarray(x, dtype=np.float64)
                           for x in (q, k, v, dq, dk, dv))
    B, H, nq, d = q.shape
    nk = k.shape[2]
    if scale is None:
        scale = float(d) ** -0.5
    dvd = v.shape[3]
    O_out = np.zeros((B, H, nq, dvd))
    dO_out = np.zeros((B, H, nq, dvd))
    lse = np.zeros((B, H, nq))
    dlse = np.zeros((B, H, nq))
    qidx = np.arange(nq)
    for b in range(B):
        for h in range(H):
            Q, tQ = q[b, h], dq[b, h]
            m = np.full(nq, -np.inf)
            s = np.zeros(nq)
            r = np.zeros(nq)
            O = np.zeros((nq, dvd))
            A = np.zeros((nq, dvd))
            Bacc = np.zeros((nq, dvd))
            for start in range(0, nk, block):
                ks = slice(start, min(start + block, nk))
                Ki, tKi = k[b, h][ks], dk[b, h][ks]
                Vi, tVi = v[b, h][ks], dv[b, h][ks]
                Si = scale * (Q @ Ki.T)
                tSi = scale * (tQ @ Ki.T + Q @ tKi.T)
                if visible is not None:
                    vis = visible(qidx, np.arange(ks.start, ks.stop))
                    Si = np.where(vis, Si, -np.inf)
                    tSi = np.where(vis, tSi, 0.0)
                m_hat = np.maximum(m, Si.max(axis=1))
                # a row whose max is still -inf has seen nothing yet
                m_use = np.where(np.isfinite(m_hat), m_hat, 0.0)
                decay = np.where(np.isfinite(m), np.exp(m - m_use), 0.0)
                Pi = np.exp(Si - m_use[:, None])
                s = decay * s + Pi.sum(axis=1)
                O = decay[:, None] * O + Pi @ Vi
                A = decay[:, None] * A + Pi @ tVi
                Hi = Pi * tSi
                r = decay * r + Hi.sum(axis=1)
                Bacc = decay[:, None] * Bacc + Hi @ Vi
                m = m_hat
            O = O / s[:, None]
            O_out[b, h] = O
            dO_out[b, h] = (A + Bacc - r[:, None] * O) / s[:, None]
            lse[b, h] = m + np.log(s)
            dlse[b, h] = r / s
    return O_out, dO_out, lse, dlse
