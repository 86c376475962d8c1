"""Float64 gradients of attention from the saved log-sum-exp (the primal
backward).

TEST INFRASTRUCTURE (the oracle): never imported by the library.

Page "带分数正则的一致性蒸馏" (gitcode.csdn.net), section 注意力, subsection 反向:
given the upstream gradient G = dL/dO of O = P V, the output product gives
dV = Pᵀ G and dP = G Vᵀ; the softmax gives dS = P ⊙ (dP − rowsum(dP ⊙ P));
the scaled scores S = s Q Kᵀ give dQ = s dS K and dK = s dSᵀ Q.  The pages
state it for equal head dims (d_qk = d_v) and for Lq ≠ Lkv alike.

P is recomputed from the scores and the stored row log-sum-exp
(P = exp(S − LSE)); the oracle takes LSE from its own forward definition.
Rows with no visible key (LSE = −∞) contribute nothing.
"""

import numpy as np

from .attention_jvp import default_scale

__all__ = ["attention_backward"]


def attention_backward(q, k, v, g, scale=None, visible=None):
    """dQ, dK, dV (float64) of sum(G ⊙ O) for O = softmax(s Q Kᵀ) V.

    q: [B, H, Nq, d]; k: [B, H, Nk, d]; v: [B, H, Nk, dv]; g: [B, H, Nq, dv].
    visible: None or a callable ``visible(qi, ki)`` -> bool [len(qi), len(ki)].
    """
    q, k, v, g = (np.asarray(x, dtype=np.float64) for x in (q, k, v, g))
    B, H, nq, d = q.shape
    nk = k.shape[2]
    s = default_scale(d) if scale is None else scale
    vis = None if visible is None else visible(np.arange(nq), np.arange(nk))
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for b in range(B):
        for h in range(H):
            sc = s * (q[b, h] @ k[b, h].T)                     # S
            if vis is not None:
                sc = np.where(vis, sc, -np.inf)
            m = sc.max(axis=1, keepdims=True)
            m = np.where(np.isfinite(m), m, 0.0)
            e = np.exp(sc - m)
            l = e.sum(axis=1, keepdims=True)
            lse = m + np.log(np.where(l > 0, l, 1.0))
            p = np.where(l > 0, np.exp(sc - lse), 0.0)           # P = exp(S - LSE)
            gb = g[b, h]
            dv[b, h] = p.T @ gb                                  # dV = Pᵀ G
            dp = gb @ v[b, h].T                                  # dP = G Vᵀ
            ds = p * (dp - (dp * p).sum(axis=1, keepdims=True))  # softmax backward
            dq[b, h] = s * (ds @ k[b, h])                        # dQ = s dS K
            dk[b, h] = s * (ds.T @ q[b, h])                      # dK = s dSᵀ Q
    return dq, dk, dv
