"""Merge of attention-JVP results over disjoint key sets (float64).

TEST INFRASTRUCTURE (the oracle): never imported by the library.

The softmax over a union of disjoint key sets K_1, ..., K_n, restricted to
K_k, is the softmax over K_k scaled by that set's share of the total mass:
P = w_k P_k on K_k with w_k = exp(LSE_k - LSE) and LSE = log sum_k
exp(LSE_k).  Hence O = sum_k w_k O_k and dLSE = sum_k w_k dLSE_k (the
softmax-weighted mean of the score tangent splits the same way).  The output
tangent follows from the product rule on O = sum_k w_k O_k, with the tangent
of w_k being w_k (dLSE_k - dLSE):  dO = sum_k w_k (dO_k + (dLSE_k - dLSE) O_k).

The per-set quantities are those of ``attention_jvp`` (page "带分数正则的一致性
蒸馏", gitcode.csdn.net, section 注意力); the identity is derived from that
definition and is not stated on the pages.  A row that sees no key of a set
has LSE_k = -inf there (weight 0); a row that sees no key at all gets the
empty-row convention O = dO = 0, LSE = -inf, dLSE = 0.
"""

import numpy as np

__all__ = ["merge_partials"]


def merge_partials(parts):
    """parts: list of (O, dO, LSE, dLSE) float64 arrays, O and dO [..., R, dv],
    LSE and dLSE [..., R], over disjoint key sets of the same query rows.
    Returns the merged (O, dO, LSE, dLSE)."""
    lses = np.stack([np.asarray(p[2], dtype=np.float64) for p in parts])
    m = lses.max(axis=0)
    empty = ~np.isfinite(m)
    m_safe = np.where(empty, 0.0, m)
    total = np.exp(lses - m_safe).sum(axis=0)
    lse = np.where(empty, -np.inf, m_safe + np.log(np.where(empty, 1.0, total)))
    lse_safe = np.where(empty, 0.0, lse)
    w = [np.where(empty, 0.0, np.exp(np.asarray(p[2], dtype=np.float64) - lse_safe))
         for p in parts]
    dlse = sum(wk * np.asarray(p[3], dtype=np.float64) for wk, p in zip(w, parts))
    o = sum(wk[..., None] * np.asarray(p[0], dtype=np.float64) for wk, p in zip(w, parts))
    do = sum(wk[..., None] * (np.asarray(p[1], dtype=np.float64)
                              + (np.asarray(p[3], dtype=np.float64) - dlse)[..., None]
                              * np.asarray(p[0], dtype=np.float64))
             for wk, p in zip(w, parts))
    return o, do, lse, dlse
