"""Parity bounds shared by the GPU tests (the HIP path against the float64
oracle), and the comparison that applies them.

Two bounds per output, both normwise, err = max|gpu - ref| / max|ref| over
the finite reference entries:

* the contract: float32 inputs O <= 1e-5 and dO <= 1e-4, bfloat16 inputs
  <= 2e-2 for every output;
* a regression ceiling from the error model of the path, well inside the
  contract, so that a partial regression (a missed rescale on a rare path, a
  dropped term in a tail tile) cannot hide under the contract's margin.

Error model (u = 2^-8, the unit roundoff of bfloat16):
  O   rounded once to bfloat16 (<= u of each element) after P~ was rounded
      to bfloat16 before P V (a relative error <= u per weight, which moves
      O by at most u * sum_j P_j |V_j| <= u * max|V|; with random signs it
      averages out to about u |O|): ceiling 2u.
  dO  the same output rounding, the rounding of P~ in P dV and of P~ . dS
      in (P . dS) V, and the cancellation against dLSE * O (dLSE is summed
      from the unrounded float32 P~ . dS): ceiling 3u.
  LSE computed in float32 from float32 scores of exactly representable
      inputs: an ABSOLUTE bound in nats (it enters the backward as
      P = exp(S - LSE), so an absolute error e is a relative error e in P):
      1e-4 for bfloat16 and 1e-5 for float32 inputs at the default scale;
      tests with scores far above unit size pass their own bound.
  dLSE summed in float32 from unrounded float32 products: normwise 1e-4
      (bfloat16 inputs) and 1e-5 (float32).
float32 inputs: the MFMA products are float32 throughout, so the O and dO
ceilings are 5e-6 and 1e-5 (observed about 1e-6).

The backward (dQ, dK, dV) of bfloat16 inputs rounds P and dS to bfloat16
before the MFMAs and the outputs once more: ceiling 3u, contract 2e-2; float32:
ceiling 1e-5, contract 1e-4.  Its denominator is max|ref| of the output
itself, except where the exact dQ and dK are zero (one key, or one visible
key per row), where the test names that case and measures against max|dV|.
"""

import numpy as np

U_BF16 = 2.0 ** -8

CONTRACT = {
    "fp32": {"O": 1e-5, "dO": 1e-4, "dLSE": 1e-4},
    "bf16": {"O": 2e-2, "dO": 2e-2, "dLSE": 2e-2},
}
CEILING = {
    "fp32": {"O": 5e-6, "dO": 1e-5, "dLSE": 1e-5},
    "bf16": {"O": 2 * U_BF16, "dO": 3 * U_BF16, "dLSE": 1e-4},
}
LSE_ABS = {"fp32": 1e-5, "bf16": 1e-4}

BWD_CONTRACT = {"fp32": 1e-4, "bf16": 2e-2}
BWD_CEILING = {"fp32": 1e-5, "bf16": 3 * U_BF16}


def say(*a):
    print(*a, flush=True)


def normwise(got, ref, den=None):
    """max|got - ref| / max|ref| over the finite entries of ref."""
    fin = np.isfinite(ref)
    if not fin.any():
        return 0.0
    if den is None:
        den = np.max(np.abs(ref[fin]))
    return float(np.max(np.abs(got[fin] - ref[fin])) / max(den, 1e-30))


def compare_fwd(gpu, ref, dtype, what, lse_abs=None, ceiling=None):
    """Check (O, dO, LSE, dLSE) against the oracle's.  Returns the errors."""
    con, cei = CONTRACT[dtype], dict(CEILING[dtype])
    if ceiling:
        cei.update(ceiling)
    lse_tol = LSE_ABS[dtype] if lse_abs is None else lse_abs
    errs = {}
    for n, g, r in zip(("O", "dO", "LSE", "dLSE"), gpu, ref):
        assert np.array_equal(np.isfinite(g), np.isfinite(r)), f"{what}: {n} finiteness"
        fin = np.isfinite(r)
        if n == "LSE":
            assert np.array_equal(g[~fin], r[~fin]), f"{what}: LSE -inf rows"
            e = float(np.max(np.abs(g[fin] - r[fin]))) if fin.any() else 0.0
            errs[n] = e
            assert e <= lse_tol, f"{what}: LSE absolute error {e:.3e} > {lse_tol:.0e} nats"
            continue
        e = normwise(g, r)
        errs[n] = e
        assert e <= con[n], f"{what}: {n} normwise error {e:.3e} > contract {con[n]:.0e}"
        assert e <= cei[n], f"{what}: {n} normwise error {e:.3e} > ceiling {cei[n]:.2e}"
    say(what, " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    return errs


def compare_bwd(gpu, ref, dtype, what, zero_dq_dk=False):
    """Check (dQ, dK, dV) against the oracle's backward.  With zero_dq_dk the
    exact dQ and dK are zero (one key, or one visible key per row): their
    errors are then measured against max|dV_ref|, the scale of the
    gradients, since the kernel returns rounding noise of dP - D there."""
    errs = {}
    dv_scale = float(np.max(np.abs(ref[2])))
    for n, a, r in zip(("dQ", "dK", "dV"), gpu, ref):
        assert np.isfinite(a).all(), f"{what}: {n} not finite"
        den = dv_scale if (zero_dq_dk and n != "dV") else None
        if zero_dq_dk and n != "dV":
            assert np.max(np.abs(r)) == 0.0, f"{what}: exact {n} is not zero"
        e = normwise(a, r, den)
        errs[n] = e
        assert e <= BWD_CONTRACT[dtype], f"{what}: {n} error {e:.3e} > contract"
        assert e <= BWD_CEILING[dtype], f"{what}: {n} error {e:.3e} > ceiling"
    return errs
