"""Acceptance criteria for GPU results against the oracle (test infrastructure).

Random-input floating-point results pass when both hold:
  * normwise:    ||C - T||_F / ||T||_F <= 1e-3
  * elementwise: |C_ij - T_ij| <= 1e-2 * scale_ij + 1e-3,
    scale_ij = |alpha| * U_ij, with U_ij = sum_k |A_ik||B_kj| from the oracle
    (the bound as the specification of the product writes it, U scaled by
    the alpha that multiplies the product).  beta * C_old and the bias enter
    T exactly; their share of the GPU's rounding (one fp32 multiply-add
    each, then the output rounding) must fit the 1e-3 absolute term and the
    1e-2 U slack, which holds at the magnitudes the tests use.
    ``rounding_fits`` checks that the bound admits the correctly rounded
    exact result itself, so that an unsuitable test input is reported as
    such rather than as a kernel error.
Integer-valued runs and the q4 dequant must match the oracle's rounded bits
exactly.  T is the oracle's binary64 result before output rounding.

bfloat16 OUTPUT: one rounding to bfloat16 alone has a relative error of up to
2^-9 per element (RMS about 2^-9/sqrt(3) = 1.1e-3 for uniformly spread
significands), which exceeds the 1e-3 normwise bound by construction.  For
that output type the normwise bound is widened by the bfloat16 unit
roundoff u = 2^-8 (1e-3 + 2^-8); the elementwise bound is unchanged (the
rounding, at most 2^-9 |T| <= 2^-9 scale, fits inside 1e-2 * scale).
Inputs in bfloat16 with fp16 or fp32 output keep the 1e-3 bound.
"""
import numpy as np

NORMWISE_TOL = 1e-3
BF16_OUT_NORMWISE_TOL = 1e-3 + 2.0 ** -8


def normwise_tol(out_type):
    """Normwise bound for an output type name ('f16', 'bf16', 'f32')."""
    return BF16_OUT_NORMWISE_TOL if out_type == "bf16" else NORMWISE_TOL


ELEM_RTOL = 1e-2
ELEM_ATOL = 1e-3


def normwise_rel_err(C, T):
    C = np.asarray(C, dtype=np.float64)
    T = np.asarray(T, dtype=np.float64)
    den = np.linalg.norm(T)
    num = np.linalg.norm(C - T)
    if den == 0.0:
        return 0.0 if num == 0.0 else np.inf
    return float(num / den)


def elem_scale(U, alpha=1.0):
    """Scale of the elementwise bound: |alpha| * U."""
    return abs(alpha) * np.asarray(U, dtype=np.float64)


def rounding_fits(T_rounded, T, scale, rtol=ELEM_RTOL, atol=ELEM_ATOL, share=0.5):
    """True when the correctly rounded exact result uses at most `share` of
    the elementwise bound everywhere (T_rounded: the oracle's T after the
    output rounding, as float64)."""
    err = np.abs(np.asarray(T_rounded, dtype=np.float64) - np.asarray(T, dtype=np.float64))
    return bool(np.all(err <= share * (rtol * scale + atol)))


def elem_violations(C, T, scale, rtol=ELEM_RTOL, atol=ELEM_ATOL):
    C = np.asarray(C, dtype=np.float64)
    T = np.asarray(T, dtype=np.float64)
    bad = ~(np.abs(C - T) <= rtol * scale + atol)
    return int(np.count_nonzero(bad))


def check_tolerance(C, T, scale, normwise_tol=NORMWISE_TOL):
    """Returns (ok, report) for the floating-point acceptance criteria."""
    nre = normwise_rel_err(C, T)
    nbad = elem_violations(C, T, scale)
    finite = bool(np.all(np.isfinite(np.asarray(C, dtype=np.float64))))
    ok = finite and nre <= normwise_tol and nbad == 0
    return ok, {"normwise_rel_err": nre, "elem_violations": nbad, "finite": finite}


def bits_mismatch(got_bits, want_bits):
    """Number of positions whose raw bits differ (NaN never expected here)."""
    got = np.asarray(got_bits)
    want = np.asarray(want_bits)
    assert got.shape == want.shape, (got.shape, want.shape)
    return int(np.count_nonzero(got != want))
