"""Comparison helpers for the GPU parity tests (tolerances written here, used everywhere).

fp32 path: max |O - O_ref| <= 1e-5 and ||O - O_ref||_2 / ||O_ref||_2 <= 1e-6.
bf16/fp16 path (P rounded for PV, fp32 state): max abs <= 2e-2 and relative L2 <= 5e-3.
Statistics m (row max of the scaled scores) and l (sum of exp(s - m)): both are governed by how
well fp32 knows each score. A d-term fp32 dot product is within d * 2^-24 * sum_c |q_c k_c| of the
exact one (the standard bound for recursive summation), so per row
    bound = d * 2^-24 * scale * max_j sum_c |q_c k_jc| + 1e-5
and the tests require |m - m_ref| <= bound and |l / l_ref - 1| <= bound (exp(x + e) = exp(x)(1 + e)).
"""
import numpy as np

# Gradients (fa_bwd, bf16 / fp16 inputs): P and dS are rounded to the input type as matrix-core
# operands (relative error <= 2^-9 for bf16, 2^-12 for fp16, per element, unbiased, so about
# 2^-9 / sqrt(3) = 1.1e-3 and 1.4e-4 in relative L2 per rounded operand), and D uses the forward's
# own O, which carries the forward's P rounding. Two such sources give ~1.6e-3 (bf16) and ~2e-4
# (fp16) measured; the bar is 2.5x that: relative L2 <= BWD_TOL[dtype][1] and
# max |g - g_ref| <= BWD_TOL[dtype][0] * max |g_ref| over the whole tensor.
BWD_TOL = {"bf16": (1e-2, 5e-3), "f16": (2e-3, 1e-3)}

TOL = {"f32": (1e-5, 1e-6), "bf16": (2e-2, 5e-3), "f16": (2e-2, 5e-3)}


def errors(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    diff = got - ref
    max_abs = float(np.max(np.abs(diff))) if diff.size else 0.0
    denom = float(np.linalg.norm(ref))
    rel_l2 = float(np.linalg.norm(diff) / denom) if denom > 0 else float(np.linalg.norm(diff))
    return max_abs, rel_l2


def assert_close(got, ref, dtype, what=""):
    max_abs, rel_l2 = errors(got, ref)
    tol_abs, tol_rel = TOL[dtype]
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    assert max_abs <= tol_abs and rel_l2 <= tol_rel, (
        f"{what}: max_abs={max_abs:.3e} (tol {tol_abs:.0e}) rel_l2={rel_l2:.3e} (tol {tol_rel:.0e})")
    return max_abs, rel_l2


def stat_bound(q_rows, k, scale):
    """Per-row score-error bound (see the module docstring); q_rows [..., n, d], k [..., Nk, d] in float64."""
    q_rows = np.abs(np.asarray(q_rows, dtype=np.float64))
    k = np.abs(np.asarray(k, dtype=np.float64))
    d = q_rows.shape[-1]
    return d * 2.0 ** -24 * float(scale) * np.max(q_rows @ np.swapaxes(k, -1, -2), axis=-1) + 1e-5


def assert_stats(m, l, m_ref, l_ref, bound, what=""):
    m = np.asarray(m, dtype=np.float64)
    l = np.asarray(l, dtype=np.float64)
    dm = np.abs(m - m_ref)
    dl = np.abs(l / l_ref - 1)
    assert np.all(dm <= bound), f"{what}: m off by {np.max(dm):.3e} (bound {np.min(bound):.1e}..)"
    assert np.all(dl <= bound), f"{what}: l off by {np.max(dl):.3e} rel (bound {np.min(bound):.1e}..)"


def assert_grad_close(got, ref, dtype, what="", zero_bound=None):
    """Gradient bar of BWD_TOL: scale-relative max error and relative L2 error.

    An all-zero reference (dQ, dK with one key: softmax is constant) has no relative scale; the
    GPU value is then the difference of two fp32 evaluations of the same dot product and must lie
    within ``zero_bound`` (elementwise, from the fp32 summation bound).
    """
    max_abs, rel_l2 = errors(got, ref)
    tol_rel_max, tol_rel = BWD_TOL[dtype]
    scale = max(float(np.max(np.abs(ref))) if np.size(ref) else 0.0, 1e-30)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    if not np.any(ref):
        assert zero_bound is not None, f"{what}: all-zero reference needs a bound"
        assert np.all(np.abs(got) <= zero_bound), f"{what}: reference is zero, max_abs={max_abs:.3e}"
        return max_abs, rel_l2
    assert max_abs <= tol_rel_max * scale and rel_l2 <= tol_rel, (
        f"{what}: max_abs={max_abs:.3e} (tol {tol_rel_max:.0e} x {scale:.2e}) rel_l2={rel_l2:.3e} (tol {tol_rel:.0e})")
    return max_abs, rel_l2
