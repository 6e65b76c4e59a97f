"""Comparison rules of the parity tests.

fp32 workloads: max |got - ref| <= 1e-5 against the fp64 oracle.  That
bound is for the unit-scale tiny workload; the larger fp32 test shapes have
sums of hundreds of O(1) terms, where one fp32 ulp already exceeds 1e-5, so
there ("fp32-scaled") the bound is 1e-5 * max(1, RMS of the reference tensor).

bf16 workloads (bf16 storage, fp32 accumulation): the relative error with a
floor,  max_i |got_i - ref_i| / max(|ref_i|, rho)  <= 2e-2,  where rho is the
RMS of the reference over the token row for [T, .] activation tensors and
over the whole compared tensor for parameters and their gradients.  A bare
elementwise relative error is meaningless for entries near zero among 10^8
values; the floor makes the bound relative to the tensor's own scale.  bf16
rounding of a stored intermediate is 2^-9 ~ 2e-3 relative, so on the narrow
test shapes correct kernels sit around 1e-3 to 5e-3 and a real fault (a wrong
index, a dropped term) lands far above 2e-2.  Wide shapes (10^7 - 10^8
entries), where upstream rounding flips leave a correct implementation no
margin end to end on the activation, dN and dx, hold those three tensors to
the same bound stage by stage (tests/stagewise.py); the bound is never raised.
"""

import numpy as np
import torch

# FP8 GEMMs.  The matrix unit sums
# each 128-long block of k with about 12 bits of precision relative to the
# block's largest product (2^-11.6 worst relative to that product and 2^-12.8
# relative to the block's sum of |products| were measured); a GEMM of codes
# given to both sides must then satisfy, per output,
#     |got - ref| <= FP8_GEMM_REL * (sum_k |a_k b_k|) * dequantisation.
FP8_GEMM_REL = 2.0 ** -10
# A whole FP8 step compares tensors that went through casts of computed
# values: where the GPU's bf16 input to a cast differs by an ulp from the
# oracle's (the block sums above put 1-5% of such inputs an ulp away), a
# rounding boundary can lie in between and the code differs by a whole FP8
# step (12.5% of the value in E4M3, 25% in E5M2).  A fraction p of flipped
# codes gives a GEMM output a relative Frobenius error of about
# sqrt(p) * 0.25; p <= 1% (0.1-0.6% measured) bounds it by 2.5%, and 2.4% was
# the worst measured (the row-sampled dx of the Llama-3-8B TP=8 step).
# Elementwise bounds do not apply to such tensors; each is compared by its
# relative Frobenius error against twice that estimate, while a wrong operand,
# index or scale moves it to O(1).  The kernels themselves are held to the
# strict bounds above on inputs whose codes both sides share.
FP8_STEP_FROB = 5e-2

FP32_ATOL = 1e-5
BF16_RTOL = 2e-2


def _np(a):
    if isinstance(a, torch.Tensor):
        return a.detach().double().cpu().numpy()
    return np.asarray(a, dtype=np.float64)


def max_abs(got, ref) -> float:
    g, r = _np(got), _np(ref)
    assert g.shape == r.shape, (g.shape, r.shape)
    return float(np.max(np.abs(g - r))) if g.size else 0.0


def floored_rel(got, ref, rowwise: bool) -> float:
    g, r = _np(got), _np(ref)
    assert g.shape == r.shape, (g.shape, r.shape)
    if g.size == 0:
        return 0.0
    if rowwise and r.ndim >= 2:
        rho = np.sqrt(np.mean(r * r, axis=-1, keepdims=True))
    else:
        rho = np.sqrt(np.mean(r * r))
    den = np.maximum(np.abs(r), rho)
    den = np.where(den > 0, den, 1.0)
    return float(np.max(np.abs(g - r) / den))


def check(name, got, ref, dtype: str, rowwise: bool = False, report=None, tol=None) -> float:
    if dtype == "fp32":
        e = max_abs(got, ref)
        if report is not None:
            report[name] = e
        assert e <= FP32_ATOL, f"{name}: max-abs {e:.3e} > {FP32_ATOL}"
    elif dtype == "fp32-scaled":
        r = _np(ref)
        scale = max(1.0, float(np.sqrt(np.mean(r * r)))) if r.size else 1.0
        e = max_abs(got, ref) / scale
        if report is not None:
            report[name] = e
        assert e <= FP32_ATOL, f"{name}: max-abs / max(1, rms) {e:.3e} > {FP32_ATOL}"
    else:
        e = floored_rel(got, ref, rowwise)
        bound = BF16_RTOL if tol is None else tol
        if report is not None:
            report[name] = e
        assert e <= bound, f"{name}: floored relative error {e:.3e} > {bound:.3e}"
    return e


def frob_rel(got, ref) -> float:
    g, r = _np(got), _np(ref)
    assert g.shape == r.shape, (g.shape, r.shape)
    n = float(np.linalg.norm(r))
    return float(np.linalg.norm(g - r)) / n if n > 0 else float(np.linalg.norm(g))


def check_fp8_gemm(name, got, ref, abs_products, deq: float, report=None) -> float:
    """Per-output bound of an FP8 GEMM of identical codes (FP8_GEMM_REL)."""
    g, r, a = _np(got), _np(ref), _np(abs_products)
    assert g.shape == r.shape == a.shape, (g.shape, r.shape, a.shape)
    bound = FP8_GEMM_REL * a * abs(deq) + 1e-30
    e = float(np.max(np.abs(g - r) / bound)) if g.size else 0.0
    if report is not None:
        report[name] = e
    assert e <= 1.0, f"{name}: error / FP8 GEMM bound {e:.3e} > 1"
    return e


def check_fp8_step(name, got, ref, report=None) -> float:
    e = frob_rel(got, ref)
    if report is not None:
        report[name] = e
    assert e <= FP8_STEP_FROB, f"{name}: relative Frobenius error {e:.3e} > {FP8_STEP_FROB}"
    return e


def check_sum_of_stored(name, got, ref, a_terms, b_terms, scale: float = 1.0, report=None) -> float:
    """The bf16 bound for C = A^T B (times `scale`, e.g. the learning rate of
    an update) where A is a stored bf16 tensor: besides the floored relative
    bound, a stored value of A can land one bf16 ulp away from the oracle's
    where its fp32 value lies within the accumulation error of a rounding
    midpoint, and a sum dominated by a few large terms then moves by that
    ulp times the other factor.  The allowance is one such flip of the largest
    term, bounded separably: 2^-7 max_t |A[t, i]| max_t |B[t, j]| (a bf16 ulp
    is at most 2^-7 of the value).  a_terms [T, M], b_terms [T, N] are the
    oracle's A and B."""
    g, r = _np(got), _np(ref)
    a, b = np.abs(_np(a_terms)), np.abs(_np(b_terms))
    assert g.shape == r.shape == (a.shape[1], b.shape[1]), (g.shape, r.shape, a.shape, b.shape)
    rho = np.sqrt(np.mean(r * r)) if r.size else 0.0
    allow = 2.0 ** -7 * np.outer(a.max(axis=0), b.max(axis=0)) * abs(scale)
    bound = BF16_RTOL * np.maximum(np.abs(r), rho) + allow
    e = float(np.max(np.abs(g - r) / np.where(bound > 0, bound, 1.0))) if g.size else 0.0
    if report is not None:
        report[name] = e
    assert e <= 1.0, f"{name}: error / (bf16 bound + one-ulp flip of the largest term) {e:.3e} > 1"
    return e

