"""Shared helpers of the GPU parity tests: tolerances and comparisons.

Tolerances (applied element by element, GPU vs the fp64 oracle on the same inputs):
  * fp32 path: max |dO| <= 1e-5;
  * bf16 inputs with fp32 accumulation: |dO| <= 2e-2 + 1e-2 * |O_ref|;
  * fp16 inputs, general path: |dO| <= 1e-4 + 2^-10 * |O_ref|; on the matrix cores:
    |dO| <= 5e-3 + 2.5e-3 * |O_ref|;
  * log-sum-exp: |dlse| <= 1e-3; rows whose oracle lse is -inf must be -inf.
"""

import os

import numpy as np

F32_ATOL = 1e-5
BF16_ATOL = 2e-2
BF16_RTOL = 1e-2
LSE_ATOL = 1e-3
# fp16 (general path: fp32 arithmetic, one rounding of O to fp16, whose half-ulp is at
# most 2^-11 |O|): |dO| <= 1e-4 + 2^-10 |O_ref|, twice the rounding plus an fp32 floor.
F16_ATOL = 1e-4
F16_RTOL = 2.0 ** -10
# fp16 on the matrix cores: the probabilities are rounded to fp16 (2^-11 relative) for
# P V, like bf16's 2^-9; fp16 has three more mantissa bits, so a quarter of the bf16
# bar (twice the 8x finer rounding): |dO| <= 5e-3 + 2.5e-3 |O_ref|.
F16_MFMA_ATOL = 5e-3
F16_MFMA_RTOL = 2.5e-3


# Error-scale bar for 16-bit inputs on the matrix cores, applied together with the bars
# above. The probabilities are rounded to the 16-bit type (relative error <= u: 2^-8 for
# bf16, 2^-11 for fp16) before the P V products, and split problems round each key
# range's partial output once more; the oracle's scale S_ik = sqrt(sum_j P_ij^2 v_jk^2)
# is the root-sum-square of the terms those roundings multiply. Bar:
#   |dO| <= 4 u S + 2 u |O_ref|
# four roundings' worth of the root-sum-square (the error of a sum of independent
# roundings has standard deviation <= u S / sqrt(3) per source, so this is > 4.9
# standard deviations with two sources), and two half-ulps of |O| (the output's own
# rounding, plus the mean part of the partial outputs' rounding).
SCALE_TOL = {"bf16": 2.0 ** -6, "f16_mfma": 2.0 ** -9}
SCALE_RTOL = {"bf16": 2.0 ** -7, "f16_mfma": 2.0 ** -10}


def to_np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def check_out(o_gpu, o_ref, dtype, where="", scale=None):
    """Element-wise bar of the dtype; with the oracle's error scale (16-bit inputs on
    the matrix cores), also the error-scale bar SCALE_TOL * S + SCALE_RTOL * |O_ref|.
    Returns max |dO|; prints the worst ratio to the error-scale bar when it is used."""
    o = to_np(o_gpu) if not isinstance(o_gpu, np.ndarray) else o_gpu
    assert np.isfinite(o).all(), f"non-finite output {where}"
    err = np.abs(o - o_ref)
    if scale is not None and dtype in SCALE_TOL and err.size:
        bar = SCALE_TOL[dtype] * scale + SCALE_RTOL[dtype] * np.abs(o_ref)
        tiny = bar <= 0  # rows whose every weight sits on zero values: exact results
        ratio = np.where(tiny, np.where(err > 0, np.inf, 0.0), err / np.where(tiny, 1.0, bar))
        worst = float(ratio.max())
        print(f"[parity] {where}: worst |dO| / error-scale bar = {worst:.3g}", flush=True)
        log = os.environ.get("FA_PARITY_LOG")
        if log:  # a record of the worst ratio per case, for the design notes
            with open(log, "a") as f:
                f.write(f"{dtype}\t{err.size}\t{worst:.4f}\t{where}\n")
        bad = ratio > 1.0
        assert not bad.any(), (f"{int(bad.sum())} elements beyond the error-scale bar {where}; "
                               f"worst |dO| / bar = {worst:.3g}")
    if dtype == "f32":
        worst = float(err.max()) if err.size else 0.0
        assert worst <= F32_ATOL, f"max |dO| = {worst:.3g} > {F32_ATOL} {where}"
    elif dtype in ("f16", "f16_mfma"):
        atol, rtol = (F16_ATOL, F16_RTOL) if dtype == "f16" else (F16_MFMA_ATOL, F16_MFMA_RTOL)
        bad = err > atol + rtol * np.abs(o_ref)
        assert not bad.any(), (f"{int(bad.sum())} elements out of tolerance {where}; "
                               f"max |dO| = {float(err.max()):.3g}")
    else:
        bound = BF16_ATOL + BF16_RTOL * np.abs(o_ref)
        bad = err > bound
        assert not bad.any(), (f"{int(bad.sum())} elements out of tolerance {where}; "
                               f"max |dO| = {float(err.max()):.3g}")
    return float(err.max()) if err.size else 0.0


def check_lse(l_gpu, l_ref, where=""):
    lg = to_np(l_gpu) if not isinstance(l_gpu, np.ndarray) else l_gpu
    neg = np.isneginf(l_ref)
    assert np.array_equal(np.isneginf(lg), neg), f"-inf pattern of lse differs {where}"
    fin = ~neg
    err = np.abs(lg[fin] - l_ref[fin])
    worst = float(err.max()) if err.size else 0.0
    assert worst <= LSE_ATOL, f"max |dlse| = {worst:.3g} > {LSE_ATOL} {where}"
    return worst



# Gradients (bf16 path). A gradient element is a long sum whose terms may cancel, so
# its error is sized by the oracle's rounding-error scale S of that element (the
# root-sum-square of the terms that bf16 roundings multiply, plus the shared error of
# D_i = dO_i . O_i; see oracle/backward.py): |dG| <= 2^-6 * S + 1e-2 * |G_ref|.
# 2^-6 is eight bf16 half-ulps (2^-9): independent roundings of P, dS, O and the
# forward's own O error, at six standard deviations over up to 10^7 elements; the
# relative term covers the final bf16 rounding of the gradient itself.
GRAD_SCALE_TOL = 2.0 ** -6
GRAD_RTOL = 1e-2
# fp16 gradients: the same form with fp16's half-ulp (2^-11): 2^-8 S + 2.5e-3 |G_ref|.
GRAD_SCALE_TOL_F16 = 2.0 ** -8
GRAD_RTOL_F16 = 2.5e-3


def check_grad(g_gpu, g_ref, scale, where="", dtype="bf16"):
    g = to_np(g_gpu) if not isinstance(g_gpu, np.ndarray) else g_gpu
    assert np.isfinite(g).all(), f"non-finite gradient {where}"
    if g_ref.size == 0:
        return 0.0
    err = np.abs(g - g_ref)
    floor = 1e-6 * float(scale.max())
    tol, rtol = (GRAD_SCALE_TOL_F16, GRAD_RTOL_F16) if dtype == "f16" else (GRAD_SCALE_TOL, GRAD_RTOL)
    bound = tol * scale + rtol * np.abs(g_ref) + floor
    bad = err > bound
    assert not bad.any(), (f"{int(bad.sum())} elements out of tolerance {where}; "
                           f"worst |dG| / bound = {float((err / bound).max()):.3g}")
    return float((err / bound).max())
