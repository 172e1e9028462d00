"""Comparison helpers for the GPU parity tests.

Tolerance for y = x . dequant(W)^T (floating point, several accumulation
orders are correct):
  * relative L2 error <= 1e-3 against the oracle's bf16-rounded result
    y_ref = bf16(y64) (rounding to bf16 alone is ~1.6e-3 from the unrounded
    product, so the unrounded value cannot be the L2 reference);
  * max |y - y64| <= 4e-3 * max |y64| against the oracle's exact float64
    product (a correctly rounded bf16 output is within half an ulp,
    <= 2^-8 |y| ~ 3.9e-3 |y|, of it; measured against the rounded reference a
    single legitimate one-ulp rounding flip in the top binade would already be
    up to 2^-7 ~ 7.8e-3 of the maximum);
  * an all-zero reference must be matched exactly.
Integer, byte and code outputs are compared bit for bit.
"""
import numpy as np

import oracle

REL_L2_TOL = 1e-3
MAX_ABS_TOL = 4e-3


def bf16_bits(t) -> np.ndarray:
    import wqd_inputs

    return wqd_inputs.bf16_tensor_to_bits(t)


def compare_y(y_bits_gpu: np.ndarray, y64: np.ndarray, what: str = "") -> dict:
    y = oracle.bf16_bits_to_f64(y_bits_gpu)
    y_ref = oracle.bf16_round(y64)
    assert y.shape == y64.shape, what
    assert np.isfinite(y).all(), f"{what}: non-finite output"
    if not np.any(y_ref):
        assert not np.any(y), f"{what}: reference is all zero, output is not"
        return {"rel_l2": 0.0, "max_rel": 0.0}
    rel_l2 = float(np.linalg.norm(y - y_ref) / np.linalg.norm(y_ref))
    max_rel = float(np.abs(y - y64).max() / np.abs(y64).max())
    assert rel_l2 <= REL_L2_TOL, f"{what}: rel L2 {rel_l2:.3e} > {REL_L2_TOL}"
    assert max_rel <= MAX_ABS_TOL, f"{what}: max |dy| / max |y| = {max_rel:.3e} > {MAX_ABS_TOL}"
    return {"rel_l2": rel_l2, "max_rel": max_rel}
