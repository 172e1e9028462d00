"""W8A8-FP8: weights and activations both in FP8-E4M3, the product on FP8 matrix units.

Test infrastructure only (see ``oracle/__init__.py``).

What it computes ("Making each token cheaper", section "Weight quantization /
Formats": E4M3 is the format for weights and activations, and values are
multiplied by a scale before the cast so that they fit its range; the common
INT8 practice is a scale per channel for weights and one per tensor for
activations; section "What quantization saves": only a format whose matrix
product itself runs at lower precision, such as FP8 W8A8 on hardware that
supports it, reduces the arithmetic of the compute-bound passes; "LLM 推理是怎么
变快的", section 4.2 B: W8A8 uses the FP8/INT8 matrix units, so the arithmetic
itself doubles in rate, for large batches and prefill):

* the weights are the FP8 weight-only format of ``oracle.quant`` (E4M3 codes,
  one float32 scale per output row);
* the activations x[M, K] (bf16 values) take ONE dynamic scale for the whole
  tensor, s_a = max |x| / 448 in float32 (the reading the weight rows use,
  applied to the tensor: 1 for an all-zero tensor, floored at 2^-126), and
  codes = nearest E4M3 of x / s_a (float32 division, ties to even,
  saturating at 448);
* y[m, n] = s_a * s_n * sum_k e4m3(xc[m, k]) * e4m3(wc[n, k]).

Every E4M3 value is a multiple of 2^-9 below 2^9, so each product is a
multiple of 2^-18 below 2^18 and a sum of up to 2^15 of them is an integer
multiple of 2^-18 below 2^33: the float64 sum is exact for K <= 32768.  The
two scale multiplications then round once each in float64, and the result is
rounded once to bfloat16.
"""
from __future__ import annotations

import numpy as np

from .formats import bf16_bits_to_f64, bf16_to_bits, e4m3_decode, e4m3_encode

E4M3_MAX = 448.0
EXACT_K_MAX = 1 << 15


def act_scale(x_bits) -> np.float32:
    """The per-tensor activation scale: float32 max |x| / 448 (1 if x is all zero)."""
    x = bf16_bits_to_f64(np.asarray(x_bits, dtype=np.uint16)).astype(np.float32)  # bf16 values are exact in f32
    a = np.float32(np.abs(x).max()) if x.size else np.float32(0)
    if a == 0:
        return np.float32(1.0)
    s = np.float32(a / np.float32(E4M3_MAX))
    return np.float32(max(s, np.float32(2.0 ** -126)))


def quantize_act(x_bits) -> dict:
    """Activation codes and scale: codes = nearest E4M3 of float32(x / s_a)."""
    x = bf16_bits_to_f64(np.asarray(x_bits, dtype=np.uint16)).astype(np.float32)
    s = act_scale(x_bits)
    return {"codes": e4m3_encode((x / s).astype(np.float32)), "scale": s}


def qgemm_w8a8_exact(xq: dict, qw: dict) -> np.ndarray:
    """y64[M, N] = s_a * s_n * (e4m3(xc) . e4m3(wc)^T), the sum exact in float64."""
    if qw["fmt"] != "fp8":
        raise ValueError("W8A8 takes FP8 weights")
    xc, wc = np.asarray(xq["codes"]), np.asarray(qw["codes"])
    if xc.shape[1] != wc.shape[1]:
        raise ValueError("K mismatch")
    if xc.shape[1] > EXACT_K_MAX:
        raise ValueError("the float64 sum is exact only up to K = 32768")
    acc = e4m3_decode(xc) @ e4m3_decode(wc).T
    return acc * np.float64(xq["scale"]) * qw["scales"].astype(np.float64)[None, :]


def qgemm_w8a8_ref(x_bits, qw: dict) -> dict:
    """The whole W8A8 layer from bf16 activations: codes, scale, the float64
    product and its bf16 rounding (bit patterns)."""
    xq = quantize_act(x_bits)
    y64 = qgemm_w8a8_exact(xq, qw)
    return {"x_codes": xq["codes"], "x_scale": xq["scale"], "y64": y64, "y_bits": bf16_to_bits(y64)}
