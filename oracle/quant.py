"""Weight quantisers and exact dequantisation, as the oracle computes them.

Test infrastructure only (see ``oracle/__init__.py``).

Three storage formats for a weight matrix W[N, K] (float32, row n = output
channel, k = input channel):

* ``bf16``  - each weight rounded to bfloat16 (2 bytes/weight).
* ``fp8``   - FP8-E4M3 codes (1 byte/weight) plus one float32 scale per output
  row ("Making each token cheaper", "Worked example: weight bytes per format":
  one 32-bit scale per row of weights; "Weight quantization / Formats": the
  value is multiplied by the scale's inverse before the cast to E4M3).
* ``w4a16`` - 4-bit integer codes in groups of 128 along K, each group with a
  16-bit scale ("Making each token cheaper", "Weight quantization / Formats":
  weight-only INT4 shares one scale per group, group size 128; dequantised to
  16-bit before the multiply-accumulate) and an unsigned 4-bit zero point
  (CS336 lecture 10 notes, section 5.2 "Quantization": quantisation with a
  scale and a zero point).  The stored format is uint4 codes q in [0, 15], an
  fp16 scale s and a uint4 zero z per (row, group); the weight is (q - z) * s.

Readings where the pages leave a step open:

* FP8 row scale s_n = max_k |W[n, k]| / 448 in float32 (the page fixes one
  32-bit scale per row and the E4M3 maximum 448; absmax-to-max is the plain
  choice).  A zero row takes s_n = 1; s_n is floored at 2^-126 so it is a
  normal float32.  Codes: nearest E4M3 value of W / s_n (float32 division),
  ties to even, saturating at 448.
* W4A16 group (min/max asymmetric round-to-nearest, the textbook scheme; the
  worked result in the CS336 notes is missing from the page):
  lo = min(0, min W_g), hi = max(0, max W_g); s = fp16(fp32(hi - lo) / 15),
  rounded to float16 *before* the codes are chosen; s == 0 becomes 2^-24 (the
  smallest fp16 step), an infinite s becomes 65504, and an all-zero group takes
  s = 1, z = 0, q = 0.  z = clamp(rint(-lo / s), 0, 15);
  q = clamp(rint(W / s) + z, 0, 15); all divisions in float32, rint ties to
  even.
"""
from __future__ import annotations

import numpy as np

from .formats import (
    bf16_bits_to_f64,
    bf16_to_bits,
    e4m3_decode,
    e4m3_encode,
    fp16_round_f32,
)

GROUP = 128
FMTS = ("bf16", "fp8", "w4a16")


# --------------------------------------------------------------------------- bf16
def quantize_bf16(W) -> dict:
    W = np.asarray(W, dtype=np.float32)
    return {"fmt": "bf16", "codes": bf16_to_bits(W.astype(np.float64))}


# --------------------------------------------------------------------------- fp8
def fp8_row_scales(W) -> np.ndarray:
    W = np.asarray(W, dtype=np.float32)
    a = np.abs(W).max(axis=1) if W.shape[1] else np.zeros(W.shape[0], np.float32)
    s = (a / np.float32(448.0)).astype(np.float32)
    s = np.maximum(s, np.float32(2.0 ** -126))
    s = np.where(a == 0, np.float32(1.0), s).astype(np.float32)
    return s


def quantize_fp8(W) -> dict:
    W = np.asarray(W, dtype=np.float32)
    s = fp8_row_scales(W)
    v = (W / s[:, None]).astype(np.float32)  # float32 division, correctly rounded
    return {"fmt": "fp8", "codes": e4m3_encode(v), "scales": s}


# --------------------------------------------------------------------------- w4a16
def w4a16_group_params(W):
    """Per-(row, group) scale (float16) and zero point (uint8 in [0, 15])."""
    W = np.asarray(W, dtype=np.float32)
    N, K = W.shape
    if K % GROUP:
        raise ValueError("w4a16 needs K % 128 == 0")
    Wg = W.reshape(N, K // GROUP, GROUP)
    lo = np.minimum(np.float32(0), Wg.min(axis=2))
    hi = np.maximum(np.float32(0), Wg.max(axis=2))
    with np.errstate(over="ignore"):
        span = (hi - lo).astype(np.float32)
        s16 = fp16_round_f32((span / np.float32(15.0)).astype(np.float32))
    s16 = np.where(s16 == 0, np.float16(2.0 ** -24), s16)
    s16 = np.where(np.isinf(s16), np.float16(65504.0), s16)
    s16 = np.where(span == 0, np.float16(1.0), s16).astype(np.float16)
    s32 = s16.astype(np.float32)
    z = np.clip(np.rint((-lo / s32).astype(np.float32)), 0, 15).astype(np.uint8)
    return s16, z


def quantize_w4a16(W) -> dict:
    W = np.asarray(W, dtype=np.float32)
    N, K = W.shape
    s16, z = w4a16_group_params(W)
    s32 = np.repeat(s16.astype(np.float32), GROUP, axis=1)
    zf = np.repeat(z.astype(np.float32), GROUP, axis=1)
    q = np.clip(np.rint((W / s32).astype(np.float32)) + zf, 0, 15).astype(np.uint8)
    return {"fmt": "w4a16", "codes": q, "scales": s16, "zeros": z}


def quantize(fmt: str, W) -> dict:
    if fmt == "bf16":
        return quantize_bf16(W)
    if fmt == "fp8":
        return quantize_fp8(W)
    if fmt == "w4a16":
        return quantize_w4a16(W)
    raise ValueError(f"unknown format {fmt!r}")


# --------------------------------------------------------------------------- dequant
def dequant_exact(qw: dict) -> np.ndarray:
    """Exact dequantised weights as float64 [N, K] (no rounding happens).

    bf16: the bf16 value.  fp8: e4m3(c) * s_n (4 x 24 significant bits, exact
    in float64).  w4a16: (q - z) * s (5 x 11 bits, exact).
    """
    fmt = qw["fmt"]
    if fmt == "bf16":
        return bf16_bits_to_f64(qw["codes"])
    if fmt == "fp8":
        return e4m3_decode(qw["codes"]) * qw["scales"].astype(np.float64)[:, None]
    if fmt == "w4a16":
        q = qw["codes"].astype(np.float64)
        z = np.repeat(qw["zeros"].astype(np.float64), GROUP, axis=1)
        s = np.repeat(qw["scales"].astype(np.float64), GROUP, axis=1)
        return (q - z) * s
    raise ValueError(f"unknown format {fmt!r}")


def dequant_f32(qw: dict) -> np.ndarray:
    """Dequantised weights as float32: the exact value rounded once (RNE).

    For bf16 and w4a16 the exact value is already a float32; for fp8 this is
    the single IEEE float32 product e4m3(c) * s_n.
    """
    return dequant_exact(qw).astype(np.float32)
