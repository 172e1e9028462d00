"""Number formats used by the oracle: bfloat16, float16 and FP8-E4M3.

Test infrastructure only (see ``oracle/__init__.py``).

Every routine works in float64, where every value of the three formats and every
product the oracle forms is exact, and rounds once, to nearest with ties to
even.  Nothing here is shared with, or imported from, the device library.

* bfloat16: 1 sign, 8 exponent (bias 127), 7 stored mantissa bits; the upper
  half of an IEEE float32.  Activations and outputs of the layer are bf16.
* float16: IEEE binary16; the W4A16 group scale is stored in it.  Rounding to
  it uses numpy's float32 -> float16 conversion (a library primitive, RNE).
* FP8-E4M3: 4 exponent bits, 3 mantissa bits, largest normal 448 ("Making each
  token cheaper", section "Weight quantization / Formats": E4M3 tops out at
  448 and values are multiplied by a scale before the cast).  A maximum normal
  of 448 fixes the OCP "E4M3FN" variant: exponent bias 7, subnormals present,
  no infinities, S.1111.111 is NaN.
"""
from __future__ import annotations

import numpy as np

BF16_MAX = float((2.0 - 2.0 ** -7) * 2.0 ** 127)
E4M3_MAX = 448.0


# --------------------------------------------------------------------------- bf16
def bf16_round(v) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 value (ties to even), as float64.

    Definition: a bf16 number has 8 significant bits; for |v| in the normal
    range the spacing is 2^(floor(log2|v|) - 7), below 2^-126 it is 2^-133.
    Values that round beyond the largest finite bf16 become +-inf; NaN stays NaN.
    """
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    with np.errstate(invalid="ignore", over="ignore"):
        _, e = np.frexp(a)  # a = m * 2**e with m in [0.5, 1)
        expo = np.maximum(e.astype(np.int64) - 1, -126)
        quantum = np.ldexp(1.0, (expo - 7).astype(np.int32))
        r = np.rint(a / quantum) * quantum
        r = np.where(r > BF16_MAX, np.inf, r)
        r = np.where(np.isnan(a), np.nan, r)
    return np.copysign(r, v)


def bf16_bits_from_value(v) -> np.ndarray:
    """Bit pattern (uint16) of float64 values that are already bf16-representable."""
    f = np.asarray(v, dtype=np.float64).astype(np.float32)
    return (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def bf16_to_bits(v) -> np.ndarray:
    """Round float64 values to bf16 (RNE) and return the uint16 bit patterns."""
    return bf16_bits_from_value(bf16_round(v))


def bf16_bits_to_f64(bits) -> np.ndarray:
    """Exact value of bf16 bit patterns (uint16) as float64."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


# --------------------------------------------------------------------------- fp16
def fp16_round_f32(v) -> np.ndarray:
    """Round float32 values to float16 (RNE, overflow to inf) via numpy's cast."""
    with np.errstate(over="ignore"):
        return np.asarray(v, dtype=np.float32).astype(np.float16)


# --------------------------------------------------------------------------- e4m3
def e4m3_decode(codes) -> np.ndarray:
    """Value of FP8-E4M3FN codes as float64 (NaN for S.1111.111).

    Closed form: normal (E > 0): (-1)^S * 2^(E-7) * (1 + M/8);
    subnormal (E == 0): (-1)^S * 2^-6 * (M/8).
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = (c >> 7) & 1
    E = (c >> 3) & 0xF
    Mt = c & 7
    mag = np.where(
        E == 0,
        np.ldexp(Mt / 8.0, -6),
        np.ldexp(1.0 + Mt / 8.0, (E - 7).astype(np.int32)),
    )
    mag = np.where((E == 15) & (Mt == 7), np.nan, mag)
    return np.where(s == 1, -mag, mag)


def e4m3_encode(v) -> np.ndarray:
    """Encode float32 values as FP8-E4M3FN codes: nearest value, ties to even
    mantissa, magnitudes above 448 saturate to 448 (0x7E / 0xFE).

    The sign bit is the sign bit of the input (so -0.0 and tiny negatives that
    round to zero give 0x80).  Inputs must not be NaN.
    """
    v = np.asarray(v, dtype=np.float32).astype(np.float64)
    if np.isnan(v).any():
        raise ValueError("e4m3_encode: NaN input")
    sign = np.signbit(v)
    a = np.minimum(np.abs(v), E4M3_MAX)
    _, e = np.frexp(a)
    expo = np.maximum(e.astype(np.int64) - 1, -6)  # binade; subnormals share 2^-6's spacing
    quantum = np.ldexp(1.0, (expo - 3).astype(np.int32))
    r = np.rint(a / quantum) * quantum  # exact in float64; never exceeds 448
    # encode the representable magnitude r
    sub = r < 2.0 ** -6
    mt_sub = np.rint(r / 2.0 ** -9).astype(np.int64)
    _, er = np.frexp(np.where(sub, 1.0, r))
    eu = er.astype(np.int64) - 1
    mt_norm = np.rint((np.ldexp(np.where(sub, 1.0, r), (-eu).astype(np.int32)) - 1.0) * 8).astype(np.int64)
    E = np.where(sub, 0, eu + 7)
    Mt = np.where(sub, mt_sub, mt_norm)
    code = (E << 3) | Mt
    code = np.where(sign, code | 0x80, code)
    return code.astype(np.uint8)
