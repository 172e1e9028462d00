"""Reference product y = x . dequant(W)^T for the decode linear layer.

Test infrastructure only (see ``oracle/__init__.py``).

The method reaches exactly (up to the order of accumulation) a plain dense
matmul with dequantised weights: a weight-only kernel multiplies the quantised
matrix by a full-precision activation vector, dequantising on the fly, and the
activations are never quantised ("Making each token cheaper", section "What
quantization saves": the GPTQ decode kernel; CS336 lecture 10 notes, section
5.2: "simulated quantisation" is quantise, dequantise, then a dense matmul).
So the oracle is that definition: x (bf16 values) times the exact dequantised
weights, in float64, then one rounding to bf16.
"""
from __future__ import annotations

import numpy as np

from .formats import bf16_bits_to_f64, bf16_to_bits
from .quant import dequant_exact


def qgemm_exact(x_bits, qw: dict) -> np.ndarray:
    """y64[M, N] = x[M, K] . Wd[N, K]^T in float64 (x given as bf16 bit patterns)."""
    x = bf16_bits_to_f64(np.asarray(x_bits, dtype=np.uint16))
    Wd = dequant_exact(qw)
    if x.shape[1] != Wd.shape[1]:
        raise ValueError("K mismatch")
    return x @ Wd.T


def qgemm_ref(x_bits, qw: dict) -> dict:
    """Reference output: the float64 product and its bf16 rounding (bit patterns)."""
    y64 = qgemm_exact(x_bits, qw)
    return {"y64": y64, "y_bits": bf16_to_bits(y64)}



def silu(g) -> np.ndarray:
    """silu(g) = g * sigmoid(g) = g / (1 + exp(-g)), float64 (an overflowing
    exp(-g) gives -0: the limit)."""
    g = np.asarray(g, dtype=np.float64)
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g))


def swiglu_exact(x_bits, qw_gate: dict, qw_up: dict) -> np.ndarray:
    """h64[M, F] = silu(x . gate^T) * (x . up^T), in float64 from the exact
    products (CS336 lecture 10 notes, section 3.2: the MLP's gate and up
    projections of the same input, multiplied after the gate's activation)."""
    return silu(qgemm_exact(x_bits, qw_gate)) * qgemm_exact(x_bits, qw_up)
