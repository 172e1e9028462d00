"""Bytes moved by a decode step, and the step's lower bound, as the pages define them.

Test infrastructure only (see ``oracle/__init__.py``).

Definitions followed ("降低每個 Token 的生成成本" / Making each token cheaper):

* section "為何 Decode 通常受記憶體頻寬限制" (Why decode is usually bandwidth
  bound): a step cannot finish before every weight byte and every sequence's
  KV bytes have crossed from HBM, nor before its 2 x parameters x positions
  multiply-add FLOPs are done; the bound is the larger of the two times.  The
  KV cache of one sequence holds a key and a value vector per layer, KV head
  and context token.
* section "完整範例：各格式的權重位元組與下限" (Worked example: weight bytes and
  bounds per format): weight bytes = parameters x bits per weight / 8, where
  the bits per weight include the per-group scale overhead (a 16-bit scale per
  128 weights adds 0.125 bits) and FP8's one 32-bit scale per row.

The per-matrix model counts each stored byte once: codes, the format's scales
and zero points, then the activation rows read (x, 2 bytes each) and the
output rows written (y, 2 bytes each).
"""
from __future__ import annotations

from fractions import Fraction

GROUP = 128

# Storage of one weight and of each piece of metadata, in bits.
CODE_BITS = {"bf16": 16, "fp8": 8, "w4a16": 4}
FP8_ROW_SCALE_BITS = 32      # one float32 scale per output row
W4A16_SCALE_BITS = 16        # one float16 scale per (row, group of 128)
W4A16_ZERO_BITS = 4          # one uint4 zero point per (row, group of 128)
ACT_BITS = 16                # bf16 activations in and out


def bits_per_weight(fmt: str, K: int) -> Fraction:
    """Average stored bits per weight of a row of K weights (exact rational)."""
    if fmt == "bf16":
        return Fraction(CODE_BITS["bf16"])
    if fmt == "fp8":
        return Fraction(CODE_BITS["fp8"]) + Fraction(FP8_ROW_SCALE_BITS, K)
    if fmt == "w4a16":
        if K % GROUP:
            raise ValueError("w4a16 needs whole groups of 128")
        return Fraction(CODE_BITS["w4a16"]) + Fraction(W4A16_SCALE_BITS + W4A16_ZERO_BITS, GROUP)
    raise ValueError(f"unknown format {fmt!r}")


def weight_bytes(fmt: str, N: int, K: int) -> dict:
    """Stored bytes of an N x K weight matrix: codes, scales, zero points."""
    if fmt not in CODE_BITS:
        raise ValueError(f"unknown format {fmt!r}")
    codes = Fraction(N * K * CODE_BITS[fmt], 8)
    if fmt == "bf16":
        scales = zeros = Fraction(0)
    elif fmt == "fp8":
        scales, zeros = Fraction(N * FP8_ROW_SCALE_BITS, 8), Fraction(0)
    else:
        if K % GROUP:
            raise ValueError("w4a16 needs whole groups of 128")
        groups = N * (K // GROUP)
        scales = Fraction(groups * W4A16_SCALE_BITS, 8)
        zeros = Fraction(groups * W4A16_ZERO_BITS, 8)
    out = {"w": codes, "s": scales, "z": zeros}
    for k, v in out.items():
        if v.denominator != 1:
            raise ValueError(f"{k} bytes of a {N} x {K} {fmt} matrix are not whole: {v}")
        out[k] = int(v)
    return out


def call_bytes(fmt: str, M: int, N: int, K: int) -> int:
    """Algorithmic bytes of one y[M, N] = x[M, K] . dequant(W)^T call."""
    wb = weight_bytes(fmt, N, K)
    act = Fraction(M * K * ACT_BITS, 8) + Fraction(M * N * ACT_BITS, 8)
    return wb["w"] + wb["s"] + wb["z"] + int(act)


def params_weight_bytes(params: int, bits: float) -> float:
    """Weight bytes of a model of `params` parameters stored at `bits` per weight."""
    return params * bits / 8


def kv_bytes_per_sequence(layers: int, kv_heads: int, head_dim: int, bytes_per_elem: int,
                          context: int) -> int:
    """KV-cache bytes of one sequence: a key and a value vector of head_dim
    elements per layer, KV head and context token."""
    return 2 * layers * kv_heads * head_dim * bytes_per_elem * context


def memory_time_s(weight_bytes_total: float, batch: int, kv_per_seq: float, hbm_bytes_per_s: float) -> float:
    """Weights once per step plus every sequence's own KV bytes, at the HBM rate."""
    return (weight_bytes_total + batch * kv_per_seq) / hbm_bytes_per_s


def compute_time_s(params: int, batch: int, positions: int, peak_flops: float) -> float:
    """One multiply and one add per parameter per position processed."""
    return 2 * params * batch * positions / peak_flops


def step_bound_s(weight_bytes_total: float, batch: int, positions: int, kv_per_seq: float, params: int,
                 hbm_bytes_per_s: float, peak_flops: float) -> float:
    """The step's lower bound: it ends no sooner than the slower of the two."""
    return max(memory_time_s(weight_bytes_total, batch, kv_per_seq, hbm_bytes_per_s),
               compute_time_s(params, batch, positions, peak_flops))
