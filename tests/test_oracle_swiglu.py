"""Pins for the oracle's SwiGLU (``oracle.gemm.silu`` / ``swiglu_exact``), CPU only.

* silu's closed forms: silu(0) = 0, silu(x) - silu(-x) = x (the logistic
  function's symmetry), silu(ln 3) = (3/4) ln 3, the limits at +-large x
  (no NaN where exp overflows);
* against torch's float64 silu (an independent library routine);
* the gate/up product against exact rational products on tiny shapes (the
  two projections' bf16-exact sums), with silu from math.exp;
* planted mistakes (sigmoid instead of silu, gate and up swapped) fail a pin.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import oracle.gemm as G
import wqd_inputs as I


def test_silu_closed_forms():
    assert G.silu(0.0) == 0.0
    x = np.random.default_rng(1).standard_normal(1000) * 6
    assert np.allclose(G.silu(x) - G.silu(-x), x, rtol=1e-14, atol=1e-14)
    assert math.isclose(float(G.silu(math.log(3.0))), 0.75 * math.log(3.0), rel_tol=1e-15)
    assert G.silu(40.0) == 40.0
    big = G.silu(np.array([-800.0, 800.0]))
    assert big[0] == 0.0 and big[1] == 800.0 and not np.isnan(big).any()


def test_silu_against_torch():
    x = np.random.default_rng(2).standard_normal(5000) * 10
    assert np.allclose(G.silu(x), torch.nn.functional.silu(torch.from_numpy(x)).numpy(), rtol=1e-15, atol=1e-300)


def exact_swiglu(x_bits, qg, qu):
    x = oracle.bf16_bits_to_f64(x_bits)
    wg, wu = oracle.dequant_exact(qg), oracle.dequant_exact(qu)
    M, F = x.shape[0], wg.shape[0]
    out = np.zeros((M, F))
    for m in range(M):
        xs = [Fraction(float(v)) for v in x[m]]
        for f in range(F):
            g = float(sum(a * Fraction(float(b)) for a, b in zip(xs, wg[f])))
            u = float(sum(a * Fraction(float(b)) for a, b in zip(xs, wu[f])))
            out[m, f] = g / (1.0 + math.exp(-g)) * u
    return out


@pytest.mark.parametrize("fmt", ["w4a16", "fp8", "bf16"])
def test_swiglu_against_exact_products(fmt):
    M, F, K = 2, 6, 128
    x = I.x_bf16_bits(31, M, K)
    qg = oracle.quantize(fmt, I.w_host(32, F, K) * np.float32(20))  # gate values of order 1
    qu = oracle.quantize(fmt, I.w_host(33, F, K))
    assert np.allclose(oracle.swiglu_exact(x, qg, qu), exact_swiglu(x, qg, qu), rtol=1e-13, atol=1e-16)


def test_pins_catch_planted_mistakes(monkeypatch):
    real = G.silu
    monkeypatch.setattr(G, "silu", lambda g: 1.0 / (1.0 + np.exp(-np.asarray(g, np.float64))))
    with pytest.raises(AssertionError):
        test_silu_closed_forms()
    monkeypatch.setattr(G, "silu", real)
    real_sw = G.swiglu_exact
    monkeypatch.setattr(oracle, "swiglu_exact", lambda x, qg, qu: real_sw(x, qu, qg))
    with pytest.raises(AssertionError):
        test_swiglu_against_exact_products("w4a16")
    monkeypatch.undo()
