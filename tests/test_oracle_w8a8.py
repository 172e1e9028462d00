"""Pins for the W8A8-FP8 oracle (``oracle/w8a8.py``), CPU only.

* exact rational brute force on tiny shapes: s_a s_n sum e4m3(xc) e4m3(wc),
  nearest bf16, bit for bit;
* the activation codes are the nearest E4M3 value of x / s_a (brute-force
  argmin over the finite codes), and the scale is one per tensor: the
  tensor's largest |x| maps to 448, a row whose own maximum is smaller does
  not reach it;
* a special case that reduces to the pinned weight-only oracle: activations
  already on the E4M3 grid times 2^j, with the largest at 448 * 2^j, give
  s_a = 2^j, codes that decode to x / 2^j exactly, and the weight-only FP8
  product;
* the activation-rounding error bound against the weight-only product;
* planted mistakes (one scale per row, the activation scale left out,
  truncating instead of rounding) fail a pin.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import oracle.w8a8 as W8
import wqd_inputs as I
from tests.test_oracle_quant_gemm import _e4m3_half_spacing, _nearest_bf16_bits

FIN = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
TABLE = oracle.e4m3_decode(FIN)


def x_bits_from_f32(x):
    import torch

    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(
        np.uint16).copy()


def brute(x_bits, qw):
    xq = W8.quantize_act(x_bits)
    xd = oracle.e4m3_decode(xq["codes"])
    wd = oracle.e4m3_decode(qw["codes"])
    sa = Fraction(float(xq["scale"]))
    M, K = xd.shape
    N = wd.shape[0]
    out = np.zeros((M, N), np.uint16)
    for m in range(M):
        xs = [Fraction(float(v)) for v in xd[m]]
        for n in range(N):
            acc = sum(a * Fraction(float(b)) for a, b in zip(xs, wd[n]))
            out[m, n] = _nearest_bf16_bits(acc * sa * Fraction(float(qw["scales"][n])))
    return out


@pytest.mark.parametrize("M,N,K", [(1, 5, 64), (3, 4, 128), (2, 7, 96)])
def test_exact_rationals(M, N, K):
    x = x_bits_from_f32(I.x_f32(60 + K, M, K) * np.float32(3.0))
    qw = oracle.quantize_fp8(I.w_host(61 + N, N, K))
    assert np.array_equal(W8.qgemm_w8a8_ref(x, qw)["y_bits"], brute(x, qw))


def check_act_codes(x_bits, xq):
    x = oracle.bf16_bits_to_f64(x_bits).astype(np.float32)
    s = xq["scale"]
    assert np.ndim(s) == 0, "one activation scale for the whole tensor"
    v = (x / s).astype(np.float32).astype(np.float64)
    got = oracle.e4m3_decode(xq["codes"])
    dist = np.abs(v[..., None] - TABLE[None, None, :])
    best = dist.min(axis=-1)
    assert np.array_equal(np.abs(v - got), best)  # nearest (either side of an exact tie)
    # one scale for the tensor: its largest |x| maps to 448
    a = np.abs(x).max()
    assert abs(float(s) * 448 - a) <= a * 2.0 ** -23
    assert np.abs(got).max() == 448.0
    return got


def test_act_codes_nearest_and_one_scale_per_tensor():
    x = I.x_f32(70, 6, 256)
    x[2] *= np.float32(0.01)  # a row far below the tensor maximum
    x[4, 17] = np.float32(-50.0)
    xb = x_bits_from_f32(x)
    xq = W8.quantize_act(xb)
    got = check_act_codes(xb, xq)
    assert np.abs(got[2]).max() < 448.0  # a per-row scale would have lifted this row to 448
    assert (xq["codes"][4, 17] & 0x7F) == 0x7E and (xq["codes"][4, 17] & 0x80)


def test_zero_and_tiny_activations():
    z = np.zeros((2, 64), np.uint16)
    xq = W8.quantize_act(z)
    assert xq["scale"] == np.float32(1.0) and not xq["codes"].any()
    qw = oracle.quantize_fp8(I.w_host(71, 3, 64))
    assert not W8.qgemm_w8a8_exact(xq, qw).any()
    # the smallest bf16 subnormal alone: the scale floors at 2^-126
    t = np.zeros((1, 64), np.uint16)
    t[0, 5] = 0x0001
    xq = W8.quantize_act(t)
    assert xq["scale"] == np.float32(2.0 ** -126)


def grid_activations(seed, M, K, j):
    """x = e4m3(c) * 2^j for random finite codes c, one of them +/-448: exactly bf16."""
    rng = np.random.default_rng(seed)
    c = FIN[rng.integers(0, len(FIN), size=(M, K))]
    c[rng.integers(0, M), rng.integers(0, K)] = 0x7E | (0x80 * int(rng.integers(0, 2)))
    x = (oracle.e4m3_decode(c) * 2.0 ** j).astype(np.float32)
    return x_bits_from_f32(x), c


@pytest.mark.parametrize("j", [-12, -3, 0, 5])
def test_grid_activations_reduce_to_weight_only(j):
    M, N, K = 4, 24, 384
    xb, c = grid_activations(80 + j, M, K, j)
    qw = oracle.quantize_fp8(I.w_host(81, N, K))
    xq = W8.quantize_act(xb)
    assert xq["scale"] == np.float32(2.0 ** j)
    assert np.array_equal(oracle.e4m3_decode(xq["codes"]), oracle.e4m3_decode(c))
    y8 = W8.qgemm_w8a8_exact(xq, qw)
    y16 = oracle.qgemm_exact(xb, qw)  # the pinned weight-only product of the same x
    assert np.allclose(y8, y16, rtol=2.0 ** -45, atol=0)
    assert np.array_equal(oracle.bf16_to_bits(y8), oracle.bf16_to_bits(y16))


def check_error_bound(xb, qw, y8):
    """|y_w8a8 - y_weight_only| <= sum_k |Wd[n, k]| s_a (half an E4M3 step at
    x/s_a + the float32 rounding of the quotient)."""
    x = oracle.bf16_bits_to_f64(xb)
    s = float(W8.act_scale(xb))
    v = x / s
    dx = s * (_e4m3_half_spacing(v) + np.abs(v) * 2.0 ** -24)
    bound = dx @ np.abs(oracle.dequant_exact(qw)).T
    err = np.abs(y8 - oracle.qgemm_exact(xb, qw))
    assert (err <= bound * (1 + 1e-12)).all(), float((err / bound).max())


def test_activation_rounding_error_bound():
    xb = I.x_bf16_bits(90, 8, 1024, outliers=False)
    qw = oracle.quantize_fp8(I.w_host(91, 40, 1024))
    check_error_bound(xb, qw, W8.qgemm_w8a8_exact(W8.quantize_act(xb), qw))


def test_k_limit_for_an_exact_sum():
    xq = {"codes": np.zeros((1, W8.EXACT_K_MAX + 128), np.uint8), "scale": np.float32(1)}
    qw = {"fmt": "fp8", "codes": np.zeros((2, W8.EXACT_K_MAX + 128), np.uint8), "scales": np.ones(2, np.float32)}
    with pytest.raises(ValueError):
        W8.qgemm_w8a8_exact(xq, qw)


def test_pins_catch_planted_mistakes(monkeypatch):
    # 1) one activation scale per row: the tensor-wide 448 pin fails
    real_scale = W8.act_scale

    def per_row_quantize(x_bits):
        x = oracle.bf16_bits_to_f64(np.asarray(x_bits, np.uint16)).astype(np.float32)
        s = (np.abs(x).max(axis=1, keepdims=True) / np.float32(448)).astype(np.float32)
        return {"codes": oracle.e4m3_encode((x / s).astype(np.float32)), "scale": s}

    monkeypatch.setattr(W8, "quantize_act", per_row_quantize)
    with pytest.raises(AssertionError):
        test_act_codes_nearest_and_one_scale_per_tensor()
    monkeypatch.undo()

    # 2) the activation scale left out of the product: the grid special case fails
    real_exact = W8.qgemm_w8a8_exact

    def no_act_scale(xq, qw):
        return real_exact({"codes": xq["codes"], "scale": np.float32(1)}, qw)

    monkeypatch.setattr(W8, "qgemm_w8a8_exact", no_act_scale)
    with pytest.raises(AssertionError):
        test_grid_activations_reduce_to_weight_only(-3)
    monkeypatch.undo()

    # 3) codes truncated toward zero instead of rounded: the nearest-code pin fails
    def truncating(x_bits):
        xq = {"scale": real_scale(x_bits)}
        x = oracle.bf16_bits_to_f64(np.asarray(x_bits, np.uint16)).astype(np.float32)
        v = (x / xq["scale"]).astype(np.float64)
        idx = np.abs(TABLE[None, None, :] - v[..., None])
        below = np.where((np.abs(TABLE)[None, None, :] <= np.abs(v)[..., None]) &
                         (np.sign(TABLE)[None, None, :] * np.sign(v)[..., None] >= 0), idx, np.inf)
        xq["codes"] = FIN[below.argmin(axis=-1)]
        return xq

    monkeypatch.setattr(W8, "quantize_act", truncating)
    with pytest.raises(AssertionError):
        test_act_codes_nearest_and_one_scale_per_tensor()
    monkeypatch.undo()
    test_act_codes_nearest_and_one_scale_per_tensor()
