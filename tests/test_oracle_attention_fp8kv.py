"""Pins for the oracle's FP8 KV cache (``oracle.attention.quantize_kv_fp8`` and
``decode_attention_fp8kv_exact``), CPU only.

* codes: the nearest E4M3 value of x / scale (brute-force argmin over the 253
  finite codes of the float32 quotient), saturating at 448 for values beyond
  448 x scale; values already on the scaled grid come back unchanged;
* the round-to-nearest error bound of the dequantised cache against the bf16
  one;
* attention over an FP8 cache with power-of-two scales, where every
  dequantised value is exact in bf16, equals the (pinned) bf16 attention on
  those values bit for bit, and with any scales equals it on the float64
  values;
* the K scale acts on the scores and the V scale on the output: a cache whose
  keys are all one code gives the mean of the values whatever k_scale is, and
  the output scales linearly with v_scale;
* planted mistakes (the K scale left out, the V scale applied to the scores,
  codes truncated toward zero) fail a pin.
"""
import numpy as np
import pytest

import oracle
import oracle.attention as A

FIN = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
TABLE = oracle.e4m3_decode(FIN)


def bits(x):
    import torch

    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(
        np.uint16).copy()


def rand_cache(seed, B=2, Hq=8, Hkv=2, L=24, D=16, spread=1.0):
    rng = np.random.default_rng(seed)
    q = bits(rng.standard_normal((B, Hq, D)))
    k = bits(rng.standard_normal((B, Hkv, L, D)) * spread)
    v = bits(rng.standard_normal((B, Hkv, L, D)) * spread)
    lens = rng.integers(1, L + 1, size=B)
    return q, k, v, lens


@pytest.mark.parametrize("scale", [0.0078125, 0.01, 1.0, 3.7])
def test_codes_nearest_and_saturating(scale):
    _, k, _, _ = rand_cache(1, spread=3.0)
    x = oracle.bf16_bits_to_f64(k).astype(np.float32)
    codes = A.quantize_kv_fp8(k, scale)
    v = (x / np.float32(scale)).astype(np.float32).astype(np.float64)
    got = oracle.e4m3_decode(codes)
    dist = np.abs(np.minimum(np.abs(v), 448.0)[..., None] * np.sign(v)[..., None] - TABLE)
    assert np.array_equal(np.abs(np.clip(v, -448, 448) - got), dist.min(axis=-1))
    big = np.abs(v) > 448
    assert np.array_equal(codes[big] & 0x7F, np.full(big.sum(), 0x7E, np.uint8))
    if scale == 0.0078125:
        assert big.any()  # the case exercises saturation


def test_grid_values_round_trip():
    rng = np.random.default_rng(2)
    for j in (-9, -2, 0, 3):
        c = FIN[rng.integers(0, len(FIN), size=(2, 2, 16, 8))]
        x = (oracle.e4m3_decode(c) * 2.0 ** j).astype(np.float32)
        codes = A.quantize_kv_fp8(bits(x), 2.0 ** j)
        assert np.array_equal(oracle.e4m3_decode(codes), oracle.e4m3_decode(c))


def test_dequantisation_error_bound():
    _, k, _, _ = rand_cache(3, spread=2.0)
    x = oracle.bf16_bits_to_f64(k)
    for s in (0.02, 1.0, 0.37):
        got = oracle.e4m3_decode(A.quantize_kv_fp8(k, s)) * float(np.float32(s))
        v = np.abs(x / s)
        e = np.floor(np.log2(np.maximum(v, 2.0 ** -6)))
        half = np.ldexp(1.0, (e - 4).astype(int))  # half the spacing of E4M3 at |v|
        inside = v <= 448  # past 448 x scale the code saturates (pinned above)
        assert inside.mean() > 0.99
        err = np.abs(got - x)[inside]
        assert (err <= (s * (half + v * 2.0 ** -24) * (1 + 1e-12))[inside]).all()


@pytest.mark.parametrize("ks,vs", [(1.0, 1.0), (0.25, 4.0), (2.0 ** -5, 2.0 ** 3)])
def test_power_of_two_scales_reduce_to_bf16_attention(ks, vs):
    q, k, v, lens = rand_cache(4, B=3, Hq=16, Hkv=4, L=40, D=32)
    kc, vc = A.quantize_kv_fp8(k, ks), A.quantize_kv_fp8(v, vs)
    o8 = A.decode_attention_fp8kv_exact(q, kc, vc, ks, vs, lens, 0.2)
    kd = bits(oracle.e4m3_decode(kc) * ks)  # exact: E4M3 values times 2^j are bf16 values
    vd = bits(oracle.e4m3_decode(vc) * vs)
    assert np.array_equal(oracle.bf16_bits_to_f64(kd), oracle.e4m3_decode(kc) * ks)
    assert np.array_equal(o8, A.decode_attention_exact(q, kd, vd, lens, 0.2))


def test_any_scales_equal_attention_on_the_dequantised_values():
    q, k, v, lens = rand_cache(5, B=2, Hq=8, Hkv=2, L=30, D=16)
    ks, vs = 0.37, 1.9
    kc, vc = A.quantize_kv_fp8(k, ks), A.quantize_kv_fp8(v, vs)
    o8 = A.decode_attention_fp8kv_exact(q, kc, vc, ks, vs, lens, 0.3)
    K = oracle.e4m3_decode(kc) * float(np.float32(ks))
    V = oracle.e4m3_decode(vc) * float(np.float32(vs))
    qd = oracle.bf16_bits_to_f64(q)
    for b in range(2):
        n = int(lens[b])
        for h in range(8):
            s = K[b, h // 4, :n] @ qd[b, h] * 0.3
            p = np.exp(s - s.max())
            assert np.allclose(o8[b, h], (p / p.sum()) @ V[b, h // 4, :n], rtol=1e-13, atol=1e-15)


def test_scales_act_on_scores_and_values():
    q, k, v, lens = rand_cache(6)
    vc = A.quantize_kv_fp8(v, 1.0)
    kc = np.full(k.shape, 0x38, np.uint8)  # every key the same code (1.0)
    for ks in (0.01, 1.0, 20.0):
        o = A.decode_attention_fp8kv_exact(q, kc, vc, ks, 1.0, lens, 0.5)
        for b in range(2):
            mean = oracle.e4m3_decode(vc[b, :, : lens[b]]).mean(axis=1)
            assert np.allclose(o[b], np.repeat(mean, 4, axis=0), rtol=1e-13, atol=1e-15)
    kc = A.quantize_kv_fp8(k, 1.0)
    o1 = A.decode_attention_fp8kv_exact(q, kc, vc, 1.0, 1.0, lens, 0.5)
    o3 = A.decode_attention_fp8kv_exact(q, kc, vc, 1.0, 3.0, lens, 0.5)
    assert np.allclose(o3, 3.0 * o1, rtol=1e-13, atol=1e-15)
    with pytest.raises(ValueError):
        A.quantize_kv_fp8(k, 0.0)
    with pytest.raises(ValueError):
        A.quantize_kv_fp8(k, float("nan"))


def test_pins_catch_planted_mistakes(monkeypatch):
    real = A.decode_attention_fp8kv_exact

    def no_k_scale(q, kc, vc, ks, vs, lens, sc):
        return real(q, kc, vc, 1.0, vs, lens, sc)

    def v_scale_on_scores(q, kc, vc, ks, vs, lens, sc):
        return real(q, kc, vc, ks * vs, 1.0, lens, sc)

    pins = (lambda: test_power_of_two_scales_reduce_to_bf16_attention(0.25, 4.0),
            test_scales_act_on_scores_and_values)
    for bad in (no_k_scale, v_scale_on_scores):
        monkeypatch.setattr(A, "decode_attention_fp8kv_exact", bad)
        caught = False
        for pin in pins:
            try:
                pin()
            except AssertionError:
                caught = True
                break
        monkeypatch.undo()
        assert caught, bad.__name__
    # codes truncated toward zero instead of rounded to nearest
    real_q = A.quantize_kv_fp8

    def truncating(x_bits, scale):
        x = oracle.bf16_bits_to_f64(np.asarray(x_bits, np.uint16)).astype(np.float32)
        v = np.clip((x / np.float32(scale)).astype(np.float64), -448, 448)
        ok = (np.abs(TABLE)[None, :] <= np.abs(v).reshape(-1, 1)) & (np.sign(TABLE)[None, :] * np.sign(
            v).reshape(-1, 1) >= 0)
        d = np.where(ok, np.abs(v).reshape(-1, 1) - np.abs(TABLE)[None, :], np.inf)
        return FIN[d.argmin(axis=1)].reshape(v.shape)

    monkeypatch.setattr(A, "quantize_kv_fp8", truncating)
    with pytest.raises(AssertionError):
        test_codes_nearest_and_saturating(1.0)
    monkeypatch.undo()
    assert real_q is A.quantize_kv_fp8
