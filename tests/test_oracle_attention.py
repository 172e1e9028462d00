"""Pins for the decode-attention oracle (``oracle/attention.py``), CPU only.

* closed forms: one position gives its value row; equal keys (or scale 0)
  give the mean of the value rows; one dominant key gives its value row; two
  keys whose scores differ by ln 3 give 3/4 and 1/4 of their value rows;
* invariances: permuting positions, changing positions past the length;
* grouped-query heads: every query head of a KV group, and only those, sees
  that group (per-group constant values come out exactly);
* against torch's float64 scaled-dot-product attention (an independent
  library routine) with the KV heads repeated per group;
* planted mistakes (heads mapped to groups round-robin, no max subtraction,
  an off-by-one length, the scale applied twice) fail a pin.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import oracle.attention as A


def bits(x):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(
        np.uint16).copy()


def val(b):
    return oracle.bf16_bits_to_f64(b)


def rand_case(seed, B=3, Hq=8, Hkv=2, L=40, D=16):
    rng = np.random.default_rng(seed)
    q = bits(rng.standard_normal((B, Hq, D)))
    k = bits(rng.standard_normal((B, Hkv, L, D)))
    v = bits(rng.standard_normal((B, Hkv, L, D)))
    lens = rng.integers(1, L + 1, size=B)
    return q, k, v, lens


def test_one_position_and_zero_length():
    q, k, v, _ = rand_case(1)
    lens = np.array([1, 0, 1])
    o = A.decode_attention_exact(q, k, v, lens, 0.25)
    group = 8 // 2
    for b in (0, 2):
        for h in range(8):
            assert np.array_equal(o[b, h], val(v)[b, h // group, 0])
    assert not o[1].any()


def test_equal_keys_and_zero_scale_give_the_mean():
    q, k, v, lens = rand_case(2)
    k_eq = k.copy()
    k_eq[:] = k[:, :, :1, :]  # every position the same key
    o = A.decode_attention_exact(q, k_eq, v, lens, 0.3)
    o0 = A.decode_attention_exact(q, k, v, lens, 0.0)
    for b in range(3):
        mean = val(v)[b, :, : lens[b]].mean(axis=1)  # [Hkv, D]
        for h in range(8):
            assert np.allclose(o[b, h], mean[h // 4], rtol=1e-13, atol=1e-15)
            assert np.allclose(o0[b, h], mean[h // 4], rtol=1e-13, atol=1e-15)


def test_dominant_key_and_three_to_one():
    D = 4
    q = bits(np.array([[[1.0, 0, 0, 0]]]))
    k = np.zeros((1, 1, 5, D), np.float32)
    k[0, 0, 2, 0] = 64.0  # a score 64 above the others: weight 1 - O(e^-64)
    v = bits(np.arange(20, dtype=np.float32).reshape(1, 1, 5, D))
    o = A.decode_attention_exact(q, bits(k), v, np.array([5]), 1.0)
    assert np.allclose(o[0, 0], val(v)[0, 0, 2], rtol=0, atol=1e-12)
    # the same with scores past the float64 range of exp (scale 16: 1024)
    o = A.decode_attention_exact(q, bits(k), v, np.array([5]), 16.0)
    assert np.array_equal(o[0, 0], val(v)[0, 0, 2])
    # two positions whose scores differ by ln 3: weights 3/4 and 1/4
    k2 = np.zeros((1, 1, 2, D), np.float32)
    k2[0, 0, 0, 0] = 1.0
    v2 = bits(np.array([[[[4.0, 0, 8, 1], [0.0, 4, 8, 2]]]]))
    o2 = A.decode_attention_exact(q, bits(k2), v2, np.array([2]), math.log(3.0))
    assert np.allclose(o2[0, 0], [3.0, 1.0, 8.0, 1.25], rtol=1e-14, atol=1e-14)


def test_invariances():
    q, k, v, lens = rand_case(3, B=2, L=24)
    lens = np.array([17, 24])
    o = A.decode_attention_exact(q, k, v, lens, 0.2)
    # permuting the first len positions (keys and values alike)
    perm = np.random.default_rng(4).permutation(17)
    k2, v2 = k.copy(), v.copy()
    k2[0, :, :17], v2[0, :, :17] = k[0][:, perm], v[0][:, perm]
    assert np.allclose(A.decode_attention_exact(q, k2, v2, lens, 0.2), o, rtol=1e-12, atol=1e-14)
    # positions past the length do not matter
    k3, v3 = k.copy(), v.copy()
    k3[0, :, 17:] = 0x7F80  # +inf
    v3[0, :, 17:] = 0x7FC0  # NaN
    assert np.array_equal(A.decode_attention_exact(q, k3, v3, lens, 0.2), o)


def test_groups_see_their_own_kv_heads():
    B, Hq, Hkv, L, D = 2, 12, 3, 9, 8
    q, k, _, lens = rand_case(5, B, Hq, Hkv, L, D)
    v = np.zeros((B, Hkv, L, D), np.float32)
    for g in range(Hkv):
        v[:, g] = g + 1.0
    o = A.decode_attention_exact(q, k, bits(v), lens, 0.5)
    for h in range(Hq):
        # softmax weights sum to 1 (to rounding)
        assert np.allclose(o[:, h], h // (Hq // Hkv) + 1.0, rtol=1e-14, atol=0)


def torch_sdpa(q, k, v, lens, scale):
    qf, kf, vf = (torch.from_numpy(val(x)) for x in (q, k, v))
    B, Hq, D = qf.shape
    Hkv = kf.shape[1]
    out = torch.zeros((B, Hq, D), dtype=torch.float64)
    for b in range(B):
        n = int(lens[b])
        kk = kf[b, :, :n].repeat_interleave(Hq // Hkv, dim=0)  # [Hq, n, D]
        vv = vf[b, :, :n].repeat_interleave(Hq // Hkv, dim=0)
        out[b] = torch.nn.functional.scaled_dot_product_attention(qf[b][:, None, :], kk, vv, scale=scale)[:, 0]
    return out.numpy()


@pytest.mark.parametrize("seed", [6, 7])
def test_against_torch_sdpa_float64(seed):
    q, k, v, lens = rand_case(seed, B=4, Hq=16, Hkv=2, L=64, D=32)
    o = A.decode_attention_exact(q, k, v, lens, 1 / math.sqrt(32))
    assert np.allclose(o, torch_sdpa(q, k, v, lens, 1 / math.sqrt(32)), rtol=1e-12, atol=1e-13)


def test_pins_catch_planted_mistakes(monkeypatch):
    real = A.decode_attention_exact

    def round_robin(q_bits, k_bits, v_bits, lengths, scale):
        # heads assigned to groups h % Hkv instead of h // (Hq / Hkv)
        qv = np.asarray(q_bits)
        Hq, Hkv = qv.shape[1], np.asarray(k_bits).shape[1]
        order = np.array([(h % Hkv) * (Hq // Hkv) + h // Hkv for h in range(Hq)])
        return real(qv[:, order], k_bits, v_bits, lengths, scale)[:, np.argsort(order)]

    def no_max(q_bits, k_bits, v_bits, lengths, scale):
        qv, K, V = (oracle.bf16_bits_to_f64(np.asarray(x, np.uint16)) for x in (q_bits, k_bits, v_bits))
        o = np.zeros(qv.shape)
        g = qv.shape[1] // K.shape[1]
        with np.errstate(all="ignore"):
            for b in range(qv.shape[0]):
                n = int(lengths[b])
                for h in range(qv.shape[1]):
                    e = np.exp(K[b, h // g, :n] @ qv[b, h] * scale)
                    o[b, h] = (e / e.sum()) @ V[b, h // g, :n] if n else 0
        return o

    def off_by_one(q_bits, k_bits, v_bits, lengths, scale):
        return real(q_bits, k_bits, v_bits, np.maximum(np.asarray(lengths) - 1, 0), scale)

    def scale_twice(q_bits, k_bits, v_bits, lengths, scale):
        return real(q_bits, k_bits, v_bits, lengths, scale * scale)

    pins = (test_one_position_and_zero_length, test_groups_see_their_own_kv_heads, test_dominant_key_and_three_to_one,
            lambda: test_against_torch_sdpa_float64(6))
    for bad in (round_robin, no_max, off_by_one, scale_twice):
        monkeypatch.setattr(A, "decode_attention_exact", bad)
        caught = False
        for pin in pins:
            try:
                pin()
            except (AssertionError, ValueError, FloatingPointError):
                caught = True
                break
        monkeypatch.undo()
        assert caught, bad.__name__
