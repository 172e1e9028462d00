"""Pins for the oracle's number formats (CPU only).

Each check ties the oracle to something other than its own formula: the
pages' printed E4M3 facts, torch's and numpy's conversions (library routines),
bit-level constructions, and brute force over exact rationals.
"""
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle


def _golden(golden_dir, name):
    out = {}
    with open(os.path.join(golden_dir, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            parts = line.split()
            out[parts[0]] = parts[1:]
    return out


# ----------------------------------------------------------------- E4M3 decode
def test_e4m3_decode_page_facts(golden_dir):
    facts = _golden(golden_dir, "e4m3_page_facts.txt")
    d = oracle.e4m3_decode(np.arange(256, dtype=np.uint8))
    assert np.nanmax(d) == float(facts["e4m3_max_normal"][0])
    assert d[0x7E] == 448.0 and d[0xFE] == -448.0
    # 2^exponent_bits * 2^mantissa_bits codes per sign
    assert 2 ** (int(facts["e4m3_exponent_bits"][0]) + int(facts["e4m3_mantissa_bits"][0])) == 128


def test_e4m3_decode_exhaustive_against_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = oracle.e4m3_decode(codes.numpy())
    nan_ref = np.isnan(ref)
    assert (nan_ref == np.isnan(got)).all()
    assert nan_ref.sum() == 2 and nan_ref[0x7F] and nan_ref[0xFF]
    assert (ref[~nan_ref] == got[~nan_ref]).all()
    assert np.array_equal(np.signbit(ref[~nan_ref]), np.signbit(got[~nan_ref]))


def test_e4m3_decode_bit_construction():
    # place the fields into an IEEE float32 directly (independent of the oracle's arithmetic)
    for c in range(256):
        s, E, Mt = c >> 7, (c >> 3) & 15, c & 7
        if E == 15 and Mt == 7:
            continue
        if E == 0:
            bits = (s << 31) | (Mt << 20) | ((127 - 6) << 23)  # (1 + Mt/8) * 2^-6, minus the implicit 2^-6
            val = float(np.array([bits], np.uint32).view(np.float32)[0]) - (-1) ** s * 2.0 ** -6
        else:
            bits = (s << 31) | ((E - 7 + 127) << 23) | (Mt << 20)
            val = float(np.array([bits], np.uint32).view(np.float32)[0])
        got = oracle.e4m3_decode(np.array([c], np.uint8))[0]
        assert got == val, hex(c)


def test_e4m3_decode_structure():
    d = oracle.e4m3_decode(np.arange(256, dtype=np.uint8))
    fin = d[~np.isnan(d)]
    assert len(fin) == 254 and len(set(fin.tolist())) == 253  # +0 and -0 coincide
    pos = d[:0x7F]
    assert (np.diff(pos) > 0).all()  # codes 0x00..0x7E strictly increase
    assert d[0x08] == 2.0 ** -6 and d[0x01] == 2.0 ** -9 and d[0x00] == 0.0
    assert np.array_equal(d[0x80:0xFF], -d[0x00:0x7F])


# ----------------------------------------------------------------- E4M3 encode
def _e4m3_table():
    d = oracle.e4m3_decode(np.arange(256, dtype=np.uint8))
    codes = np.array([c for c in range(256) if not np.isnan(d[c])], dtype=np.int64)
    return codes, d[codes]


def _brute_encode(v: float) -> int:
    """Nearest finite E4M3 by exact rational distance, ties to even mantissa, saturating."""
    codes, vals = _e4m3_table()
    fv = Fraction(float(np.float32(v)))
    neg = np.signbit(np.float32(v))
    best = None
    for c, val in zip(codes, vals):
        if (c >> 7) != int(neg):
            continue
        dist = abs(Fraction(float(val)) - fv)
        key = (dist, c & 1)
        if best is None or key < best[0]:
            best = (key, int(c))
    return best[1]


def _adversarial_values():
    codes, vals = _e4m3_table()
    pos = np.unique(np.abs(vals))
    mids = (pos[:-1] + pos[1:]) / 2
    cand = [0.0, 2.0 ** -6, 2.0 ** -9, 2.0 ** -10, 448.0, 464.0, 1e6, 2.0 ** -6 - 2.0 ** -10]
    for m in mids:
        for eps in (0.0, 2.0 ** -20, -(2.0 ** -20)):
            cand.append(m * (1 + eps))
    for p in pos:
        f = np.float32(p)
        cand += [float(np.nextafter(f, np.float32(np.inf))), float(np.nextafter(f, np.float32(0)))]
    cand = np.array(cand, dtype=np.float32)
    return np.concatenate([cand, -cand])


def test_e4m3_encode_brute_force_adversarial():
    vals = _adversarial_values()
    got = oracle.e4m3_encode(vals)
    for v, g in zip(vals, got):
        assert int(g) == _brute_encode(float(v)), (v, hex(g))


def test_e4m3_encode_brute_force_random():
    rng = np.random.default_rng(11)
    v = np.concatenate([
        rng.standard_normal(600).astype(np.float32) * np.float32(100),
        (rng.standard_normal(300) * 2.0 ** rng.integers(-12, 9, 300)).astype(np.float32),
    ])
    got = oracle.e4m3_encode(v)
    for x, g in zip(v, got):
        assert int(g) == _brute_encode(float(x)), (x, hex(g))


def test_e4m3_encode_against_torch_in_range():
    # torch's float -> float8_e4m3fn conversion rounds to nearest even and does
    # not saturate (it gives NaN past the 448/NaN midpoint), so compare below 464.
    rng = np.random.default_rng(12)
    v = (rng.standard_normal(2_000_000) * 2.0 ** rng.integers(-14, 9, 2_000_000)).astype(np.float32)
    v = v[np.abs(v) < 464]
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = oracle.e4m3_encode(v)
    assert np.array_equal(ref, got)


def test_e4m3_encode_saturates_and_roundtrips():
    assert oracle.e4m3_encode(np.array([1e30, -1e30, 464.0, 500.0], np.float32)).tolist() == [0x7E, 0xFE, 0x7E, 0x7E]
    codes, vals = _e4m3_table()
    rt = oracle.e4m3_encode(vals.astype(np.float32))
    nz = vals != 0
    assert np.array_equal(rt[nz], codes[nz].astype(np.uint8))
    assert oracle.e4m3_encode(np.array([-0.0], np.float32))[0] == 0x80


# ----------------------------------------------------------------- bf16
def test_bf16_round_f32_matches_torch():
    rng = np.random.default_rng(3)
    with np.errstate(over="ignore"):
        v = (rng.standard_normal(3_000_000) * 2.0 ** rng.integers(-140, 128, 3_000_000)).astype(np.float32)
    special = np.array([0.0, -0.0, 1.0, 3.3895314e38, 3.39e38, 1e-40, -1e-45, np.inf, -np.inf], np.float32)
    v = np.concatenate([v, special])
    # every bf16 rounding boundary: odd/even midpoints of random bf16 pairs
    b = rng.integers(0, 0x7F7F, 100_000).astype(np.uint32)
    mid = ((b << 16) | 0x8000).view(np.float32)
    v = np.concatenate([v, mid, -mid])
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.bf16_to_bits(v.astype(np.float64))
    assert np.array_equal(ref, got)


def _brute_bf16_bits(v: float) -> int:
    """Nearest bf16 to a float64 value by exact rational comparison (ties to even)."""
    f32 = np.array([v], np.float64).astype(np.float32)  # any float32 near v
    base = int(f32.view(np.uint32)[0] >> 16) & 0x7FFF
    sign = 0x8000 if v < 0 else 0
    fv = Fraction(abs(v))
    best = None
    for cand in range(max(base - 2, 0), min(base + 3, 0x7F81)):
        val = np.array([cand << 16], np.uint32).view(np.float32)[0]
        if np.isinf(val):
            continue
        key = (abs(Fraction(float(val)) - fv), cand & 1)
        if best is None or key < best[0]:
            best = (key, cand)
    return best[1] | sign


def test_bf16_round_f64_no_double_rounding():
    rng = np.random.default_rng(5)
    vals = []
    # midpoints between bf16 neighbours nudged by less than a float32 ulp: rounding
    # through float32 first would land on the tie and pick the even side wrongly
    for _ in range(2000):
        hb = int(rng.integers(0x0080, 0x7F00))
        lo = float(np.array([hb << 16], np.uint32).view(np.float32)[0])
        hi = float(np.array([(hb + 1) << 16], np.uint32).view(np.float32)[0])
        mid = (lo + hi) / 2
        for nud in (2.0 ** -40, -(2.0 ** -40), 0.0):
            vals.append(mid * (1 + nud))
    vals += list(rng.standard_normal(2000) * 10.0 ** rng.integers(-30, 30, 2000))
    vals = np.array(vals)
    got = oracle.bf16_to_bits(vals)
    for v, g in zip(vals, got):
        assert int(g) == _brute_bf16_bits(float(v)), v


def test_bf16_overflow_to_inf():
    assert np.isinf(oracle.bf16_round(np.array([3.4e38]))[0])
    assert oracle.bf16_round(np.array([oracle.BF16_MAX]))[0] == oracle.BF16_MAX


# ----------------------------------------------------------------- fp16
def test_fp16_round_matches_torch():
    rng = np.random.default_rng(9)
    v = (rng.standard_normal(1_000_000) * 2.0 ** rng.integers(-30, 17, 1_000_000)).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.float16).numpy()
    got = oracle.fp16_round_f32(v)
    assert np.array_equal(ref.view(np.uint16), got.view(np.uint16))
