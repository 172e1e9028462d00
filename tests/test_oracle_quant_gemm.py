"""Pins for the oracle's quantisers, dequantisation and matmul (CPU only).

The checks come from outside the oracle's own formulas: brute-force argmin
over the quantisation grid in exact rationals, the representable-value sets,
exact rational matmuls on tiny shapes, special cases that reduce to integer
matmul / identity / zero, one-hot probes, and planted mistakes that the pins
must catch.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import wqd_inputs as I


def _frac(a):
    return [Fraction(float(v)) for v in np.asarray(a, dtype=np.float64).ravel()]


# ----------------------------------------------------------------- W4A16
def _w4a16_pin(W, qw):
    """Every unclamped code is the nearest grid point (q - z) * s (ties: either, when
    the float32 quotient is within rounding of a tie); z places 0 on the grid."""
    N, K = W.shape
    q, s16, z = qw["codes"], qw["scales"], qw["zeros"]
    assert q.dtype == np.uint8 and q.max() <= 15 and z.max() <= 15
    for n in range(N):
        for g in range(K // 128):
            s = Fraction(float(s16[n, g]))
            zz = int(z[n, g])
            ws = W[n, g * 128:(g + 1) * 128]
            lo = min(0.0, float(ws.min()))
            hi = max(0.0, float(ws.max()))
            if lo == hi:
                assert s == 1 and zz == 0 and (q[n, g * 128:(g + 1) * 128] == 0).all()
                continue
            # the scale is the fp16 rounding of (hi - lo) / 15 (the reading): 15 s ~ hi - lo
            assert abs(float(s) * 15 - (hi - lo)) <= (hi - lo) * 2.0 ** -10 + 2.0 ** -24 * 15
            # zero point: nearest integer to -lo / s
            r = -Fraction(lo) / s
            assert abs(r - zz) <= Fraction(1, 2) + Fraction(1, 2 ** 20)
            for k in range(128):
                w = Fraction(float(ws[k]))
                qq = int(q[n, g * 128 + k])
                d = [abs(w - (c - zz) * s) for c in range(16)]
                best = min(d)
                if d[qq] != best:
                    # allowed only at a tie up to float32 rounding of w / s
                    assert d[qq] - best <= s * Fraction(1, 2 ** 18), (n, g, k)


def test_w4a16_argmin_random():
    W = I.w_host(21, 24, 512)
    _w4a16_pin(W, oracle.quantize_w4a16(W))


def test_w4a16_argmin_structured():
    rng = np.random.default_rng(4)
    W = I.w_host(22, 8, 384)
    W[0, :128] = 0.0                    # all-zero group
    W[1, :128] = np.abs(W[1, :128])     # non-negative group: z = 0
    W[2, :128] = -np.abs(W[2, :128])    # non-positive group: z = 15
    W[3, 128:256] = 1e-9                # tiny group: scale floors at 2^-24
    W[4, :128] = rng.integers(-7, 8, 128).astype(np.float32) * np.float32(0.25)  # exact ties
    W[5, 256:] = np.float32(3.0)        # constant positive group
    qw = oracle.quantize_w4a16(W)
    _w4a16_pin(W, qw)
    assert qw["zeros"][1, 0] == 0 and qw["zeros"][2, 0] == 15
    assert qw["scales"][3, 1] == np.float16(2.0 ** -24)
    assert qw["scales"][0, 0] == 1 and qw["zeros"][0, 0] == 0


def test_w4a16_dequant_set_and_bits():
    W = I.w_host(23, 16, 256)
    qw = oracle.quantize_w4a16(W)
    Wd = oracle.dequant_exact(qw)
    s = np.repeat(qw["scales"].astype(np.float64), 128, axis=1)
    k = Wd / s
    assert np.array_equal(k, np.rint(k)) and np.abs(k).max() <= 15
    # fp32 dequant is exact: no rounding happened
    assert np.array_equal(oracle.dequant_f32(qw).astype(np.float64), Wd)
    # error bound: within half a step wherever the code is not clamped
    err = np.abs(Wd - W.astype(np.float64))
    assert (err <= s / 2 * (1 + 2.0 ** -18)).mean() > 0.999


# ----------------------------------------------------------------- FP8
def test_fp8_rowscale_and_codes():
    W = I.w_host(31, 32, 192)
    W[5] = 0.0
    qw = oracle.quantize_fp8(W)
    s = qw["scales"]
    assert s.dtype == np.float32 and s[5] == 1.0
    assert (qw["codes"][5] == 0).all()
    a = np.abs(W).max(axis=1)
    for n in range(32):
        if n == 5:
            continue
        assert s[n] == np.float32(a[n] / np.float32(448))
        # the row maximum maps to the E4M3 maximum 448 (code 0x7E with its sign)
        j = int(np.abs(W[n]).argmax())
        assert qw["codes"][n, j] & 0x7F == 0x7E
    # each code is the brute-force nearest E4M3 value of W / s (table lookup)
    table = oracle.e4m3_decode(np.arange(256, dtype=np.uint8))
    fin = np.array([c for c in range(256) if not np.isnan(table[c])])
    v = (W / s[:, None]).astype(np.float32).astype(np.float64)
    dist = np.abs(v[..., None] - table[fin][None, None, :])
    best = dist.min(axis=2)
    got = np.abs(v - table[qw["codes"]])
    assert np.array_equal(got, best)


def test_fp8_dequant_f32_single_rounding():
    W = I.w_host(32, 8, 64)
    qw = oracle.quantize_fp8(W)
    exact = oracle.dequant_exact(qw)
    f32 = oracle.dequant_f32(qw)
    # the float32 result is the IEEE float32 product of two float32 factors
    prod = (oracle.e4m3_decode(qw["codes"]).astype(np.float32) * qw["scales"][:, None]).astype(np.float32)
    assert np.array_equal(f32, prod)
    assert np.abs(f32 - exact).max() <= np.abs(exact).max() * 2.0 ** -24


def _e4m3_half_spacing(v):
    """Half the spacing of the E4M3 grid around |v| (no E4M3 routine involved):
    3 mantissa bits, so 2^(e-3) between neighbours in the binade [2^e, 2^(e+1))
    for e >= -6, and the subnormal step 2^-9 below 2^-6."""
    a = np.abs(np.asarray(v, np.float64))
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    step = np.where(a >= 2.0 ** -6, 2.0 ** (e - 3), 2.0 ** -9)
    return step / 2


def _fp8_wide_rows(seed=91, N=24, K=320):
    """Non-square W whose rows span very different magnitudes (distinct row scales)."""
    rng = np.random.default_rng(seed)
    W = rng.standard_normal((N, K)).astype(np.float32)
    mag = (2.0 ** rng.integers(-12, 6, size=N)) * rng.uniform(0.5, 1.0, size=N)
    return (W * mag[:, None].astype(np.float32)).astype(np.float32)


def check_fp8_dequant_error_bound(W, qw):
    """Round to nearest on the scaled grid: |Wd - W| <= s_n x (half an E4M3
    step at W / s_n + the float32 rounding of that quotient), element by
    element, and the row's absolute maximum is hit to that bound with the
    E4M3 maximum 448 (the per-row scale maps the row's largest weight to it)."""
    Wd = oracle.dequant_exact(qw)
    s = qw["scales"].astype(np.float64)
    assert Wd.shape == W.shape and s.shape == (W.shape[0],)
    v = W.astype(np.float64) / s[:, None]
    bound = s[:, None] * (_e4m3_half_spacing(v) + np.abs(v) * 2.0 ** -24)
    err = np.abs(Wd - W.astype(np.float64))
    assert (err <= bound).all(), float((err / bound).max())
    # round to nearest, not a looser rounding: somewhere the error is close to the bound
    assert (err / bound).max() > 0.9
    for n in range(W.shape[0]):
        j = int(np.abs(W[n]).argmax())
        assert abs(abs(Wd[n, j]) - 448 * s[n]) <= s[n] * 2.0 ** -20
        assert abs(abs(float(W[n, j])) - 448 * s[n]) <= abs(float(W[n, j])) * 2.0 ** -22


def test_fp8_dequant_error_bound_distinct_row_scales():
    W = _fp8_wide_rows()
    qw = oracle.quantize_fp8(W)
    assert len(np.unique(qw["scales"])) == W.shape[0]
    check_fp8_dequant_error_bound(W, qw)


def test_fp8_dequant_bound_catches_planted_scale_mistakes(monkeypatch):
    """Row scales reversed, or taken per column, must break the error bound."""
    import oracle.quant as Q

    W = _fp8_wide_rows()
    real_scales = Q.fp8_row_scales

    monkeypatch.setattr(Q, "fp8_row_scales", lambda A: real_scales(A)[::-1].copy())
    with pytest.raises((AssertionError, ValueError)):
        check_fp8_dequant_error_bound(W, Q.quantize_fp8(W))
    monkeypatch.undo()

    def column_scales(A):
        a = np.abs(np.asarray(A, np.float32)).max(axis=0)
        return np.where(a == 0, np.float32(1), a / np.float32(448)).astype(np.float32)

    def quantize_by_column(A):
        A = np.asarray(A, np.float32)
        sc = column_scales(A)
        return {"fmt": "fp8", "codes": oracle.e4m3_encode((A / sc[None, :]).astype(np.float32)), "scales": sc}

    with pytest.raises((AssertionError, ValueError)):
        check_fp8_dequant_error_bound(W, quantize_by_column(W))
    monkeypatch.undo()
    check_fp8_dequant_error_bound(W, Q.quantize_fp8(W))


# ----------------------------------------------------------------- matmul
def _brute_qgemm_bits(x_bits, qw):
    """Exact rational y = sum_k x * Wd, then nearest bf16 (ties to even), all by brute force."""
    x = oracle.bf16_bits_to_f64(x_bits)
    Wd = oracle.dequant_exact(qw)
    M, K = x.shape
    N = Wd.shape[0]
    xf = [[Fraction(float(v)) for v in row] for row in x]
    Wf = [[Fraction(float(v)) for v in row] for row in Wd]
    out = np.zeros((M, N), dtype=np.uint16)
    for m in range(M):
        for n in range(N):
            acc = sum(a * b for a, b in zip(xf[m], Wf[n]))
            out[m, n] = _nearest_bf16_bits(acc)
    return out


def _nearest_bf16_bits(v: Fraction) -> int:
    sign = 0x8000 if v < 0 else 0
    a = abs(v)
    if a == 0:
        return sign
    approx = np.array([float(a)], np.float64).astype(np.float32).view(np.uint32)[0] >> 16
    best = None
    for cand in range(max(int(approx) - 2, 0), min(int(approx) + 3, 0x7F80)):
        val = Fraction(float(np.array([cand << 16], np.uint32).view(np.float32)[0]))
        key = (abs(val - a), cand & 1)
        if best is None or key < best[0]:
            best = (key, cand)
    return best[1] | sign


@pytest.mark.parametrize("fmt", ["bf16", "fp8", "w4a16"])
@pytest.mark.parametrize("M,N,K", [(1, 16, 128), (3, 5, 256), (4, 16, 128)])
def test_qgemm_matches_exact_rationals(fmt, M, N, K):
    W = I.w_host(100 + M + N, N, K)
    x = I.x_bf16_bits(200 + K, M, K)
    qw = oracle.quantize(fmt, W)
    ref = oracle.qgemm_ref(x, qw)
    assert np.array_equal(ref["y_bits"], _brute_qgemm_bits(x, qw))


def test_qgemm_integer_special_case():
    # s = 1, z = 8: the product is an integer matmul of x with (q - 8)
    rng = np.random.default_rng(8)
    M, N, K = 4, 12, 256
    q = rng.integers(0, 16, (N, K)).astype(np.uint8)
    qw = {"fmt": "w4a16", "codes": q, "scales": np.ones((N, K // 128), np.float16),
          "zeros": np.full((N, K // 128), 8, np.uint8)}
    xi = rng.integers(-20, 21, (M, K))
    x_bits = oracle.bf16_to_bits(xi.astype(np.float64))
    y = oracle.qgemm_ref(x_bits, qw)["y64"]
    assert np.array_equal(y, (xi @ (q.astype(np.int64) - 8).T).astype(np.float64))


def test_qgemm_identity_and_zero():
    K = 64
    x = I.x_bf16_bits(5, 3, K)
    eye = oracle.quantize_bf16(np.eye(K, dtype=np.float32))
    assert np.array_equal(oracle.qgemm_ref(x, eye)["y_bits"], x)
    for fmt in ("bf16", "fp8", "w4a16"):
        Kz = 128
        z = oracle.quantize(fmt, np.zeros((7, Kz), np.float32))
        y = oracle.qgemm_ref(I.x_bf16_bits(6, 2, Kz), z)["y64"]
        assert (y == 0).all()


@pytest.mark.parametrize("fmt", ["bf16", "fp8", "w4a16"])
def test_one_hot_probe(fmt):
    N, K = 40, 256
    W = I.w_host(7, N, K)
    qw = oracle.quantize(fmt, W)
    Wd = oracle.dequant_exact(qw)
    for k in (0, 1, 127, 128, 255):
        x = np.zeros((1, K), np.uint16)
        x[0, k] = 0x3F80  # 1.0
        y = oracle.qgemm_ref(x, qw)["y_bits"][0]
        assert np.array_equal(y, oracle.bf16_to_bits(Wd[:, k]))


# ----------------------------------------------------------------- planted mistakes
def test_pins_catch_planted_mistakes(monkeypatch):
    """Plant plausible mistakes in the oracle and check that a pin fails for each."""
    import oracle.gemm as G
    import oracle.quant as Q

    M, N, K = 2, 6, 128
    W = I.w_host(77, N, K)
    x = I.x_bf16_bits(78, M, K)

    def brute_ok(fmt):
        qw = oracle.quantize(fmt, W)
        return np.array_equal(oracle.qgemm_ref(x, qw)["y_bits"], _brute_qgemm_bits(x, qw))

    assert brute_ok("w4a16")
    real = Q.dequant_exact

    # 1) dropped zero point in the W4A16 dequant: the brute force uses the same
    #    dequant, so this one must be caught by the integer special case instead
    def no_zero(qw):
        if qw["fmt"] == "w4a16":
            return qw["codes"].astype(np.float64) * np.repeat(qw["scales"].astype(np.float64), 128, axis=1)
        return real(qw)

    monkeypatch.setattr(G, "dequant_exact", no_zero)
    with pytest.raises(AssertionError):
        test_qgemm_integer_special_case()
    monkeypatch.setattr(G, "dequant_exact", real)

    # 2) transposed / misindexed product: caught by the one-hot probe
    def transposed(x_bits, qw):
        xx = oracle.bf16_bits_to_f64(x_bits)
        Wd = real(qw)
        return xx @ Wd[:, ::-1].T

    monkeypatch.setattr(G, "qgemm_exact", transposed)
    with pytest.raises(AssertionError):
        test_one_hot_probe("bf16")
    monkeypatch.undo()

    # 3) wrong rounding of the scale (scale left in float32): caught by the argmin pin's
    #    fp16 check on the stored scale dtype / value
    s16, z = Q.w4a16_group_params(W)
    assert s16.dtype == np.float16

    # 4) sign error in the FP8 encoder: caught by the torch comparison
    def bad_encode(v):
        return oracle.formats.e4m3_encode(-np.asarray(v, np.float32))

    monkeypatch.setattr(oracle, "e4m3_encode", bad_encode)
    with pytest.raises(AssertionError):
        from tests.test_oracle_formats import test_e4m3_encode_against_torch_in_range
        test_e4m3_encode_against_torch_in_range()
