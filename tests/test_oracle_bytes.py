"""Pins of the oracle's byte model (``oracle/bytes.py``) to the numbers the pages print.

Every GB/s and roofline fraction this project reports divides algorithmic
bytes by time.  Those bytes come from ``workloads.py``; the oracle computes
them independently and is pinned here to the pages' own closed forms
(``tests/golden/bytes_page_values.txt``, each value with its source):

* "Making each token cheaper", section "Why decode is usually bandwidth bound":
  70e9 BF16 parameters are 140e9 bytes; the batch-1 floor at 3.0 TB/s is
  46.667 ms and the compute time at 1,000 TFLOP/s 0.140 ms; one sequence's KV
  cache at 80 layers x 8 KV heads x 128 x 2 bytes x 2,048 tokens is 671,088,640
  bytes, and batch 32 raises the floor to 53.825 ms.
* same page, "Worked example: weight bytes and bounds per format": FP8 70.0 GB
  (a 32-bit scale per 8,192-weight row adds under 0.004 bits per weight),
  INT4 g128 at 4.15 bits 36.3125 GB (a 16-bit scale per 128 weights adds 0.125
  bits, GPTQ's estimate is about 0.15).
* same page, "Building a per-token cost calculator", the expected values:
  batch-1 23.333 / 12.104 ms, batch-32 30.492 / 19.262 ms, INT4 verify cost
  ratio 1.1629 for 5 positions per sequence.
* same page, the hands-on lab, exercise 5 and its reference values: with a
  1-byte FP8 KV cache (scales ignored) the INT4 batch-32 bound is 15.683 ms.
* CS336 lecture 10 notes, section 10, exercise 4: a 4096 x 4096 INT4 matrix
  with groups of 128 and an FP16 scale takes 4.125 bits per weight, about
  8.65 MB, against 33.6 MB in BF16.

The format stored here adds a uint4 zero point per group: 4 + 16/128 + 4/128 =
4.15625 bits.  The page's 4.15 is GPTQ's rounded estimate; the difference,
0.00625 bits per weight, is checked as exactly the zero points' bytes.

A last test plants plausible mistakes in the oracle's byte model (zero points
dropped, scale bytes doubled, FP8 scales counted per column) and checks that
these pins catch each one.
"""
import os
from fractions import Fraction

import pytest

import oracle.bytes as B

PARAMS_70B = 70_000_000_000
HBM_PAGE = 3.0e12          # the page's hypothetical part, bytes per second
PEAK_PAGE = 1.0e15         # its dense FLOP/s
# 70e9 parameters as one matrix of whole 128-weight groups (70e9 = 546,875,000 x 128)
N_70B_AS_ROWS, K_GROUP = 546_875_000, 128


def golden(golden_dir):
    vals = {}
    with open(os.path.join(golden_dir, "bytes_page_values.txt")) as f:
        for ln in f:
            ln = ln.strip()
            if not ln or ln.startswith("#"):
                continue
            key, value, tol, src = ln.split()
            vals[key] = (float(value), float(tol), src)
    return vals


USED_KEYS = set()


def close(got, key, g):
    USED_KEYS.add(key)
    value, tol, src = g[key]
    assert abs(got - value) <= tol, f"{key}: {got} vs the page's {value} (source {src})"


# ------------------------------------------------------------------ checks (shared by the planted-mistake test)
def check_bf16(g):
    wb = B.weight_bytes("bf16", N_70B_AS_ROWS, K_GROUP)
    close(sum(wb.values()), "bf16_weight_bytes_70b", g)
    bf16_4096 = sum(B.weight_bytes("bf16", 4096, 4096).values())
    close(bf16_4096 / 1e6, "bf16_4096sq_mb", g)


def check_fp8(g):
    wb = B.weight_bytes("fp8", N_70B_AS_ROWS, K_GROUP)
    close(wb["w"] / 1e9, "fp8_weight_gb_70b", g)
    # one 32-bit scale per row of 8,192 weights adds under 0.004 bits per
    # weight; checked on a short-N 70B matrix (k: 1024 x 8192), where counting
    # one scale per column instead would add 0.03 bits
    for N, K in ((1024, 8192), (8192, 8192), (28672, 8192)):
        wb = B.weight_bytes("fp8", N, K)
        extra_bits = Fraction(8 * wb["s"], N * K)
        assert 0 < extra_bits < Fraction(4, 1000), (N, K, float(extra_bits))
        assert wb["w"] == N * K and wb["z"] == 0


def check_w4a16(g):
    # CS336 exercise 4: codes and fp16 scales of a 4096 x 4096 INT4 g128 matrix
    wb = B.weight_bytes("w4a16", 4096, 4096)
    close(wb["w"] + wb["s"], "int4_g128_4096sq_bytes_scale_only", g)
    close((wb["w"] + wb["s"]) / 1e6, "int4_g128_4096sq_mb", g)
    close(float(Fraction(8 * (wb["w"] + wb["s"]), 4096 * 4096)), "int4_g128_fp16scale_bits_per_weight", g)
    # GPTQ's estimate: about 0.15 extra bits per weight for scale and zero
    # together (the page rounds to two decimals; allow one unit in the last)
    total_bits = Fraction(8 * sum(wb.values()), 4096 * 4096)
    assert abs(float(total_bits) - 4.15) <= 0.01, float(total_bits)
    # at 70e9 parameters the page's 4.15-bit figure is 36.3125 GB; this format
    # is the codes' 35 GB plus its scale and zero bytes, and the two differ by
    # exactly 70e9 x (bits - 4.15) / 8
    wb70 = B.weight_bytes("w4a16", N_70B_AS_ROWS, K_GROUP)
    page = B.params_weight_bytes(PARAMS_70B, 4.15)
    close(page / 1e9, "int4_weight_gb_70b_at_4.15_bits", g)
    assert wb70["w"] == PARAMS_70B // 2
    ours = sum(wb70.values())
    assert abs((ours - page) - PARAMS_70B * (float(total_bits) - 4.15) / 8) < 1.0
    # the bits per weight of a row are the same whatever N (groups are row-local)
    for N, K in ((8192, 8192), (1024, 8192), (8192, 28672)):
        wbN = B.weight_bytes("w4a16", N, K)
        assert Fraction(8 * sum(wbN.values()), N * K) == total_bits == B.bits_per_weight("w4a16", K)


def check_bounds(g):
    kv = B.kv_bytes_per_sequence(layers=80, kv_heads=8, head_dim=128, bytes_per_elem=2, context=2048)
    close(kv, "kv_bytes_per_sequence", g)
    w_bf16 = sum(B.weight_bytes("bf16", N_70B_AS_ROWS, K_GROUP).values())
    # the batch-1 bound counts the weights alone
    close(1e3 * B.memory_time_s(w_bf16, 1, 0, HBM_PAGE), "bound_bf16_batch1_ms", g)
    close(1e3 * B.compute_time_s(PARAMS_70B, 1, 1, PEAK_PAGE), "compute_bf16_batch1_ms", g)
    close(1e3 * B.step_bound_s(w_bf16, 32, 1, kv, PARAMS_70B, HBM_PAGE, PEAK_PAGE), "bound_bf16_batch32_ms", g)
    # FP8 and INT4 at the page's bits per weight (the table ignores FP8's scales)
    for fmt_key, bits in (("fp8", 8.0), ("int4", 4.15)):
        wbytes = B.params_weight_bytes(PARAMS_70B, bits)
        close(1e3 * B.memory_time_s(wbytes, 1, 0, HBM_PAGE), f"bound_{fmt_key}_batch1_ms", g)
        close(1e3 * B.step_bound_s(wbytes, 32, 1, kv, PARAMS_70B, HBM_PAGE, PEAK_PAGE),
              f"bound_{fmt_key}_batch32_ms", g)
    # a 1-byte (FP8) KV cache, scales ignored as the lab's exercise says: the
    # INT4 batch-32 bound drops from 19.262 to 15.683 ms
    kv8 = B.kv_bytes_per_sequence(layers=80, kv_heads=8, head_dim=128, bytes_per_elem=1, context=2048)
    assert 2 * kv8 == kv
    w4 = B.params_weight_bytes(PARAMS_70B, 4.15)
    close(1e3 * B.step_bound_s(w4, 32, 1, kv8, PARAMS_70B, HBM_PAGE, PEAK_PAGE), "bound_int4_batch32_fp8kv_ms", g)
    # verifying 4 drafts + 1 position per sequence turns INT4's batch-32 step
    # compute bound; BF16 and FP8 stay memory bound (ratio exactly 1)
    for bits, key in ((16.0, None), (8.0, None), (4.15, "int4_verify_cost_ratio")):
        wbytes = B.params_weight_bytes(PARAMS_70B, bits)
        plain = B.step_bound_s(wbytes, 32, 1, kv, PARAMS_70B, HBM_PAGE, PEAK_PAGE)
        verify = B.step_bound_s(wbytes, 32, 5, kv, PARAMS_70B, HBM_PAGE, PEAK_PAGE)
        if key is None:
            assert verify / plain == 1.0
        else:
            close(verify / plain, key, g)


ALL_CHECKS = (check_bf16, check_fp8, check_w4a16, check_bounds)


# ------------------------------------------------------------------ the pins
@pytest.mark.parametrize("check", ALL_CHECKS, ids=lambda c: c.__name__)
def test_byte_model_against_page_values(check, golden_dir):
    check(golden(golden_dir))


def test_every_golden_value_is_checked(golden_dir):
    g = golden(golden_dir)
    USED_KEYS.clear()
    for c in ALL_CHECKS:
        c(g)
    assert USED_KEYS == set(g), sorted(set(g) ^ USED_KEYS)


def test_call_bytes_counts_x_and_y_once():
    # M activation rows of K bf16 in, M output rows of N bf16 out
    for fmt in ("bf16", "fp8", "w4a16"):
        w = sum(B.weight_bytes(fmt, 8192, 8192).values())
        for M in (1, 8, 1024):
            assert B.call_bytes(fmt, M, 8192, 8192) == w + 2 * M * 8192 + 2 * M * 8192


# ------------------------------------------------------------------ the reported byte counts
def _config_shapes():
    import wqd_inputs as I

    shapes = set((N, K) for _, N, K in I.LAYER_70B + I.LAYER_7B)
    shapes |= {(4096, 4096), (10240, 8192), (57344, 8192), (12288, 4096), (22016, 4096)}
    return sorted(shapes)


def test_workload_bytes_equal_oracle_model():
    """The byte counts behind every reported GB/s (workloads.py) agree with the pinned oracle model."""
    from weight_only_quantized_decode_amd import workloads as WL

    for fmt in ("bf16", "fp8", "w4a16"):
        for N, K in _config_shapes():
            assert WL.weight_bytes(fmt, N, K) == B.weight_bytes(fmt, N, K), (fmt, N, K)
            for M in (1, 4, 8, 16, 32, 48, 128, 1024):
                assert WL.call_bytes(fmt, M, N, K) == B.call_bytes(fmt, M, N, K), (fmt, M, N, K)


def test_stack_step_bytes():
    """Whole-stack bytes from the oracle model: 80 70B layers, 32 7B layers."""
    import wqd_inputs as I
    from weight_only_quantized_decode_amd import workloads as WL

    # fused layout: q/k/v and gate/up each one matrix, so their x is read once
    fused_70b = ((10240, 8192), (8192, 8192), (57344, 8192), (8192, 28672))
    fused_7b = ((12288, 4096), (4096, 4096), (22016, 4096), (4096, 11008))
    for fmt, M, fused in (("w4a16", 1, True), ("w4a16", 1, False), ("w4a16", 8, True), ("fp8", 1, True),
                          ("fp8", 8, False)):
        wl = WL.stack_70b(fmt, M, 80, fused)
        shapes = fused_70b if fused else [(N, K) for _, N, K in I.LAYER_70B]
        assert wl.step_bytes() == 80 * sum(B.call_bytes(fmt, M, N, K) for N, K in shapes)
    # the same weights either way: only the x bytes of the merged launches differ
    for fmt in ("w4a16", "fp8"):
        sep, fus = WL.stack_70b(fmt, 1, 80, False), WL.stack_70b(fmt, 1, 80, True)
        assert sep.step_bytes() - fus.step_bytes() == 80 * 2 * (2 + 1) * 8192
    wl = WL.stack_7b_bf16(1, 32, True)
    assert wl.step_bytes() == 32 * sum(B.call_bytes("bf16", 1, N, K) for N, K in fused_7b)


# ------------------------------------------------------------------ planted mistakes
def test_pins_catch_planted_byte_mistakes(golden_dir, monkeypatch):
    g = golden(golden_dir)

    def fails():
        for c in ALL_CHECKS:
            try:
                c(g)
            except (AssertionError, ValueError):
                return True
        return False

    assert not fails()
    # zero points dropped from the W4A16 bytes
    monkeypatch.setattr(B, "W4A16_ZERO_BITS", 0)
    assert fails(), "dropped zero points"
    monkeypatch.undo()
    # scale bytes doubled (a float32 scale counted instead of fp16)
    monkeypatch.setattr(B, "W4A16_SCALE_BITS", 32)
    assert fails(), "doubled scale bytes"
    monkeypatch.undo()
    # FP8 scales counted once per column instead of once per row
    real = B.weight_bytes

    def column_scales(fmt, N, K):
        wb = real(fmt, N, K)
        if fmt == "fp8":
            wb["s"] = 4 * K
        return wb

    monkeypatch.setattr(B, "weight_bytes", column_scales)
    assert fails(), "column scales"
    monkeypatch.undo()
    # the KV cache counting only keys (a dropped factor of 2)
    realkv = B.kv_bytes_per_sequence
    monkeypatch.setattr(B, "kv_bytes_per_sequence", lambda *a, **k: realkv(*a, **k) // 2)
    assert fails(), "keys only"
    monkeypatch.undo()
    assert not fails()
