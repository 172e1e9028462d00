"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Integer work (codes, scales, zero points, dequantised weights) is compared
bit for bit; y within the tolerance in tests/parity.py.  Small cases span
several 64-row tiles, several K tiles and ragged tails in N and K; the
full-size cases use the exact shapes and launch plans of the benchmark and
check sampled output channels, which the oracle computes one by one.
"""
import numpy as np
import pytest
import torch

import oracle
import weight_only_quantized_decode_amd as wqd
import wqd_inputs as I
from tests.parity import bf16_bits, compare_y

pytestmark = pytest.mark.gpu

FMTS = ("bf16", "fp8", "w4a16")


def dev():
    return torch.device("cuda", 0)


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


def x_dev(x_bits):
    return to_dev(x_bits.view(np.int16)).view(torch.bfloat16)


def small_shapes(fmt):
    # (N, K): several tiles, ragged N; ragged K tiles where the format allows it
    if fmt == "w4a16":
        return [(357, 896), (64, 128), (1, 128), (130, 512), (200, 4096)]
    return [(357, 904), (64, 64), (1, 8), (130, 512), (200, 4096)]


def check_unpack(fmt, pw, qw):
    codes, scales, zeros = wqd.unpack(pw)
    torch.cuda.synchronize()
    if fmt == "bf16":
        assert np.array_equal(codes.cpu().numpy().view(np.uint16), qw["codes"])
    elif fmt == "fp8":
        assert np.array_equal(codes.cpu().numpy(), qw["codes"])
        assert np.array_equal(scales.cpu().numpy().view(np.uint32), qw["scales"].view(np.uint32))
    else:
        assert np.array_equal(codes.cpu().numpy(), qw["codes"])
        assert np.array_equal(scales.cpu().numpy().view(np.uint16), qw["scales"].view(np.uint16))
        assert np.array_equal(zeros.cpu().numpy(), qw["zeros"])


# --------------------------------------------------------------------------- formats
def test_decode_e4m3_exhaustive():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8).to(dev())
    got = wqd.decode_e4m3(codes).cpu().numpy().astype(np.float64)
    ref = oracle.e4m3_decode(np.arange(256, dtype=np.uint8))
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(got[fin], ref[fin])
    assert np.array_equal(np.signbit(got[fin]), np.signbit(ref[fin]))
    assert np.nanmax(got) == 448.0


@pytest.mark.parametrize("fmt", FMTS)
def test_pack_unpack_and_dequant_bitexact(fmt):
    for N, K in small_shapes(fmt):
        print(f"pack/unpack/dequant {fmt} N={N} K={K}", flush=True)
        W = I.w_host(11 + N + K, N, K)
        qw = oracle.quantize(fmt, W)
        pw = wqd.pack_weights(fmt, to_dev(W))
        check_unpack(fmt, pw, qw)
        Wd = wqd.dequant(pw).cpu().numpy()
        assert np.array_equal(Wd.view(np.uint32), oracle.dequant_f32(qw).view(np.uint32)), (fmt, N, K)


def test_pack_degenerate_groups_and_rows():
    rng = np.random.default_rng(3)
    W = I.w_host(5, 70, 384)
    W[0, :] = 0.0                             # zero row (fp8 scale 1) and zero groups
    W[1, :128] = np.abs(W[1, :128])           # z = 0
    W[2, 128:256] = -np.abs(W[2, 128:256])    # z = 15
    W[3, 256:] = 1e-9                         # tiny groups: fp16 scale floors at 2^-24
    W[4, :] = np.float32(3.0)                 # constant row
    W[5, :128] = rng.integers(-7, 8, 128).astype(np.float32) * np.float32(0.25)  # exact ties
    W[6, :] = -0.0
    W[7, 5] = np.float32(1e4)                 # one outlier inflating its group / row scale
    for fmt in FMTS:
        qw = oracle.quantize(fmt, W)
        pw = wqd.pack_weights(fmt, to_dev(W))
        check_unpack(fmt, pw, qw)
        Wd = wqd.dequant(pw).cpu().numpy()
        assert np.array_equal(Wd.view(np.uint32), oracle.dequant_f32(qw).view(np.uint32)), fmt


# --------------------------------------------------------------------------- qgemm small
@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 6, 7, 8, 9, 16, 33])
def test_qgemm_small_shapes(fmt, M):
    for N, K in small_shapes(fmt):
        print(f"qgemm {fmt} M={M} N={N} K={K}", flush=True)
        W = I.w_host(1000 + N + K, N, K)
        qw = oracle.quantize(fmt, W)
        pw = wqd.pack_weights(fmt, to_dev(W))
        x = I.x_bf16_bits(7 * M + K, M, K)
        y = wqd.qgemm(x_dev(x), pw)
        torch.cuda.synchronize()
        compare_y(bf16_bits(y), oracle.qgemm_exact(x, qw), f"{fmt} M={M} N={N} K={K}")


def bcast_shapes(fmt):
    # (N, K) for the broadcast kernel: shares of 1, 3, 5 (partial groups), 16
    # tiles, 4 / 8 / 16 wavefronts per block, and K long enough that it falls
    # back to the staged kernel (more than 512 tiles; 256 for two W4A16 rows)
    if fmt == "w4a16":
        return [(16, 128), (40, 384), (200, 640), (72, 2176), (1024, 8192), (96, 12800), (64, 28672), (16, 32896),
                (16, 65664)]
    if fmt == "fp8":
        return [(16, 8), (40, 72), (200, 1000), (1024, 8192), (64, 16384), (16, 16448), (16, 32832)]
    return [(16, 8), (40, 72), (200, 1000), (1024, 8192), (16, 8200), (16, 16416)]


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("M", [1, 2, 3, 5, 8])
def test_qgemm_broadcast_rows(fmt, M):
    for N, K in bcast_shapes(fmt):
        print(f"qgemm {fmt} M={M} N={N} K={K}", flush=True)
        W = I.w_host(2000 + N + K, N, K)
        qw = oracle.quantize(fmt, W)
        pw = wqd.pack_weights(fmt, to_dev(W))
        x = I.x_bf16_bits(11 * M + K, M, K)
        y = wqd.qgemm(x_dev(x), pw)
        torch.cuda.synchronize()
        compare_y(bf16_bits(y), oracle.qgemm_exact(x, qw), f"{fmt} M={M} N={N} K={K}")


@pytest.mark.parametrize("fmt,N,K,waves", [("w4a16", 4096, 20608, 8), ("fp8", 4096, 12352, 8),
                                           ("bf16", 2048, 10976, 16)])
def test_qgemm_long_shares(fmt, N, K, waves):
    """One row, shares of 24-28 tiles (eight groups; two x-sum registers for
    W4A16), a partial last group and an idle last wavefront."""
    assert wqd.kernel_path(fmt, 1, N, K) == ("bcast", waves)
    print(f"qgemm {fmt} M=1 N={N} K={K}", flush=True)
    W = I.w_host(3000 + K, N, K)
    qw = oracle.quantize(fmt, W)
    pw = wqd.pack_weights(fmt, to_dev(W))
    x = I.x_bf16_bits(17 + K, 1, K)
    y = wqd.qgemm(x_dev(x), pw)
    torch.cuda.synchronize()
    compare_y(bf16_bits(y), oracle.qgemm_exact(x, qw), f"{fmt} M=1 N={N} K={K}")


@pytest.mark.parametrize("fmt", FMTS)
def test_qgemm_two_blocks_per_wave(fmt):
    """Streaming matrix-core kernel with two 16-row blocks per wavefront, an odd
    block count (the last workgroup's second block is past N) and a ragged N."""
    N, K, M = 16392, 1024, 6
    assert wqd.kernel_path(fmt, M, N, K)[0] == "mc"
    print(f"qgemm {fmt} M={M} N={N} K={K}", flush=True)
    W = I.w_host(4000 + N, N, K)
    qw = oracle.quantize(fmt, W)
    pw = wqd.pack_weights(fmt, to_dev(W))
    x = I.x_bf16_bits(23, M, K)
    y = wqd.qgemm(x_dev(x), pw)
    torch.cuda.synchronize()
    compare_y(bf16_bits(y), oracle.qgemm_exact(x, qw), f"{fmt} M={M} N={N} K={K}")


@pytest.mark.parametrize("fmt", ["w4a16", "fp8"])
def test_qgemm_three_blocks_per_wave(fmt):
    """Streaming matrix-core kernel with three 16-row blocks per wavefront (640
    row blocks: 214 workgroups instead of 320 of two), and a ragged N whose
    last workgroup holds one partial block and two past N."""
    for N in (10240, 10232):
        K = 1024
        W = I.w_host(4100 + N, N, K)
        qw = oracle.quantize(fmt, W)
        pw = wqd.pack_weights(fmt, to_dev(W))
        for M in ((2, 6, 8) if fmt == "w4a16" else (6, 8)):
            assert wqd.kernel_path(fmt, M, N, K) == ("mc", 4)
            print(f"qgemm {fmt} M={M} N={N} K={K}", flush=True)
            x = I.x_bf16_bits(29 + M, M, K)
            y = wqd.qgemm(x_dev(x), pw)
            torch.cuda.synchronize()
            compare_y(bf16_bits(y), oracle.qgemm_exact(x, qw), f"{fmt} M={M} N={N} K={K}")


def skinny_shapes(fmt):
    # (N, K) for the skinny matrix-core kernel, in tiles of TK k.  With the
    # planner's choices: 13 tiles (shares shorter than one loop body; 7
    # consumers of one row block), 5 tiles over 3073 row blocks (7 consumers
    # of two row blocks, no K split, a half-live last workgroup), 512 row blocks
    # of 64 tiles (4 consumers of two row blocks, 4-way K split), 257 and 63 row
    # blocks (ragged last groups, K splits), a 7-way split whose last split
    # is short (28 of 32 tiles), and 640 row blocks of 64 tiles (5 consumers
    # of two row blocks, 4-way K split)
    tk = {"w4a16": 128, "fp8": 64, "bf16": 32}[fmt]
    return [(2000, 13 * tk), (49160, 5 * tk), (8192, 64 * tk), (4104, 64 * tk), (1000, 8192), (300, 220 * tk),
            (10240, 64 * tk)]


@pytest.mark.parametrize("fmt", FMTS)
def test_qgemm_skinny(fmt):
    """x staged in LDS by a producer wavefront and shared by 4 consumer
    wavefronts (two 16-row blocks each), K split over
    workgroups with the fixed-order partial sum."""
    for N, K in skinny_shapes(fmt):
        W = I.w_host(5000 + N + K, N, K)
        qw = oracle.quantize(fmt, W)
        pw = wqd.pack_weights(fmt, to_dev(W))
        for M in (9, 16, 17, 32, 40, 64):
            # up to 16 rows, matrices up to 8192 x 8192 that it would split go to
            # the streaming matrix-core kernel (tested below)
            assert wqd.kernel_path(fmt, M, N, K)[0] in (("skinny", "mc") if M <= 16 else ("skinny",))
            print(f"qgemm {fmt} M={M} N={N} K={K} ws={wqd.workspace_bytes(fmt, M, N, K)}", flush=True)
            x = I.x_bf16_bits(29 * M + K, M, K)
            y = wqd.qgemm(x_dev(x), pw)
            torch.cuda.synchronize()
            compare_y(bf16_bits(y), oracle.qgemm_exact(x, qw), f"{fmt} M={M} N={N} K={K}")


def mc_wide_row_shapes(fmt):
    # (N, K) that take the streaming matrix-core kernel from 9 to 16 rows: a
    # ragged N of 63 row blocks with long shares (16 wavefronts for BF16), 129
    # row blocks, and 257 row blocks over the longest K it takes
    return [(1000, 8192), (2056, 4096), (4104, 8192)]


@pytest.mark.parametrize("fmt", FMTS)
def test_qgemm_mc_rows_9_to_16(fmt):
    """9 to 16 activation rows in one 16-row x block of the streaming matrix-core kernel."""
    for N, K in mc_wide_row_shapes(fmt):
        W = I.w_host(9000 + N + K, N, K)
        qw = oracle.quantize(fmt, W)
        pw = wqd.pack_weights(fmt, to_dev(W))
        for M in (9, 12, 16):
            assert wqd.kernel_path(fmt, M, N, K)[0] == "mc"
            print(f"qgemm {fmt} M={M} N={N} K={K}", flush=True)
            x = I.x_bf16_bits(41 * M + K, M, K)
            y = wqd.qgemm(x_dev(x), pw)
            torch.cuda.synchronize()
            compare_y(bf16_bits(y), oracle.qgemm_exact(x, qw), f"{fmt} M={M} N={N} K={K}")


def tiled_shapes(fmt):
    # (N, K) for the tiled matrix-core kernel (at least 16 column blocks of
    # 256): a partial column block, odd chunk counts (11, 19; W4A16 5, 9), K
    # splits over few workgroups, and a K that ends inside a tile (x past K
    # reads as zero; W4A16 K is whole groups)
    if fmt == "w4a16":
        return [(3900, 640), (4000, 1152), (4104, 4096)]
    return [(3900, 648), (4000, 1160), (4104, 4096)]


@pytest.mark.parametrize("fmt", FMTS)
def test_qgemm_tiled(fmt):
    """Wide verify batches: 64- and 128-row tiles of y with a ragged last row block."""
    for N, K in tiled_shapes(fmt):
        W = I.w_host(6000 + N + K, N, K)
        qw = oracle.quantize(fmt, W)
        pw = wqd.pack_weights(fmt, to_dev(W))
        for M in (65, 100, 128, 129, 257, 300, 384):
            assert wqd.kernel_path(fmt, M, N, K)[0] == "gemm"
            print(f"qgemm {fmt} M={M} N={N} K={K} ws={wqd.workspace_bytes(fmt, M, N, K)}", flush=True)
            x = I.x_bf16_bits(31 * M + K, M, K)
            y = wqd.qgemm(x_dev(x), pw)
            torch.cuda.synchronize()
            compare_y(bf16_bits(y), oracle.qgemm_exact(x, qw), f"{fmt} M={M} N={N} K={K}")


@pytest.mark.parametrize("N,K,Ms", [(16392, 640, (200,)), (16392, 2048, (65, 200)), (12296, 4096, (65,))])
def test_qgemm_tiled_w4a16_128_rows(N, K, Ms):
    """W4A16 on 128-row wavefront tiles (the planner's time model picks them for
    these shapes): no K split with an odd chunk count (5) and an even one
    (16), K splits of 3 and 5 with both remainders, and ragged rows."""
    fmt = "w4a16"
    W = I.w_host(6100 + N + K, N, K)
    qw = oracle.quantize(fmt, W)
    pw = wqd.pack_weights(fmt, to_dev(W))
    for M in Ms:
        assert wqd.kernel_path(fmt, M, N, K) == ("gemm", 8)
        print(f"qgemm {fmt} M={M} N={N} K={K} ws={wqd.workspace_bytes(fmt, M, N, K)}", flush=True)
        x = I.x_bf16_bits(37 * M + K, M, K)
        y = wqd.qgemm(x_dev(x), pw)
        torch.cuda.synchronize()
        compare_y(bf16_bits(y), oracle.qgemm_exact(x, qw), f"{fmt} M={M} N={N} K={K}")


@pytest.mark.parametrize("fmt,N,K,M", [("bf16", 8224, 4096, 200), ("bf16", 8232, 4104, 193)])
def test_qgemm_tiled_256_rows_padded(fmt, N, K, M):
    """BF16 on 256-row tiles below 256 rows (the planner's time model picks them
    for these shapes with a K split): padded rows, ragged N, ragged K."""
    W = I.w_host(6200 + N + K, N, K)
    qw = oracle.quantize(fmt, W)
    pw = wqd.pack_weights(fmt, to_dev(W))
    assert wqd.kernel_path(fmt, M, N, K) == ("gemm", 8)
    print(f"qgemm {fmt} M={M} N={N} K={K} ws={wqd.workspace_bytes(fmt, M, N, K)}", flush=True)
    x = I.x_bf16_bits(41 * M + K, M, K)
    y = wqd.qgemm(x_dev(x), pw)
    torch.cuda.synchronize()
    compare_y(bf16_bits(y), oracle.qgemm_exact(x, qw), f"{fmt} M={M} N={N} K={K}")


@pytest.mark.parametrize("N,K,M,R,TC,TS", [(28680, 2048, 300, 64, 4104, 2), (36872, 8192, 700, 128, 4104, 3),
                                          (24584, 2048, 1024, 128, 8, 4), (28672, 8192, 777, 128, 2048, 4),
                                          (10240, 8192, 1024, 64, 2048, 2)])
def test_qgemm_tiled_tail_split(N, K, M, R, TC, TS):
    """W4A16 on the tiled kernel with a tail split: the last TC columns of y
    run as TS K splits after the other column blocks (filling the launch's
    last round) and a second launch sums their partials.  Ragged N (the tail
    ending inside a 16-row block, or a tail of 8 columns), ragged M, 64- and
    128-row tiles, 2 to 4 splits; the oracle checks sampled columns on both
    sides of the tail's edge and the last ones, over every row."""
    assert wqd.kernel_path("w4a16", M, N, K)[0] == "gemm"
    assert wqd.gemm_tile("w4a16", M, N, K, tail=True) == (R, 256, 1, TC, TS)
    W = I.w_host(6500 + N + K, N, K)
    rng = np.random.default_rng(N + K + M)
    edge = N - TC
    fixed = [0, 15, 255, edge - 9, edge - 1, edge, edge + 7, edge + 8, N - 17, N - 9, N - 1]
    cols = np.unique(np.concatenate([rng.choice(N, 48, replace=False), [c for c in fixed if 0 <= c < N]]))
    qw = oracle.quantize("w4a16", W[cols])
    pw = wqd.pack_weights("w4a16", to_dev(W))
    print(f"qgemm tail M={M} N={N} K={K} tail {TC} x {TS}", flush=True)
    x = I.x_bf16_bits(47 * M + K, M, K)
    y = wqd.qgemm(x_dev(x), pw)
    torch.cuda.synchronize()
    compare_y(bf16_bits(y)[:, cols], oracle.qgemm_exact(x, qw), f"w4a16 tail M={M} N={N} K={K}")


@pytest.mark.parametrize("fmt,N,K,M,S,R,C", [
    ("bf16", 8208, 8224, 513, 2, 256, 224), ("bf16", 16392, 2048, 513, 1, 256, 224),
    ("bf16", 28672, 1056, 300, 1, 256, 224), ("bf16", 12296, 4096, 777, 1, 256, 224),
    ("bf16", 11008, 4096, 777, 1, 256, 224), ("bf16", 13456, 2048, 1000, 1, 256, 224),
    ("bf16", 8192, 28704, 513, 5, 256, 256), ("bf16", 12288, 28672, 700, 5, 256, 256),
    ("fp8", 8208, 8256, 1000, 3, 256, 224), ("fp8", 28672, 1088, 1023, 1, 256, 224),
    ("fp8", 28680, 4096, 900, 1, 256, 256), ("fp8", 8200, 28672, 1024, 3, 256, 224),
    ("fp8", 20488, 8192, 1023, 2, 256, 224), ("fp8", 13456, 2048, 1000, 1, 256, 224),
    ("fp8", 28672, 8192, 1024, 1, 128, 448), ("fp8", 28664, 8192, 1000, 1, 128, 448),
    ("fp8", 29104, 4096, 777, 1, 128, 448), ("fp8", 57352, 2048, 777, 1, 128, 448)])
def test_qgemm_tiled_lds(fmt, N, K, M, S, R, C):
    """BF16 and FP8 on the tiled kernel that stages x and the weights in LDS
    (R x C tiles: 256 x 256, 256 x 224, for FP8 also 128 x 448): ragged N
    inside a 16-row block, last column blocks of one row block (of 16, 14 and
    28) and of 7, 9 or 27, ragged M (last row blocks of 1 to 255 rows), chunk
    counts leaving each remainder of the loop (BF16: 4 chunks of 32 k, FP8: 3
    of 64 k), and K splits of 2, 3 and 5.  The oracle checks a sample of output
    columns, the first and last ones and those on either side of the first
    column blocks' edges included, over every row."""
    assert wqd.kernel_path(fmt, M, N, K) == ("gemm_lds", 8)
    assert wqd.gemm_tile(fmt, M, N, K) == (R, C, S)
    ws = wqd.workspace_bytes(fmt, M, N, K)
    assert (ws // (M * N * 4) if ws else 1) == S
    W = I.w_host(6300 + N + K, N, K)
    rng = np.random.default_rng(N + K)
    edges = [0, 15, C - 1, C, 2 * C - 1, 2 * C, N - 17, N - 9, N - 1]
    cols = np.unique(np.concatenate([rng.choice(N, 48, replace=False), edges]))
    qw = oracle.quantize(fmt, W[cols])
    pw = wqd.pack_weights(fmt, to_dev(W))
    print(f"qgemm lds M={M} N={N} K={K} S={S}", flush=True)
    x = I.x_bf16_bits(43 * M + K, M, K)
    y = wqd.qgemm(x_dev(x), pw)
    torch.cuda.synchronize()
    compare_y(bf16_bits(y)[:, cols], oracle.qgemm_exact(x, qw), f"{fmt} lds M={M} N={N} K={K}")
    if fmt == "fp8":  # the row scales of the sampled columns, bit for bit
        _, sc, _ = wqd.unpack(pw)
        torch.cuda.synchronize()
        assert np.array_equal(sc.cpu().numpy()[cols].view(np.uint32), qw["scales"].view(np.uint32))


def mfma_wide_shapes(fmt):
    # (N, K) that the LDS matrix-core kernel takes above 64 rows (below 16
    # column blocks of 256): ragged N, ragged K tiles where the format allows
    # them, and a K split
    if fmt == "w4a16":
        return [(357, 896), (1000, 1152), (3840, 1024)]
    return [(357, 904), (1000, 1160), (3840, 512)]


@pytest.mark.parametrize("fmt", FMTS)
def test_qgemm_mfma_wide(fmt):
    """Wide batches on narrow matrices: 16 to 64 rows per block of the LDS kernel."""
    for N, K in mfma_wide_shapes(fmt):
        W = I.w_host(7000 + N + K, N, K)
        qw = oracle.quantize(fmt, W)
        pw = wqd.pack_weights(fmt, to_dev(W))
        for M in (65, 100, 200, 300):
            assert wqd.kernel_path(fmt, M, N, K)[0] == "mfma"
            print(f"qgemm {fmt} M={M} N={N} K={K} ws={wqd.workspace_bytes(fmt, M, N, K)}", flush=True)
            x = I.x_bf16_bits(37 * M + K, M, K)
            y = wqd.qgemm(x_dev(x), pw)
            torch.cuda.synchronize()
            compare_y(bf16_bits(y), oracle.qgemm_exact(x, qw), f"{fmt} M={M} N={N} K={K}")


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("rows", [1, 2, 8, 10, 16])
def test_one_hot_probes_exact(fmt, rows):
    """x = e_k gives y[:, n] = bf16(Wd[n, k]) exactly: ties the kernel's own dequant to the oracle.

    Wd is the float32 dequantised weight (exact for bf16 and W4A16; for FP8 the
    kernel applies the row scale in float32, so the single float32 product
    e4m3 * s_n is the value it rounds to bf16)."""
    N, K = 200, 512
    W = I.w_host(77, N, K)
    qw = oracle.quantize(fmt, W)
    Wd = oracle.dequant_f32(qw).astype(np.float64)
    pw = wqd.pack_weights(fmt, to_dev(W))
    ks = [0, 1, 7, 8, 63, 64, 127, 128, 300, 511]
    x = np.zeros((len(ks), K), np.uint16)
    for i, k in enumerate(ks):
        x[i, k] = 0x3F80  # 1.0
    for M0 in range(0, len(ks), rows):
        xb = x[M0:M0 + rows]
        y = bf16_bits(wqd.qgemm(x_dev(xb), pw))
        for i in range(xb.shape[0]):
            assert np.array_equal(y[i], oracle.bf16_to_bits(Wd[:, ks[M0 + i]])), (fmt, ks[M0 + i])


@pytest.mark.parametrize("fmt", FMTS)
def test_zero_weights_give_exact_zero(fmt):
    N, K = 130, 512
    pw = wqd.pack_weights(fmt, torch.zeros((N, K), dtype=torch.float32, device=dev()))
    for M in (1, 2, 4, 16, 40, 64, 100):
        y = wqd.qgemm(x_dev(I.x_bf16_bits(3 + M, M, K)), pw)
        torch.cuda.synchronize()
        assert (y.float() == 0).all(), M


@pytest.mark.parametrize("fmt", FMTS)
def test_deterministic_and_every_output_written(fmt):
    N, K = 1000, 2048
    W = I.w_host(9, N, K)
    pw = wqd.pack_weights(fmt, to_dev(W))
    for M in (1, 5, 8, 24, 40, 150):
        x = x_dev(I.x_bf16_bits(10 + M, M, K))
        y1 = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=dev())
        y2 = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=dev())
        wqd.qgemm(x, pw, y=y1)
        wqd.qgemm(x, pw, y=y2)
        torch.cuda.synchronize()
        assert torch.isfinite(y1.float()).all()
        assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))


def test_workspace_use():
    """No workspace for M <= 8; the split-K matrix-core path writes its partials
    into a caller workspace (any contents) and still matches the oracle."""
    fmt, N, K = "w4a16", 640, 4096
    for M in (1, 8, 3):
        assert wqd.workspace_bytes(fmt, M, N, K) == 0
    W = I.w_host(1, N, K)
    qw = oracle.quantize(fmt, W)
    pw = wqd.pack_weights(fmt, to_dev(W))
    x = I.x_bf16_bits(5, 3, K)
    y = wqd.qgemm(x_dev(x), pw, workspace=None)
    torch.cuda.synchronize()
    compare_y(bf16_bits(y), oracle.qgemm_exact(x, qw), "no workspace")
    M = 40
    need = wqd.workspace_bytes(fmt, M, N, K)
    assert need > 0
    ws = torch.full((need // 4,), float("nan"), dtype=torch.float32, device=dev())
    x = I.x_bf16_bits(6, M, K)
    y = wqd.qgemm(x_dev(x), pw, workspace=ws)
    y2 = wqd.qgemm(x_dev(x), pw, workspace=ws)
    torch.cuda.synchronize()
    compare_y(bf16_bits(y), oracle.qgemm_exact(x, qw), "split-K workspace")
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))
