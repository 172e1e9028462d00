"""GPU parity at the full sizes of the decode workloads, in the launch plans the
benchmark uses.  The weights are drawn on the device; the oracle quantises and
multiplies a sample of output channels (every format is row-local: a row's
codes depend only on that row), so it checks those outputs one by one.

Workloads (hidden 8192, GQA 8 KV heads x 128, FFN 28672 for the 70B-class
layer; Llama-2-7B for the BF16 stack):
  * W4A16-g128 GEMV 4096 x 4096, M = 1 (all 4096 outputs checked);
  * 7B BF16 layer shapes, M = 1;
  * 70B FP8-E4M3 layer shapes, M = 1, 8, 32;
  * 70B W4A16 layer shapes with 6 outlier hidden channels at 20x, M = 1, 4, 16, 32;
  * speculative-verify widths M = batch x (k + 1) on q / gate / down shapes in
    W4A16, BF16 and FP8.
"""
import numpy as np
import pytest
import torch

import oracle
import weight_only_quantized_decode_amd as wqd
import wqd_inputs as I
from tests.parity import bf16_bits, compare_y

pytestmark = pytest.mark.gpu

DEV = "cuda"
N_SAMPLE = 40


def sample_rows(N, seed):
    rng = np.random.default_rng(seed)
    rows = set(rng.choice(N, size=min(N, N_SAMPLE - 4), replace=False).tolist())
    rows |= {0, 15, N - 16, N - 1}  # first / last 16-row blocks
    return np.array(sorted(r for r in rows if 0 <= r < N))


WORST = {}


def x_bits_for(M, K, outliers):
    """Activation rows as bf16 bits; `outliers` = "long" puts the six 20x
    channels of the hidden width into a K = 28672 input as well."""
    if outliers == "long":
        import torch as _t

        x = I.x_f32(I.x_seed(0, M, K), M, K)
        x[:, I.outlier_channels(I.HIDDEN)] *= np.float32(I.OUTLIER_SCALE)
        return _t.from_numpy(x).to(_t.bfloat16).view(_t.int16).numpy().view(np.uint16).copy()
    return I.x_bf16_bits(I.x_seed(0, M, K), M, K, outliers=bool(outliers))


def run_case(fmt, N, K, Ms, seed, outliers, full=False):
    W = I.w_device(seed, N, K, device=DEV)
    pw = wqd.pack_weights(fmt, W)
    rows = np.arange(N) if full else sample_rows(N, seed)
    W_rows = W[torch.from_numpy(rows).to(DEV)].cpu().numpy()
    del W
    qw = oracle.quantize(fmt, W_rows)
    # dequantised weights of the sampled rows, bit for bit
    Wd = wqd.dequant(pw)
    Wd_rows = Wd[torch.from_numpy(rows).to(DEV)].cpu().numpy()
    del Wd
    assert np.array_equal(Wd_rows.view(np.uint32), oracle.dequant_f32(qw).view(np.uint32)), (fmt, N, K)
    for M in Ms:
        path = wqd.kernel_path(fmt, M, N, K)
        print(f"fullsize {fmt} N={N} K={K} M={M} path={path}", flush=True)
        x = x_bits_for(M, K, outliers)
        xd = torch.from_numpy(x.view(np.int16)).to(DEV).view(torch.bfloat16)
        y = wqd.qgemm(xd, pw)
        torch.cuda.synchronize()
        yb = bf16_bits(y)[:, rows]
        st = compare_y(yb, oracle.qgemm_exact(x, qw), f"{fmt} N={N} K={K} M={M}")
        print(f"  rel L2 {st['rel_l2']:.3e}  max {st['max_rel']:.3e}", flush=True)
        if st["rel_l2"] > WORST.get(fmt, (0.0,))[0]:
            WORST[fmt] = (st["rel_l2"], st["max_rel"], N, K, M, path)


def test_w4a16_gemv_4096_all_outputs():
    run_case("w4a16", 4096, 4096, [1], 101, outliers=False, full=True)


@pytest.mark.parametrize("N,K", [(4096, 4096), (11008, 4096), (4096, 11008)])
def test_llama7b_bf16_shapes(N, K):
    run_case("bf16", N, K, [1], 200 + N % 97, outliers=False)


@pytest.mark.parametrize("N,K", [(8192, 8192), (1024, 8192), (28672, 8192), (8192, 28672)])
def test_70b_fp8_shapes(N, K):
    run_case("fp8", N, K, [1, 8, 32], 300 + N % 97 + K % 89, outliers=False)


@pytest.mark.parametrize("N,K", [(8192, 8192), (1024, 8192), (28672, 8192), (8192, 28672)])
def test_70b_w4a16_shapes_with_outliers(N, K):
    run_case("w4a16", N, K, [1, 2, 4, 8, 16, 32], 400 + N % 97 + K % 89, outliers=True)


@pytest.mark.parametrize("fmt,Ms", [("w4a16", [1, 2, 4, 8, 16]), ("fp8", [1, 8, 32]), ("bf16", [1, 4])])
@pytest.mark.parametrize("N,K", [(10240, 8192), (57344, 8192)])
def test_70b_fused_qkv_and_gate_up(fmt, Ms, N, K):
    """The fused q/k/v (10240 rows: three row blocks per wavefront on the
    streaming matrix-core kernel, full-K shares) and gate/up (57344 rows)
    matrices the headline stack launches, at the widths each layout times."""
    run_case(fmt, N, K, Ms, 700 + N % 97 + len(fmt), outliers=fmt != "bf16")


def test_w4a16_long_k_with_outlier_channels():
    """W4A16 down projection (K = 28672) with six 20x channels in its input:
    the offset-128 products cancel a term ~128x the result over the longest K."""
    run_case("w4a16", 8192, 28672, [1, 8, 16, 64, 1024], 801, outliers="long")


@pytest.mark.parametrize("fmt", ["w4a16", "bf16", "fp8"])
@pytest.mark.parametrize("N,K", [(8192, 8192), (28672, 8192), (8192, 28672)])
def test_verify_widths(fmt, N, K):
    run_case(fmt, N, K, [6, 16, 48, 128, 192, 200, 384, 512, 1024], 500 + N % 97 + K % 89, outliers=True)


@pytest.mark.parametrize("fmt,N,K,M", [("bf16", 8192, 8192, 129), ("fp8", 8192, 28672, 200)])
def test_tall_tiles_below_256_rows(fmt, N, K, M):
    """BF16 / FP8 on 256-row tiles with padded rows and an 8-way K split."""
    assert wqd.kernel_path(fmt, M, N, K) == ("gemm", 8)
    run_case(fmt, N, K, [M], 600 + N % 97 + K % 89, outliers=False)


def test_zz_report_worst_margins():
    """Prints the largest error seen per format in this module (a record of the
    margin under the 1e-3 / 4e-3 bar)."""
    for fmt, (rel, mx, N, K, M, path) in sorted(WORST.items()):
        print(f"worst {fmt}: rel L2 {rel:.3e} max {mx:.3e} at N={N} K={K} M={M} {path}", flush=True)
