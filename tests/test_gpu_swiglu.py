"""GPU parity of the SwiGLU path (wqd_pack_gate_up / wqd_qgemm_swiglu) against
the oracle's swiglu_exact: h = silu(x . gate^T) * (x . up^T).

Cases: every kernel family the planner picks for a 2F x K matrix (broadcast,
streaming matrix-core, skinny with and without a K split, staged, tiled with a
K split, LDS matrix-core with and without), all three formats; the 70B gate/up
pair (F = 28672, K = 8192) at decode and verify widths on sampled output
columns; the interleaved packing's dequantised rows, bit for bit."""
import numpy as np
import pytest
import torch

import oracle
import weight_only_quantized_decode_amd as wqd
import wqd_inputs as I
from tests.parity import bf16_bits, compare_y

pytestmark = pytest.mark.gpu

DEV = "cuda"


def src_row(n, F):
    b, r = n // 16, n % 16
    return 8 * b + r if r < 8 else F + 8 * b + r - 8


def run(fmt, M, F, K, seed, cols=None, gate_gain=8.0):
    W = I.w_device(seed, 2 * F, K, device=DEV)
    W[:F] *= gate_gain  # gate values of order 1, where silu bends
    path = wqd.kernel_path(fmt, M, 2 * F, K)
    print(f"swiglu {fmt} M={M} F={F} K={K} path={path} workspace={wqd.workspace_bytes(fmt, M, 2 * F, K)}",
          flush=True)
    pw = wqd.pack_gate_up(fmt, W)
    cols = np.arange(F) if cols is None else cols
    idx = torch.from_numpy(np.concatenate([cols, F + cols])).to(DEV)
    Wh = W[idx].cpu().numpy()
    qg, qu = oracle.quantize(fmt, Wh[: len(cols)]), oracle.quantize(fmt, Wh[len(cols):])
    # the interleaved packing: packed row n is source row src_row(n), dequantised bit for bit
    Wd = wqd.dequant(pw)
    rows = np.array(sorted({n for c in cols[:8] for n in (16 * (c // 8) + c % 8, 16 * (c // 8) + 8 + c % 8)}))
    got = Wd[torch.from_numpy(rows).to(DEV)].cpu().numpy()
    want = oracle.dequant_f32(oracle.quantize(fmt, W[torch.from_numpy(np.array([src_row(n, F) for n in rows])).to(
        DEV)].cpu().numpy()))
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    del W, Wd
    x = I.x_bf16_bits(I.x_seed(seed, M, K), M, K, outliers=K == 8192)
    h = wqd.qgemm_swiglu(torch.from_numpy(x.view(np.int16)).to(DEV).view(torch.bfloat16), pw)
    torch.cuda.synchronize()
    assert tuple(h.shape) == (M, F)
    st = compare_y(bf16_bits(h)[:, cols], oracle.swiglu_exact(x, qg, qu), f"swiglu {fmt} M={M} F={F} K={K}")
    print(f"  rel L2 {st['rel_l2']:.2e} max {st['max_rel']:.2e}", flush=True)
    return path


CASES = [("bf16", 1, 200, 512), ("bf16", 8, 200, 512), ("bf16", 9, 200, 512), ("bf16", 24, 200, 1024),
         ("bf16", 1, 200, 28672), ("bf16", 65, 2048, 512), ("bf16", 100, 4096, 512), ("bf16", 65, 200, 512),
         ("bf16", 65, 200, 1024),
         ("fp8", 1, 200, 512), ("fp8", 3, 200, 512), ("fp8", 8, 200, 512), ("fp8", 24, 200, 8192),
         ("fp8", 1, 200, 65536), ("fp8", 65, 2048, 512), ("fp8", 65, 200, 1024),
         ("w4a16", 1, 200, 512), ("w4a16", 2, 200, 512), ("w4a16", 9, 200, 512), ("w4a16", 24, 200, 8192),
         ("w4a16", 1, 200, 131072), ("w4a16", 65, 2048, 512), ("w4a16", 65, 200, 512), ("w4a16", 65, 200, 1024)]


@pytest.mark.parametrize("fmt,M,F,K", CASES)
def test_every_kernel_family(fmt, M, F, K):
    run(fmt, M, F, K, 100 + M + F % 97 + K % 89)


@pytest.mark.parametrize("fmt,Ms", [("w4a16", [1, 4, 8, 16, 32, 128, 512, 1024]), ("fp8", [1, 8, 32, 512, 1024]),
                                    ("bf16", [1, 4, 192, 512])])
def test_70b_gate_up(fmt, Ms):
    F, K = 28672, 8192
    rng = np.random.default_rng(5)
    cols = np.array(sorted(set(rng.choice(F, 40, replace=False).tolist()) | {0, 7, 8, F - 1}))
    for M in Ms:
        run(fmt, M, F, K, 700 + M, cols=cols)


def test_shape_errors():
    W = torch.zeros((2 * 12, 256), dtype=torch.float32, device=DEV)  # F = 12: not a multiple of 8
    with pytest.raises(wqd.WqdError) as e:
        wqd.pack_gate_up("w4a16", W)
    assert e.value.status == 2
