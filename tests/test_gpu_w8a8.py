"""GPU parity of the W8A8-FP8 path: wqd_act_quant_fp8 (activation codes and
the per-tensor scale, bit for bit against the oracle) and wqd_qgemm_w8a8
(the product within the tolerance of tests/parity.py against the oracle's
exact float64 product of the same codes).

Cases: small ragged shapes through every tile height (32, 64 and 128 rows)
with and without a K split; the 70B verify shapes (q, gate, down) at the
verify widths on sampled output rows; activations with 20x outlier channels;
an all-zero tensor; shape errors."""
import numpy as np
import pytest
import torch

import oracle
import oracle.w8a8 as W8
import weight_only_quantized_decode_amd as wqd
import wqd_inputs as I
from tests.parity import bf16_bits, compare_y

pytestmark = pytest.mark.gpu

DEV = "cuda"


def bits_to_dev(xb):
    return torch.from_numpy(xb.view(np.int16)).to(DEV).view(torch.bfloat16)


def check_act(xb):
    codes, scale = wqd.act_quant_fp8(bits_to_dev(xb))
    torch.cuda.synchronize()
    ref = W8.quantize_act(xb)
    assert scale.cpu().numpy()[0].view(np.uint32) == np.float32(ref["scale"]).view(np.uint32)
    got = codes.cpu().numpy()
    assert np.array_equal(got, ref["codes"]), np.argwhere(got != ref["codes"])[:5]
    return codes, scale, ref


@pytest.mark.parametrize("M,K,outl", [(1, 8192, True), (3, 4096, False), (64, 28672, False), (1024, 8192, True),
                                      (7, 1040, False)])
def test_act_quant_bitexact(M, K, outl):
    xb = I.x_bf16_bits(I.x_seed(9, M, K), M, K, outliers=outl)
    print(f"act_quant M={M} K={K}", flush=True)
    check_act(xb)


def test_act_quant_zero_and_tiny():
    check_act(np.zeros((4, 256), np.uint16))
    t = np.zeros((2, 512), np.uint16)
    t[1, 300] = 0x8001  # -smallest subnormal
    codes, scale, ref = check_act(t)
    assert ref["scale"] == np.float32(2.0 ** -126)


def test_act_quant_rounding_cases():
    """Scale 1 (the tensor holds 448): every finite E4M3 value, the midpoints
    between neighbours (ties to even), one bf16 step either side of each, the
    subnormal range and values that round to +-0 (the sign kept)."""
    import torch as _t

    fin = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    vals = np.sort(np.unique(oracle.e4m3_decode(fin)))
    mids = (vals[:-1] + vals[1:]) / 2
    b = _t.from_numpy(np.concatenate([vals, mids]).astype(np.float32)).to(_t.bfloat16)
    bits = b.view(_t.int16).numpy().view(np.uint16).astype(np.int32)
    mid_bits = bits[len(vals):]
    near = np.concatenate([mid_bits + 1, mid_bits - 1])
    near = near[(near & 0x7FFF) != 0]  # keep to values next to the midpoints
    tiny = np.array([0x0001, 0x8001, 0x3A00, 0xBA00, 0x3A80, 0xBA80, 0x8000, 0x3B00], np.int32)  # below 2^-9
    allb = np.concatenate([bits, near, tiny, [0x43E0]]).astype(np.uint16)  # 0x43E0 = 448
    n = (len(allb) + 15) // 16 * 16
    xb = np.zeros(n, np.uint16)
    xb[:len(allb)] = allb
    codes, scale, ref = check_act(xb.reshape(n // 16, 16))
    assert ref["scale"] == np.float32(1.0)


def run_product(M, N, K, seed, rows=None, outl=False):
    W = I.w_device(seed, N, K, device=DEV)
    pw = wqd.pack_weights("fp8", W)
    rows = np.arange(N) if rows is None else rows
    qw = oracle.quantize_fp8(W[torch.from_numpy(rows).to(DEV)].cpu().numpy())
    del W
    xb = I.x_bf16_bits(I.x_seed(seed, M, K), M, K, outliers=outl)
    codes, scale, xq = check_act(xb)
    print(f"w8a8 M={M} N={N} K={K} workspace={wqd.w8a8_workspace_bytes(M, N, K)}", flush=True)
    y = wqd.qgemm_w8a8(codes, scale, pw)
    torch.cuda.synchronize()
    st = compare_y(bf16_bits(y)[:, rows], W8.qgemm_w8a8_exact(xq, qw), f"w8a8 M={M} N={N} K={K}")
    print(f"  rel L2 {st['rel_l2']:.3e} max {st['max_rel']:.3e}", flush=True)


@pytest.mark.parametrize("M", [1, 5, 32, 33, 64, 65, 100, 128, 200])
def test_small_ragged(M):
    # N = 300 (a ragged last 16-row block and 256-column block), K = 1040
    # (8 full 128-k chunks and a 16-k remainder), split over K or not
    run_product(M, 300, 1040, 500 + M)


@pytest.mark.parametrize("M", [16, 128, 512, 1024])
@pytest.mark.parametrize("N,K", [(8192, 8192), (28672, 8192), (8192, 28672)])
def test_verify_shapes_sampled(M, N, K):
    rng = np.random.default_rng(N + K + M)
    rows = np.array(sorted(set(rng.choice(N, 36, replace=False).tolist()) | {0, 15, N - 16, N - 1}))
    run_product(M, N, K, 600 + M, rows=rows, outl=K == 8192)


@pytest.mark.parametrize("M,N,K,R,C,S", [(513, 43008, 2176, 128, 448, 1), (256, 16400, 4224, 128, 448, 3),
                                         (257, 8200, 28672, 128, 448, 7), (257, 28672, 2176, 256, 224, 1),
                                         (256, 13456, 8192, 256, 224, 4), (256, 8200, 28672, 256, 224, 6),
                                         (256, 57352, 2176, 256, 256, 1), (300, 8200, 2176, 256, 256, 3),
                                         (1000, 29104, 4096, 256, 256, 1)])
def test_lds_staged_ragged(M, N, K, R, C, S):
    """From 256 rows (K a whole number of 128-k chunks, tiles that fill the
    compute units' rounds) both operands are staged in LDS on 256 x 256,
    256 x 224 or 128 x 448 tiles: ragged N inside
    a 16-row block and last column blocks of 1 to 27 row blocks, ragged M (last
    row blocks of 1 to 127 rows), odd and even chunk counts per split (the
    two-stage loop's remainder) and K splits of 2 to 7.  Sampled columns
    include the first column blocks' edges."""
    assert wqd.w8a8_tile(M, N, K) == (R, C, S)
    rng = np.random.default_rng(N + K + M)
    edges = {0, 15, C - 1, C, 2 * C - 1, 2 * C, N - 17, N - 9, N - 1}
    rows = np.array(sorted(set(rng.choice(N, 40, replace=False).tolist()) | edges))
    run_product(M, N, K, 700 + M, rows=rows)


def test_deterministic():
    M, N, K = 256, 4096, 4096
    pw = wqd.pack_weights("fp8", I.w_device(77, N, K, device=DEV))
    x = bits_to_dev(I.x_bf16_bits(78, M, K))
    y1 = wqd.w8a8(x, pw)
    y2 = wqd.w8a8(x, pw)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))


def test_shape_errors():
    x = torch.zeros((2, 100), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(wqd.WqdError) as e:
        wqd.act_quant_fp8(x)
    assert e.value.status == 2  # WQD_E_SHAPE: K % 16 != 0
    pw = wqd.pack_weights("fp8", torch.zeros((32, 104), dtype=torch.float32, device=DEV))
    codes = torch.zeros((2, 104), dtype=torch.uint8, device=DEV)
    with pytest.raises(wqd.WqdError) as e:
        wqd.qgemm_w8a8(codes, torch.ones(1, device=DEV), pw)
    assert e.value.status == 2
