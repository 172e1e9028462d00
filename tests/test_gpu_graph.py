"""qgemm captured in a HIP graph (as the benchmark replays it) against eager calls.

One case per kernel family, including the K-split paths (workspace partials and
the second launch) and the W4A16 x-sum first kernel of the tiled path.  The
graph is replayed several times with new x written between replays from
outside the graph and y poisoned with NaNs, and every replay must give the
eager result bit for bit (every kernel is deterministic), which also ties the
graph to the oracle through the eager result.
"""
import numpy as np
import pytest
import torch

import oracle
import weight_only_quantized_decode_amd as wqd
import wqd_inputs as I
from tests.parity import bf16_bits, compare_y

pytestmark = pytest.mark.gpu

# (fmt, M, N, K, kernel family)
CASES = [
    ("w4a16", 1, 4104, 4096, "bcast"),
    ("w4a16", 4, 8192, 2048, "mc"),
    ("w4a16", 4, 10232, 1024, "mc"),         # three row blocks per wavefront, ragged N
    ("fp8", 16, 10240, 2048, "skinny"),      # K split: partials + second launch
    ("w4a16", 300, 4104, 4096, "gemm"),      # x sums, K split
    ("bf16", 200, 4000, 1160, "gemm"),
    ("bf16", 513, 8208, 8224, "gemm_lds"),   # weights staged in LDS too, K split, ragged M and N
    ("fp8", 1000, 8208, 8256, "gemm_lds"),   # the FP8 form: 3-way K split, ragged M and N
    ("w4a16", 100, 1000, 1152, "mfma"),
]


def x_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to("cuda").view(torch.bfloat16)


@pytest.mark.parametrize("fmt,M,N,K,family", CASES)
def test_graph_replay_matches_eager(fmt, M, N, K, family):
    assert wqd.kernel_path(fmt, M, N, K)[0] == family
    print(f"graph {fmt} {family} M={M} N={N} K={K} ws={wqd.workspace_bytes(fmt, M, N, K)}", flush=True)
    W = I.w_host(11000 + N + K, N, K)
    qw = oracle.quantize(fmt, W)
    pw = wqd.pack_weights(fmt, torch.from_numpy(W).to("cuda"))
    xs = [I.x_bf16_bits(500 + 7 * i + M, M, K) for i in range(3)]
    eager = []
    for xb in xs:
        y = wqd.qgemm(x_dev(xb), pw)
        torch.cuda.synchronize()
        eager.append(y.clone())
    compare_y(bf16_bits(eager[0]), oracle.qgemm_exact(xs[0], qw), f"eager {fmt} M={M} N={N} K={K}")

    x_buf = x_dev(xs[0])
    y_buf = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        wqd.qgemm(x_buf, pw, y=y_buf)  # the workspace is allocated here, outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        wqd.qgemm(x_buf, pw, y=y_buf)
    for i in (0, 1, 2, 1, 0):
        x_buf.copy_(x_dev(xs[i]))
        y_buf.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y_buf.view(torch.int16), eager[i].view(torch.int16)), (fmt, family, M, i)


def replay_check(run_eager, set_input, out_buf, capture, n_inputs=3):
    """Eager results for each input, then one captured graph replayed over the
    inputs in the order 0, 1, 2, 1, 0 with the output poisoned between
    replays; every replay must match its eager result bit for bit."""
    eager = []
    for i in range(n_inputs):
        set_input(i)
        run_eager()
        torch.cuda.synchronize()
        eager.append(out_buf.clone())
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        capture()  # workspaces are allocated here, outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        capture()
    for i in (0, 1, 2, 1, 0):
        set_input(i)
        out_buf.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_buf.view(torch.int16), eager[i].view(torch.int16)), i


@pytest.mark.parametrize("M,N,K", [(256, 8192, 4096), (48, 4096, 8192)])
def test_graph_w8a8(M, N, K):
    """Activation quantisation (absmax partials, codes) and the FP8 product,
    with a K split at 48 rows."""
    pw = wqd.pack_weights("fp8", I.w_device(41, N, K))
    xs = [x_dev(I.x_bf16_bits(60 + i, M, K)) for i in range(3)]
    x_buf = torch.empty_like(xs[0])
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    print(f"graph w8a8 M={M} N={N} K={K} ws={wqd.w8a8_workspace_bytes(M, N, K)}", flush=True)

    def run():
        wqd.w8a8(x_buf, pw, y=y)

    replay_check(run, lambda i: x_buf.copy_(xs[i]), y, run)


@pytest.mark.parametrize("B", [2, 32])
def test_graph_decode_attention(B):
    """B = 2 splits the context (partials and the merge launch); B = 32 does not."""
    Hq, Hkv, L = 64, 8, 2048
    cache = wqd.alloc_kv_cache(B, Hkv, L)
    g0 = torch.Generator(device="cuda").manual_seed(3)
    cache.k.normal_(generator=g0)
    cache.v.normal_(generator=g0)
    qs = [torch.randn((B, Hq, 128), generator=g0, device="cuda").to(torch.bfloat16) for _ in range(3)]
    q_buf = torch.empty_like(qs[0])
    lens = torch.tensor([(L * (b + 1)) // B for b in range(B)], dtype=torch.int32, device="cuda")
    out = torch.empty_like(q_buf)
    print(f"graph attention B={B} ws={wqd.attn_workspace_bytes(B, Hq, Hkv, L)}", flush=True)

    def run():
        wqd.decode_attention(q_buf, cache, lens, 0.088, out=out)

    replay_check(run, lambda i: q_buf.copy_(qs[i]), out, run)


@pytest.mark.parametrize("fmt,M,F,K", [("w4a16", 1, 28672, 8192), ("fp8", 24, 200, 8192), ("w4a16", 65, 2048, 512)])
def test_graph_swiglu(fmt, M, F, K):
    """SwiGLU epilogue on the broadcast kernel, on the skinny kernel's split-K
    sum, and on the tiled kernel's."""
    pw = wqd.pack_gate_up(fmt, I.w_device(43, 2 * F, K))
    xs = [x_dev(I.x_bf16_bits(70 + i, M, K)) for i in range(3)]
    x_buf = torch.empty_like(xs[0])
    h = torch.empty((M, F), dtype=torch.bfloat16, device="cuda")
    print(f"graph swiglu {fmt} M={M} F={F} K={K} path={wqd.kernel_path(fmt, M, 2 * F, K)}", flush=True)

    def run():
        wqd.qgemm_swiglu(x_buf, pw, h=h)

    replay_check(run, lambda i: x_buf.copy_(xs[i]), h, run)
