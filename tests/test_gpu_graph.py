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
