"""The measurement kernels that bench.py compares the decode kernels with: the
HBM read stream (per-workgroup XOR checksums), the copy, and the matrix-core
ceiling (back-to-back multiplies from registers)."""
import numpy as np
import pytest
import torch

import weight_only_quantized_decode_amd as wqd

pytestmark = pytest.mark.gpu


def test_stream_read_checksums():
    nbytes = (3 << 20) + 16 * 37  # not a multiple of the workgroup ranges
    host = np.random.default_rng(5).integers(0, 1 << 32, nbytes // 4, dtype=np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).to("cuda")
    sink = wqd.stream_read(buf)
    torch.cuda.synchronize()
    got = sink.cpu().numpy().view(np.uint32)
    n16 = nbytes // 16
    blocks = wqd.lib().wqd_stream_sink_words(nbytes)
    per = -(-n16 // blocks)
    words = host.reshape(-1, 4)
    want = [np.bitwise_xor.reduce(words[b * per: min((b + 1) * per, n16)].ravel()) if b * per < n16 else 0
            for b in range(blocks)]
    assert got.tolist() == [int(w) for w in want]


@pytest.mark.parametrize("words", [(1 << 20) + 12, (16 << 20) + 12])
def test_stream_copy(words):
    # the larger size runs the 8-loads-in-flight loop and a ragged remainder in
    # every workgroup; nothing past the end is written
    src = torch.randint(-2**31, 2**31 - 1, (words,), dtype=torch.int32, device="cuda")
    dst = torch.full((words + 64,), 0x5A5A5A5A, dtype=torch.int32, device="cuda")
    wqd.stream_copy(dst, src)
    torch.cuda.synchronize()
    assert torch.equal(dst[:words], src)
    assert (dst[words:] == 0x5A5A5A5A).all()


def test_mfma_peak():
    sink = torch.full((wqd.mfma_peak_sink_words(),), float("nan"), dtype=torch.float32, device="cuda")
    wqd.mfma_peak(10, sink)  # warm-up
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    flops = wqd.mfma_peak(2000, sink)
    e1.record()
    torch.cuda.synchronize()
    tflops = flops / (e0.elapsed_time(e1) * 1e-3) / 1e12
    print(f"matrix-core ceiling {tflops:.0f} TFLOP/s", flush=True)
    assert torch.isfinite(sink).all() and (sink != 0).all()
    # dense bf16 peak 2500 TFLOP/s; the clock drops under this load
    assert 1000 < tflops < 2600
