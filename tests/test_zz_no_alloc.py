"""wqd_qgemm_noalloc (the entry point for callers that cannot allocate) against
wqd_qgemm: the same kernels, so the outputs must be bit-identical.

Two calls in a row on shapes that use the scratch array (the second smaller
than the first, so stale contents from the first are present), a repeated
shape with new activations, a shape that needs no scratch, and a shape whose
workspace exceeds the array (rejected before anything is enqueued)."""
import numpy as np
import pytest
import torch

import weight_only_quantized_decode_amd as wqd
import wqd_inputs as I

pytestmark = pytest.mark.gpu

DEV = "cuda"


def packed(fmt, N, K, seed):
    return wqd.pack_weights(fmt, I.w_device(seed, N, K, device=DEV))


def x_dev(M, K, seed):
    return I.x_bf16(seed, M, K, outliers=K == I.HIDDEN).to(DEV)


def both(x, pw):
    ref = wqd.qgemm(x, pw)
    y = torch.full((x.shape[0], pw.N), float("nan"), dtype=torch.bfloat16, device=DEV)
    wqd.qgemm_noalloc(x, pw, y)
    torch.cuda.synchronize()
    return ref, y


def check(fmt, M, N, K, seed, expect_scratch=True):
    need = wqd.workspace_bytes(fmt, M, N, K)
    print(f"noalloc {fmt} M={M} N={N} K={K} path={wqd.kernel_path(fmt, M, N, K)} scratch={need}", flush=True)
    assert (need > 0) == expect_scratch and need <= wqd.NOALLOC_SCRATCH_BYTES
    pw = packed(fmt, N, K, seed)
    ref, y = both(x_dev(M, K, seed + 1), pw)
    assert torch.equal(ref.view(torch.int16), y.view(torch.int16)), (fmt, M, N, K)
    return pw


def test_two_calls_second_smaller():
    # 60 MiB of scratch (W4A16 group x sums and a K split on the tiled
    # kernel), then 7 MiB (the skinny kernel's split partials) written over
    # the first call's contents
    check("w4a16", 512, 10240, 8192, 11)
    check("w4a16", 32, 8192, 28672, 13)


def test_every_format_and_a_repeat():
    for fmt, M, N, K, seed in (("fp8", 256, 8192, 28672, 21), ("bf16", 256, 10240, 8192, 23),
                               ("fp8", 16, 8192, 28672, 25), ("bf16", 32, 8192, 8192, 27)):
        check(fmt, M, N, K, seed)
    pw = check("w4a16", 128, 8192, 8192, 29)
    # the same shape again with new activations: nothing left from the last call shows
    ref, y = both(x_dev(128, 8192, 99), pw)
    assert torch.equal(ref.view(torch.int16), y.view(torch.int16))


def test_no_scratch_needed_and_too_large():
    check("w4a16", 1, 8192, 8192, 31, expect_scratch=False)
    check("w4a16", 16, 8192, 8192, 32, expect_scratch=False)
    need = wqd.workspace_bytes("bf16", 1024, 10240, 8192)
    assert need > wqd.NOALLOC_SCRATCH_BYTES
    pw = packed("bf16", 10240, 8192, 33)
    x = x_dev(1024, 8192, 34)
    y = torch.zeros((1024, 10240), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(wqd.WqdError) as e:
        wqd.qgemm_noalloc(x, pw, y)
    assert e.value.status == 4  # WQD_E_WORKSPACE
    torch.cuda.synchronize()
    assert not torch.any(y.view(torch.int16))  # nothing was enqueued
