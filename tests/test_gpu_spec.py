"""GPU parity of the speculative-sampling accept / reject step (wqd_spec_accept).

The kernel and the oracle take every decision the same way (the float32
accept products, the draws in integer units of 2^-32), so the kept counts and
the tokens must agree exactly.  Cases: vocabularies from 3 tokens to 128256
(not a multiple of the 256 segments), 1 to 16 drafts, and the degenerate
cases (draft equal to target, a draft token the target never emits, an empty
residual, an out-of-range token, no drafts).
"""
import numpy as np
import pytest
import torch

import oracle
import weight_only_quantized_decode_amd as wqd
import wqd_inputs as I

pytestmark = pytest.mark.gpu


def run(target, draft, tokens, u, v):
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to("cuda")  # noqa: E731
    n, out = wqd.spec_accept(dev(target), dev(draft), dev(tokens), dev(u), dev(v))
    torch.cuda.synchronize()
    return n.cpu().numpy(), out.cpu().numpy()


def check(target, draft, tokens, u, v, what):
    print(f"spec {what} B={target.shape[0]} k={target.shape[1] - 1} V={target.shape[2]}", flush=True)
    n, out = run(target, draft, tokens, u, v)
    n_ref, out_ref = oracle.spec_accept(target, draft, tokens, u, v)
    assert np.array_equal(n, n_ref), (what, n, n_ref)
    assert np.array_equal(out, out_ref), (what, np.argwhere(out != out_ref)[:5])
    return n


@pytest.mark.parametrize("B,k,V", [(64, 1, 3), (64, 4, 1000), (32, 7, 32000), (8, 16, 4099), (8, 4, 128256),
                                   (1, 4, 128256), (1024, 2, 1000)])
def test_spec_accept_matches_oracle(B, k, V):
    n = check(*I.spec_inputs(900 + V + k, B, k, V), f"random V={V}")
    assert 0 < n.mean() < k or k == 1  # a mix of early rejections and kept drafts


def test_spec_accept_degenerate_cases():
    B, k, V = 6, 3, 700
    t, d, x, u, v = I.spec_inputs(77, B, k, V)
    d = d.copy(); t = t.copy(); x = x.copy()
    d[0] = t[0, :k]                          # draft equals target: every draft kept, bonus draw
    d[1, 0] = t[1, 0]; t[1, 1, x[1, 1]] = 0  # kept at 0, rejected at 1
    t[2, 0, x[2, 0]] = 0; d[2, 0] = t[2, 0]  # empty residual: draw from the target row
    x[3, 0] = V                              # out-of-range token: rejected
    x[4, 2] = -1
    n = check(t, d, x, u, v, "degenerate")
    assert n[0] == k and n[1] == 1 and n[2] == 0 and n[3] == 0 and n[4] <= 2
    # no drafts: the draw from target row 0 only
    t0, _, _, _, v0 = I.spec_inputs(78, 5, 1, 300)
    check(t0[:, :1], np.zeros((5, 0, 300), np.float32), np.zeros((5, 0), np.int32),
          np.zeros((5, 0), np.float32), v0, "k=0")


def test_spec_accept_uniform_range_ends_and_zero_rows():
    """u_draw at 1 (a (0, 1] generator), above 1, NaN and 0; an all-zero target
    row after every draft is kept (token -1); NaN and out-of-range weights."""
    B, k, V = 8, 2, 1500
    t, d, x, u, v = I.spec_inputs(79, B, k, V)
    t = t.copy(); d = d.copy(); v = v.copy()
    v[0], v[1], v[2], v[3] = 1.0, 1.25, np.nan, 0.0
    d[4] = t[4, :k]; t[4, k] = 0.0              # every draft kept, then an all-zero row: -1
    d[5] = t[5, :k]; t[5, k] = 0.0; v[5] = 1.0
    t[6, 0, 3] = np.nan; t[6, 0, 9] = 1.5       # malformed weights count as clamped
    d[6, 0, 5] = np.nan
    n, out = run(t, d, x, u, v)
    n_ref, out_ref = oracle.spec_accept(t, d, x, u, v)
    assert np.array_equal(n, n_ref) and np.array_equal(out, out_ref), (n, n_ref, out, out_ref)
    assert out[4, k] == -1 and out[5, k] == -1
    assert (out[:, :] >= -1).all() and (out < V).all()
