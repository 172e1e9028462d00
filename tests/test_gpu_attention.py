"""GPU parity of decode attention (wqd_decode_attention) against the oracle,
and of the KV cache writers (wqd_kv_pack / wqd_kv_append / wqd_kv_unpack).

Cases: grouped-query groups of 1, 4, 8 and 16 query heads per KV head;
lengths from 0 to Lmax in one batch (ragged last steps, empty sequences,
splits past a sequence's end); cache slots past each length filled with NaN
and infinities (never used); the 70B layer at the pages' batch-32 snapshot
(64 query heads, 8 KV heads of 128, 2048 positions) on sampled heads;
determinism; the cache layout round trip, bit for bit, and a decode step's
append.  Tolerance as for the linear layer (tests/parity.py)."""
import math

import numpy as np
import pytest
import torch

import oracle
import weight_only_quantized_decode_amd as wqd
from tests.parity import bf16_bits, compare_y

pytestmark = pytest.mark.gpu

DEV = "cuda"


def make(seed, B, Hq, Hkv, Lmax, lens, poison=True):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn((B, Hq, 128), generator=g).to(torch.bfloat16)
    k = torch.randn((B, Hkv, Lmax, 128), generator=g).to(torch.bfloat16)
    v = torch.randn((B, Hkv, Lmax, 128), generator=g).to(torch.bfloat16)
    if poison:  # stale slots past each length: NaN keys, infinite values
        for b, n in enumerate(lens):
            k[b, :, n:] = float("nan")
            v[b, :, n:] = float("inf")
    return q, k, v


def packed(k, v):
    B, Hkv, Lmax, _ = k.shape
    cache = wqd.alloc_kv_cache(B, Hkv, Lmax, device=DEV)
    return wqd.kv_pack(k.to(DEV), v.to(DEV), cache)


def run(q, k, v, lens, scale):
    lens_d = torch.tensor(lens, dtype=torch.int32, device=DEV)
    out = wqd.decode_attention(q.to(DEV), packed(k, v), lens_d, scale)
    torch.cuda.synchronize()
    return out


def bits(t):
    return t.view(torch.int16).numpy().view(np.uint16)


def check(q, k, v, lens, scale, what, heads=None):
    out = run(q, k, v, lens, scale)
    o64 = oracle.decode_attention_exact(bits(q), bits(k), bits(v), np.array(lens), scale)
    ob = bf16_bits(out)
    B, Hq, D = o64.shape
    if heads is not None:
        ob, o64 = ob.reshape(B * Hq, D)[heads], o64.reshape(B * Hq, D)[heads]
    st = compare_y(ob.reshape(-1, D), o64.reshape(-1, D), what)
    print(f"{what}: rel L2 {st['rel_l2']:.2e} max {st['max_rel']:.2e}", flush=True)
    return out


@pytest.mark.parametrize("Hq,Hkv", [(8, 8), (8, 2), (64, 8), (32, 2)])
def test_groups_and_ragged_lengths(Hq, Hkv):
    Lmax = 1024
    lens = [1, 31, 32, 33, 1024, 517, 0, 1000]
    q, k, v = make(Hq + Hkv, len(lens), Hq, Hkv, Lmax, lens)
    out = check(q, k, v, lens, 1 / math.sqrt(128), f"attn Hq={Hq} Hkv={Hkv}")
    assert not torch.any(out[6].view(torch.int16))  # the empty sequence gives zeros


def test_large_scores():
    # scale 1: scores of order 10, a sharply peaked softmax
    lens = [300, 2048]
    q, k, v = make(5, 2, 16, 2, 2048, lens)
    check(q, k, v, lens, 1.0, "attn scale 1")


def test_70b_layer_batch32_sampled():
    B, Hq, Hkv, L = 32, 64, 8, 2048
    lens = [L] * B
    q, k, v = make(7, B, Hq, Hkv, L, lens, poison=False)
    rng = np.random.default_rng(8)
    heads = np.sort(rng.choice(B * Hq, 96, replace=False))
    print(f"splits: workspace {wqd.attn_workspace_bytes(B, Hq, Hkv, L)} bytes", flush=True)
    check(q, k, v, lens, 1 / math.sqrt(128), "attn 70B batch 32", heads=heads)


def test_deterministic_and_shape_errors():
    lens = [700, 2048, 5]
    q, k, v = make(9, 3, 64, 8, 2048, lens)
    a = run(q, k, v, lens, 0.088)
    b = run(q, k, v, lens, 0.088)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    with pytest.raises(wqd.WqdError) as e:
        wqd.attn_workspace_bytes(1, 64, 8, 1000)  # Lmax % 32
    assert e.value.status == 2
    with pytest.raises(wqd.WqdError) as e:
        wqd.attn_workspace_bytes(1, 64, 2, 1024)  # 32 query heads per KV head
    assert e.value.status == 2


def test_cache_layout_round_trip_and_append():
    B, Hkv, Lmax = 3, 8, 256
    g = torch.Generator().manual_seed(11)
    k = torch.randn((B, Hkv, Lmax, 128), generator=g).to(torch.bfloat16)
    v = torch.randn((B, Hkv, Lmax, 128), generator=g).to(torch.bfloat16)
    cache = packed(k, v)
    k2, v2 = wqd.kv_unpack(cache)
    torch.cuda.synchronize()
    assert torch.equal(k2.cpu().view(torch.int16), k.view(torch.int16))
    assert torch.equal(v2.cpu().view(torch.int16), v.view(torch.int16))
    # a decode step: append one position per sequence, then attend over it
    kn = torch.randn((B, Hkv, 128), generator=g).to(torch.bfloat16)
    vn = torch.randn((B, Hkv, 128), generator=g).to(torch.bfloat16)
    pos = [17, 255, 300]  # the last is outside the cache: nothing written
    wqd.kv_append(kn.to(DEV), vn.to(DEV), torch.tensor(pos, dtype=torch.int32, device=DEV), cache)
    k3, v3 = wqd.kv_unpack(cache)
    torch.cuda.synchronize()
    k_ref, v_ref = k.clone(), v.clone()
    for b, t in enumerate(pos[:2]):
        k_ref[b, :, t], v_ref[b, :, t] = kn[b], vn[b]
    assert torch.equal(k3.cpu().view(torch.int16), k_ref.view(torch.int16))
    assert torch.equal(v3.cpu().view(torch.int16), v_ref.view(torch.int16))
    q = torch.randn((B, 64, 128), generator=g).to(torch.bfloat16)
    lens = [18, 256, 200]
    out = wqd.decode_attention(q.to(DEV), cache, torch.tensor(lens, dtype=torch.int32, device=DEV), 0.09)
    torch.cuda.synchronize()
    o64 = oracle.decode_attention_exact(bits(q), bits(k_ref), bits(v_ref), np.array(lens), 0.09)
    compare_y(bf16_bits(out).reshape(-1, 128), o64.reshape(-1, 128), "attention after append")
