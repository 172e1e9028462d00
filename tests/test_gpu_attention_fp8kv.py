"""GPU parity of decode attention over an FP8-E4M3 KV cache
(wqd_decode_attention_fp8kv) against the oracle, and of the FP8 cache writers
(wqd_kv_pack_fp8 / wqd_kv_append_fp8 / wqd_kv_unpack_fp8).

The oracle quantises the bf16 keys and values itself
(oracle.attention.quantize_kv_fp8); the device's codes must equal them bit for
bit, and the attention output is compared with the oracle's attention on the
oracle's own codes.  Cases: grouped-query groups of 1, 4, 8 and 16 query heads
per KV head; lengths from 0 to Lmax in one batch (ragged 64-position steps,
empty sequences, contexts split over several workgroups); cache slots past
each length holding the E4M3 NaN code (never used); scales that saturate,
power-of-two scales and a sharply peaked softmax; the 70B layer at batch 32
over 2048 positions on sampled heads; determinism and argument errors.
Tolerance as for the linear layer (tests/parity.py)."""
import math

import numpy as np
import pytest
import torch

import oracle
import oracle.attention as A
import weight_only_quantized_decode_amd as wqd
from tests.parity import bf16_bits, compare_y

pytestmark = pytest.mark.gpu

DEV = "cuda"
NAN_CODE = 0x7F


def make(seed, B, Hq, Hkv, Lmax, spread=1.0):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn((B, Hq, 128), generator=g).to(torch.bfloat16)
    k = (torch.randn((B, Hkv, Lmax, 128), generator=g) * spread).to(torch.bfloat16)
    v = (torch.randn((B, Hkv, Lmax, 128), generator=g) * spread).to(torch.bfloat16)
    return q, k, v


def bits(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def pack_ragged(k, v, lens, ks, vs):
    """An FP8 cache whose slots past each length hold the NaN code: every
    byte starts as NaN, then each sequence packs only its first len[b]
    positions."""
    B, Hkv, Lmax, D = k.shape
    cache = wqd.alloc_kv_cache_fp8(B, Hkv, Lmax, ks, vs, device=DEV)
    cache.k.fill_(NAN_CODE)
    cache.v.fill_(NAN_CODE)
    n = Hkv * Lmax * D
    for b, L in enumerate(lens):
        if L == 0:
            continue
        sub = wqd.KVCacheFP8(1, Hkv, Lmax, cache.k[b * n:(b + 1) * n], cache.v[b * n:(b + 1) * n], ks, vs)
        wqd.kv_pack_fp8(k[b:b + 1, :, :L].contiguous().to(DEV), v[b:b + 1, :, :L].contiguous().to(DEV), sub)
    return cache


def oracle_out(q, k, v, lens, ks, vs, scale):
    kc = A.quantize_kv_fp8(bits(k), ks)
    vc = A.quantize_kv_fp8(bits(v), vs)
    return A.decode_attention_fp8kv_exact(bits(q), kc, vc, ks, vs, np.array(lens), scale)


def check(q, k, v, lens, ks, vs, scale, what, heads=None):
    cache = pack_ragged(k, v, lens, ks, vs)
    lens_d = torch.tensor(lens, dtype=torch.int32, device=DEV)
    out = wqd.decode_attention_fp8kv(q.to(DEV), cache, lens_d, scale)
    torch.cuda.synchronize()
    o64 = oracle_out(q, k, v, lens, ks, vs, scale)
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
    lens = [1, 31, 32, 33, 63, 64, 65, 1024, 517, 0, 1000]
    q, k, v = make(Hq + Hkv, len(lens), Hq, Hkv, Lmax)
    print(f"splits {wqd.attn_fp8kv_splits(len(lens), Hq, Hkv, Lmax)}", flush=True)
    out = check(q, k, v, lens, 0.0117, 0.0093, 1 / math.sqrt(128), f"fp8 kv attn Hq={Hq} Hkv={Hkv}")
    assert not torch.any(out[9].view(torch.int16))  # the empty sequence gives zeros


def test_many_splits_and_lmax_not_multiple_of_64():
    # one sequence, a long context: the context is split over many workgroups;
    # Lmax = 4000 is a multiple of 32, not of 64 (the last step reads past it)
    Lmax = 4000
    assert wqd.attn_fp8kv_splits(1, 16, 2, Lmax) > 1
    lens = [Lmax]
    q, k, v = make(21, 1, 16, 2, Lmax)
    check(q, k, v, lens, 0.02, 0.015, 1 / math.sqrt(128), "fp8 kv attn 4000 positions")
    lens = [3969]
    check(q, k, v, lens, 0.02, 0.015, 1 / math.sqrt(128), "fp8 kv attn 3969 of 4000")


@pytest.mark.parametrize("ks,vs", [(2.0 ** -6, 2.0 ** -5), (1e-3, 4e-3)])
def test_scales_pow2_and_saturating(ks, vs):
    # 1e-3 saturates every |k| > 0.448 at 448 codes: the oracle saturates too
    lens = [300, 2048]
    q, k, v = make(5, 2, 16, 2, 2048)
    check(q, k, v, lens, ks, vs, 1 / math.sqrt(128), f"fp8 kv attn scales {ks:g} {vs:g}")


def test_large_scores():
    lens = [300, 2048]
    q, k, v = make(6, 2, 16, 2, 2048)
    check(q, k, v, lens, 0.0117, 0.0117, 1.0, "fp8 kv attn scale 1")


def test_70b_layer_batch32_sampled():
    B, Hq, Hkv, L = 32, 64, 8, 2048
    lens = [L] * B
    q, k, v = make(7, B, Hq, Hkv, L)
    rng = np.random.default_rng(8)
    heads = np.sort(rng.choice(B * Hq, 96, replace=False))
    print(f"splits {wqd.attn_fp8kv_splits(B, Hq, Hkv, L)}", flush=True)
    check(q, k, v, lens, 0.0117, 0.0117, 1 / math.sqrt(128), "fp8 kv attn 70B batch 32", heads=heads)


def test_codes_layout_and_append():
    B, Hkv, Lmax = 3, 8, 256
    ks, vs = 0.0117, 0.0093
    g = torch.Generator().manual_seed(11)
    k = (torch.randn((B, Hkv, Lmax, 128), generator=g) * 2).to(torch.bfloat16)
    v = (torch.randn((B, Hkv, Lmax, 128), generator=g) * 2).to(torch.bfloat16)
    cache = wqd.alloc_kv_cache_fp8(B, Hkv, Lmax, ks, vs, device=DEV)
    wqd.kv_pack_fp8(k.to(DEV), v.to(DEV), cache)
    kc, vc = wqd.kv_unpack_fp8(cache)
    torch.cuda.synchronize()
    k_ref, v_ref = A.quantize_kv_fp8(bits(k), ks), A.quantize_kv_fp8(bits(v), vs)
    assert np.array_equal(kc.cpu().numpy(), k_ref)
    assert np.array_equal(vc.cpu().numpy(), v_ref)
    assert (np.abs(oracle.e4m3_decode(k_ref)) == 448).any()  # the case exercises saturation
    # a decode step: append one position per sequence, then attend over it
    kn = (torch.randn((B, Hkv, 128), generator=g) * 2).to(torch.bfloat16)
    vn = (torch.randn((B, Hkv, 128), generator=g) * 2).to(torch.bfloat16)
    pos = [17, 255, 300]  # the last is outside the cache: nothing written
    wqd.kv_append_fp8(kn.to(DEV), vn.to(DEV), torch.tensor(pos, dtype=torch.int32, device=DEV), cache)
    kc3, vc3 = wqd.kv_unpack_fp8(cache)
    torch.cuda.synchronize()
    k2, v2 = k.clone(), v.clone()
    for b, t in enumerate(pos[:2]):
        k2[b, :, t], v2[b, :, t] = kn[b], vn[b]
    assert np.array_equal(kc3.cpu().numpy(), A.quantize_kv_fp8(bits(k2), ks))
    assert np.array_equal(vc3.cpu().numpy(), A.quantize_kv_fp8(bits(v2), vs))
    q = torch.randn((B, 64, 128), generator=g).to(torch.bfloat16)
    lens = [18, 256, 200]
    out = wqd.decode_attention_fp8kv(q.to(DEV), cache, torch.tensor(lens, dtype=torch.int32, device=DEV), 0.09)
    torch.cuda.synchronize()
    o64 = oracle_out(q, k2, v2, lens, ks, vs, 0.09)
    compare_y(bf16_bits(out).reshape(-1, 128), o64.reshape(-1, 128), "fp8 kv attention after append")


def test_deterministic_and_argument_errors():
    lens = [700, 2048, 5]
    q, k, v = make(9, 3, 64, 8, 2048)
    cache = pack_ragged(k, v, lens, 0.0117, 0.0117)
    lens_d = torch.tensor(lens, dtype=torch.int32, device=DEV)
    a = wqd.decode_attention_fp8kv(q.to(DEV), cache, lens_d, 0.088)
    b = wqd.decode_attention_fp8kv(q.to(DEV), cache, lens_d, 0.088)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    for bad in (0.0, -1.0, float("nan"), float("inf")):
        c = wqd.KVCacheFP8(cache.B, cache.Hkv, cache.Lmax, cache.k, cache.v, bad, 0.01)
        with pytest.raises(wqd.WqdError) as e:
            wqd.decode_attention_fp8kv(q.to(DEV), c, lens_d, 0.088)
        assert e.value.status == 1
        with pytest.raises(wqd.WqdError) as e:
            wqd.kv_pack_fp8(k[:, :, :4].contiguous().to(DEV), v[:, :, :4].contiguous().to(DEV), c)
        assert e.value.status == 1
    with pytest.raises(wqd.WqdError) as e:
        wqd.attn_fp8kv_workspace_bytes(1, 64, 8, 1000)  # Lmax % 32
    assert e.value.status == 2
