"""Decode attention over a KV cache with grouped-query heads.

Test infrastructure only (see ``oracle/__init__.py``).

What it computes ("Making each token cheaper", section "Why kernels matter
most for long prefill": a decode step has one query per sequence, so its
score row is as long as the context, and decode attention is dominated by
reading the KV cache; "LLM 推理是怎么变快的", section 2.3: with grouped-query
attention several query heads share one KV head, e.g. 32 query heads on 8 KV
heads; section 1 on the KV cache: every earlier position's key and value are
kept and read again at each step):

    for each sequence b and query head h (KV head g = h // (Hq / Hkv)),
    over the first len[b] positions t of the cache:
        s_t = scale * (q[b, h] . K[b, g, t])
        p_t = exp(s_t - max_t s_t) / sum_t exp(s_t - max_t s_t)
        o[b, h] = sum_t p_t V[b, g, t]

in float64 from the bf16 inputs, rounded once to bfloat16.  Readings where the
pages leave it open: the softmax scale is an input (1 / sqrt(head_dim) in the
usual model); a sequence of length 0 gives a zero output row.

An FP8 cache ("LLM 推理是怎么变快的", section 4, C: keys and values stored in
FP8 halve the cache's bytes; "Making each token cheaper", the hands-on lab,
exercise 5: the step bound with a 1-byte KV cache) holds E4M3FN codes of K and
V.  The pages leave the scales open (the exercise ignores them); read here as
one float32 scale per tensor for K and one for V, given by the caller:
code = nearest E4M3 of x / scale (float32 division, ties to even, saturating
at 448, as the FP8 weight rows are quantised), value = e4m3(code) * scale.

The split-and-merge of Flash-Decoding is the kernel's business: softmax over
the whole row is the definition, and merging per-chunk maxima, sums and
partial outputs reaches it exactly in real arithmetic.
"""
from __future__ import annotations

import numpy as np

from .formats import bf16_bits_to_f64, bf16_to_bits, e4m3_decode, e4m3_encode


def decode_attention_exact(q_bits, k_bits, v_bits, lengths, scale: float) -> np.ndarray:
    """o64[B, Hq, D] from q [B, Hq, D], K and V [B, Hkv, L, D] (bf16 bit
    patterns, position-major: row t of head g is K[b, g, t, :]), lengths [B]."""
    q = bf16_bits_to_f64(np.asarray(q_bits, np.uint16))
    K = bf16_bits_to_f64(np.asarray(k_bits, np.uint16))
    V = bf16_bits_to_f64(np.asarray(v_bits, np.uint16))
    return _attention_f64(q, K, V, lengths, scale)


def quantize_kv_fp8(x_bits, scale) -> np.ndarray:
    """E4M3 codes (uint8, same shape) of bf16 keys or values for one per-tensor
    scale: the nearest E4M3FN value of x / scale in float32, ties to even,
    saturating at 448.  The scale must be finite and positive."""
    s = np.float32(scale)
    if not (np.isfinite(s) and s > 0):
        raise ValueError("the KV scale must be finite and positive")
    x = bf16_bits_to_f64(np.asarray(x_bits, np.uint16)).astype(np.float32)
    return e4m3_encode((x / s).astype(np.float32))


def decode_attention_fp8kv_exact(q_bits, k_codes, v_codes, k_scale, v_scale, lengths, scale: float) -> np.ndarray:
    """o64[B, Hq, D] over an FP8 cache: K = e4m3(k_codes) * k_scale and
    V = e4m3(v_codes) * v_scale (exact in float64; codes [B, Hkv, L, D],
    position-major), then the softmax of decode_attention_exact."""
    q = bf16_bits_to_f64(np.asarray(q_bits, np.uint16))
    K = e4m3_decode(np.asarray(k_codes, np.uint8)) * float(np.float32(k_scale))
    V = e4m3_decode(np.asarray(v_codes, np.uint8)) * float(np.float32(v_scale))
    return _attention_f64(q, K, V, lengths, scale)


def decode_attention_fp8kv_ref(q_bits, k_codes, v_codes, k_scale, v_scale, lengths, scale: float) -> dict:
    o64 = decode_attention_fp8kv_exact(q_bits, k_codes, v_codes, k_scale, v_scale, lengths, scale)
    return {"o64": o64, "o_bits": bf16_to_bits(o64)}


def _attention_f64(q, K, V, lengths, scale: float) -> np.ndarray:
    """The definition above on float64 arrays q [B, Hq, D], K, V [B, Hkv, L, D]."""
    B, Hq, D = q.shape
    _, Hkv, L, Dk = K.shape
    if Dk != D or V.shape != K.shape or Hq % Hkv:
        raise ValueError("shape mismatch")
    group = Hq // Hkv
    o = np.zeros((B, Hq, D))
    for b in range(B):
        n = int(lengths[b])
        if n < 0 or n > L:
            raise ValueError("length out of range")
        if n == 0:
            continue
        for h in range(Hq):
            g = h // group
            s = (K[b, g, :n] @ q[b, h]) * float(scale)
            e = np.exp(s - s.max())
            o[b, h] = (e / e.sum()) @ V[b, g, :n]
    return o


def decode_attention_ref(q_bits, k_bits, v_bits, lengths, scale: float) -> dict:
    o64 = decode_attention_exact(q_bits, k_bits, v_bits, lengths, scale)
    return {"o64": o64, "o_bits": bf16_to_bits(o64)}
