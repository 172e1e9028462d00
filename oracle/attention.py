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

The split-and-merge of Flash-Decoding is the kernel's business: softmax over
the whole row is the definition, and merging per-chunk maxima, sums and
partial outputs reaches it exactly in real arithmetic.
"""
from __future__ import annotations

import numpy as np

from .formats import bf16_bits_to_f64, bf16_to_bits


def decode_attention_exact(q_bits, k_bits, v_bits, lengths, scale: float) -> np.ndarray:
    """o64[B, Hq, D] from q [B, Hq, D], K and V [B, Hkv, L, D] (bf16 bit
    patterns, position-major: row t of head g is K[b, g, t, :]), lengths [B]."""
    q = bf16_bits_to_f64(np.asarray(q_bits, np.uint16))
    K = bf16_bits_to_f64(np.asarray(k_bits, np.uint16))
    V = bf16_bits_to_f64(np.asarray(v_bits, np.uint16))
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
