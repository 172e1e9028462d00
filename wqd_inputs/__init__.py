"""Seeded synthetic inputs for the weight-only quantized decode linear layer.

This module is shared by the CPU oracle, the tests and the benchmark.  It holds
no arithmetic of the method itself (no quantisation, no dequantisation, no
matmul): it only draws random numbers and stores them in the types the layer
consumes (activations as bfloat16, weights as float32, probabilities as float32).

Recipe (all draws seeded, nothing read from disk):

* activations ``x[M, K]``: float32 from N(0, 1); for inputs whose K equals the
  8192-wide hidden size of the 70B-class shapes, six seeded hidden channels are
  multiplied by 20 (emergent outlier features reach about 20x the typical
  magnitude on a handful of hidden dimensions: "Making each token cheaper",
  section on why outliers defeat plain INT8); then rounded to bfloat16
  (round-to-nearest-even, done by torch's dtype conversion).
* weights ``W[N, K]``: float32 from N(0, sigma=0.02).
* speculative accept / reject inputs: target rows softmax(N(0, 2.5) logits) over
  V tokens, draft rows softmax of the same logits plus N(0, 1) noise, draft
  tokens drawn from the draft rows, uniforms as multiples of 2^-24 in [0, 1).

Host draws use numpy's PCG64; device draws use torch's CUDA generator.  The two
streams differ for the same seed, so a test always takes one of them and moves
the data to the other side when both need it.
"""
from __future__ import annotations

import numpy as np

HIDDEN = 8192
OUTLIER_SEED = 7
N_OUTLIERS = 6
OUTLIER_SCALE = 20.0
W_SIGMA = 0.02

# 70B-class decode layer (hidden 8192, GQA 64 q / 8 kv heads of 128, FFN 28672)
# and the Llama-2-7B layer, as (name, N, K) with y[M, N] = x[M, K] W[N, K]^T.
LAYER_70B = (
    ("q", 8192, 8192),
    ("k", 1024, 8192),
    ("v", 1024, 8192),
    ("o", 8192, 8192),
    ("gate", 28672, 8192),
    ("up", 28672, 8192),
    ("down", 8192, 28672),
)
LAYER_7B = (
    ("q", 4096, 4096),
    ("k", 4096, 4096),
    ("v", 4096, 4096),
    ("o", 4096, 4096),
    ("gate", 11008, 4096),
    ("up", 11008, 4096),
    ("down", 4096, 11008),
)


def outlier_channels(K: int) -> np.ndarray:
    """The six seeded hidden channels that carry 20x outliers (empty if K != 8192)."""
    if K != HIDDEN:
        return np.zeros(0, dtype=np.int64)
    rng = np.random.Generator(np.random.PCG64(OUTLIER_SEED))
    return np.sort(rng.choice(HIDDEN, size=N_OUTLIERS, replace=False)).astype(np.int64)


def x_f32(seed: int, M: int, K: int, outliers: bool = False) -> np.ndarray:
    """Activations before the bfloat16 cast, float32 [M, K]."""
    rng = np.random.Generator(np.random.PCG64(seed))
    x = rng.standard_normal((M, K), dtype=np.float32)
    if outliers:
        idx = outlier_channels(K)
        x[:, idx] *= np.float32(OUTLIER_SCALE)
    return x


def x_bf16(seed: int, M: int, K: int, outliers: bool = False):
    """Activations as a torch bfloat16 CPU tensor [M, K]."""
    import torch

    return torch.from_numpy(x_f32(seed, M, K, outliers)).to(torch.bfloat16)


def x_bf16_bits(seed: int, M: int, K: int, outliers: bool = False) -> np.ndarray:
    """Activations as raw bfloat16 bit patterns, uint16 [M, K]."""
    import torch

    return x_bf16(seed, M, K, outliers).view(torch.int16).numpy().view(np.uint16).copy()


def bf16_tensor_to_bits(t) -> np.ndarray:
    """Raw bit patterns of a bfloat16 torch tensor (any device) as uint16 numpy."""
    import torch

    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16).copy()


def w_host(seed: int, N: int, K: int, sigma: float = W_SIGMA) -> np.ndarray:
    """Weights float32 [N, K] ~ N(0, sigma), drawn on the host."""
    rng = np.random.Generator(np.random.PCG64(seed))
    w = rng.standard_normal((N, K), dtype=np.float32)
    w *= np.float32(sigma)
    return w


def w_device(seed: int, N: int, K: int, device="cuda", sigma: float = W_SIGMA):
    """Weights float32 [N, K] ~ N(0, sigma), drawn on the device (large stacks)."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(seed)
    w = torch.randn((N, K), generator=g, device=device, dtype=torch.float32)
    w.mul_(sigma)
    return w


def stack_seed(cfg: int, layer: int, matrix: int) -> int:
    """Seed of one weight matrix of a layer stack (matrix index q=0 .. down=6)."""
    return 1000 * cfg + 10 * layer + matrix


def x_seed(cfg: int, M: int, K: int) -> int:
    """Seed of the activation rows fed to every matrix with input width K."""
    return 1000 * cfg + M + 7919 * K


def uniform_f32(rng, shape) -> np.ndarray:
    """Uniform float32 numbers in [0, 1): multiples of 2^-24, so none rounds up to 1."""
    return (rng.integers(0, 1 << 24, size=shape) / float(1 << 24)).astype(np.float32)


def spec_inputs(seed: int, B: int, k: int, V: int, noise: float = 1.0, temp: float = 2.5):
    """Inputs of the speculative accept / reject step for B sequences of k drafts.

    Target rows: softmax of N(0, temp) logits over V tokens (float32), k + 1 per
    sequence.  Draft rows: softmax of the same logits plus N(0, noise) (a cheap
    model close to the target), k per sequence.  Draft tokens: drawn from the
    draft rows.  Uniforms: u_accept [B, k] and v [B] in [0, 1).
    """
    rng = np.random.default_rng(seed)
    logits = rng.normal(0.0, temp, size=(B, k + 1, V))

    def softmax(z):
        e = np.exp(z - z.max(axis=-1, keepdims=True))
        return (e / e.sum(axis=-1, keepdims=True)).astype(np.float32)

    target = softmax(logits)
    draft = softmax(logits[:, :k] + rng.normal(0.0, noise, size=(B, k, V)))
    tokens = np.zeros((B, k), dtype=np.int32)
    for b in range(B):
        for i in range(k):
            p = draft[b, i].astype(np.float64)
            tokens[b, i] = rng.choice(V, p=p / p.sum())
    return target, draft, tokens, uniform_f32(rng, (B, k)), uniform_f32(rng, (B,))
