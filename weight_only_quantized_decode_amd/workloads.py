"""Decode workloads (layer stacks and single matrices) and their algorithmic byte counts.

Algorithmic bytes of one y[M, N] = x[M, K] . W[N, K]^T call: packed weights +
scales + zero points + x + y, each counted once:
  bf16   2 B/weight;
  fp8    1 B/weight + 4 B per output row (one 32-bit scale per row);
  w4a16  0.5 B/weight + (2 B scale + 0.5 B zero) per 128-weight group,
         i.e. 4 + 16/128 + 4/128 = 4.15625 bits/weight;
  x      2 B * M * K;   y  2 B * M * N.
"""
from __future__ import annotations

from dataclasses import dataclass

import wqd_inputs as I

WEIGHT_BITS = {"bf16": 16.0, "fp8": 8.0, "w4a16": 4.0}


def weight_bytes(fmt: str, N: int, K: int) -> dict:
    if fmt == "bf16":
        return {"w": 2 * N * K, "s": 0, "z": 0}
    if fmt == "fp8":
        return {"w": N * K, "s": 4 * N, "z": 0}
    if fmt == "w4a16":
        g = N * (K // 128)
        return {"w": N * K // 2, "s": 2 * g, "z": g // 2}
    raise ValueError(fmt)


def call_bytes(fmt: str, M: int, N: int, K: int) -> int:
    wb = weight_bytes(fmt, N, K)
    return wb["w"] + wb["s"] + wb["z"] + 2 * M * K + 2 * M * N


def call_bytes_w8a8(M: int, N: int, K: int) -> int:
    """The W8A8 product: FP8 weights and row scales, activation codes (1 B
    each) in, y (bf16) out."""
    wb = weight_bytes("fp8", N, K)
    return wb["w"] + wb["s"] + M * K + 2 * M * N


def act_quant_bytes(M: int, K: int) -> int:
    """The activation quantisation: x read twice (maximum, then codes), codes written."""
    return 2 * 2 * M * K + M * K


def call_flops(M: int, N: int, K: int) -> int:
    return 2 * M * N * K


@dataclass(frozen=True)
class Workload:
    name: str
    fmt: str
    M: int
    layers: int
    mats: tuple  # ((name, N, K), ...) per layer
    outliers: bool
    cfg: int
    act: str = "bf16"  # "fp8": W8A8, activations quantised per tensor before each product
    swiglu: bool = False  # gate_up writes silu(gate) * up (N / 2 columns), which down reads

    @property
    def launches(self) -> int:
        return self.layers * len(self.mats)

    def call_bytes(self, N: int, K: int, name: str = "") -> int:
        if self.act == "fp8":
            return call_bytes_w8a8(self.M, N, K)
        if self.swiglu and name == "gate_up":  # y holds N / 2 columns
            return call_bytes(self.fmt, self.M, N, K) - 2 * self.M * (N // 2)
        return call_bytes(self.fmt, self.M, N, K)

    def step_bytes(self) -> int:
        return self.layers * sum(self.call_bytes(N, K, name) for name, N, K in self.mats)

    def step_flops(self) -> int:
        return self.layers * sum(call_flops(self.M, N, K) for _, N, K in self.mats)

    def weight_stream_bytes(self) -> int:
        return self.layers * sum(sum(weight_bytes(self.fmt, N, K).values()) for _, N, K in self.mats)


def fuse_layer(mats) -> tuple:
    """q/k/v and gate/up concatenated along N (they share their input x).

    Row-concatenation leaves every row's codes, scales and zero points
    unchanged (all three formats quantise row-locally), so a fused matrix
    holds exactly the bytes of its parts and computes their outputs side by
    side, in one launch instead of several.
    """
    d = {name: (N, K) for name, N, K in mats}
    out = []
    if all(n in d for n in ("q", "k", "v")):
        out.append(("qkv", d["q"][0] + d["k"][0] + d["v"][0], d["q"][1]))
    out.append(("o", *d["o"]))
    if "gate" in d and "up" in d:
        out.append(("gate_up", d["gate"][0] + d["up"][0], d["gate"][1]))
    out.append(("down", *d["down"]))
    return tuple(out)


FUSED_PARTS = {"qkv": ("q", "k", "v"), "gate_up": ("gate", "up")}


def stack_70b(fmt: str, M: int, layers: int = 80, fused: bool = False, swiglu: bool = False) -> Workload:
    """swiglu: the fused layout with gate/up packed for the SwiGLU epilogue;
    gate_up writes h = silu(gate) * up and the down projection reads h."""
    cfg = 3 if fmt == "fp8" else 4
    mats = fuse_layer(I.LAYER_70B) if fused or swiglu else I.LAYER_70B
    tag = "_swiglu" if swiglu else "_fused" if fused else ""
    return Workload(f"70b_{fmt}_stack_{layers}l_m{M}{tag}", fmt, M, layers, mats, fmt == "w4a16", cfg,
                    swiglu=swiglu)


def stack_7b_bf16(M: int = 1, layers: int = 32, fused: bool = False) -> Workload:
    mats = fuse_layer(I.LAYER_7B) if fused else I.LAYER_7B
    tag = "_fused" if fused else ""
    return Workload(f"llama2_7b_bf16_stack_{layers}l_m{M}{tag}", "bf16", M, layers, mats, False, 2)


def gemv_4096_w4a16() -> Workload:
    return Workload("w4a16_gemv_4096x4096_m1", "w4a16", 1, 1, (("w", 4096, 4096),), False, 1)


def verify_matrix(fmt: str, mat: str, M: int) -> Workload:
    shapes = {"q": (8192, 8192), "o": (8192, 8192), "gate": (28672, 8192), "up": (28672, 8192),
              "down": (8192, 28672)}
    N, K = shapes[mat]
    return Workload(f"verify_{fmt}_{mat}_m{M}", fmt, M, 1, ((mat, N, K),), True, 5)


def verify_w8a8(mat: str, M: int) -> Workload:
    """A 70B verify-shape matrix in W8A8-FP8: FP8 weights, activations
    quantised to FP8 per tensor, the product on the FP8 matrix cores."""
    wl = verify_matrix("fp8", mat, M)
    return Workload(f"verify_w8a8_{mat}_m{M}", "fp8", M, 1, wl.mats, True, 5, "fp8")


VERIFY_M = (6, 16, 48, 128, 192, 384, 512, 1024)
