"""Weight-only quantized decode linear layer for MI355X (gfx950).

A thin ctypes binding over ``libwqd.so`` (C ABI in ``include/wqd.h``).  It only
marshals arguments: torch provides device memory and the current HIP stream,
and every step of the computation runs in the library's HIP kernels.  If the
library is missing, every call raises: there is no fallback.

    import weight_only_quantized_decode_amd as wqd
    pw = wqd.pack_weights("w4a16", W)        # W: cuda float32 [N, K]
    y = wqd.qgemm(x, pw)                     # x: cuda bfloat16 [M, K] -> y [M, N]
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libwqd.so")

FMT = {"bf16": 0, "fp8": 1, "w4a16": 2}
FMT_NAMES = {v: k for k, v in FMT.items()}
GROUP = 128

_lib = None


class WqdError(RuntimeError):
    def __init__(self, status: int, where: str, hip_error: int = 0):
        self.status = status
        self.hip_error = hip_error
        msg = f"{where}: {lib().wqd_status_str(status).decode()} (status {status})"
        if hip_error:
            msg += f", hipError {hip_error}"
        super().__init__(msg)


_SIGNATURE_NAMES: list = []


class ChainCallC(ctypes.Structure):
    """wqd_chain_call."""
    _fields_ = [("w_packed", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("zeros", ctypes.c_void_p),
                ("x", ctypes.c_void_p), ("y", ctypes.c_void_p), ("N", ctypes.c_int64), ("K", ctypes.c_int64),
                ("wait_for", ctypes.c_int32), ("swiglu", ctypes.c_int32)]


class ChainPlanC(ctypes.Structure):
    """wqd_chain_plan."""
    _fields_ = [("fmt", ctypes.c_int32), ("M", ctypes.c_int32), ("ncalls", ctypes.c_int32),
                ("total_items", ctypes.c_int32), ("workgroups", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("wait_ticks", ctypes.c_int64)]


def lib() -> ctypes.CDLL:
    """The loaded C library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m weight_only_quantized_decode_amd.build` "
                "(the decode path has no fallback)"
            )
        L = ctypes.CDLL(LIB_PATH)
        i64, sz, vp, i32 = ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int
        f32 = ctypes.c_float
        psz = ctypes.POINTER(ctypes.c_size_t)
        sig = {
            "wqd_version": (i32, []),
            "wqd_status_str": (ctypes.c_char_p, [i32]),
            "wqd_last_hip_error": (i32, []),
            "wqd_packed_sizes": (i32, [i32, i64, i64, psz, psz, psz]),
            "wqd_workspace_bytes": (i32, [i32, i64, i64, i64, psz]),
            "wqd_kernel_path": (i32, [i32, i64, i64, i64, ctypes.POINTER(i32), ctypes.POINTER(i32)]),
            "wqd_gemm_tile": (i32, [i32, i64, i64, i64] + [ctypes.POINTER(i32)] * 5),
            "wqd_w8a8_tile": (i32, [i64, i64, i64, ctypes.POINTER(i32), ctypes.POINTER(i32), ctypes.POINTER(i32)]),
            "wqd_pack_weights": (i32, [i32, vp, i64, i64, vp, vp, vp, vp]),
            "wqd_qgemm": (i32, [i32, vp, i64, i64, i64, vp, vp, vp, vp, vp, sz, vp]),
            "wqd_qgemm_noalloc": (i32, [i32, vp, i64, i64, i64, vp, vp, vp, vp, vp]),
            "wqd_pack_gate_up": (i32, [i32, vp, i64, i64, vp, vp, vp, vp]),
            "wqd_qgemm_swiglu": (i32, [i32, vp, i64, i64, i64, vp, vp, vp, vp, vp, sz, vp]),
            "wqd_act_quant_fp8": (i32, [vp, i64, i64, vp, vp, vp, sz, vp]),
            "wqd_attn_workspace_bytes": (i32, [i64, i64, i64, i64, i64, psz]),
            "wqd_attn_splits": (i32, [i64, i64, i64, i64, i64, ctypes.POINTER(ctypes.c_int)]),
            "wqd_decode_attention": (i32, [vp, vp, vp, vp, i64, i64, i64, i64, i64, ctypes.c_float, vp, vp, sz,
                                            vp]),
            "wqd_kv_pack": (i32, [vp, vp, i64, i64, i64, i64, i64, vp, vp, vp]),
            "wqd_kv_append": (i32, [vp, vp, vp, i64, i64, i64, i64, vp, vp, vp]),
            "wqd_kv_unpack": (i32, [vp, vp, i64, i64, i64, i64, vp, vp, vp]),
            "wqd_attn_fp8kv_workspace_bytes": (i32, [i64, i64, i64, i64, i64, psz]),
            "wqd_attn_fp8kv_splits": (i32, [i64, i64, i64, i64, i64, ctypes.POINTER(ctypes.c_int)]),
            "wqd_decode_attention_fp8kv": (i32, [vp, vp, vp, f32, f32, vp, i64, i64, i64, i64, i64, f32, vp, vp,
                                                 sz, vp]),
            "wqd_kv_pack_fp8": (i32, [vp, vp, f32, f32, i64, i64, i64, i64, i64, vp, vp, vp]),
            "wqd_kv_append_fp8": (i32, [vp, vp, f32, f32, vp, i64, i64, i64, i64, vp, vp, vp]),
            "wqd_kv_unpack_fp8": (i32, [vp, vp, i64, i64, i64, i64, vp, vp, vp]),
            "wqd_w8a8_workspace_bytes": (i32, [i64, i64, i64, psz]),
            "wqd_qgemm_w8a8": (i32, [vp, vp, i64, i64, i64, vp, vp, vp, vp, sz, vp]),
            "wqd_chain_workspace_bytes": (i32, [i64, psz]),
            "wqd_chain_prepare": (i32, [i32, i64, i64, ctypes.POINTER(ChainCallC), i32, vp, sz,
                                        ctypes.POINTER(ChainPlanC)]),
            "wqd_chain_run": (i32, [ctypes.POINTER(ChainPlanC), vp, vp]),
            "wqd_chain_status": (i32, [vp, vp]),
            "wqd_dequant": (i32, [i32, vp, vp, vp, i64, i64, vp, vp]),
            "wqd_unpack": (i32, [i32, vp, vp, vp, i64, i64, vp, vp, vp, vp]),
            "wqd_decode_e4m3": (i32, [vp, vp, i64, vp]),
            "wqd_spec_workspace_bytes": (i32, [i64, i64, psz]),
            "wqd_spec_accept": (i32, [vp, vp, vp, vp, vp, i64, i64, i64, vp, vp, vp, sz, vp]),
            "wqd_stream_read": (i32, [vp, sz, vp, vp]),
            "wqd_stream_sink_words": (sz, [sz]),
            "wqd_stream_copy": (i32, [vp, vp, sz, vp]),
            "wqd_mfma_peak": (i32, [i64, vp, vp]),
            "wqd_mfma_peak_sink_words": (sz, []),
            "wqd_mfma_peak_flops": (ctypes.c_double, [i64]),
        }
        _SIGNATURE_NAMES[:] = list(sig)
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def exported_symbols():
    """Names of the C entry points this binding declares (all must resolve)."""
    lib()
    return list(_SIGNATURE_NAMES)


def _check(status: int, where: str):
    if status != 0:
        raise WqdError(status, where, lib().wqd_last_hip_error() if status == 5 else 0)


def _fmt(fmt) -> int:
    if isinstance(fmt, str):
        if fmt not in FMT:
            raise ValueError(f"unknown format {fmt!r}; expected one of {sorted(FMT)}")
        return FMT[fmt]
    return int(fmt)


def _stream(stream=None):
    import torch

    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


# ----------------------------------------------------------------------------- host queries
def packed_sizes(fmt, N: int, K: int):
    w, s, z = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    _check(lib().wqd_packed_sizes(_fmt(fmt), N, K, ctypes.byref(w), ctypes.byref(s), ctypes.byref(z)),
           "wqd_packed_sizes")
    return w.value, s.value, z.value


def workspace_bytes(fmt, M: int, N: int, K: int) -> int:
    b = ctypes.c_size_t()
    _check(lib().wqd_workspace_bytes(_fmt(fmt), M, N, K, ctypes.byref(b)), "wqd_workspace_bytes")
    return b.value


KERNEL_PATHS = ("bcast", "staged", "mfma", "mc", "skinny", "gemm", "gemm_lds")


def kernel_path(fmt, M: int, N: int, K: int):
    """(family, wavefronts per workgroup) of the kernel qgemm launches for this shape."""
    p, w = ctypes.c_int(), ctypes.c_int()
    _check(lib().wqd_kernel_path(_fmt(fmt), M, N, K, ctypes.byref(p), ctypes.byref(w)), "wqd_kernel_path")
    return KERNEL_PATHS[p.value], w.value


def gemm_tile(fmt, M: int, N: int, K: int, tail: bool = False):
    """(rows, columns, K splits) of the tile of y each workgroup computes, for
    shapes on a tiled matrix-core kernel (WqdError with WQD_E_UNSUPPORTED for
    the others); with tail=True also (tail columns, tail splits), (0, 0) when
    there is no tail split."""
    r, c, s, tc, ts = (ctypes.c_int() for _ in range(5))
    _check(lib().wqd_gemm_tile(_fmt(fmt), M, N, K, ctypes.byref(r), ctypes.byref(c), ctypes.byref(s),
                               ctypes.byref(tc), ctypes.byref(ts)), "wqd_gemm_tile")
    return (r.value, c.value, s.value) + ((tc.value, ts.value) if tail else ())


def w8a8_tile(M: int, N: int, K: int):
    """(rows, columns, K splits) of the tile of y each workgroup of qgemm_w8a8
    computes for this shape."""
    r, c, s = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    _check(lib().wqd_w8a8_tile(M, N, K, ctypes.byref(r), ctypes.byref(c), ctypes.byref(s)), "wqd_w8a8_tile")
    return r.value, c.value, s.value


# ----------------------------------------------------------------------------- packed weights
@dataclass
class PackedWeight:
    fmt: str
    N: int
    K: int
    w: "object"                 # torch uint8 device tensor
    scales: "Optional[object]"  # torch uint8 device tensor (or None)
    zeros: "Optional[object]"

    @property
    def nbytes(self) -> int:
        return sum(t.numel() for t in (self.w, self.scales, self.zeros) if t is not None)


def alloc_packed(fmt, N: int, K: int, device="cuda") -> PackedWeight:
    import torch

    wb, sb, zb = packed_sizes(fmt, N, K)
    w = torch.empty(wb, dtype=torch.uint8, device=device)
    s = torch.empty(sb, dtype=torch.uint8, device=device) if sb else None
    z = torch.empty(zb, dtype=torch.uint8, device=device) if zb else None
    return PackedWeight(FMT_NAMES[_fmt(fmt)], N, K, w, s, z)


def pack_weights(fmt, W, out: Optional[PackedWeight] = None, stream=None) -> PackedWeight:
    """Quantise float32 W[N, K] (cuda) into the packed layout."""
    import torch

    if W.dtype != torch.float32 or not W.is_cuda or W.dim() != 2:
        raise ValueError("W must be a cuda float32 [N, K] tensor")
    W = W.contiguous()
    N, K = W.shape
    pw = out if out is not None else alloc_packed(fmt, N, K, W.device)
    _check(lib().wqd_pack_weights(_fmt(fmt), W.data_ptr(), N, K, _ptr(pw.w), _ptr(pw.scales), _ptr(pw.zeros),
                                  _stream(stream)), "wqd_pack_weights")
    return pw


def pack_gate_up(fmt, W, out: Optional[PackedWeight] = None, stream=None) -> PackedWeight:
    """wqd_pack_gate_up: W float32 [2F, K] (cuda; gate rows, then up rows),
    packed for the SwiGLU epilogue.  The PackedWeight has N = 2F rows."""
    import torch

    if W.dtype != torch.float32 or not W.is_cuda or W.dim() != 2 or W.shape[0] % 2:
        raise ValueError("W must be a cuda float32 [2F, K] tensor (gate rows, then up rows)")
    W = W.contiguous()
    N, K = W.shape
    pw = out if out is not None else alloc_packed(fmt, N, K, W.device)
    _check(lib().wqd_pack_gate_up(_fmt(fmt), W.data_ptr(), N // 2, K, _ptr(pw.w), _ptr(pw.scales), _ptr(pw.zeros),
                                  _stream(stream)), "wqd_pack_gate_up")
    return pw


def qgemm_swiglu(x, pw: PackedWeight, h=None, workspace=None, stream=None):
    """wqd_qgemm_swiglu: h[M, F] (bfloat16) = silu(x . gate^T) * (x . up^T),
    pw packed by pack_gate_up (N = 2F)."""
    import torch

    if x.dtype != torch.bfloat16 or x.dim() != 2 or not x.is_contiguous():
        raise ValueError("x must be a contiguous bfloat16 [M, K] tensor")
    M, K = x.shape
    F = pw.N // 2
    if K != pw.K:
        raise ValueError(f"K mismatch: x has {K}, weights have {pw.K}")
    if h is None:
        h = torch.empty((M, F), dtype=torch.bfloat16, device=x.device)
    need = workspace_bytes(pw.fmt, M, pw.N, K)
    if workspace is None:
        workspace = get_workspace(need, x.device)
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().wqd_qgemm_swiglu(_fmt(pw.fmt), x.data_ptr(), M, F, K, _ptr(pw.w), _ptr(pw.scales), _ptr(pw.zeros),
                                  h.data_ptr(), _ptr(workspace), wsb, _stream(stream)), "wqd_qgemm_swiglu")
    return h


# ----------------------------------------------------------------------------- workspace
_ws_cache = {}


def get_workspace(nbytes: int, device=None):
    """A workspace of at least nbytes, cached per device (grow-only).

    Its contents on entry do not matter to wqd_qgemm (every byte it reads was
    written earlier in the same call), so consecutive calls on one stream can
    share it; calls that may run at the same time must not.
    """
    import torch

    if nbytes == 0:
        return None
    dev = torch.device(device) if device is not None else torch.device("cuda", torch.cuda.current_device())
    cur = _ws_cache.get(dev)
    if cur is None or cur.numel() < nbytes:
        cur = torch.zeros(max(nbytes, 1 << 20), dtype=torch.uint8, device=dev)
        _ws_cache[dev] = cur
    return cur


def qgemm(x, pw: PackedWeight, y=None, workspace=None, stream=None):
    """y[M, N] (bfloat16) = x[M, K] (bfloat16) . dequant(W)^T."""
    import torch

    if x.dtype != torch.bfloat16 or x.dim() != 2 or not x.is_contiguous():
        raise ValueError("x must be a contiguous bfloat16 [M, K] tensor")
    M, K = x.shape
    if K != pw.K:
        raise ValueError(f"K mismatch: x has {K}, weights have {pw.K}")
    if y is None:
        y = torch.empty((M, pw.N), dtype=torch.bfloat16, device=x.device)
    need = workspace_bytes(pw.fmt, M, pw.N, K)
    if workspace is None:
        workspace = get_workspace(need, x.device)
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().wqd_qgemm(_fmt(pw.fmt), x.data_ptr(), M, pw.N, K, _ptr(pw.w), _ptr(pw.scales), _ptr(pw.zeros),
                           y.data_ptr(), _ptr(workspace), wsb, _stream(stream)), "wqd_qgemm")
    return y


NOALLOC_SCRATCH_BYTES = 64 << 20  # WQD_NOALLOC_SCRATCH_BYTES


def qgemm_noalloc(x, pw: PackedWeight, y, stream=None):
    """wqd_qgemm_noalloc: y = x . dequant(W)^T with the library's per-GPU
    scratch array instead of a workspace; allocates nothing (y is the
    caller's).  Calls that can overlap on one GPU must not use it."""
    import torch

    if x.dtype != torch.bfloat16 or x.dim() != 2 or not x.is_contiguous():
        raise ValueError("x must be a contiguous bfloat16 [M, K] tensor")
    M, K = x.shape
    if K != pw.K or y.dtype != torch.bfloat16 or tuple(y.shape) != (M, pw.N) or not y.is_contiguous():
        raise ValueError("x / y shapes do not match the packed weights")
    _check(lib().wqd_qgemm_noalloc(_fmt(pw.fmt), x.data_ptr(), M, pw.N, K, _ptr(pw.w), _ptr(pw.scales),
                                   _ptr(pw.zeros), y.data_ptr(), _stream(stream)), "wqd_qgemm_noalloc")
    return y


# ----------------------------------------------------------------------------- chains
@dataclass
class ChainStep:
    """One call of a chain: y = x . dequant(pw)^T (swiglu: the SwiGLU of a
    pack_gate_up pair, y with N / 2 columns); wait_for = index of the earlier
    step whose y this x is (or is part of), -1 when x is ready beforehand."""
    x: "object"
    pw: PackedWeight
    y: "object"
    wait_for: int = -1
    swiglu: bool = False


@dataclass
class Chain:
    plan: ChainPlanC
    workspace: "object"   # torch uint8 device tensor holding the call table and counters
    steps: list           # the ChainSteps (their tensors stay referenced)


def chain_workspace_bytes(ncalls: int) -> int:
    b = ctypes.c_size_t()
    _check(lib().wqd_chain_workspace_bytes(ncalls, ctypes.byref(b)), "wqd_chain_workspace_bytes")
    return b.value


def chain_prepare(steps, workgroups: int = 0, workspace=None) -> Chain:
    """wqd_chain_prepare: validate the steps (one format, the same M rows of
    x for all) and write the call table into a device workspace."""
    import torch

    if not steps:
        raise ValueError("a chain needs at least one step")
    fmt = _fmt(steps[0].pw.fmt)
    M = steps[0].x.shape[0]
    arr = (ChainCallC * len(steps))()
    for i, st in enumerate(steps):
        if _fmt(st.pw.fmt) != fmt:
            raise ValueError("every step of a chain uses one weight format")
        if st.x.dtype != torch.bfloat16 or st.x.dim() != 2 or not st.x.is_contiguous() or st.x.shape[0] != M:
            raise ValueError(f"step {i}: x must be a contiguous bfloat16 [{M}, K] tensor")
        if st.x.shape[1] != st.pw.K:
            raise ValueError(f"step {i}: K mismatch: x has {st.x.shape[1]}, weights have {st.pw.K}")
        cols = st.pw.N // 2 if st.swiglu else st.pw.N
        if st.y.dtype != torch.bfloat16 or tuple(st.y.shape) != (M, cols) or not st.y.is_contiguous():
            raise ValueError(f"step {i}: y must be a contiguous bfloat16 [{M}, {cols}] tensor")
        arr[i] = ChainCallC(_ptr(st.pw.w), _ptr(st.pw.scales), _ptr(st.pw.zeros), st.x.data_ptr(), st.y.data_ptr(),
                            st.pw.N, st.pw.K, int(st.wait_for), 1 if st.swiglu else 0)
    need = chain_workspace_bytes(len(steps))
    if workspace is None:
        workspace = torch.zeros(need, dtype=torch.uint8, device=steps[0].x.device)
    plan = ChainPlanC()
    _check(lib().wqd_chain_prepare(fmt, M, len(steps), arr, workgroups, workspace.data_ptr(),
                                   workspace.numel() * workspace.element_size(), ctypes.byref(plan)),
           "wqd_chain_prepare")
    return Chain(plan, workspace, list(steps))


def chain_run(chain: Chain, stream=None):
    """wqd_chain_run: the whole chain in one persistent launch (after a small
    clearing launch), on the current stream; graph-capturable."""
    _check(lib().wqd_chain_run(ctypes.byref(chain.plan), chain.workspace.data_ptr(), _stream(stream)),
           "wqd_chain_run")


def chain_status(chain: Chain, stream=None) -> int:
    """wqd_chain_status: synchronizes the stream; 0 when the last run
    completed, WQD_E_TIMEOUT (7) when it abandoned a wait, WQD_E_ARG (1) when
    the plan did not match the table."""
    return int(lib().wqd_chain_status(chain.workspace.data_ptr(), _stream(stream)))


ACT_QUANT_WORKSPACE_BYTES = 4096  # WQD_ACT_QUANT_WORKSPACE_BYTES


def act_quant_fp8(x, codes=None, scale=None, workspace=None, stream=None):
    """wqd_act_quant_fp8: (codes uint8 [M, K], scale float32 [1]) of bf16 x."""
    import torch

    if x.dtype != torch.bfloat16 or x.dim() != 2 or not x.is_contiguous():
        raise ValueError("x must be a contiguous bfloat16 [M, K] tensor")
    M, K = x.shape
    if codes is None:
        codes = torch.empty((M, K), dtype=torch.uint8, device=x.device)
    if scale is None:
        scale = torch.empty(1, dtype=torch.float32, device=x.device)
    if workspace is None:
        workspace = get_workspace(ACT_QUANT_WORKSPACE_BYTES, x.device)
    _check(lib().wqd_act_quant_fp8(x.data_ptr(), M, K, codes.data_ptr(), scale.data_ptr(), _ptr(workspace),
                                   workspace.numel() * workspace.element_size(), _stream(stream)),
           "wqd_act_quant_fp8")
    return codes, scale


def w8a8_workspace_bytes(M: int, N: int, K: int) -> int:
    b = ctypes.c_size_t()
    _check(lib().wqd_w8a8_workspace_bytes(M, N, K, ctypes.byref(b)), "wqd_w8a8_workspace_bytes")
    return b.value


def qgemm_w8a8(codes, scale, pw: PackedWeight, y=None, workspace=None, stream=None):
    """wqd_qgemm_w8a8: y[M, N] (bfloat16) from activation codes / scale and FP8 packed weights."""
    import torch

    if pw.fmt != "fp8":
        raise ValueError("W8A8 takes FP8 packed weights")
    M, K = codes.shape
    if K != pw.K or codes.dtype != torch.uint8 or not codes.is_contiguous():
        raise ValueError("codes must be a contiguous uint8 [M, K] tensor matching the weights")
    if y is None:
        y = torch.empty((M, pw.N), dtype=torch.bfloat16, device=codes.device)
    need = w8a8_workspace_bytes(M, pw.N, K)
    if workspace is None:
        workspace = get_workspace(need, codes.device)
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().wqd_qgemm_w8a8(codes.data_ptr(), scale.data_ptr(), M, pw.N, K, _ptr(pw.w), _ptr(pw.scales),
                                y.data_ptr(), _ptr(workspace), wsb, _stream(stream)), "wqd_qgemm_w8a8")
    return y


def w8a8(x, pw: PackedWeight, y=None, stream=None):
    """The W8A8-FP8 layer from bf16 x: activation quantisation, then the product."""
    codes, scale = act_quant_fp8(x, stream=stream)
    return qgemm_w8a8(codes, scale, pw, y=y, stream=stream)


def attn_workspace_bytes(B: int, Hq: int, Hkv: int, Lmax: int, D: int = 128) -> int:
    b = ctypes.c_size_t()
    _check(lib().wqd_attn_workspace_bytes(B, Hq, Hkv, Lmax, D, ctypes.byref(b)), "wqd_attn_workspace_bytes")
    return b.value


def attn_splits(B: int, Hq: int, Hkv: int, Lmax: int, D: int = 128) -> int:
    s = ctypes.c_int()
    _check(lib().wqd_attn_splits(B, Hq, Hkv, Lmax, D, ctypes.byref(s)), "wqd_attn_splits")
    return s.value


@dataclass
class KVCache:
    """One layer's KV cache in the library's tiled layout (device bf16)."""
    B: int
    Hkv: int
    Lmax: int
    k: "object"
    v: "object"
    D: int = 128


def alloc_kv_cache(B: int, Hkv: int, Lmax: int, D: int = 128, device="cuda") -> KVCache:
    import torch

    n = B * Hkv * Lmax * D
    return KVCache(B, Hkv, Lmax, torch.zeros(n, dtype=torch.bfloat16, device=device),
                   torch.zeros(n, dtype=torch.bfloat16, device=device), D)


def kv_pack(k, v, cache: KVCache, stream=None) -> KVCache:
    """wqd_kv_pack: logical k, v bf16 [B, Hkv, L, D] into positions 0 .. L - 1."""
    B, Hkv, L, D = k.shape
    if tuple(v.shape) != (B, Hkv, L, D) or not (k.is_contiguous() and v.is_contiguous()):
        raise ValueError("k and v must be contiguous [B, Hkv, L, D] tensors")
    _check(lib().wqd_kv_pack(k.data_ptr(), v.data_ptr(), B, Hkv, L, cache.Lmax, D, cache.k.data_ptr(),
                             cache.v.data_ptr(), _stream(stream)), "wqd_kv_pack")
    return cache


def kv_append(k_new, v_new, positions, cache: KVCache, stream=None) -> KVCache:
    """wqd_kv_append: k_new, v_new bf16 [B, Hkv, D] at positions int32 [B]."""
    _check(lib().wqd_kv_append(k_new.data_ptr(), v_new.data_ptr(), positions.data_ptr(), cache.B, cache.Hkv,
                               cache.Lmax, cache.D, cache.k.data_ptr(), cache.v.data_ptr(), _stream(stream)),
           "wqd_kv_append")
    return cache


def kv_unpack(cache: KVCache, stream=None):
    """wqd_kv_unpack: (k, v) logical bf16 [B, Hkv, Lmax, D]."""
    import torch

    shape = (cache.B, cache.Hkv, cache.Lmax, cache.D)
    k = torch.empty(shape, dtype=torch.bfloat16, device=cache.k.device)
    v = torch.empty(shape, dtype=torch.bfloat16, device=cache.k.device)
    _check(lib().wqd_kv_unpack(cache.k.data_ptr(), cache.v.data_ptr(), cache.B, cache.Hkv, cache.Lmax, cache.D,
                               k.data_ptr(), v.data_ptr(), _stream(stream)), "wqd_kv_unpack")
    return k, v


def decode_attention(q, cache: KVCache, lengths, scale: float, out=None, workspace=None, stream=None):
    """wqd_decode_attention: q bf16 [B, Hq, D] against a KVCache, lengths
    int32 [B] -> out bf16 [B, Hq, D]."""
    import torch

    B, Hq, D = q.shape
    if (B, D) != (cache.B, cache.D) or q.dtype != torch.bfloat16 or not q.is_contiguous():
        raise ValueError("q must be a contiguous bfloat16 [B, Hq, D] tensor matching the cache")
    if tuple(lengths.shape) != (B,) or lengths.dtype != torch.int32:
        raise ValueError("lengths must be int32 [B]")
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=q.device)
    if workspace is None:
        workspace = get_workspace(attn_workspace_bytes(B, Hq, cache.Hkv, cache.Lmax, D), q.device)
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().wqd_decode_attention(q.data_ptr(), cache.k.data_ptr(), cache.v.data_ptr(), lengths.data_ptr(), B,
                                      Hq, cache.Hkv, cache.Lmax, D, float(scale), out.data_ptr(),
                                      _ptr(workspace), wsb, _stream(stream)), "wqd_decode_attention")
    return out


def attn_fp8kv_workspace_bytes(B: int, Hq: int, Hkv: int, Lmax: int, D: int = 128) -> int:
    b = ctypes.c_size_t()
    _check(lib().wqd_attn_fp8kv_workspace_bytes(B, Hq, Hkv, Lmax, D, ctypes.byref(b)),
           "wqd_attn_fp8kv_workspace_bytes")
    return b.value


def attn_fp8kv_splits(B: int, Hq: int, Hkv: int, Lmax: int, D: int = 128) -> int:
    s = ctypes.c_int()
    _check(lib().wqd_attn_fp8kv_splits(B, Hq, Hkv, Lmax, D, ctypes.byref(s)), "wqd_attn_fp8kv_splits")
    return s.value


@dataclass
class KVCacheFP8:
    """One layer's FP8-E4M3 KV cache in the library's tiled layout (device
    uint8 codes) with its per-tensor scales."""
    B: int
    Hkv: int
    Lmax: int
    k: "object"
    v: "object"
    k_scale: float
    v_scale: float
    D: int = 128


def alloc_kv_cache_fp8(B: int, Hkv: int, Lmax: int, k_scale: float, v_scale: float, D: int = 128,
                       device="cuda") -> KVCacheFP8:
    import torch

    n = B * Hkv * Lmax * D
    return KVCacheFP8(B, Hkv, Lmax, torch.zeros(n, dtype=torch.uint8, device=device),
                      torch.zeros(n, dtype=torch.uint8, device=device), float(k_scale), float(v_scale), D)


def kv_pack_fp8(k, v, cache: KVCacheFP8, stream=None) -> KVCacheFP8:
    """wqd_kv_pack_fp8: logical k, v bf16 [B, Hkv, L, D], quantised with the
    cache's scales, into positions 0 .. L - 1."""
    B, Hkv, L, D = k.shape
    if tuple(v.shape) != (B, Hkv, L, D) or not (k.is_contiguous() and v.is_contiguous()):
        raise ValueError("k and v must be contiguous [B, Hkv, L, D] tensors")
    _check(lib().wqd_kv_pack_fp8(k.data_ptr(), v.data_ptr(), cache.k_scale, cache.v_scale, B, Hkv, L, cache.Lmax,
                                 D, cache.k.data_ptr(), cache.v.data_ptr(), _stream(stream)), "wqd_kv_pack_fp8")
    return cache


def kv_append_fp8(k_new, v_new, positions, cache: KVCacheFP8, stream=None) -> KVCacheFP8:
    """wqd_kv_append_fp8: k_new, v_new bf16 [B, Hkv, D] at positions int32 [B]."""
    _check(lib().wqd_kv_append_fp8(k_new.data_ptr(), v_new.data_ptr(), cache.k_scale, cache.v_scale,
                                   positions.data_ptr(), cache.B, cache.Hkv, cache.Lmax, cache.D,
                                   cache.k.data_ptr(), cache.v.data_ptr(), _stream(stream)), "wqd_kv_append_fp8")
    return cache


def kv_unpack_fp8(cache: KVCacheFP8, stream=None):
    """wqd_kv_unpack_fp8: (k_codes, v_codes) logical uint8 [B, Hkv, Lmax, D]."""
    import torch

    shape = (cache.B, cache.Hkv, cache.Lmax, cache.D)
    k = torch.empty(shape, dtype=torch.uint8, device=cache.k.device)
    v = torch.empty(shape, dtype=torch.uint8, device=cache.k.device)
    _check(lib().wqd_kv_unpack_fp8(cache.k.data_ptr(), cache.v.data_ptr(), cache.B, cache.Hkv, cache.Lmax,
                                   cache.D, k.data_ptr(), v.data_ptr(), _stream(stream)), "wqd_kv_unpack_fp8")
    return k, v


def decode_attention_fp8kv(q, cache: KVCacheFP8, lengths, scale: float, out=None, workspace=None, stream=None):
    """wqd_decode_attention_fp8kv: q bf16 [B, Hq, D] against a KVCacheFP8,
    lengths int32 [B] -> out bf16 [B, Hq, D]."""
    import torch

    B, Hq, D = q.shape
    if (B, D) != (cache.B, cache.D) or q.dtype != torch.bfloat16 or not q.is_contiguous():
        raise ValueError("q must be a contiguous bfloat16 [B, Hq, D] tensor matching the cache")
    if tuple(lengths.shape) != (B,) or lengths.dtype != torch.int32:
        raise ValueError("lengths must be int32 [B]")
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=q.device)
    if workspace is None:
        workspace = get_workspace(attn_fp8kv_workspace_bytes(B, Hq, cache.Hkv, cache.Lmax, D), q.device)
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().wqd_decode_attention_fp8kv(q.data_ptr(), cache.k.data_ptr(), cache.v.data_ptr(), cache.k_scale,
                                            cache.v_scale, lengths.data_ptr(), B, Hq, cache.Hkv, cache.Lmax, D,
                                            float(scale), out.data_ptr(), _ptr(workspace), wsb, _stream(stream)),
           "wqd_decode_attention_fp8kv")
    return out


def dequant(pw: PackedWeight, out=None, stream=None):
    import torch

    if out is None:
        out = torch.empty((pw.N, pw.K), dtype=torch.float32, device=pw.w.device)
    _check(lib().wqd_dequant(_fmt(pw.fmt), _ptr(pw.w), _ptr(pw.scales), _ptr(pw.zeros), pw.N, pw.K, out.data_ptr(),
                             _stream(stream)), "wqd_dequant")
    return out


def unpack(pw: PackedWeight, stream=None):
    """Logical (codes, scales, zeros) of a packed weight, as device tensors."""
    import torch

    dev = pw.w.device
    G = pw.K // GROUP
    if pw.fmt == "bf16":
        codes = torch.empty((pw.N, pw.K), dtype=torch.int16, device=dev)
        scales = zeros = None
    elif pw.fmt == "fp8":
        codes = torch.empty((pw.N, pw.K), dtype=torch.uint8, device=dev)
        scales = torch.empty((pw.N,), dtype=torch.float32, device=dev)
        zeros = None
    else:
        codes = torch.empty((pw.N, pw.K), dtype=torch.uint8, device=dev)
        scales = torch.empty((pw.N, G), dtype=torch.int16, device=dev)
        zeros = torch.empty((pw.N, G), dtype=torch.uint8, device=dev)
    _check(lib().wqd_unpack(_fmt(pw.fmt), _ptr(pw.w), _ptr(pw.scales), _ptr(pw.zeros), pw.N, pw.K,
                            codes.data_ptr(), _ptr(scales), _ptr(zeros), _stream(stream)), "wqd_unpack")
    return codes, scales, zeros


def decode_e4m3(codes, stream=None):
    import torch

    out = torch.empty(codes.shape, dtype=torch.float32, device=codes.device)
    _check(lib().wqd_decode_e4m3(codes.data_ptr(), out.data_ptr(), codes.numel(), _stream(stream)),
           "wqd_decode_e4m3")
    return out


def spec_accept(target, draft, draft_tokens, u_accept, u_draw, workspace=None, stream=None):
    """Speculative accept / reject on the device (``wqd_spec_accept``).

    target float32 [B, k+1, V], draft float32 [B, k, V], draft_tokens int32
    [B, k], u_accept float32 [B, k], u_draw float32 [B], all contiguous on one
    device.  Returns (n_kept int32 [B], out_tokens int32 [B, k+1]).
    """
    import torch

    B, k1, V = target.shape
    k = k1 - 1
    want = ((target, torch.float32, (B, k1, V)), (draft, torch.float32, (B, k, V)),
            (draft_tokens, torch.int32, (B, k)), (u_accept, torch.float32, (B, k)), (u_draw, torch.float32, (B,)))
    for t, dt, shape in want:
        if t.dtype != dt or tuple(t.shape) != shape or not t.is_contiguous() or t.device != target.device:
            raise ValueError(f"spec_accept: expected a contiguous {dt} tensor of shape {shape} on {target.device}")
    n_kept = torch.empty(B, dtype=torch.int32, device=target.device)
    out = torch.empty((B, k1), dtype=torch.int32, device=target.device)
    ptr = lambda t: t.data_ptr() if t.numel() else None  # noqa: E731
    if workspace is None:
        workspace = get_workspace(spec_workspace_bytes(B, V), target.device)
    wsb = workspace.numel() * workspace.element_size()
    _check(lib().wqd_spec_accept(target.data_ptr(), ptr(draft), ptr(draft_tokens), ptr(u_accept), u_draw.data_ptr(),
                                 B, k, V, n_kept.data_ptr(), out.data_ptr(), workspace.data_ptr(), wsb,
                                 _stream(stream)), "wqd_spec_accept")
    return n_kept, out


def spec_workspace_bytes(B: int, V: int) -> int:
    b = ctypes.c_size_t()
    _check(lib().wqd_spec_workspace_bytes(B, V, ctypes.byref(b)), "wqd_spec_workspace_bytes")
    return b.value


def stream_read(buf, sink=None, stream=None):
    import torch

    nbytes = buf.numel() * buf.element_size()
    words = lib().wqd_stream_sink_words(nbytes)
    if sink is None:
        sink = torch.empty(words, dtype=torch.int32, device=buf.device)
    _check(lib().wqd_stream_read(buf.data_ptr(), nbytes, sink.data_ptr(), _stream(stream)), "wqd_stream_read")
    return sink


def stream_copy(dst, src, stream=None):
    nbytes = src.numel() * src.element_size()
    _check(lib().wqd_stream_copy(dst.data_ptr(), src.data_ptr(), nbytes, _stream(stream)), "wqd_stream_copy")
    return dst


def mfma_peak(iters, sink, stream=None):
    """Launch the matrix-core ceiling kernel (`iters` x 16 multiplies per
    wavefront, see wqd_mfma_peak); returns the FLOP count of the launch."""
    _check(lib().wqd_mfma_peak(int(iters), sink.data_ptr(), _stream(stream)), "wqd_mfma_peak")
    return lib().wqd_mfma_peak_flops(int(iters))


def mfma_peak_sink_words():
    return lib().wqd_mfma_peak_sink_words()
