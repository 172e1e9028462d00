"""GPU parity of a chain of decode layers in one persistent launch
(wqd_chain_prepare / wqd_chain_run / wqd_chain_status) against the oracle.

Every output buffer is filled with NaN before a run, and each call is checked
against the oracle on the input it actually read (the bf16 output of the call
it waited for, copied back after the run).  A call that read its x before the
call writing it had finished would therefore see NaN or stale values and fail,
so the checks cover the ordering as well as the arithmetic.

Cases: chains of six calls per format and row count (dependencies on the
previous call and on an earlier one, an independent call in the middle, a
SwiGLU gate/up pair, ragged N and, for FP8 / BF16, ragged K), with the
library's grid and with 1 and 5 workgroups (each workgroup then runs many
items back to back); determinism and graph replays; two full 70B layers in
the fused layout (W4A16 at one row, FP8 at two; sampled rows); a plan that
does not match the prepared table, and a wait bound of zero (runs that stop
early report it and leave the next run correct)."""
import numpy as np
import pytest
import torch

import oracle
import weight_only_quantized_decode_amd as wqd
import wqd_inputs as I
from tests.parity import bf16_bits, compare_y

pytestmark = pytest.mark.gpu

DEV = "cuda"
NAN_BF16 = 0x7FC0


def to_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV).view(torch.bfloat16)


class Case:
    """A chain built from (N, K, wait_for, swiglu) specs; x of a call that
    waits is the y of the call it waits for (whose columns must equal K)."""

    def __init__(self, fmt, M, specs, seed):
        self.fmt, self.M = fmt, M
        self.steps, self.q, self.ext = [], [], {}
        for i, (N, K, dep, sw) in enumerate(specs):
            # weights of scale 1 / sqrt(K): every call's outputs stay of order 1
            W = I.w_host(seed + 17 * i, N, K, sigma=float(K) ** -0.5)
            Wd = torch.from_numpy(W).to(DEV)
            if sw:
                pw = wqd.pack_gate_up(fmt, Wd)
                self.q.append((oracle.quantize(fmt, W[: N // 2]), oracle.quantize(fmt, W[N // 2:])))
            else:
                pw = wqd.pack_weights(fmt, Wd)
                self.q.append(oracle.quantize(fmt, W))
            if dep < 0:
                xb = I.x_bf16_bits(seed + 1000 + i, M, K)
                self.ext[i] = xb
                x = to_dev(xb)
            else:
                x = self.steps[dep].y
                assert tuple(x.shape) == (M, K), (i, dep, tuple(x.shape), K)
            y = torch.empty((M, N // 2 if sw else N), dtype=torch.bfloat16, device=DEV)
            self.steps.append(wqd.ChainStep(x, pw, y, dep, bool(sw)))

    def poison(self):
        for st in self.steps:
            st.y.view(torch.int16).fill_(NAN_BF16)

    def outputs(self):
        return [bf16_bits(st.y) for st in self.steps]

    def check(self, what):
        ys = self.outputs()
        for i, st in enumerate(self.steps):
            xb = self.ext[i] if st.wait_for < 0 else ys[st.wait_for]
            if st.swiglu:
                ref = oracle.swiglu_exact(xb, *self.q[i])
            else:
                ref = oracle.qgemm_exact(xb, self.q[i])
            s = compare_y(ys[i], ref, f"{what} call {i}")
            print(f"  call {i}: rel L2 {s['rel_l2']:.2e} max {s['max_rel']:.2e}", flush=True)
        return ys


def specs_for(fmt):
    if fmt == "w4a16":  # K whole groups of 128
        return [(384, 512, -1, 0), (1280, 384, 0, 1), (512, 640, 1, 0), (200, 256, -1, 0), (1024, 512, 2, 0),
                (64, 384, 0, 0)]
    # FP8 / BF16: ragged K (208, 96, 40 are not whole tiles of 64 or 32 k) and ragged N
    return [(96, 208, -1, 0), (416, 96, 0, 1), (40, 208, 1, 0), (200, 40, 2, 0), (1024, 200, 3, 0),
            (48, 96, 0, 0)]


def run_chain(case, workgroups=0):
    chain = wqd.chain_prepare(case.steps, workgroups=workgroups)
    case.poison()
    wqd.chain_run(chain)
    st = wqd.chain_status(chain)
    assert st == 0, wqd.lib().wqd_status_str(st)
    return chain


@pytest.mark.parametrize("fmt", ["w4a16", "fp8", "bf16"])
@pytest.mark.parametrize("M", [1, 2])
@pytest.mark.parametrize("workgroups", [0, 1, 5])
def test_small_chains(fmt, M, workgroups):
    case = Case(fmt, M, specs_for(fmt), 300 + 7 * M + workgroups)
    print(f"chain {fmt} M={M} workgroups={workgroups}", flush=True)
    chain = run_chain(case, workgroups)
    assert chain.plan.workgroups == (workgroups or chain.plan.workgroups) and chain.plan.workgroups >= 1
    case.check(f"chain {fmt} M={M} wg={workgroups}")


def test_deterministic_and_graph_replays():
    case = Case("w4a16", 1, specs_for("w4a16"), 41)
    print("chain determinism and graph replays", flush=True)
    chain = run_chain(case)
    first = case.check("eager")
    case.poison()
    wqd.chain_run(chain)
    assert wqd.chain_status(chain) == 0
    assert all(np.array_equal(a, b) for a, b in zip(first, case.outputs()))
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        wqd.chain_run(chain, stream=s)  # warm up on the capture stream
    s.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        wqd.chain_run(chain, stream=s)
    for r in range(3):
        case.poison()  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert wqd.chain_status(chain) == 0
        assert all(np.array_equal(a, b) for a, b in zip(first, case.outputs())), f"replay {r}"


@pytest.mark.parametrize("fmt,M", [("w4a16", 1), ("fp8", 2)])
def test_70b_two_layers_fused(fmt, M):
    """qkv (10240 x 8192) -> o (x = the first M x 8192 outputs of qkv, standing
    in for attention) -> gate/up SwiGLU (57344 x 8192 packed pairs) -> down
    (8192 x 28672) -> the next layer's qkv on down's output."""
    K = 8192
    shapes = [("qkv", 10240, 8192), ("o", 8192, 8192), ("gate_up", 57344, 8192), ("down", 8192, 28672)]
    rng = np.random.default_rng(9)
    steps, samples = [], []
    x0 = I.x_bf16_bits(I.x_seed(8, M, K), M, K, outliers=True)
    prev = to_dev(x0)
    for layer in range(2):
        for j, (name, N, Kc) in enumerate(shapes):
            i = 4 * layer + j
            W = I.w_device(9000 + i, N, Kc, device=DEV)
            sw = name == "gate_up"
            pw = wqd.pack_gate_up(fmt, W) if sw else wqd.pack_weights(fmt, W)
            cols_out = N // 2 if sw else N
            pick = np.array(sorted(set(rng.choice(cols_out, 24, replace=False).tolist()) | {0, cols_out - 1}))
            if sw:
                idx = torch.from_numpy(np.concatenate([pick, N // 2 + pick])).to(DEV)
                Wh = W[idx].cpu().numpy()
                q = (oracle.quantize(fmt, Wh[: len(pick)]), oracle.quantize(fmt, Wh[len(pick):]))
            else:
                q = oracle.quantize(fmt, W[torch.from_numpy(pick).to(DEV)].cpu().numpy())
            del W
            x = prev if name != "o" else prev.reshape(-1)[: M * 8192].view(M, 8192)
            y = torch.empty((M, cols_out), dtype=torch.bfloat16, device=DEV)
            steps.append(wqd.ChainStep(x, pw, y, i - 1, sw))
            samples.append((pick, q))
            prev = y
    steps[0].wait_for = -1
    print(f"chain 70B {fmt} M={M}, 2 layers (8 calls)", flush=True)
    chain = wqd.chain_prepare(steps)
    for st in steps:
        st.y.view(torch.int16).fill_(NAN_BF16)
    wqd.chain_run(chain)
    assert wqd.chain_status(chain) == 0
    ys = [bf16_bits(st.y) for st in steps]
    for i, st in enumerate(steps):
        xb = x0 if i == 0 else (ys[i - 1].reshape(-1)[: M * 8192].reshape(M, 8192) if i % 4 == 1 else ys[i - 1])
        pick, q = samples[i]
        ref = oracle.swiglu_exact(xb, *q) if st.swiglu else oracle.qgemm_exact(xb, q)
        s = compare_y(ys[i][:, pick], ref, f"70B chain call {i}")
        print(f"  call {i}: rel L2 {s['rel_l2']:.2e}", flush=True)


def test_plan_mismatch_and_zero_wait_bound():
    case = Case("fp8", 1, specs_for("fp8"), 77)
    chain = run_chain(case)
    good = case.check("reference run")
    # a plan that does not match the prepared table: the kernel stops at once
    bad = wqd.ChainPlanC.from_buffer_copy(chain.plan)
    bad.total_items += 1
    st = wqd.lib().wqd_chain_run(bad, chain.workspace.data_ptr(), None)
    assert st == 0
    assert wqd.chain_status(chain) == 1
    # a wait bound of zero: every wait that is not already satisfied is
    # abandoned, the other workgroups stop at their next wait
    zero = wqd.ChainPlanC.from_buffer_copy(chain.plan)
    zero.wait_ticks = 0
    case.poison()
    assert wqd.lib().wqd_chain_run(zero, chain.workspace.data_ptr(), None) == 0
    st = wqd.chain_status(chain)
    print(f"zero wait bound: status {st}", flush=True)
    assert st in (0, 7)
    # the next run clears counters and flag and is whole again
    case.poison()
    wqd.chain_run(chain)
    assert wqd.chain_status(chain) == 0
    assert all(np.array_equal(a, b) for a, b in zip(good, case.outputs()))
