"""Pins of the oracle's speculative-sampling accept / reject step (CPU only).

The step is pinned against what the pages and the mathematics fix, not against
its own formulas: the worked three-token example printed with its answers
(tests/golden/spec_sampling_page_example.txt), the theorem that the output is
distributed exactly as the target (integrated over grids of the uniforms), a
pure-Python walk of the inverse cumulative distribution, and special cases.
"""
import os

import numpy as np
import pytest

import oracle
import wqd_inputs as I

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "spec_sampling_page_example.txt")


def golden():
    g = {}
    for line in open(GOLDEN):
        if line.startswith("#") or not line.strip():
            continue
        key, vals, tol, _src = line.split()
        g[key] = (np.array([float(v) for v in vals.split(",")]), float(tol))
    return g


def midpoints(n):
    return ((np.arange(n) + 0.5) / n).astype(np.float32)


def accept_prob(d_x, t_x, n=12000):
    return np.mean([oracle.accept(u, d_x, t_x) for u in midpoints(n)])


def draw_freq(w, V, n=12000):
    units = oracle.draw_units(w)
    f = np.zeros(V)
    for v in midpoints(n):
        f[oracle.inverse_cdf_draw(units, v)] += 1
    return f / n


def test_page_example_three_tokens():
    g = golden()
    t, d = g["target"][0].astype(np.float32), g["draft"][0].astype(np.float32)
    # (a) acceptance per step: sum over draft tokens x of d(x) P(keep | x)
    pa = sum(float(d[x]) * accept_prob(d[x], t[x]) for x in range(3))
    assert abs(pa - g["accept_prob"][0][0]) <= 1e-4
    # (b) the residual distribution
    res = draw_freq(np.maximum(t - d, np.float32(0)), 3)
    assert np.allclose(res, g["residual"][0], atol=1e-4)
    # (c) the whole step on a product grid of (u, v), one draft position, each
    # draft token weighted by its draft probability: the output is the target
    n = 120  # 1/3 and 3/4 fall between midpoints, so the grid is exact
    out = np.zeros(3)
    for x in range(3):
        for u in midpoints(n):
            for v in midpoints(n):
                nk, toks = oracle.spec_accept_one(np.stack([t, t]), d[None], [x], [u], v)
                out[toks[0]] += float(d[x]) / (n * n)
    assert np.allclose(out, g["output"][0], atol=1e-6)


def test_page_example_two_tokens():
    g = golden()
    t = g["two_token_target"][0].astype(np.float32)
    d = g["two_token_draft"][0].astype(np.float32)
    assert d[0] > t[0]  # the draft overestimates A
    assert np.allclose(draw_freq(np.maximum(t - d, np.float32(0)), 2), g["two_token_residual"][0], atol=1e-6)


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_output_is_distributed_as_target(seed):
    """Leviathan / Chen: keep-or-resample yields an exact sample of the target."""
    rng = np.random.default_rng(seed)
    V = 5
    t = rng.dirichlet(np.ones(V)).astype(np.float32)
    d = rng.dirichlet(np.ones(V)).astype(np.float32)
    res = draw_freq(np.maximum(t - d, np.float32(0)), V, n=20000)
    out = np.zeros(V)
    for x in range(V):
        pk = accept_prob(d[x], t[x], n=20000)
        out[x] += float(d[x]) * pk
        out += float(d[x]) * (1.0 - pk) * res
    assert np.allclose(out, t, atol=3e-4), (out, t)
    # the acceptance rate is sum(min(d, t))
    pa = sum(float(d[x]) * accept_prob(d[x], t[x], n=20000) for x in range(V))
    assert abs(pa - float(np.minimum(d, t).sum())) <= 2e-4


def test_inverse_cdf_against_a_walk():
    rng = np.random.default_rng(7)
    for _ in range(300):
        V = int(rng.integers(1, 12))
        units = rng.integers(0, 50, size=V) * (rng.random(V) < 0.7)
        vs = list(I.uniform_f32(rng, (5,))) + [np.float32(0.0), np.float32(1 - 2.0 ** -24)]
        for v in vs:
            T = int(units.sum())
            if T == 0:
                assert oracle.inverse_cdf_draw(units, v) == -1
                continue
            U = int(np.floor(float(v) * T))  # exact here: T is small
            acc, j = 0, -1
            for i in range(V):
                acc += int(units[i])
                if acc > U:
                    j = i
                    break
            got = oracle.inverse_cdf_draw(units, v)
            assert got == j and units[got] > 0, (units, v, got, j)


def test_draw_at_the_ends_of_the_uniform_range():
    # u = 1 (a generator whose range is (0, 1]) and anything above it draws the
    # last token of positive weight; NaN or a negative u draws like u = 0
    units = np.array([0, 3, 0, 5, 2, 0, 0], dtype=np.int64)
    for v in (1.0, 1.5, np.inf):
        assert oracle.inverse_cdf_draw(units, v) == 4
    for v in (np.nan, -0.25, 0.0):
        assert oracle.inverse_cdf_draw(units, v) == 1
    assert oracle.inverse_cdf_draw(units, 1 - 2.0 ** -24) == 4
    assert oracle.inverse_cdf_draw(np.zeros(5, np.int64), 1.0) == -1


def test_malformed_weights_count_as_clamped():
    w = np.array([np.nan, -0.5, 2.0, 0.25], dtype=np.float32)
    assert oracle.draw_units(w).tolist() == [0, 0, 1 << 32, 1 << 30]


def test_draw_units_exact():
    w = np.array([0.0, 2.0 ** -32, 2.0 ** -33, 0.5, 1.0, 0.1], dtype=np.float32)
    units = oracle.draw_units(w)
    assert units.tolist()[:5] == [0, 1, 0, 1 << 31, 1 << 32]
    assert units[5] == int(np.floor(float(np.float32(0.1)) * 2.0 ** 32))


def test_special_cases():
    V, k = 16, 3
    t, d, x, u, v = I.spec_inputs(11, 1, k, V)
    t, d, x, u, v = t[0], d[0], x[0], u[0], v[0]
    # draft equal to target: every draft kept (u < 1), then the bonus from t_k
    n, out = oracle.spec_accept_one(t, t[:k], x, u, v)
    assert n == k and out[:k].tolist() == x.tolist()
    assert out[k] == oracle.inverse_cdf_draw(oracle.draw_units(t[k]), v)
    # a draft token the target never emits is rejected there; later drafts dropped
    t2 = t.copy(); d2 = d.copy()
    d2[0] = t2[0]                       # position 0 kept
    t2[1, x[1]] = 0.0                   # position 1 rejected
    n, out = oracle.spec_accept_one(t2, d2, x, u, v)
    assert n == 1 and out[0] == x[0] and out[2:].tolist() == [-1] * (k - 1)
    assert out[1] != x[1] and t2[1, out[1]] > d2[1, out[1]]
    # no mass under either distribution and equal elsewhere: the residual is
    # empty, the draw falls back to the target row
    t3 = t.copy(); d3 = d.copy()
    t3[0, x[0]] = 0.0
    d3[0] = t3[0]
    n, out = oracle.spec_accept_one(t3, d3, x, u, v)
    assert n == 0 and out[0] == oracle.inverse_cdf_draw(oracle.draw_units(t3[0]), v)
    # out-of-range draft token: rejected
    n, out = oracle.spec_accept_one(t, t[:k], np.array([V, 0, 0]), u, v)
    assert n == 0
    # an all-zero target row (every draft kept): token -1, whatever u
    t4 = t.copy(); t4[k] = 0.0
    for vv in (v, np.float32(1.0)):
        n, out = oracle.spec_accept_one(t4, t4[:k], x, u, vv)
        assert n == k and out[k] == -1
    # k = 0: only the draw from t_0
    n, out = oracle.spec_accept_one(t[:1], np.zeros((0, V), np.float32), [], [], v)
    assert n == 0 and out.tolist() == [oracle.inverse_cdf_draw(oracle.draw_units(t[0]), v)]


def test_pins_catch_planted_mistakes(monkeypatch):
    """Plant plausible mistakes in the oracle's step and check that a pin fails for each."""
    import oracle.spec as S

    real_accept, real_draw, real_units, real_res = S.accept, S.inverse_cdf_draw, S.draw_units, S.residual
    plants = [
        # ratio inverted in the accept test: the page's acceptance 0.6 fails
        ("accept", lambda u, d_x, t_x: bool(np.float32(u) * np.float32(t_x) < np.float32(d_x)), test_page_example_three_tokens),
        # residual with the operands swapped: the output is no longer the target
        ("residual", lambda t_row, d_row: real_res(d_row, t_row), test_page_example_three_tokens),
        # inverse CDF one token early (first prefix sum >= the threshold)
        ("inverse_cdf_draw", lambda units, v: int(np.searchsorted(np.cumsum(np.asarray(units, np.int64)),
                                                                  int(np.floor(float(np.float32(v)) * int(np.sum(units)))), side="left")),
         test_inverse_cdf_against_a_walk),
        # units rounded up instead of down
        ("draw_units", lambda w: np.ceil(np.asarray(w, np.float32).astype(np.float64) * S.UNIT).astype(np.int64), test_draw_units_exact),
    ]
    for name, bad, pin in plants:
        monkeypatch.setattr(S, name, bad)
        monkeypatch.setattr(oracle, name, bad)
        with pytest.raises(AssertionError):
            pin()
        monkeypatch.undo()
    assert (S.accept, S.inverse_cdf_draw, S.draw_units, S.residual) == (real_accept, real_draw, real_units, real_res)
