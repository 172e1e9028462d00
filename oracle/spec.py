"""Speculative-sampling accept / reject step over the verify pass's distributions.

Test infrastructure only (see ``oracle/__init__.py``).

What it computes (CS336 lecture 10 notes, section 6.1, the four steps of
speculative sampling, and section 6.2, why the output is an exact sample of the
target; "Making each token cheaper", section on why the acceptance rule keeps
the target distribution).  Per sequence, with the target's distributions
t_0 .. t_k over V tokens (the verify pass scores k + 1 positions), the draft's
d_0 .. d_{k-1}, the draft tokens x_0 .. x_{k-1} (drawn from the d_i), and the
uniform numbers in [0, 1) that the method draws (passed in: u_i for the
accept tests, one v for the final draw):

1. left to right, draft token x_i is kept with probability min(1, t_i(x_i) /
   d_i(x_i)), i.e. when u_i < that ratio;
2. at the first rejection, at position i, one token is drawn from the
   residual distribution max(t_i - d_i, 0) / sum(max(t_i - d_i, 0)) and the
   round ends (the later drafts are dropped);
3. if all k drafts are kept, one more token is drawn from t_k.

Readings where the pages leave the arithmetic open:

* the accept test is taken in float32 as ``u * d(x) < t(x)`` (the product form
  of u < min(1, t/d): for d > 0 the two agree in real arithmetic; with
  d(x) = 0 a token is kept iff t(x) > 0).  An out-of-range draft token is
  rejected;
* a draw from non-negative float32 weights w (the residual max(t - d, 0) in
  float32, or t_k itself) counts each weight in units of 2^-32:
  W_j = floor(w_j * 2^32), an exact integer, so the draw does not depend on an
  order of summation.  With T = sum W_j and U = floor(v * T) (the product in
  float64, rounded to nearest), the drawn token is the smallest j whose prefix
  sum W_0 + .. + W_j exceeds U: the inverse of the cumulative distribution.
  Mass below 2^-32 per token is dropped (at most V * 2^-32 in total).  U is
  kept below T: a v of 1 or more (a generator whose range is (0, 1]) draws
  the last token of positive weight, and a NaN or negative v counts as 0.  A
  weight outside [0, 1] counts as the nearest end of that range, a NaN weight
  as 0 (probabilities are in [0, 1]; this only fixes what malformed input
  gives);
* a residual whose units sum to zero (the rejected draft had no mass under
  either distribution, and the two agree everywhere else) draws from t_i
  instead; a row of all-zero target units draws token -1.

Outputs: the number of kept drafts n (0 .. k) and k + 1 tokens: the n kept
drafts, then the drawn token, then -1.
"""
from __future__ import annotations

import numpy as np

UNIT = 2.0 ** 32


def draw_units(w) -> np.ndarray:
    """Integer weights W_j = floor(w_j * 2^32) of float32 weights w >= 0."""
    w = np.asarray(w, dtype=np.float32)
    w = np.clip(np.where(np.isnan(w), np.float32(0), w), 0, 1)
    return np.floor(w.astype(np.float64) * UNIT).astype(np.int64)


def inverse_cdf_draw(units, v) -> int:
    """Smallest j with units[0] + .. + units[j] > floor(v * T); -1 if T = 0."""
    units = np.asarray(units, dtype=np.int64)
    T = int(units.sum())
    if T == 0:
        return -1
    v = np.float32(v)
    p = np.float64(v) if v > 0 else np.float64(0)
    f = np.floor(p * np.float64(T))
    U = T - 1 if f >= T else int(f)
    return int(np.searchsorted(np.cumsum(units), U, side="right"))


def residual(t_row, d_row) -> np.ndarray:
    """max(t - d, 0) in float32: the weights of the draw after a rejection."""
    return np.maximum(np.asarray(t_row, np.float32) - np.asarray(d_row, np.float32), np.float32(0))


def accept(u, d_x, t_x) -> bool:
    """The accept test u < min(1, t/d) in float32 product form."""
    return bool(np.float32(u) * np.float32(d_x) < np.float32(t_x))


def spec_accept_one(target, draft, tokens, u_accept, v):
    """One sequence: target [k+1, V], draft [k, V] float32, tokens [k], u_accept [k], v.

    Returns (n_kept, out[k+1]).
    """
    target = np.asarray(target, dtype=np.float32)
    draft = np.asarray(draft, dtype=np.float32)
    k1, V = target.shape
    k = k1 - 1
    out = np.full(k + 1, -1, dtype=np.int32)
    for i in range(k):
        x = int(tokens[i])
        if 0 <= x < V and accept(u_accept[i], draft[i, x], target[i, x]):
            out[i] = x
            continue
        units = draw_units(residual(target[i], draft[i]))
        if units.sum() == 0:
            units = draw_units(target[i])
        out[i] = inverse_cdf_draw(units, v)
        return i, out
    out[k] = inverse_cdf_draw(draw_units(target[k]), v)
    return k, out


def spec_accept(target, draft, tokens, u_accept, v):
    """Batch of B sequences: target [B, k+1, V], draft [B, k, V], tokens [B, k] int,
    u_accept [B, k], v [B] float32.  Returns (n_kept [B] int32, out [B, k+1] int32)."""
    target = np.asarray(target, dtype=np.float32)
    B, k1, _ = target.shape
    n = np.zeros(B, dtype=np.int32)
    out = np.zeros((B, k1), dtype=np.int32)
    for b in range(B):
        n[b], out[b] = spec_accept_one(target[b], draft[b], tokens[b], u_accept[b], v[b])
    return n, out
