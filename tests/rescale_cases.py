"""Inputs that drive the reference-point move of the online softmax.

The kernels exponentiate each key tile against the row's current reference
point and move the reference (rescaling the running sum and the output
accumulator by exp2(m_old - m_new), the merge identity of "The math of Flash
Attention", unite.ai) only when a lane's sum of a tile's exponentials leaves
(0, limit]. With i.i.d. N(0,1) inputs that never happens after a row's first
tile, so these builders plant scores that force it:

* ``outlier``: every key scores about 0 (log2 units) except one key, late in
  the row, that scores ``jump`` higher. With ~10^5 flat keys the keys before
  the outlier still carry a large share of the softmax weight after being
  rescaled by 2^-jump, and V is offset by +1 before the outlier and -1 after
  it, so a wrong rescale factor moves the output well past the tolerances.
* ``ramp``: each 32-key block scores ``step`` higher than the previous one,
  so the reference moves at every block.

``jump_rows`` replays the condition on the CPU so a test can assert that its
inputs really cross the limit: a key tile whose best score exceeds the best
score of all earlier keys of the row by more than log2(limit) forces the move
whatever the reference was, since the reference is always at most the best
earlier score.

Test infrastructure: builds inputs only; no attention arithmetic.
"""
from __future__ import annotations

import math

import numpy as np

import attn_inputs as ai

LOG2E = 1.4426950408889634


def c_log2(scale: float) -> float:
    """The factor that takes a raw score q.k to log2 units, as the kernels form it."""
    return float(np.float32(np.float32(scale) * np.float32(LOG2E)))


def _unit(d: int) -> np.ndarray:
    return np.full(d, 1.0 / math.sqrt(d))


def outlier(seed: int, Nq: int, Nk: int, d: int, j_out: int, jump: float, scale: float, H: int = 1,
            a: float = 4.0, noise: float = 0.05):
    """q [H,Nq,d], k/v [H,Nk,d] float32 (before rounding) with key j_out
    scoring about ``jump`` log2 units above the other keys (which score about
    0), V offset +1 before j_out and -1 after it."""
    rng = np.random.default_rng([seed, 11])
    u = _unit(d)
    c = c_log2(scale)
    q = (a * u + noise * rng.standard_normal((H, Nq, d))).astype(np.float32)
    k = (noise * rng.standard_normal((H, Nk, d))).astype(np.float32)
    k[:, j_out] += (jump / (c * a)) * u
    v = rng.standard_normal((H, Nk, d)).astype(np.float32)
    v[:, :j_out] += 1.0
    v[:, j_out + 1:] -= 1.0
    return q, k, v


def ramp(seed: int, Nq: int, Nk: int, d: int, step: float, scale: float, H: int = 1, a: float = 4.0,
         block: int = 32):
    """Each ``block`` keys score ``step`` log2 units above the previous block."""
    rng = np.random.default_rng([seed, 12])
    u = _unit(d)
    c = c_log2(scale)
    q = (a * u + 0.05 * rng.standard_normal((H, Nq, d))).astype(np.float32)
    lev = (np.arange(Nk) // block) * step / (c * a)
    k = (lev[None, :, None] * u + 0.05 * rng.standard_normal((H, Nk, d))).astype(np.float32)
    v = rng.standard_normal((H, Nk, d)).astype(np.float32)
    return q, k, v


def rounded(x: np.ndarray, dtype: str):
    """(bits, float64 values) of x rounded to the 16-bit type."""
    bits = ai.round_to_bits(np.ascontiguousarray(x, np.float32), dtype)
    return bits, ai.bits_to_f64(bits, dtype)


def jump_rows(q64: np.ndarray, k64: np.ndarray, scale: float, tile: int, limit: float,
              causal: bool = False) -> int:
    """Rows (of one head) with a key tile t >= 1 whose best visible score, in
    log2 units, exceeds the best visible score of all earlier keys by more
    than log2(limit)."""
    s = (q64 @ k64.T) * c_log2(scale)
    Nq, Nk = s.shape
    if causal:
        vis = np.arange(Nk)[None, :] <= np.arange(Nq)[:, None] + (Nk - Nq)
        s = np.where(vis, s, -np.inf)
    n_t = (Nk + tile - 1) // tile
    pad = np.full((Nq, n_t * tile - Nk), -np.inf)
    tmax = np.concatenate([s, pad], axis=1).reshape(Nq, n_t, tile).max(axis=2)
    prev = np.maximum.accumulate(tmax, axis=1)[:, :-1]
    return int(np.sum(np.any(tmax[:, 1:] > prev + math.log2(limit), axis=1)))
