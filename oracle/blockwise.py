"""Attention from block-wise partial softmaxes and the merge identity, in
float64 (TEST INFRASTRUCTURE).

Source: "Flash Attention: Revolutionizing Transformer Efficiency" (unite.ai),
section "The math of Flash Attention": the softmax over the union of two sets
of scores follows from the softmaxes of the parts, each rescaled by the
exponential of its own maximum minus the maximum of the union; section
"Flash Attention algorithm": the scores are taken block by block and never
held whole.

Reading of the merge identity: the page prints the merge wrapped in a second
softmax, which its own code does not do. The plainest reading the rest of the
page supports keeps unnormalised partials. For a set x of scores of one row,
m(x) = max x, f(x) = exp(x - m(x)), l(x) = sum f(x) and acc(x) = f(x) V(x).
For disjoint x and y with m = max(m(x), m(y)):
    l(x u y)   = exp(m(x) - m) l(x)   + exp(m(y) - m) l(y)
    acc(x u y) = exp(m(x) - m) acc(x) + exp(m(y) - m) acc(y)
and the result is O = acc / l, LSE = m + log l. (The FlashAttention-2 form
of the output update, with the division by l deferred to the end.)

Here each (query block, key block) partial is computed on its own and the
partials of a query block are folded pairwise as a balanced tree (adjacent
pairs first), so the identity is pinned for partials of any sizes in any
grouping, not only as a running update. ``merge_partials`` is the same
identity for normalised parts in LSE form (used by the split-key decode).

This module pins the identity against the one-shot definition in
``exact.py``; it is test infrastructure.
"""
from __future__ import annotations

import numpy as np

from .exact import as_fp32_scale


def block_partial(q, k, v, sigma, rows, cols, Nk_minus_Nq, causal):
    """(m, l, acc) of one query block against one key block.

    rows / cols are the absolute query / key indices of the blocks; a key
    is visible to a query iff causal is off or col <= row + (Nk - Nq). Rows
    with no visible key get m = -inf, l = 0, acc = 0."""
    s = sigma * (q @ k.T)
    vis = (cols[None, :] <= rows[:, None] + Nk_minus_Nq) if causal else np.ones_like(s, bool)
    s = np.where(vis, s, -np.inf)
    m = s.max(axis=1) if s.shape[1] else np.full(s.shape[0], -np.inf)
    ref = np.where(np.isfinite(m), m, 0.0)
    f = np.where(vis, np.exp(s - ref[:, None]), 0.0)
    return m, f.sum(axis=1), f @ v


def merge_two(a, b):
    """The merge identity for two unnormalised partials over disjoint keys."""
    (ma, la, acca), (mb, lb, accb) = a, b
    m = np.maximum(ma, mb)
    ref = np.where(np.isfinite(m), m, 0.0)
    wa = np.where(np.isfinite(ma), np.exp(ma - ref), 0.0)
    wb = np.where(np.isfinite(mb), np.exp(mb - ref), 0.0)
    return m, wa * la + wb * lb, wa[:, None] * acca + wb[:, None] * accb


def fold(parts):
    """Merge a list of partials as a balanced tree of adjacent pairs."""
    while len(parts) > 1:
        parts = [merge_two(parts[i], parts[i + 1]) if i + 1 < len(parts) else parts[i]
                 for i in range(0, len(parts), 2)]
    return parts[0]


def blockwise_attention_head(q, k, v, scale, causal=False, block_q=64, block_k=64):
    """One head from block partials merged by the identity; float64 throughout."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    Nq, Nk = q.shape[0], k.shape[0]
    sigma = as_fp32_scale(scale)
    O = np.zeros((Nq, v.shape[1]))
    LSE = np.full(Nq, -np.inf)
    for i0 in range(0, Nq, block_q):
        qi = q[i0:i0 + block_q]
        rows = np.arange(i0, i0 + qi.shape[0])
        parts = [block_partial(qi, k[j0:j0 + block_k], v[j0:j0 + block_k], sigma, rows,
                               np.arange(j0, min(j0 + block_k, Nk)), Nk - Nq, causal)
                 for j0 in range(0, Nk, block_k)]
        if not parts:
            continue
        m, l, acc = fold(parts)
        ok = l > 0
        O[rows] = np.where(ok[:, None], acc / np.where(ok, l, 1.0)[:, None], 0.0)
        with np.errstate(divide="ignore"):
            LSE[rows] = np.where(ok, m + np.log(np.where(ok, l, 1.0)), -np.inf)
    return O, LSE


def merge_partials(O_parts, lse_parts):
    """Merge normalised partial results over disjoint key sets.

    Given O_s (normalised within part s) and LSE_s, the union has
    LSE = log sum_s exp(LSE_s) and O = sum_s exp(LSE_s - LSE) O_s.
    Parts with LSE_s = -inf (no keys) contribute nothing.
    """
    O_parts = [np.asarray(o, np.float64) for o in O_parts]
    lse_parts = np.stack([np.asarray(x, np.float64) for x in lse_parts])
    lse = np.logaddexp.reduce(lse_parts, axis=0)
    out = np.zeros_like(O_parts[0])
    ok = np.isfinite(lse)
    safe = np.where(ok, lse, 0.0)
    for o, ls in zip(O_parts, lse_parts):
        w = np.where(ok & np.isfinite(ls), np.exp(ls - safe), 0.0)
        out = out + w[..., None] * o
    return out, lse
