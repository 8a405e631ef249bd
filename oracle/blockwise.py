"""The block-by-block softmax of FlashAttention, in float64 (TEST INFRASTRUCTURE).

Source: "Flash Attention: Revolutionizing Transformer Efficiency" (unite.ai),
sections "The math of Flash Attention" (softmax decomposition and the merge of
two partial softmaxes) and "Implementation details" (an outer loop over query
blocks, an inner loop over key/value blocks, running row maximum M and running
sum L).

Reading of the merge identity: the page's printed merge wraps the rescaled
partial results in a second softmax, which is not what its own loop does. The
plainest reading that the loop supports: keep the unnormalised partial
f(x) = exp(x - m_x) with l(x) = sum f(x); for two parts with m = max(m_x, m_y),
f(x u y) is the concatenation of exp(m_x - m) f(x) and exp(m_y - m) f(y), and
l(x u y) = exp(m_x - m) l(x) + exp(m_y - m) l(y).

Reading of the output update: the page's loop multiplies the already
normalised output by the rescale factor alone and divides by the new sum, which
is wrong as soon as a row spans more than one key block. The reading used here
keeps the unnormalised accumulator acc = alpha * acc + P V and divides by l once
after the last block (the deferred normalisation of FlashAttention-2).

This module exists to pin the identity against the one-shot definition in
``attention.py``; it is test infrastructure.
"""
from __future__ import annotations

import numpy as np

from .exact import as_fp32_scale


def blockwise_attention_head(q, k, v, scale, causal=False, block_q=64, block_k=64):
    """Tiled attention for one head with running (m, l, acc); float64 throughout."""
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
        m = np.full(qi.shape[0], -np.inf)
        l = np.zeros(qi.shape[0])
        acc = np.zeros((qi.shape[0], v.shape[1]))
        for j0 in range(0, Nk, block_k):
            kj, vj = k[j0:j0 + block_k], v[j0:j0 + block_k]
            s = sigma * (qi @ kj.T)
            cols = np.arange(j0, j0 + kj.shape[0])
            vis = (cols[None, :] <= rows[:, None] + (Nk - Nq)) if causal else np.ones_like(s, bool)
            s = np.where(vis, s, -np.inf)
            m_new = np.maximum(m, s.max(axis=1))
            ref = np.where(np.isfinite(m_new), m_new, 0.0)  # nothing visible yet: keep zeros
            alpha = np.exp(m - ref)
            p = np.where(vis, np.exp(s - ref[:, None]), 0.0)
            l = alpha * l + p.sum(axis=1)
            acc = alpha[:, None] * acc + p @ vj
            m = m_new
        ok = l > 0
        O[i0:i0 + qi.shape[0]] = np.where(ok[:, None], acc / np.where(ok, l, 1.0)[:, None], 0.0)
        with np.errstate(divide="ignore"):
            LSE[i0:i0 + qi.shape[0]] = np.where(ok, m + np.log(np.where(ok, l, 1.0)), -np.inf)
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
