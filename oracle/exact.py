"""Plain float64 attention: the definition, written out (TEST INFRASTRUCTURE).

Source: "Flash Attention: Revolutionizing Transformer Efficiency" (unite.ai),
the standard-attention listing that opens the page: scores are Q times K
transposed divided by the square root of the head width, a softmax over the
key axis, then a product with V. The same page, section "The math of Flash
Attention", gives the softmax decomposition used here (subtract the row maximum
before exponentiating); that only guards against overflow and leaves the exact
value unchanged. FlashAttention computes exactly this result, not an
approximation (same page, section "Impact of Flash Attention", point 3).

Readings where the pages are silent (each is listed with its reason in the
design notes of the repository):
  * scale: the caller passes it; the library receives a float32, so the oracle
    uses the float64 value of that float32 (``as_fp32_scale``).
  * causal mask (SDPA page, Example 3, ``is_causal``): bottom-right aligned,
    key j is visible to query i iff j <= i + (Nk - Nq).
  * grouped-query heads (SDPA page, Example 5): q-head h reads kv-head
    h // (Hq // Hkv), i.e. K/V repeated contiguously along the head axis.
  * LSE: natural log of the sum of exp over the visible, scaled scores.
  * a row with no visible key: O = 0 and LSE = -inf.
  * decode (throughput page, "Memory requirements"): the new token of
    sequence b attends, unmasked, to cache rows [0, L_b).
  * packed variable-length prefill (throughput page, "Continuous
    batching"): sequences of different lengths share one slab per head
    without padding; sequence b owns rows cu_q[b]..cu_q[b+1]-1 of queries and
    cu_k[b]..cu_k[b+1]-1 of keys, and attends only to its own keys.
  * paged decode (throughput page, "Paged attention"): the cache of a
    sequence lives in fixed-size pages found through a per-sequence page
    table; logical row j is row j % P of page table[b, j // P]. A page-table
    entry that names no page makes that sequence's output NaN.

This module is test infrastructure. Only tests, the smoke check and the CPU
baseline of the benchmark may use it.
"""
from __future__ import annotations

import numpy as np


def as_fp32_scale(scale: float) -> float:
    """The float64 value of the float32 the C boundary receives."""
    return float(np.float32(scale))


def scores(q: np.ndarray, k: np.ndarray, scale: float) -> np.ndarray:
    """S = scale * Q K^T for one head: q [Nq,d], k [Nk,d] -> [Nq,Nk] float64."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    return as_fp32_scale(scale) * (q @ k.T)


def visibility(Nq: int, Nk: int, causal: bool) -> np.ndarray:
    """Boolean [Nq,Nk]: which keys each query may attend to."""
    if not causal:
        return np.ones((Nq, Nk), dtype=bool)
    i = np.arange(Nq)[:, None]
    j = np.arange(Nk)[None, :]
    return j <= i + (Nk - Nq)


def softmax_rows(S: np.ndarray, vis: np.ndarray):
    """Row softmax over visible entries. Returns (P, m, l).

    m is the row maximum over visible scores, l = sum exp(S - m) over visible
    entries, P = exp(S - m) / l (0 where hidden). Rows with nothing visible get
    m = -inf, l = 0, P = 0.
    """
    Sm = np.where(vis, S, -np.inf)
    m = Sm.max(axis=1) if Sm.shape[1] else np.full(Sm.shape[0], -np.inf)
    finite = np.isfinite(m)
    m_safe = np.where(finite, m, 0.0)
    e = np.where(vis, np.exp(Sm - m_safe[:, None]), 0.0)
    l = e.sum(axis=1)
    with np.errstate(invalid="ignore", divide="ignore"):
        P = np.where(l[:, None] > 0, e / np.where(l > 0, l, 1.0)[:, None], 0.0)
    return P, m, l


def attention_head(q, k, v, scale, causal=False):
    """One head: q [Nq,d], k/v [Nk,d] -> (O [Nq,d], LSE [Nq]) in float64."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    S = scores(q, k, scale)
    P, m, l = softmax_rows(S, visibility(q.shape[0], k.shape[0], causal))
    O = P @ v
    with np.errstate(divide="ignore"):
        lse = np.where(l > 0, m + np.log(np.where(l > 0, l, 1.0)), -np.inf)
    return O, lse


def _kv_head(h: int, Hq: int, Hkv: int) -> int:
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    return h // (Hq // Hkv)


def attention(q, k, v, scale, causal=False):
    """q [B,Hq,Nq,d], k/v [B,Hkv,Nk,d] (float64) -> O [B,Hq,Nq,d], LSE [B,Hq,Nq]."""
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    O = np.zeros((B, Hq, Nq, v.shape[3]), np.float64)
    L = np.zeros((B, Hq, Nq), np.float64)
    for b in range(B):
        for h in range(Hq):
            g = _kv_head(h, Hq, Hkv)
            O[b, h], L[b, h] = attention_head(q[b, h], k[b, g], v[b, g], scale, causal)
    return O, L


def attention_rows(q_rows, rows, k, v, scale, causal, Nq):
    """Selected query rows of one head.

    q_rows [R,d] are the query vectors of rows ``rows`` (absolute indices in a
    query sequence of length Nq); k/v [Nk,d]. Exactly the rows of
    ``attention_head`` over the full sequence, without the other rows.
    """
    q_rows = np.asarray(q_rows, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    rows = np.asarray(rows, np.int64)
    Nk = k.shape[0]
    S = scores(q_rows, k, scale)
    if causal:
        vis = np.arange(Nk)[None, :] <= rows[:, None] + (Nk - Nq)
    else:
        vis = np.ones_like(S, dtype=bool)
    P, m, l = softmax_rows(S, vis)
    with np.errstate(divide="ignore"):
        lse = np.where(l > 0, m + np.log(np.where(l > 0, l, 1.0)), -np.inf)
    return P @ v, lse


def varlen_bounds(cu, b, total):
    """Rows [lo, hi) of sequence b: offsets clamped into [0, total], hi >= lo."""
    lo = min(max(int(cu[b]), 0), total)
    hi = min(max(int(cu[b + 1]), lo), total)
    return lo, hi


def attention_varlen(q, k, v, cu_q, cu_k, scale, causal=False):
    """Packed batch: q [Hq,total_q,d], k/v [Hkv,total_k,d], cu_* [B+1].

    Each sequence is ``attention`` on its own rows and keys; rows that belong
    to no sequence stay 0 (O) and NaN (LSE)."""
    Hq, total_q, d = q.shape
    Hkv, total_k = k.shape[0], k.shape[1]
    O = np.zeros((Hq, total_q, v.shape[2]), np.float64)
    L = np.full((Hq, total_q), np.nan)
    for b in range(len(cu_q) - 1):
        q_lo, q_hi = varlen_bounds(cu_q, b, total_q)
        k_lo, k_hi = varlen_bounds(cu_k, b, total_k)
        if q_hi == q_lo:
            continue
        for h in range(Hq):
            g = _kv_head(h, Hq, Hkv)
            if k_hi == k_lo:
                O[h, q_lo:q_hi] = 0.0
                L[h, q_lo:q_hi] = -np.inf
                continue
            o, lse = attention_head(q[h, q_lo:q_hi], k[g, k_lo:k_hi], v[g, k_lo:k_hi], scale, causal)
            O[h, q_lo:q_hi], L[h, q_lo:q_hi] = o, lse
    return O, L


def decode(q, k_cache, v_cache, seqlens, scale):
    """One new token per sequence against its cache.

    q [B,Hq,d]; caches [B,Hkv,Lcap,d]; seqlens [B] -> O [B,Hq,d], LSE [B,Hq].
    Rows at or beyond L_b are never read (they may hold NaN).
    """
    B, Hq, d = q.shape
    Hkv, Lcap = k_cache.shape[1], k_cache.shape[2]
    O = np.zeros((B, Hq, v_cache.shape[3]), np.float64)
    L = np.full((B, Hq), -np.inf)
    for b in range(B):
        n = int(min(max(int(seqlens[b]), 0), Lcap))
        for h in range(Hq):
            g = _kv_head(h, Hq, Hkv)
            o, lse = attention_head(np.asarray(q[b, h], np.float64)[None, :],
                                    np.asarray(k_cache[b, g, :n], np.float64),
                                    np.asarray(v_cache[b, g, :n], np.float64), scale, False)
            O[b, h], L[b, h] = o[0], lse[0]
    return O, L


def paged_rows(table_row, n, P):
    """Page id and row within the page of logical cache rows 0..n-1."""
    rows = np.arange(n)
    return np.asarray(table_row, np.int64)[rows // P], rows % P


def decode_paged(q, k_pages, v_pages, block_table, seqlens, scale):
    """Decode against a paged cache.

    q [B,Hq,d]; pages [num_pages,Hkv,P,d]; block_table [B,max_pages];
    seqlens [B] (clamped to [0, max_pages*P]). The logical cache rows of each
    sequence are gathered through its page table, then attended to exactly as
    in ``decode``. If a page needed for rows [0, L_b) is outside
    [0, num_pages), O and LSE of sequence b are NaN.
    """
    B, Hq, d = q.shape
    num_pages, Hkv, P, _ = k_pages.shape
    max_pages = block_table.shape[1]
    Lcap = max_pages * P
    O = np.zeros((B, Hq, v_pages.shape[3]), np.float64)
    L = np.full((B, Hq), -np.inf)
    for b in range(B):
        n = int(min(max(int(seqlens[b]), 0), Lcap))
        ids = np.asarray(block_table[b, : (n + P - 1) // P], np.int64)
        if np.any((ids < 0) | (ids >= num_pages)):
            O[b] = np.nan
            L[b] = np.nan
            continue
        pages, within = paged_rows(ids, n, P)
        for h in range(Hq):
            g = _kv_head(h, Hq, Hkv)
            k = np.asarray(k_pages[pages, g, within], np.float64)
            v = np.asarray(v_pages[pages, g, within], np.float64)
            o, lse = attention_head(np.asarray(q[b, h], np.float64)[None, :], k, v, scale, False)
            O[b, h], L[b, h] = o[0], lse[0]
    return O, L
