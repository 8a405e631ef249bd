"""Plain float64 attention gradients: the chain rule through the definition
(TEST INFRASTRUCTURE).

Source of what is differentiated: the standard-attention definition of
"Flash Attention: Revolutionizing Transformer Efficiency" (unite.ai), the same
function ``exact.attention_head`` computes (scores, row softmax over visible
keys, product with V). That page's "Enter Flash Attention" list (point 2,
recomputation) says the backward pass recomputes the parts of the attention
matrix it needs instead of storing it; its FlashAttention-2 section (point 2)
says the backward pass was brought close to the forward in speed. The pages
give no backward formulas, so this module writes out the gradient of the
forward definition for an upstream gradient dO of O (the loss is
sum(dO * O)):

    S  = scale * Q K^T,  P = softmax over visible keys (0 where hidden),
    O  = P V
    dV = P^T dO
    dP = dO V^T
    D  = rowsum(dO * O)              (= rowsum(P * dP))
    dS = P * (dP - D)                (softmax Jacobian applied row by row)
    dQ = scale * dS K
    dK = scale * dS^T Q

Grouped-query heads: a kv-head's dK and dV sum the contributions of every
q-head that reads it. A row with no visible key has P = 0 and contributes
nothing. Everything is float64 and materialises the score matrix.

Pinned in ``tests/oracle_pins.py`` by central finite differences of the
forward oracle, by closed forms (equal V rows give dQ = dK = 0; a causal
first row gives dQ = 0) and by invariants (column sums of dV equal the
column sums of dO; dS rows sum to zero).

This module is test infrastructure. Only tests, the smoke check and the CPU
baseline of the benchmark may use it.
"""
from __future__ import annotations

import numpy as np

from .exact import _kv_head, as_fp32_scale, scores, softmax_rows, visibility


def attention_head_bwd(q, k, v, do, scale, causal=False):
    """One head: q [Nq,d], k/v [Nk,d], do [Nq,d] -> (dQ, dK, dV) in float64."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    do = np.asarray(do, np.float64)
    s = as_fp32_scale(scale)
    P, _, _ = softmax_rows(scores(q, k, scale), visibility(q.shape[0], k.shape[0], causal))
    O = P @ v
    dV = P.T @ do
    dP = do @ v.T
    D = np.sum(do * O, axis=1)
    dS = P * (dP - D[:, None])
    dQ = s * (dS @ k)
    dK = s * (dS.T @ q)
    return dQ, dK, dV


def attention_bwd(q, k, v, do, scale, causal=False):
    """q, do [B,Hq,Nq,d], k/v [B,Hkv,Nk,d] (float64) -> dQ [B,Hq,Nq,d],
    dK, dV [B,Hkv,Nk,d]."""
    B, Hq, Nq, d = q.shape
    Hkv = k.shape[1]
    dQ = np.zeros(q.shape, np.float64)
    dK = np.zeros(k.shape, np.float64)
    dV = np.zeros(v.shape, np.float64)
    for b in range(B):
        for h in range(Hq):
            g = _kv_head(h, Hq, Hkv)
            gq, gk, gv = attention_head_bwd(q[b, h], k[b, g], v[b, g], do[b, h], scale, causal)
            dQ[b, h] = gq
            dK[b, g] += gk
            dV[b, g] += gv
    return dQ, dK, dV
