"""Plant plausible mistakes in the oracle (on the CPU) and check a pin catches each.

A pin set that lets a dropped term, a wrong sign or index, or a transposed
operand through would not be pinning anything; every mutation below must make
at least one pin in ``oracle_pins`` fail.
"""
import numpy as np
import pytest

import oracle
from oracle import blockwise as ob
from oracle import exact as oe
from oracle_pins import ALL_PINS


def _some_pin_fails():
    for pin in ALL_PINS:
        try:
            pin()
        except Exception:  # AssertionError, or a shape error from a transposed operand
            return pin.__name__
    return None


def _scores_no_scale(q, k, scale):
    return np.asarray(q, np.float64) @ np.asarray(k, np.float64).T


def _scores_transposed(q, k, scale):
    return oe.as_fp32_scale(scale) * (np.asarray(k, np.float64) @ np.asarray(q, np.float64).T)


def _scores_wrong_sign(q, k, scale):
    return -oe.as_fp32_scale(scale) * (np.asarray(q, np.float64) @ np.asarray(k, np.float64).T)


def _vis_strict(Nq, Nk, causal):
    if not causal:
        return np.ones((Nq, Nk), bool)
    return np.arange(Nk)[None, :] < np.arange(Nq)[:, None] + (Nk - Nq)


def _vis_top_left(Nq, Nk, causal):
    if not causal:
        return np.ones((Nq, Nk), bool)
    return np.arange(Nk)[None, :] <= np.arange(Nq)[:, None]


_real_softmax = oe.softmax_rows


def _softmax_wrong_axis(S, vis):
    Sm = np.where(vis, S, -np.inf)
    m = Sm.max(axis=1)
    e = np.where(vis, np.exp(Sm - m[:, None]), 0.0)
    l = e.sum(axis=1)
    return e / e.sum(axis=0, keepdims=True).clip(1e-300), m, l


def _softmax_m_dropped_from_lse(S, vis):
    P, m, l = _real_softmax(S, vis)
    return P, np.zeros_like(m), l


def _softmax_unmasked_sum(S, vis):
    P, m, l = _real_softmax(S, vis)
    e = np.exp(np.where(np.isfinite(S), S, 0) - np.where(np.isfinite(m), m, 0)[:, None])
    l2 = e.sum(axis=1)
    return P * (l / l2)[:, None], m, l2


def _kv_head_modulo(h, Hq, Hkv):
    return h % Hkv


def _merge_unnormalised(O_parts, lse_parts):
    lse = np.logaddexp.reduce(np.stack(lse_parts), axis=0)
    out = sum(np.exp(ls)[..., None] * o for o, ls in zip(O_parts, lse_parts))
    return out, lse


_real_blockwise = ob.blockwise_attention_head


def _blockwise_no_rescale(q, k, v, scale, causal=False, block_q=64, block_k=64):
    """The output update without the running-sum factor: normalise every block."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    Nq, Nk = q.shape[0], k.shape[0]
    sig = oe.as_fp32_scale(scale)
    O = np.zeros((Nq, v.shape[1]))
    LSE = np.zeros(Nq)
    for i0 in range(0, Nq, block_q):
        qi = q[i0:i0 + block_q]
        rows = np.arange(i0, i0 + qi.shape[0])
        m = np.full(len(qi), -np.inf)
        l = np.zeros(len(qi))
        o = np.zeros((len(qi), v.shape[1]))
        for j0 in range(0, Nk, block_k):
            s = sig * (qi @ k[j0:j0 + block_k].T)
            cols = np.arange(j0, j0 + s.shape[1])
            vis = (cols[None, :] <= rows[:, None] + (Nk - Nq)) if causal else np.ones_like(s, bool)
            s = np.where(vis, s, -np.inf)
            m_new = np.maximum(m, s.max(axis=1))
            ref = np.where(np.isfinite(m_new), m_new, 0.0)
            a = np.exp(m - ref)
            p = np.where(vis, np.exp(s - ref[:, None]), 0.0)
            l_new = a * l + p.sum(axis=1)
            o = (a[:, None] * o + p @ v[j0:j0 + block_k]) / np.where(l_new > 0, l_new, 1)[:, None]
            l, m = l_new, m_new
        O[i0:i0 + len(qi)] = o
        LSE[i0:i0 + len(qi)] = m + np.log(l)
    return O, LSE


_real_decode = oe.decode


def _decode_whole_cache(q, k_cache, v_cache, seqlens, scale):
    return _real_decode(q, k_cache, v_cache, np.full_like(np.asarray(seqlens), k_cache.shape[2]), scale)


def _decode_off_by_one(q, k_cache, v_cache, seqlens, scale):
    return _real_decode(q, k_cache, v_cache, np.maximum(np.asarray(seqlens) - 1, 0), scale)


def _paged_rows_swapped(table_row, n, P):
    rows = np.arange(n)
    return np.asarray(table_row, np.int64)[rows % P], rows // P


def _paged_rows_ignore_table(table_row, n, P):
    rows = np.arange(n)
    return rows // P, rows % P


def _varlen_bounds_next(cu, b, total):
    lo = min(max(int(cu[b]), 0), total)
    hi = min(max(int(cu[b + 1]) + 1, lo), total)
    return lo, hi


def _varlen_bounds_unclamped(cu, b, total):
    return int(cu[b]), int(cu[b + 1])


def _scale_not_rounded(scale):
    return float(scale)


from oracle import backward as obw  # noqa: E402


def _bwd_variant(mistake):
    """attention_head_bwd with one planted mistake."""
    def f(q, k, v, do, scale, causal=False):
        q, k, v, do = (np.asarray(x, np.float64) for x in (q, k, v, do))
        s = oe.as_fp32_scale(scale)
        P, _, _ = oe.softmax_rows(oe.scores(q, k, scale), oe.visibility(q.shape[0], k.shape[0], causal))
        O = P @ v
        dV = P.T @ do
        dP = do @ v.T
        D = np.sum(do * O, axis=1)
        if mistake == "no_D":
            dS = P * dP
        elif mistake == "D_sign":
            dS = P * (dP + D[:, None])
        else:
            dS = P * (dP - D[:, None])
        dQ = (dS @ k) if mistake == "dq_no_scale" else s * (dS @ k)
        dK = s * (dS.T @ q)
        if mistake == "dk_from_dp":
            dK = s * ((P * dP).T @ q)
        if mistake == "dv_from_o":
            dV = P.T @ (do - O)
        return dQ, dK, dV
    return f


def _bwd_gqa_overwrite(q, k, v, do, scale, causal=False):
    B, Hq = q.shape[:2]
    Hkv = k.shape[1]
    dQ, dK, dV = np.zeros(q.shape), np.zeros(k.shape), np.zeros(v.shape)
    for b in range(B):
        for h in range(Hq):
            g = h // (Hq // Hkv)
            dQ[b, h], dK[b, g], dV[b, g] = obw.attention_head_bwd(q[b, h], k[b, g], v[b, g], do[b, h], scale, causal)
    return dQ, dK, dV


MUTATIONS = [
    ("bwd_no_D", obw, "attention_head_bwd", _bwd_variant("no_D")),
    ("bwd_D_sign", obw, "attention_head_bwd", _bwd_variant("D_sign")),
    ("bwd_dq_no_scale", obw, "attention_head_bwd", _bwd_variant("dq_no_scale")),
    ("bwd_dk_from_dp", obw, "attention_head_bwd", _bwd_variant("dk_from_dp")),
    ("bwd_dv_from_o", obw, "attention_head_bwd", _bwd_variant("dv_from_o")),
    ("bwd_gqa_overwrite", oracle, "attention_bwd", _bwd_gqa_overwrite),
    ("scores_no_scale", oe, "scores", _scores_no_scale),
    ("scores_transposed", oe, "scores", _scores_transposed),
    ("scores_wrong_sign", oe, "scores", _scores_wrong_sign),
    ("causal_strict_less", oe, "visibility", _vis_strict),
    ("causal_top_left", oe, "visibility", _vis_top_left),
    ("softmax_wrong_axis", oe, "softmax_rows", _softmax_wrong_axis),
    ("lse_drops_max", oe, "softmax_rows", _softmax_m_dropped_from_lse),
    ("softmax_sums_hidden", oe, "softmax_rows", _softmax_unmasked_sum),
    ("gqa_modulo_map", oe, "_kv_head", _kv_head_modulo),
    ("merge_unnormalised", oracle, "merge_partials", _merge_unnormalised),
    ("blockwise_no_rescale", oracle, "blockwise_attention_head", _blockwise_no_rescale),
    ("decode_whole_cache", oracle, "decode", _decode_whole_cache),
    ("decode_off_by_one", oracle, "decode", _decode_off_by_one),
    ("scale_not_fp32", oe, "as_fp32_scale", _scale_not_rounded),
    ("paged_rows_swapped", oe, "paged_rows", _paged_rows_swapped),
    ("paged_rows_ignore_table", oe, "paged_rows", _paged_rows_ignore_table),
    ("varlen_bounds_overrun", oe, "varlen_bounds", _varlen_bounds_next),
    ("varlen_bounds_unclamped", oe, "varlen_bounds", _varlen_bounds_unclamped),
]


@pytest.mark.parametrize("name,mod,attr,fn", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_mutation_is_caught(monkeypatch, name, mod, attr, fn):
    monkeypatch.setattr(mod, attr, fn)
    if mod is oe and hasattr(oracle, attr):
        monkeypatch.setattr(oracle, attr, fn)
    caught = _some_pin_fails()
    assert caught is not None, f"no pin catches mutation {name}"


def test_unmutated_oracle_passes_all_pins():
    assert _some_pin_fails() is None
