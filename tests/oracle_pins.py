"""Checks that pin the float64 oracle to facts that do not come from itself.

Each ``pin_*`` function raises AssertionError when the oracle disagrees with a
closed form, an invariant, a pure-Python brute force, a library routine, or a
hand-worked fixture. ``test_oracle_pins.py`` runs them on the real oracle;
``test_oracle_mutations.py`` plants plausible mistakes in the oracle and checks
that at least one pin then fails.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

import oracle
from oracle import exact as oa

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
TOL = 1e-12


def _rng(seed):
    return np.random.default_rng(seed)


def _expr(s: str) -> float:
    return float(eval(s, {"__builtins__": {}}, {"exp": math.exp, "log": math.log}))


def load_golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- brute force
def brute_force(q, k, v, scale, causal):
    """Pure-Python scalar loops, no NumPy arithmetic: q [B,Hq,Nq,d] nested lists."""
    B, Hq, Nq = len(q), len(q[0]), len(q[0][0])
    Hkv, Nk = len(k[0]), len(k[0][0])
    sigma = float(np.float32(scale))
    grp = Hq // Hkv
    O, L = [], []
    for b in range(B):
        Ob, Lb = [], []
        for h in range(Hq):
            g = h // grp
            Oh, Lh = [], []
            for i in range(Nq):
                s = {}
                for j in range(Nk):
                    if causal and j > i + (Nk - Nq):
                        continue
                    acc = 0.0
                    for t in range(len(q[b][h][i])):
                        acc += q[b][h][i][t] * k[b][g][j][t]
                    s[j] = sigma * acc
                if not s:
                    Oh.append([0.0] * len(v[b][g][0]))
                    Lh.append(-math.inf)
                    continue
                m = max(s.values())
                e = {j: math.exp(x - m) for j, x in s.items()}
                l = sum(e.values())
                Oh.append([sum(e[j] * v[b][g][j][c] for j in e) / l for c in range(len(v[b][g][0]))])
                Lh.append(m + math.log(l))
            Ob.append(Oh)
            Lb.append(Lh)
        O.append(Ob)
        L.append(Lb)
    return np.array(O), np.array(L)


def pin_brute_force():
    r = _rng(11)
    cases = [(1, 1, 1, 1, 1, 1), (1, 2, 2, 2, 2, 2), (1, 2, 2, 3, 3, 4), (2, 4, 1, 5, 5, 8),
             (1, 4, 2, 17, 17, 4), (1, 4, 1, 3, 7, 2), (1, 2, 2, 5, 9, 8)]
    for (B, Hq, Hkv, Nq, Nk, d) in cases:
        q = r.standard_normal((B, Hq, Nq, d)) * 1.5
        k = r.standard_normal((B, Hkv, Nk, d))
        v = r.standard_normal((B, Hkv, Nk, d))
        scale = 1.0 / math.sqrt(d)
        for causal in (False, True):
            if causal and Nq > Nk:
                continue
            O, L = oracle.attention(q, k, v, scale, causal)
            Ob, Lb = brute_force(q.tolist(), k.tolist(), v.tolist(), scale, causal)
            assert np.abs(O - Ob).max() <= TOL, (B, Hq, Hkv, Nq, Nk, d, causal)
            assert np.abs(L - Lb).max() <= TOL, (B, Hq, Hkv, Nq, Nk, d, causal)


# ---------------------------------------------------------------- closed forms
def pin_single_key_and_causal_row0():
    r = _rng(12)
    for d in (1, 4, 64):
        q = r.standard_normal((1, d))
        k = r.standard_normal((1, d))
        v = r.standard_normal((1, d))
        O, L = oracle.attention_head(q, k, v, 0.3)
        assert np.array_equal(O[0], v[0])
        s00 = float(np.float32(0.3)) * float(np.dot(q[0], k[0]))
        assert abs(L[0] - s00) <= TOL * max(1.0, abs(s00))
    q = r.standard_normal((9, 8))
    k = r.standard_normal((9, 8))
    v = r.standard_normal((9, 8))
    O, L = oracle.attention_head(q, k, v, 0.25, causal=True)
    assert np.array_equal(O[0], v[0])
    assert abs(L[0] - float(np.float32(0.25)) * float(np.dot(q[0], k[0]))) <= TOL


def pin_two_keys():
    r = _rng(13)
    for d in (1, 3, 16):
        q = r.standard_normal((3, d))
        k = r.standard_normal((2, d))
        v = r.standard_normal((2, d))
        sc = 0.7
        O, L = oracle.attention_head(q, k, v, sc)
        s = float(np.float32(sc)) * (q @ k.T)
        exp_o = v[1][None, :] + (v[0] - v[1])[None, :] / (1.0 + np.exp(s[:, 1] - s[:, 0]))[:, None]
        assert np.abs(O - exp_o).max() <= TOL
        assert np.abs(L - np.logaddexp(s[:, 0], s[:, 1])).max() <= TOL


def pin_golden_fixtures():
    g = load_golden("two_keys_d2.json")
    O, L = oracle.attention_head(np.array(g["q"]), np.array(g["k"]), np.array(g["v"]), g["scale"], g["causal"])
    want_o = np.array([[_expr(x) for x in row] for row in g["expected_o"]])
    want_l = np.array([_expr(x) for x in g["expected_lse"]])
    assert np.abs(O - want_o).max() <= TOL and np.abs(L - want_l).max() <= TOL
    u = load_golden("uniform_q0.json")
    for causal, ko, kl in ((False, "noncausal_o", "noncausal_lse"), (True, "causal_o", "causal_lse")):
        O, L = oracle.attention_head(np.array(u["q"]), np.array(u["k"]), np.array(u["v"]), u["scale"], causal)
        want_o = np.array([[_expr(x) for x in row] for row in u[ko]])
        want_l = np.array([_expr(x) for x in u[kl]])
        assert np.abs(O - want_o).max() <= TOL and np.abs(L - want_l).max() <= TOL


def pin_zero_query():
    r = _rng(14)
    N, d = 33, 8
    k = r.standard_normal((N, d))
    v = r.standard_normal((N, d))
    q = np.zeros((N, d))
    O, L = oracle.attention_head(q, k, v, 0.5)
    assert np.abs(O - v.mean(axis=0)[None, :]).max() <= TOL
    assert np.abs(L - math.log(N)).max() <= TOL
    O, L = oracle.attention_head(q, k, v, 0.5, causal=True)
    prefix = np.cumsum(v, axis=0) / np.arange(1, N + 1)[:, None]
    assert np.abs(O - prefix).max() <= TOL
    assert np.abs(L - np.log(np.arange(1, N + 1))).max() <= TOL


# ---------------------------------------------------------------- invariants
def pin_rows_sum_to_one():
    r = _rng(15)
    S = r.standard_normal((20, 30)) * 4
    for causal in (False, True):
        vis = oa.visibility(20, 30, causal)
        P, m, l = oa.softmax_rows(S, vis)
        assert np.abs(P.sum(axis=1) - 1.0).max() <= TOL
        assert np.all(P[~vis] == 0)
        assert np.all(P[vis] > 0)
    q = r.standard_normal((10, 4))
    k = r.standard_normal((12, 4))
    O, _ = oracle.attention_head(q, k, np.ones((12, 3)), 1.0, causal=True)
    assert np.abs(O - 1.0).max() <= TOL


def pin_merge_identity():
    r = _rng(16)
    N, d = 300, 8
    q = r.standard_normal((N, d))
    k = r.standard_normal((N, d))
    v = r.standard_normal((N, d))
    for causal in (False, True):
        O, L = oracle.attention_head(q, k, v, 0.35, causal)
        for bq, bk in ((1, 1), (7, 7), (64, 64), (256, 256), (N, N), (64, 7), (13, 256)):
            Ob, Lb = oracle.blockwise_attention_head(q, k, v, 0.35, causal, bq, bk)
            assert np.abs(Ob - O).max() <= TOL and np.abs(Lb - L).max() <= TOL, (bq, bk, causal)
    # random split of the keys into chunks, each normalised on its own, then merged
    O, L = oracle.attention_head(q, k, v, 0.35)
    cuts = np.sort(r.choice(np.arange(1, N), size=5, replace=False))
    bounds = [0, *cuts.tolist(), N]
    parts = [oracle.attention_head(q, k[a:b], v[a:b], 0.35) for a, b in zip(bounds[:-1], bounds[1:])]
    Om, Lm = oracle.merge_partials([p[0] for p in parts], [p[1] for p in parts])
    assert np.abs(Om - O).max() <= TOL and np.abs(Lm - L).max() <= TOL
    # an empty part (no keys) contributes nothing
    empty_o, empty_l = np.zeros_like(O), np.full(N, -np.inf)
    Om2, Lm2 = oracle.merge_partials([p[0] for p in parts] + [empty_o], [p[1] for p in parts] + [empty_l])
    assert np.abs(Om2 - O).max() <= TOL and np.abs(Lm2 - L).max() <= TOL


def pin_shift_invariance():
    r = _rng(17)
    q = r.standard_normal((6, 5))
    k = r.standard_normal((9, 5))
    v = r.standard_normal((9, 5))
    u = r.standard_normal(5)
    sc = 0.6
    O, L = oracle.attention_head(q, k, v, sc)
    O2, L2 = oracle.attention_head(q, k + u[None, :], v, sc)
    assert np.abs(O2 - O).max() <= 1e-11
    assert np.abs(L2 - (L + float(np.float32(sc)) * (q @ u))).max() <= 1e-11


def pin_permutation():
    r = _rng(18)
    q = r.standard_normal((7, 4))
    k = r.standard_normal((11, 4))
    v = r.standard_normal((11, 4))
    O, L = oracle.attention_head(q, k, v, 0.9)
    pk = r.permutation(11)
    O2, L2 = oracle.attention_head(q, k[pk], v[pk], 0.9)
    assert np.abs(O2 - O).max() <= TOL and np.abs(L2 - L).max() <= TOL
    pq = r.permutation(7)
    O3, L3 = oracle.attention_head(q[pq], k, v, 0.9)
    assert np.abs(O3 - O[pq]).max() <= TOL and np.abs(L3 - L[pq]).max() <= TOL


def pin_convex_hull():
    r = _rng(19)
    q = r.standard_normal((12, 4)) * 3
    k = r.standard_normal((12, 4))
    v = r.standard_normal((12, 6))
    for causal in (False, True):
        O, _ = oracle.attention_head(q, k, v, 1.0, causal)
        vis = oa.visibility(12, 12, causal)
        for i in range(12):
            lo = v[vis[i]].min(axis=0)
            hi = v[vis[i]].max(axis=0)
            assert np.all(O[i] >= lo - TOL) and np.all(O[i] <= hi + TOL)


def pin_causal_is_prefix():
    r = _rng(20)
    Nq, Nk, d = 6, 10, 4
    q = r.standard_normal((Nq, d))
    k = r.standard_normal((Nk, d))
    v = r.standard_normal((Nk, d))
    O, L = oracle.attention_head(q, k, v, 0.5, causal=True)
    for i in range(Nq):
        n = i + (Nk - Nq) + 1
        Oi, Li = oracle.attention_head(q[i:i + 1], k[:n], v[:n], 0.5)
        assert np.abs(Oi[0] - O[i]).max() <= TOL and abs(Li[0] - L[i]) <= TOL


def pin_gqa_is_repeated_mha():
    r = _rng(21)
    B, Hq, Hkv, N, d = 2, 8, 2, 9, 4
    q = r.standard_normal((B, Hq, N, d))
    k = r.standard_normal((B, Hkv, N, d))
    v = r.standard_normal((B, Hkv, N, d))
    for causal in (False, True):
        O, L = oracle.attention(q, k, v, 0.5, causal)
        kr = np.repeat(k, Hq // Hkv, axis=1)
        vr = np.repeat(v, Hq // Hkv, axis=1)
        for b in range(B):
            for h in range(Hq):
                Oh, Lh = oracle.attention_head(q[b, h], kr[b, h], vr[b, h], 0.5, causal)
                assert np.abs(Oh - O[b, h]).max() <= TOL and np.abs(Lh - L[b, h]).max() <= TOL


def pin_decode_is_single_query():
    r = _rng(22)
    B, Hq, Hkv, Lcap, d = 3, 4, 2, 20, 8
    lens = np.array([1, 13, 20])
    q = r.standard_normal((B, Hq, d))
    kc = r.standard_normal((B, Hkv, Lcap, d))
    vc = r.standard_normal((B, Hkv, Lcap, d))
    for b in range(B):
        kc[b, :, lens[b]:] = np.nan
        vc[b, :, lens[b]:] = np.nan
    O, L = oracle.decode(q, kc, vc, lens, 0.4)
    assert np.all(np.isfinite(O)) and np.all(np.isfinite(L))
    for b in range(B):
        for h in range(Hq):
            g = h // (Hq // Hkv)
            Oh, Lh = brute_force([[[q[b, h].tolist()]]], [[kc[b, g, :lens[b]].tolist()]],
                                 [[vc[b, g, :lens[b]].tolist()]], 0.4, False)
            assert np.abs(Oh[0, 0, 0] - O[b, h]).max() <= TOL and abs(Lh[0, 0, 0] - L[b, h]) <= TOL
    # an empty sequence yields zeros and -inf
    O0, L0 = oracle.decode(q[:1], kc[:1], vc[:1], np.array([0]), 0.4)
    assert np.all(O0 == 0) and np.all(np.isneginf(L0))


def pin_lse_library():
    r = _rng(23)
    q = r.standard_normal((8, 4)) * 2
    k = r.standard_normal((8, 4)) * 2
    v = r.standard_normal((8, 4))
    for causal in (False, True):
        _, L = oracle.attention_head(q, k, v, 0.8, causal)
        s = float(np.float32(0.8)) * (q @ k.T)
        vis = oa.visibility(8, 8, causal)
        for i in range(8):
            assert abs(L[i] - np.logaddexp.reduce(s[i][vis[i]])) <= TOL


def pin_sampled_rows_match_full():
    r = _rng(24)
    N, d = 40, 8
    q = r.standard_normal((N, d))
    k = r.standard_normal((N, d))
    v = r.standard_normal((N, d))
    rows = np.array([0, 3, 17, 39])
    for causal in (False, True):
        O, L = oracle.attention_head(q, k, v, 0.5, causal)
        Os, Ls = oracle.attention_rows(q[rows], rows, k, v, 0.5, causal, N)
        assert np.abs(Os - O[rows]).max() <= TOL and np.abs(Ls - L[rows]).max() <= TOL


def pin_paged_decode_is_decode():
    # Scatter a cache into pages by hand, in a shuffled page order; following
    # the page table must give back exactly the contiguous-cache decode.
    r = _rng(25)
    B, Hq, Hkv, P, max_pages, d = 3, 4, 2, 4, 5, 8
    Lcap = P * max_pages
    lens = np.array([1, 9, 20])
    q = r.standard_normal((B, Hq, d))
    kc = r.standard_normal((B, Hkv, Lcap, d))
    vc = r.standard_normal((B, Hkv, Lcap, d))
    for b in range(B):
        kc[b, :, lens[b]:] = np.nan
        vc[b, :, lens[b]:] = np.nan
    num_pages = B * max_pages + 2
    order = r.permutation(num_pages)
    table = np.zeros((B, max_pages), np.int64)
    kp = np.full((num_pages, Hkv, P, d), np.nan)
    vp = np.full((num_pages, Hkv, P, d), np.nan)
    for b in range(B):
        for j in range(max_pages):
            pid = order[b * max_pages + j]
            table[b, j] = pid
            for g in range(Hkv):
                for t in range(P):
                    kp[pid, g, t] = kc[b, g, j * P + t]
                    vp[pid, g, t] = vc[b, g, j * P + t]
    O, L = oracle.decode(q, kc, vc, lens, 0.3)
    Op, Lp = oracle.decode_paged(q, kp, vp, table, lens, 0.3)
    assert np.array_equal(O, Op) and np.array_equal(L, Lp)
    # entries past the pages a sequence needs are never followed
    t2 = table.copy()
    t2[0, 1:] = -5
    t2[1, 3:] = num_pages + 7
    Op2, Lp2 = oracle.decode_paged(q, kp, vp, t2, lens, 0.3)
    assert np.array_equal(O, Op2) and np.array_equal(L, Lp2)
    # a needed entry that names no page poisons that sequence only
    t3 = table.copy()
    t3[2, 4] = num_pages
    Op3, Lp3 = oracle.decode_paged(q, kp, vp, t3, lens, 0.3)
    assert np.all(np.isnan(Op3[2])) and np.all(np.isnan(Lp3[2]))
    assert np.array_equal(Op3[:2], O[:2]) and np.array_equal(Lp3[:2], L[:2])


def pin_varlen_is_per_sequence():
    # A packed batch is each sequence's own attention (checked against the
    # brute force), with no key shared across sequences.
    r = _rng(26)
    Hq, Hkv, d = 4, 2, 6
    nq = [3, 0, 5, 2, 4]
    nk = [4, 3, 5, 0, 2]          # sequence 4: causal with Nq > Nk leaves rows that see nothing
    cu_q = np.concatenate([[0], np.cumsum(nq)])
    cu_k = np.concatenate([[0], np.cumsum(nk)])
    tq, tk = int(cu_q[-1]) + 2, int(cu_k[-1])   # two trailing rows belong to no sequence
    q = r.standard_normal((Hq, tq, d))
    k = r.standard_normal((Hkv, tk, d))
    v = r.standard_normal((Hkv, tk, d))
    for causal in (False, True):
        O, L = oracle.attention_varlen(q, k, v, cu_q, cu_k, 0.45, causal)
        for b in range(len(nq)):
            for h in range(Hq):
                g = h // (Hq // Hkv)
                rows = slice(cu_q[b], cu_q[b + 1])
                if nk[b] == 0:
                    assert np.all(O[h, rows] == 0) and np.all(np.isneginf(L[h, rows]))
                    continue
                for i in range(nq[b]):
                    vis = [j for j in range(nk[b]) if not causal or j <= i + nk[b] - nq[b]]
                    if not vis:
                        assert np.all(O[h, cu_q[b] + i] == 0) and np.isneginf(L[h, cu_q[b] + i])
                        continue
                    kk = [k[g, cu_k[b] + j].tolist() for j in vis]
                    vv = [v[g, cu_k[b] + j].tolist() for j in vis]
                    Ob, Lb = brute_force([[[q[h, cu_q[b] + i].tolist()]]], [[kk]], [[vv]], 0.45, False)
                    assert np.abs(Ob[0, 0, 0] - O[h, cu_q[b] + i]).max() <= TOL
                    assert abs(Lb[0, 0, 0] - L[h, cu_q[b] + i]) <= TOL
        assert np.all(O[:, -2:] == 0) and np.all(np.isnan(L[:, -2:]))
    # changing another sequence's keys leaves sequence 2 alone
    k2 = k.copy()
    k2[:, cu_k[0]:cu_k[1]] += 3.0
    O2, L2 = oracle.attention_varlen(q, k2, v, cu_q, cu_k, 0.45, True)
    O1, L1 = oracle.attention_varlen(q, k, v, cu_q, cu_k, 0.45, True)
    sl = slice(cu_q[2], cu_q[3])
    assert np.array_equal(O2[:, sl], O1[:, sl]) and np.array_equal(L2[:, sl], L1[:, sl])
    # offsets outside [0, total] are clamped: [-2, 3) reads rows [0, 3)
    Oc, Lc = oracle.attention_varlen(q, k, v, [-2, 3, 1000], [-7, 4, 1000], 0.45, False)
    Od, Ld = oracle.attention_varlen(q, k, v, [0, 3, tq], [0, 4, tk], 0.45, False)
    assert np.array_equal(Oc, Od) and np.array_equal(Lc, Ld) and np.all(np.isfinite(Lc))


# ---------------------------------------------------------------- backward
def _loss_grad_fd(q, k, v, do, scale, causal, eps=1e-6):
    """Central finite differences of L = sum(dO * O) through the forward oracle,
    for each element of q, k and v in turn."""
    def loss(args):
        O, _ = oracle.attention(*args, scale, causal)
        return float(np.sum(do * O))
    grads = []
    for which in range(3):
        base = [q, k, v]
        t = base[which]
        g = np.zeros_like(t)
        for idx in np.ndindex(t.shape):
            tp, tm = t.copy(), t.copy()
            tp[idx] += eps
            tm[idx] -= eps
            g[idx] = (loss([tp if i == which else base[i] for i in range(3)])
                      - loss([tm if i == which else base[i] for i in range(3)])) / (2 * eps)
        grads.append(g)
    return grads


def pin_bwd_finite_differences():
    """The backward oracle is the derivative of the forward oracle: central
    differences of sum(dO * O) on tiny GQA inputs, causal (with Nq < Nk) and
    not."""
    r = _rng(61)
    for causal, (Nq, Nk) in ((False, (5, 7)), (True, (5, 7)), (True, (6, 6))):
        q = r.standard_normal((1, 2, Nq, 4))
        k = r.standard_normal((1, 1, Nk, 4))
        v = r.standard_normal((1, 1, Nk, 4))
        do = r.standard_normal((1, 2, Nq, 4))
        dq, dk, dv = oracle.attention_bwd(q, k, v, do, 0.7, causal)
        fq, fk, fv = _loss_grad_fd(q, k, v, do, 0.7, causal)
        for a, b in ((dq, fq), (dk, fk), (dv, fv)):
            assert a.shape == b.shape
            assert np.max(np.abs(a - b)) < 1e-7 * max(1.0, np.max(np.abs(b))), np.max(np.abs(a - b))


def pin_bwd_equal_value_rows():
    """If every V row is the same vector, O does not depend on the scores, so
    dQ = dK = 0 exactly (up to rounding), and dV_j = sum_i P_ij dO_i."""
    r = _rng(62)
    q = r.standard_normal((1, 2, 9, 8))
    k = r.standard_normal((1, 2, 11, 8))
    v = np.broadcast_to(r.standard_normal(8), (1, 2, 11, 8)).copy()
    do = r.standard_normal((1, 2, 9, 8))
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, 0.4, True)
    assert np.max(np.abs(dq)) < 1e-12 and np.max(np.abs(dk)) < 1e-12
    # dV sums over queries: column sums equal those of dO
    assert np.allclose(dv.sum(axis=2), do.sum(axis=2), atol=1e-12)


def pin_bwd_dv_column_sums_and_causal_row0():
    """Rows of P sum to one, so the key-sum of dV equals the query-sum of dO;
    a causal first row (Nq = Nk) sees only key 0, so its dQ is zero; the last
    key is seen only by the last row, so its dV is that row's dO weighted by
    the row's softmax weight on it (a direct softmax of one score row)."""
    r = _rng(63)
    B, Hq, Hkv, N, d, sc = 2, 4, 2, 12, 8, 0.3
    q = r.standard_normal((B, Hq, N, d))
    k = r.standard_normal((B, Hkv, N, d))
    v = r.standard_normal((B, Hkv, N, d))
    do = r.standard_normal((B, Hq, N, d))
    grp = Hq // Hkv
    for causal in (False, True):
        dq, dk, dv = oracle.attention_bwd(q, k, v, do, sc, causal)
        assert np.allclose(dv.sum(axis=2), do.reshape(B, Hkv, grp, N, d).sum(axis=(2, 3)), atol=1e-12)
    assert np.max(np.abs(dq[:, :, 0])) < 1e-14
    sigma = float(np.float32(sc))
    for b in range(B):
        for g in range(Hkv):
            want = np.zeros(d)
            for h in range(g * grp, (g + 1) * grp):
                row = [sigma * sum(q[b, h, -1, t] * k[b, g, j, t] for t in range(d)) for j in range(N)]
                mx = max(row)
                w = [math.exp(x - mx) for x in row]
                want += (w[-1] / sum(w)) * do[b, h, -1]
            assert np.allclose(dv[b, g, -1], want, atol=1e-12)


def pin_bwd_gqa_is_repeated_mha():
    """Grouped heads: a kv-head's dK and dV are the sums over its q-heads of
    the gradients with K and V repeated per q-head."""
    r = _rng(64)
    q = r.standard_normal((1, 6, 7, 8))
    k = r.standard_normal((1, 2, 9, 8))
    v = r.standard_normal((1, 2, 9, 8))
    do = r.standard_normal((1, 6, 7, 8))
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, 0.5, True)
    kr, vr = np.repeat(k, 3, axis=1), np.repeat(v, 3, axis=1)
    dq2, dk2, dv2 = oracle.attention_bwd(q, kr, vr, do, 0.5, True)
    assert np.allclose(dq, dq2, atol=1e-13)
    assert np.allclose(dk, dk2.reshape(1, 2, 3, 9, 8).sum(axis=2), atol=1e-13)
    assert np.allclose(dv, dv2.reshape(1, 2, 3, 9, 8).sum(axis=2), atol=1e-13)


ALL_PINS = [
    pin_brute_force, pin_single_key_and_causal_row0, pin_two_keys, pin_golden_fixtures,
    pin_zero_query, pin_rows_sum_to_one, pin_merge_identity, pin_shift_invariance,
    pin_permutation, pin_convex_hull, pin_causal_is_prefix, pin_gqa_is_repeated_mha,
    pin_decode_is_single_query, pin_lse_library, pin_sampled_rows_match_full,
    pin_paged_decode_is_decode, pin_varlen_is_per_sequence, pin_bwd_finite_differences,
    pin_bwd_equal_value_rows, pin_bwd_dv_column_sums_and_causal_row0, pin_bwd_gqa_is_repeated_mha,
]
