"""Where the FP8 tolerance comes from (CPU only).

The pages give no accuracy target for FP8 (unite.ai, FlashAttention-3
section: low-precision FP8, "incoherent processing" named but not
described). The FP8 prefill rounds 2^4 P to E4M3 (3 mantissa bits, smallest
subnormal 2^-9) for the second product while the running sum adds the
unrounded P, and moves its reference point only when a lane's sum of 2^4 P
would exceed 448. ``simulate`` applies exactly that rounding to float64
probabilities, tile by tile and lane half by lane half as the kernel holds
them, on the values the 8-bit inputs stand for; the error it leaves against
the oracle is the error the arithmetic itself makes.

Pinned here:
  * on the FP8 parity workloads the simulated error is rel-L2 1.9-2.6e-2
    and max-abs 1.3e-2-6.8e-2 (largest on early causal rows, where few keys
    are averaged); the bar the GPU tests use (rel-L2 5e-2, max-abs 0.1)
    sits above that by 1.9x and 1.5x, so it is not below what the
    arithmetic itself gives (the GPU measures the same 1.9-2.6e-2);
  * the limit of that rounding: a probability below 2^-13 of the reference
    (2^4 P under the smallest subnormal) counts 0 in P V but fully in the
    sum, so 4 10^4 such keys after an outlier key bias O by ~0.29 (the GPU
    run shows 0.26), while the same keys before the outlier (added at full
    weight, then rescaled in fp32) come out right.
"""
import math

import numpy as np
import pytest

import attn_inputs as ai
import oracle
import rescale_cases as rc

O_REL_L2_BAR = 5e-2
O_MAX_ABS_BAR = 0.1
TILE = 64


def _e4m3(x):
    return ai.fp8_decode(ai.fp8_encode(x))


def _half_of_key():
    """Lane half (0/1) holding each key of a 64-key tile in the S^T
    accumulator: key 32 kb + 8 (r // 4) + 4 h + r % 4."""
    h = np.empty(TILE, np.int64)
    for kb in range(2):
        for r in range(16):
            for half in range(2):
                h[32 * kb + 8 * (r // 4) + 4 * half + r % 4] = half
    return h


def simulate(q, k, v, scale, causal):
    """One head: O of the FP8 kernel's arithmetic, in float64."""
    c = rc.c_log2(scale)
    Nq, Nk = q.shape[0], k.shape[0]
    s = (q @ k.T) * c
    if causal:
        vis = np.arange(Nk)[None, :] <= np.arange(Nq)[:, None] + (Nk - Nq)
        s = np.where(vis, s, -np.inf)
    half = _half_of_key()
    m = np.full(Nq, -np.inf)
    l = np.zeros(Nq)
    acc = np.zeros((Nq, v.shape[1]))
    for t0 in range(0, Nk, TILE):
        st = s[:, t0:t0 + TILE]
        hk = half[:st.shape[1]]
        with np.errstate(invalid="ignore", over="ignore"):
            p = np.exp2(st - np.where(np.isfinite(m), m, 0.0)[:, None])
            lane = np.stack([(16 * p[:, hk == h]).sum(axis=1) for h in (0, 1)], axis=1)
        move = ~np.isfinite(m) | np.any(~(lane <= 448.0), axis=1)
        if np.any(move):
            m_new = np.maximum(m, st.max(axis=1))
            alpha = np.where(np.isfinite(m), np.exp2(m - m_new), 0.0)
            acc[move] *= alpha[move, None]
            l[move] *= alpha[move]
            m = np.where(move, m_new, m)
            p = np.exp2(st - m[:, None])
        p = np.where(np.isfinite(st), p, 0.0)
        acc += (_e4m3(16 * p) / 16) @ v[t0:t0 + TILE]
        l += p.sum(axis=1)
    return acc / l[:, None]


def _errors(O_sim, O_ref):
    err = O_sim - O_ref
    return float(np.linalg.norm(err) / np.linalg.norm(O_ref)), float(np.abs(err).max())


def _fp8_case(seed, B, Hq, Hkv, Nq, Nk, causal):
    x = ai.prefill_inputs_fp8(seed, B, Hq, Hkv, Nq, 128, Nk=Nk)
    f = {n: ai.fp8_to_f64(x[n], x[n + "_descale"]) for n in "qkv"}
    scale = 1.0 / math.sqrt(128)
    O_ref, _ = oracle.attention(f["q"], f["k"], f["v"], scale, causal)
    O_sim = np.empty_like(O_ref)
    for b in range(B):
        for h in range(Hq):
            g = h // (Hq // Hkv)
            O_sim[b, h] = simulate(f["q"][b, h], f["k"][b, g], f["v"][b, g], scale, causal)
    return _errors(O_sim, O_ref)


# The FP8 GPU parity workloads (seeds 700 + index, as there).
CASES = [
    (1, 4, 2, 256, 256, True),
    (1, 8, 8, 300, 520, False),
    (2, 4, 1, 200, 700, True),
    (1, 4, 4, 333, 333, True),
    (1, 32, 8, 1024, 1024, True),
]


@pytest.mark.parametrize("case", CASES, ids=[f"c{i}" for i in range(len(CASES))])
def test_fp8_rounding_error_within_the_bar(case):
    rel, mx = _fp8_case(700 + CASES.index(case), *case)
    print(f"simulated FP8 error {case}: rel-L2 {rel:.3e}, max-abs {mx:.3e}")
    assert rel <= O_REL_L2_BAR / 1.8 and mx <= O_MAX_ABS_BAR / 1.4
    assert rel >= 5e-3  # the rounding of P is really simulated (16-bit paths stay near 1e-3)


@pytest.mark.parametrize("j_from_end,flushed", [(200, False), (40001, True)])
def test_fp8_flush_below_smallest_subnormal(j_from_end, flushed):
    d, Nq, Nk = 128, 6, 100001
    scale = 1.0 / math.sqrt(d)
    q, k, v = rc.outlier(6, Nq, Nk, d, Nk - j_from_end, 17.0, scale, H=1)
    vals = {}
    for n, x in (("q", q[0]), ("k", k[0]), ("v", v[0])):
        codes, ds = ai.fp8_quantize(x)
        vals[n] = ai.fp8_decode(codes) * ds
    O_ref, _ = oracle.attention_head(vals["q"], vals["k"], vals["v"], scale, False)
    rel, mx = _errors(simulate(vals["q"], vals["k"], vals["v"], scale, False), O_ref)
    print(f"outlier {j_from_end} keys from the end: rel-L2 {rel:.3e}, max-abs {mx:.3e}")
    if flushed:
        assert rel > 0.2  # ~0.29: 40000 keys at 2^-17 flushed from P V, kept in the sum
    else:
        assert rel <= O_REL_L2_BAR / 10 and mx <= O_MAX_ABS_BAR / 10
