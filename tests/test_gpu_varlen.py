"""Packed variable-length prefill on the GPU (through the C ABI) against the
float64 oracle: sequences of different lengths share one slab per head with
no padding ("Continuous batching", cabseo.com), each attending only to its
own keys, per-sequence causal alignment."""
import math

import numpy as np
import pytest

import attn_inputs as ai
import oracle
from gpu_util import announce, compare, from_dev, to_dev

pytestmark = pytest.mark.gpu


def run(fa, x, causal, max_q=None, cu_q=None, cu_k=None):
    import torch
    dt = x["dtype"]
    q, k, v = to_dev(x["q"], dt), to_dev(x["k"], dt), to_dev(x["v"], dt)
    cq = torch.from_numpy(np.asarray(x["cu_q"] if cu_q is None else cu_q, np.int32)).cuda()
    ck = torch.from_numpy(np.asarray(x["cu_k"] if cu_k is None else cu_k, np.int32)).cuda()
    if max_q is None:
        max_q = int(np.max(np.diff(x["cu_q"])))
    o = torch.zeros_like(q)
    lse = torch.full((q.shape[0], q.shape[1]), float("nan"), dtype=torch.float32, device="cuda")
    fa.attention_varlen(q, k, v, cq, ck, max_q, causal=causal, out=o, lse=lse)
    torch.cuda.synchronize()
    return from_dev(o, dt), lse.cpu().numpy()


def check(fa, seed, lens_q, lens_k, Hq, Hkv, d, dt, causal):
    announce(f"varlen lens_q={lens_q} lens_k={lens_k} Hq={Hq} Hkv={Hkv} d={d} {dt} causal={causal}")
    x = ai.varlen_inputs(seed, lens_q, lens_k, Hq, Hkv, d, dt)
    o, lse = run(fa, x, causal)
    f = lambda a: ai.bits_to_f64(a, dt)
    O_ref, L_ref = oracle.attention_varlen(f(x["q"]), f(x["k"]), f(x["v"]), x["cu_q"], x["cu_k"],
                                           1.0 / math.sqrt(d), causal)
    fin = np.isfinite(L_ref)
    assert np.all(o[~fin] == 0) and np.array_equal(np.isneginf(lse), np.isneginf(L_ref))
    compare(o[fin], O_ref[fin], lse[fin], L_ref[fin], f"varlen d{d} {dt} causal={causal}")


CASES = [
    # lens_q, lens_k, Hq, Hkv, d, dtype, causal
    ([1, 255, 256, 257, 1000], [1, 255, 256, 257, 1000], 8, 2, 128, ai.BF16, True),
    ([1, 255, 256, 257, 1000], [3, 300, 256, 700, 1000], 8, 2, 128, ai.BF16, False),
    ([64, 200, 513], [128, 200, 1024], 4, 4, 128, ai.FP16, True),      # chunked prefill: Nq < Nk
    ([300, 0, 77], [300, 5, 77], 8, 8, 64, ai.FP16, True),            # an empty sequence
    ([100, 40], [100, 0], 4, 1, 64, ai.BF16, False),                  # a sequence with no keys
    ([129, 1, 600], [129, 1, 600], 32, 8, 128, ai.BF16, True),
]


@pytest.mark.parametrize("case", CASES, ids=[f"c{i}" for i in range(len(CASES))])
def test_varlen_vs_oracle(fa, case):
    check(fa, 400 + CASES.index(case), *case)


def test_varlen_single_sequence_equals_fwd_bitwise(fa):
    import torch
    announce("varlen B=1 == fa_fwd")
    N = 1500
    x = ai.varlen_inputs(410, [N], [N], 8, 2, 128, ai.BF16)
    p = ai.prefill_inputs(410, 1, 8, 2, N, 128, ai.BF16)
    assert np.array_equal(p["q"][0], x["q"]) and np.array_equal(p["k"][0], x["k"])
    # The packed path always runs 256-row tiles; the contiguous one would take
    # the split schedule for this small causal grid (another order of the
    # fp32 sums), so it is pinned to tiles for the bitwise comparison.
    prev = fa.fa_set_prefill_schedule(fa.FA_SCHEDULE_TILES)
    try:
        for causal in (False, True):
            o1, l1 = run(fa, x, causal)
            q, k, v = (to_dev(p[n], ai.BF16) for n in "qkv")
            o2, l2 = fa.attention(q, k, v, causal=causal)
            torch.cuda.synchronize()
            assert np.array_equal(o1, from_dev(o2, ai.BF16)[0]) and np.array_equal(l1, l2.cpu().numpy()[0])
    finally:
        fa.fa_set_prefill_schedule(prev)


def test_varlen_clamps_offsets_and_leaves_other_rows(fa):
    announce("varlen offsets out of range")
    x = ai.varlen_inputs(411, [100, 300], [100, 300], 4, 2, 128, ai.BF16)
    tq, tk = x["q"].shape[1], x["k"].shape[1]
    # a negative start and an end past the total: clamped to [0, 100) and [100, tq)
    o, lse = run(fa, x, True, max_q=tq, cu_q=[-50, 100, tq + 500], cu_k=[-9, 100, tk + 77])
    o_ok, l_ok = run(fa, x, True)
    assert np.array_equal(o, o_ok) and np.array_equal(lse, l_ok)
    # rows that belong to no sequence are not written (zeros / NaN sentinels stay)
    o2, l2 = run(fa, x, True, cu_q=[0, 100, 250], cu_k=[0, 100, 250])
    assert np.all(o2[:, 250:] == 0) and np.all(np.isnan(l2[:, 250:]))
