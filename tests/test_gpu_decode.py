"""Split-KV decode on the GPU (through the C ABI) against the float64 oracle."""
import math

import numpy as np
import pytest

import attn_inputs as ai
import oracle
from gpu_util import announce, compare, from_dev, to_dev

pytestmark = pytest.mark.gpu


def dev_inputs(x):
    import torch
    dt = x["dtype"]
    return (to_dev(x["q"], dt), to_dev(x["k_cache"], dt), to_dev(x["v_cache"], dt),
            torch.from_numpy(np.asarray(x["seqlens"], np.int32)).cuda())


def oracle_decode(x, scale):
    dt = x["dtype"]
    B, Hq, d = x["q"].shape
    O = np.zeros((B, Hq, d))
    L = np.zeros((B, Hq))
    for b in range(B):
        n = int(min(max(x["seqlens"][b], 0), x["k_cache"].shape[2]))
        O[b:b + 1], L[b:b + 1] = oracle.decode(ai.bits_to_f64(x["q"][b:b + 1], dt),
                                              ai.bits_to_f64(x["k_cache"][b:b + 1, :, :n], dt),
                                              ai.bits_to_f64(x["v_cache"][b:b + 1, :, :n], dt), [n], scale)
    return O, L


def decode_case(fa, seed, B, Hq, Hkv, Lcap, d, dt, lens, num_splits=0):
    import torch
    announce(f"decode B={B} Hq={Hq} Hkv={Hkv} Lcap={Lcap} d={d} {dt} splits={num_splits} lens={list(lens)[:8]}")
    x = ai.decode_inputs(seed, B, Hq, Hkv, Lcap, d, dt, np.asarray(lens, np.int32))
    q, kc, vc, sl = dev_inputs(x)
    o, lse = fa.decode(q, kc, vc, sl, num_splits=num_splits)
    torch.cuda.synchronize()
    O_ref, L_ref = oracle_decode(x, 1.0 / math.sqrt(d))
    m = compare(from_dev(o, dt), O_ref, lse.cpu().numpy(), L_ref, f"decode B{B} Hq{Hq} Hkv{Hkv} L{Lcap} d{d} {dt}")
    return x, o, lse, m


def test_decode_32seq_gqa_full(fa):
    c = ai.CONFIGS["decode_32seq_gqa"]
    lens = ai.decode_lengths(c["seed"], c["B"], c["len_lo"], c["len_hi"])
    decode_case(fa, c["seed"], c["B"], c["Hq"], c["Hkv"], c["Lcap"], c["d"], c["dtype"], lens)


SMALL = [
    # B, Hq, Hkv, Lcap, d, dtype, lens
    (3, 8, 2, 1000, 128, ai.BF16, [1, 999, 1000]),
    (2, 4, 4, 300, 64, ai.FP16, [127, 129]),
    (4, 32, 1, 700, 128, ai.BF16, [64, 128, 513, 700]),   # 32 q-heads per kv-head
    (2, 8, 8, 2048, 64, ai.BF16, [2048, 1]),
    (3, 16, 4, 5000, 128, ai.FP16, [4097, 31, 2500]),
]


@pytest.mark.parametrize("case", SMALL, ids=[f"B{c[0]}Hq{c[1]}Hkv{c[2]}L{c[3]}d{c[4]}{c[5]}" for c in SMALL])
def test_small_decode(fa, case):
    decode_case(fa, 200 + SMALL.index(case), *case)


def test_empty_sequence(fa):
    import torch
    announce("decode empty sequence")
    x = ai.decode_inputs(21, 2, 4, 2, 256, 128, ai.BF16, np.array([0, 100], np.int32))
    q, kc, vc, sl = dev_inputs(x)
    o, lse = fa.decode(q, kc, vc, sl)
    torch.cuda.synchronize()
    assert torch.all(o[0] == 0) and torch.all(torch.isneginf(lse[0]))
    assert torch.all(torch.isfinite(lse[1]))


@pytest.mark.parametrize("splits", [1, 3, 16, 100])
def test_num_splits_invariance(fa, splits):
    announce(f"decode num_splits={splits}")
    decode_case(fa, 22, 2, 8, 2, 3000, 128, ai.BF16, [3000, 1777], num_splits=splits)


def test_decode_matches_prefill_single_query(fa):
    import torch
    announce("decode vs fa_fwd(Nq=1)")
    x, o, lse, _ = decode_case(fa, 23, 2, 8, 2, 640, 128, ai.BF16, [640, 333])
    for b, n in enumerate([640, 333]):
        q = to_dev(x["q"][b][None, :, None, :], ai.BF16)
        k = to_dev(np.ascontiguousarray(x["k_cache"][b][None, :, :n]), ai.BF16)
        v = to_dev(np.ascontiguousarray(x["v_cache"][b][None, :, :n]), ai.BF16)
        o1, l1 = fa.attention(q, k, v)
        torch.cuda.synchronize()
        assert (o1[0, :, 0].float() - o[b].float()).abs().max().item() <= 1.6e-2
        assert (l1[0, :, 0] - lse[b]).abs().max().item() <= 1e-3


def test_decode_deterministic(fa):
    import torch
    announce("decode determinism")
    x = ai.decode_inputs(24, 4, 32, 8, 4096, 128, ai.BF16, np.array([4096, 17, 2222, 3000], np.int32))
    q, kc, vc, sl = dev_inputs(x)
    o1, l1 = fa.decode(q, kc, vc, sl)
    o2, l2 = fa.decode(q, kc, vc, sl)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_many_sequences(fa):
    # More than 64 sequences (the split walks the sequences 64 at a time),
    # short caches (a wave's share spans several (sequence, kv-head) pairs
    # and pairs are cut between waves), every 7th sequence empty.
    import torch
    lens = np.random.default_rng(25).integers(0, 301, 150).astype(np.int32)
    lens[::7] = 0
    announce(f"decode many sequences B=150 lens={list(lens[:8])}")
    x = ai.decode_inputs(25, 150, 8, 2, 300, 64, ai.BF16, lens)
    q, kc, vc, sl = dev_inputs(x)
    o, lse = fa.decode(q, kc, vc, sl)
    torch.cuda.synchronize()
    o_np, l_np = from_dev(o, ai.BF16), lse.cpu().numpy()
    empty = lens == 0
    assert np.all(o_np[empty] == 0) and np.all(np.isneginf(l_np[empty]))
    xs = {k: (v[~empty] if k in ("q", "k_cache", "v_cache", "seqlens") else v) for k, v in x.items()}
    O_ref, L_ref = oracle_decode(xs, 1.0 / math.sqrt(64))
    compare(o_np[~empty], O_ref, l_np[~empty], L_ref, "decode B150")


def test_most_partials_per_pair(fa):
    # Sequence 0 (6 blocks of 32) shifts sequence 1 (32 blocks) into the
    # middle of the first wave's share; with 384-row shares sequence 1 then
    # gets ceil(1000 / 384) + 1 = 4 partials, the most the workspace holds.
    decode_case(fa, 26, 2, 4, 1, 1000, 64, ai.BF16, [192, 1000], num_splits=3)


def _random_cases(n=16, seed=27):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        B = int(rng.integers(1, 100))
        Hkv = int(rng.choice([1, 2, 4, 8]))
        grp = int(rng.choice([1, 2, 4, 8]))
        Lcap = int(rng.integers(1, 1500))
        d = int(rng.choice([64, 128]))
        dt = ai.BF16 if rng.random() < 0.5 else ai.FP16
        lens = rng.integers(0, Lcap + 1, B).astype(np.int32)
        lens[rng.random(B) < 0.1] = 0
        splits = int(rng.choice([0, 0, 1, 2, 7]))
        cases.append((100 + i, B, Hkv * grp, Hkv, Lcap, d, dt, lens, splits))
    return cases


@pytest.mark.parametrize("case", _random_cases(), ids=lambda c: f"s{c[0]}B{c[1]}Hq{c[2]}Hkv{c[3]}L{c[4]}d{c[5]}{c[6]}n{c[8]}")
def test_decode_random_shapes(fa, case):
    # Seeded shapes around the split's edges: many or few sequences, empty
    # ones, short caches (shares spanning many pairs), explicit split counts.
    import torch
    seed, B, Hq, Hkv, Lcap, d, dt, lens, splits = case
    announce(f"decode random seed={seed} B={B} Hq={Hq} Hkv={Hkv} Lcap={Lcap} d={d} {dt} splits={splits}")
    x = ai.decode_inputs(seed, B, Hq, Hkv, Lcap, d, dt, lens)
    q, kc, vc, sl = dev_inputs(x)
    o, lse = fa.decode(q, kc, vc, sl, num_splits=splits)
    torch.cuda.synchronize()
    o_np, l_np = from_dev(o, dt), lse.cpu().numpy()
    empty = lens == 0
    assert np.all(o_np[empty] == 0) and np.all(np.isneginf(l_np[empty]))
    if np.all(empty):
        return
    xs = {k: (v[~empty] if k in ("q", "k_cache", "v_cache", "seqlens") else v) for k, v in x.items()}
    O_ref, L_ref = oracle_decode(xs, 1.0 / math.sqrt(d))
    compare(o_np[~empty], O_ref, l_np[~empty], L_ref, f"decode random seed {seed}")
