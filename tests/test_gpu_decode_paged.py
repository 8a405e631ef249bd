"""Paged-cache decode on the GPU (through the C ABI) against the float64 oracle.

The cache of each sequence is scattered over fixed-size pages in a seeded
random page order ("Paged attention", cabseo.com); the kernel follows the
page table. Checks: the oracle's paged decode within tolerance, bit-identical
results to the contiguous-cache decode with the same split plan, and the
documented handling of a page-table entry that names no page.
"""
import math

import numpy as np
import pytest

import attn_inputs as ai
import oracle
from gpu_util import announce, compare, from_dev, to_dev

pytestmark = pytest.mark.gpu


def paged_case(seed, B, Hq, Hkv, Lcap, d, dt, lens, page_size, spare=3):
    x = ai.decode_inputs(seed, B, Hq, Hkv, Lcap, d, dt, np.asarray(lens, np.int32))
    pl = ai.paged_layout(x["k_cache"], x["v_cache"], page_size, seed, dt, spare_pages=spare)
    return x, pl


def dev_paged(x, pl):
    import torch
    dt = x["dtype"]
    return (to_dev(x["q"], dt), to_dev(pl["k_pages"], dt), to_dev(pl["v_pages"], dt),
            torch.from_numpy(np.ascontiguousarray(pl["block_table"], np.int32)).cuda(),
            torch.from_numpy(np.asarray(x["seqlens"], np.int32)).cuda())


SMALL = [
    # B, Hq, Hkv, Lcap, d, dtype, lens, page_size
    (3, 8, 2, 1024, 128, ai.BF16, [1, 1000, 1024], 32),
    (4, 32, 8, 2048, 128, ai.BF16, [0, 129, 2047, 640], 128),
    (2, 4, 4, 512, 64, ai.FP16, [511, 64], 64),
    (2, 16, 2, 4096, 128, ai.FP16, [4096, 3333], 256),
    # more than 64 sequences, short caches: shares span several pairs
    (70, 8, 2, 256, 128, ai.BF16, [int(v) for v in np.random.default_rng(31).integers(0, 257, 70)], 32),
]


@pytest.mark.parametrize("case", SMALL, ids=[f"B{c[0]}Hq{c[1]}Hkv{c[2]}L{c[3]}d{c[4]}{c[5]}P{c[7]}" for c in SMALL])
def test_paged_decode_vs_oracle(fa, case):
    import torch
    B, Hq, Hkv, Lcap, d, dt, lens, P = case
    announce(f"paged decode B={B} Hq={Hq} Hkv={Hkv} Lcap={Lcap} d={d} {dt} P={P} lens={lens}")
    x, pl = paged_case(300 + SMALL.index(case), B, Hq, Hkv, Lcap, d, dt, lens, P)
    q, kp, vp, table, sl = dev_paged(x, pl)
    o, lse = fa.decode_paged(q, kp, vp, table, sl)
    torch.cuda.synchronize()
    f = lambda a: ai.bits_to_f64(a, dt)
    O_ref, L_ref = oracle.decode_paged(f(x["q"]), f(pl["k_pages"]), f(pl["v_pages"]), pl["block_table"],
                                       x["seqlens"], 1.0 / math.sqrt(d))
    empty = np.asarray(lens) == 0
    o_np, l_np = from_dev(o, dt), lse.cpu().numpy()
    assert np.all(o_np[empty] == 0) and np.all(np.isneginf(l_np[empty]))
    compare(o_np[~empty], O_ref[~empty], l_np[~empty], L_ref[~empty], f"paged decode P{P}")


@pytest.mark.parametrize("splits", [0, 1, 5])
def test_paged_equals_contiguous_bitwise(fa, splits):
    import torch
    announce(f"paged == contiguous, splits={splits}")
    x, pl = paged_case(310, 4, 32, 8, 2048, 128, ai.BF16, [2048, 700, 33, 1500], 128)
    q, kp, vp, table, sl = dev_paged(x, pl)
    o1, l1 = fa.decode_paged(q, kp, vp, table, sl, num_splits=splits)
    kc, vc = to_dev(x["k_cache"], ai.BF16), to_dev(x["v_cache"], ai.BF16)
    o2, l2 = fa.decode(q, kc, vc, sl, num_splits=splits)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_paged_32seq_gqa_bitwise(fa):
    # The 32-sequence decode workload with 128-row pages: identical bits to the
    # contiguous decode (itself checked against the oracle in the decode tests).
    import torch
    c = ai.CONFIGS["decode_32seq_gqa"]
    announce("paged decode_32seq_gqa P=128")
    lens = ai.decode_lengths(c["seed"], c["B"], c["len_lo"], c["len_hi"])
    x, pl = paged_case(c["seed"], c["B"], c["Hq"], c["Hkv"], c["Lcap"], c["d"], c["dtype"], lens, 128, spare=0)
    q, kp, vp, table, sl = dev_paged(x, pl)
    o1, l1 = fa.decode_paged(q, kp, vp, table, sl)
    del kp, vp
    kc, vc = to_dev(x["k_cache"], c["dtype"]), to_dev(x["v_cache"], c["dtype"])
    o2, l2 = fa.decode(q, kc, vc, sl)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_bad_page_entry_poisons_only_its_sequence(fa):
    import torch
    announce("paged decode with an out-of-range page entry")
    x, pl = paged_case(320, 3, 8, 2, 1024, 128, ai.BF16, [1024, 600, 300], 64)
    table = pl["block_table"].copy()
    num_pages = pl["k_pages"].shape[0]
    table[1, 5] = num_pages + 100   # needed by sequence 1 (rows 320..383)
    table[2, 10] = -1               # past the 5 pages sequence 2 needs: never followed
    pl2 = dict(pl, block_table=table)
    q, kp, vp, tb, sl = dev_paged(x, pl2)
    o, lse = fa.decode_paged(q, kp, vp, tb, sl)
    q0, kp0, vp0, tb0, _ = dev_paged(x, pl)
    o_ok, l_ok = fa.decode_paged(q0, kp0, vp0, tb0, sl)
    torch.cuda.synchronize()
    assert torch.all(torch.isnan(o[1].float())) and torch.all(torch.isnan(lse[1]))
    assert torch.equal(o[0], o_ok[0]) and torch.equal(lse[0], l_ok[0])
    assert torch.equal(o[2], o_ok[2]) and torch.equal(lse[2], l_ok[2])


def _random_paged_cases(n=8, seed=29):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        B = int(rng.integers(1, 80))
        Hkv = int(rng.choice([1, 2, 8]))
        grp = int(rng.choice([1, 4]))
        P = int(rng.choice([32, 64, 128]))
        Lcap = P * int(rng.integers(1, 20))
        d = int(rng.choice([64, 128]))
        dt = ai.BF16 if rng.random() < 0.5 else ai.FP16
        lens = [int(v) for v in rng.integers(0, Lcap + 1, B)]
        cases.append((400 + i, B, Hkv * grp, Hkv, Lcap, d, dt, lens, P))
    return cases


@pytest.mark.parametrize("case", _random_paged_cases(), ids=lambda c: f"s{c[0]}B{c[1]}Hq{c[2]}L{c[4]}d{c[5]}{c[6]}P{c[8]}")
def test_paged_decode_random_shapes(fa, case):
    import torch
    seed, B, Hq, Hkv, Lcap, d, dt, lens, P = case
    announce(f"paged decode random seed={seed} B={B} Hq={Hq} Hkv={Hkv} Lcap={Lcap} d={d} {dt} P={P}")
    x, pl = paged_case(seed, B, Hq, Hkv, Lcap, d, dt, lens, P)
    q, kp, vp, table, sl = dev_paged(x, pl)
    o, lse = fa.decode_paged(q, kp, vp, table, sl)
    torch.cuda.synchronize()
    empty = np.asarray(lens) == 0
    o_np, l_np = from_dev(o, dt), lse.cpu().numpy()
    assert np.all(o_np[empty] == 0) and np.all(np.isneginf(l_np[empty]))
    if np.all(empty):
        return
    f = lambda a: ai.bits_to_f64(a, dt)
    O_ref, L_ref = oracle.decode_paged(f(x["q"]), f(pl["k_pages"]), f(pl["v_pages"]), pl["block_table"],
                                       x["seqlens"], 1.0 / math.sqrt(d))
    compare(o_np[~empty], O_ref[~empty], l_np[~empty], L_ref[~empty], f"paged decode random seed {seed}")
