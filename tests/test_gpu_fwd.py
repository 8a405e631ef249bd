"""Prefill forward on the GPU (through the C ABI) against the float64 oracle."""
import math

import numpy as np
import pytest

import attn_inputs as ai
import oracle
from gpu_util import announce, compare, from_dev, to_dev

pytestmark = pytest.mark.gpu


def run_fwd(fa, x, causal, scale=None):
    import torch
    q, k, v = to_dev(x["q"], x["dtype"]), to_dev(x["k"], x["dtype"]), to_dev(x["v"], x["dtype"])
    o, lse = fa.attention(q, k, v, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return o, lse


def full_case(fa, seed, B, Hq, Hkv, Nq, Nk, d, dtype, causal):
    announce(f"fwd full B={B} Hq={Hq} Hkv={Hkv} Nq={Nq} Nk={Nk} d={d} {dtype} causal={causal}")
    x = ai.prefill_inputs(seed, B, Hq, Hkv, Nq, d, dtype, Nk=Nk)
    o, lse = run_fwd(fa, x, causal)
    scale = 1.0 / math.sqrt(d)
    O_ref, L_ref = oracle.attention(ai.bits_to_f64(x["q"], dtype), ai.bits_to_f64(x["k"], dtype),
                                    ai.bits_to_f64(x["v"], dtype), scale, causal)
    return compare(from_dev(o, dtype), O_ref, lse.cpu().numpy(), L_ref,
                   f"B{B} Hq{Hq} Hkv{Hkv} Nq{Nq} Nk{Nk} d{d} {dtype} causal={causal}")


def test_tiny_mha_n128(fa):
    c = ai.CONFIGS["tiny_mha_n128"]
    full_case(fa, c["seed"], c["B"], c["Hq"], c["Hkv"], c["N"], c["N"], c["d"], c["dtype"], False)


SMALL = [
    # B, Hq, Hkv, Nq, Nk, d, dtype, causal
    (1, 2, 1, 1, 1, 64, ai.BF16, False),
    (1, 2, 1, 1, 1, 128, ai.BF16, True),
    (1, 2, 2, 17, 17, 128, ai.BF16, False),
    (2, 4, 2, 100, 100, 64, ai.BF16, True),
    (1, 4, 1, 300, 300, 128, ai.BF16, True),
    (1, 2, 2, 1000, 1000, 64, ai.FP16, True),
    (1, 2, 2, 1000, 1000, 64, ai.FP16, False),
    (1, 4, 2, 77, 300, 128, ai.BF16, True),     # Nq < Nk, bottom-right causal
    (1, 4, 4, 130, 1000, 64, ai.FP16, False),
    (1, 8, 1, 200, 200, 128, ai.FP16, True),    # multi-query
    (2, 8, 2, 257, 257, 128, ai.BF16, False),
    (1, 2, 1, 513, 700, 64, ai.BF16, True),
]


@pytest.mark.parametrize("case", SMALL, ids=[f"B{c[0]}Hq{c[1]}Hkv{c[2]}Nq{c[3]}Nk{c[4]}d{c[5]}{c[6]}{'c' if c[7] else 'n'}" for c in SMALL])
def test_small_shapes(fa, case):
    full_case(fa, 100 + SMALL.index(case), *case)


# Key counts that are whole tiles (64 keys at d = 128, 128 at d = 64) with
# only a few tiles: the last two steps of every such launch issue their loads
# without a branch, re-reading tile 0 into the slot of a tile that does not
# exist, so these shapes are mostly such steps.
ALIGNED = [
    # B, Hq, Hkv, Nq, Nk, d, dtype, causal
    (1, 4, 2, 64, 64, 128, ai.BF16, False),
    (1, 4, 2, 128, 128, 128, ai.BF16, True),
    (2, 4, 1, 192, 192, 128, ai.FP16, True),
    (1, 8, 2, 100, 320, 128, ai.BF16, True),    # Nq < Nk, bottom-right causal
    (1, 2, 2, 300, 192, 128, ai.BF16, False),   # Nq > Nk
    (1, 4, 4, 128, 128, 64, ai.FP16, True),
    (2, 4, 2, 256, 256, 64, ai.BF16, False),
    (1, 8, 2, 384, 384, 64, ai.FP16, True),
    (1, 4, 1, 50, 512, 64, ai.BF16, True),
]


@pytest.mark.parametrize("case", ALIGNED,
                         ids=[f"B{c[0]}Hq{c[1]}Hkv{c[2]}Nq{c[3]}Nk{c[4]}d{c[5]}{c[6]}{'c' if c[7] else 'n'}" for c in ALIGNED])
def test_aligned_few_tiles(fa, case):
    full_case(fa, 200 + ALIGNED.index(case), *case)


def sampled_case(fa, name, causal, rows_per_head):
    c = ai.CONFIGS[name]
    B, Hq, Hkv, N, d, dt = c["B"], c["Hq"], c["Hkv"], c["N"], c["d"], c["dtype"]
    announce(f"fwd sampled {name} causal={causal}")
    x = ai.prefill_inputs(c["seed"], B, Hq, Hkv, N, d, dt)
    o, lse = run_fwd(fa, x, causal)
    o_np = from_dev(o, dt)
    lse_np = lse.cpu().numpy()
    scale = 1.0 / math.sqrt(d)
    grp = Hq // Hkv
    got, ref, gl, rl = [], [], [], []
    for b in range(B):
        kv_cache = {}
        for h in range(Hq):
            g = h // grp
            if g not in kv_cache:
                kv_cache = {g: (ai.bits_to_f64(x["k"][b, g], dt), ai.bits_to_f64(x["v"][b, g], dt))}
            k64, v64 = kv_cache[g]
            rows = ai.sample_rows(c["seed"], b * Hq + h, N, rows_per_head)
            O_r, L_r = oracle.attention_rows(ai.bits_to_f64(x["q"][b, h, rows], dt), rows, k64, v64, scale, causal, N)
            got.append(o_np[b, h, rows])
            ref.append(O_r)
            gl.append(lse_np[b, h, rows])
            rl.append(L_r)
    return compare(np.concatenate(got), np.concatenate(ref), np.concatenate(gl), np.concatenate(rl),
                   f"{name} causal={causal} ({rows_per_head} rows/head)")


def config_case(fa, name, causal):
    """A whole configuration against the oracle: every row of every head,
    rel-L2 over the whole O tensor, LSE over all rows."""
    c = ai.CONFIGS[name]
    return full_case(fa, c["seed"], c["B"], c["Hq"], c["Hkv"], c["N"], c["N"], c["d"], c["dtype"], causal)


@pytest.mark.parametrize("causal", [False, True])
def test_mha_n4096_fp16_full(fa, causal):
    config_case(fa, "mha_n4096_fp16", causal)


def test_llama3_gqa_n8192_full(fa):
    # 32 heads of 8192 x 8192 float64 scores, one head at a time (~15-40 s on the host)
    config_case(fa, "llama3_8b_gqa_n8192", True)


@pytest.mark.slow
def test_llama3_8b_gqa_n131072_sampled(fa):
    sampled_case(fa, "llama3_8b_gqa_n131072", True, ai.CONFIGS["llama3_8b_gqa_n131072"]["sample_rows"])


# ---------------------------------------------------------------- GPU-side pins
def test_zero_query_gives_mean(fa):
    import torch
    announce("fwd Q=0 pin")
    B, H, N, d = 1, 2, 300, 128
    x = ai.prefill_inputs(7, B, H, H, N, d, ai.BF16)
    x["q"][:] = 0
    for causal in (False, True):
        o, lse = run_fwd(fa, x, causal)
        v = ai.bits_to_f64(x["v"], ai.BF16)
        if causal:
            want = np.cumsum(v, axis=2) / np.arange(1, N + 1)[None, None, :, None]
            want_l = np.broadcast_to(np.log(np.arange(1, N + 1)), (B, H, N))
        else:
            want = np.broadcast_to(v.mean(axis=2, keepdims=True), v.shape)
            want_l = np.full((B, H, N), math.log(N))
        compare(from_dev(o, ai.BF16), want, lse.cpu().numpy(), want_l, f"Q=0 causal={causal}")


def test_ones_value_gives_ones(fa):
    announce("fwd V=1 pin")
    x = ai.prefill_inputs(8, 1, 4, 2, 333, 64, ai.FP16)
    x["v"][:] = ai.round_to_bits(np.ones(1, np.float32), ai.FP16)[0]
    for causal in (False, True):
        o, _ = run_fwd(fa, x, causal)
        assert np.abs(from_dev(o, ai.FP16) - 1.0).max() <= 4e-3


def test_causal_row0_is_v0_bitwise(fa):
    announce("fwd causal row 0 pin")
    for dt, d in ((ai.BF16, 128), (ai.FP16, 64)):
        x = ai.prefill_inputs(9, 1, 4, 4, 200, d, dt)
        o, lse = run_fwd(fa, x, True)
        o_bits = o.cpu().view(__import__("torch").int16).numpy().view(np.uint16)
        assert np.array_equal(o_bits[0, :, 0], x["v"][0, :, 0])
        q = ai.bits_to_f64(x["q"][0, :, 0], dt)
        k = ai.bits_to_f64(x["k"][0, :, 0], dt)
        s00 = float(np.float32(1.0 / math.sqrt(d))) * (q * k).sum(axis=1)
        assert np.abs(lse.cpu().numpy()[0, :, 0] - s00).max() <= 1e-4


def test_gqa_equals_repeated_mha_bitwise(fa):
    import torch
    announce("fwd GQA == repeated MHA pin")
    x = ai.prefill_inputs(10, 2, 8, 2, 250, 128, ai.BF16)
    for causal in (False, True):
        o1, l1 = run_fwd(fa, x, causal)
        xr = dict(x, k=np.repeat(x["k"], 4, axis=1), v=np.repeat(x["v"], 4, axis=1))
        o2, l2 = run_fwd(fa, xr, causal)
        assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_deterministic_bitwise(fa):
    import torch
    announce("fwd determinism")
    c = ai.CONFIGS["llama3_8b_gqa_n8192"]
    x = ai.prefill_inputs(c["seed"], 1, 32, 8, 2048, 128, ai.BF16)
    o1, l1 = run_fwd(fa, x, True)
    o2, l2 = run_fwd(fa, x, True)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_lse_optional_and_errors_raise(fa):
    import torch
    announce("fwd lse=None and error mapping")
    x = ai.prefill_inputs(11, 1, 2, 2, 64, 64, ai.BF16)
    q, k, v = to_dev(x["q"], ai.BF16), to_dev(x["k"], ai.BF16), to_dev(x["v"], ai.BF16)
    o = torch.empty_like(q)
    st = fa.fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), None, 1, 2, 2, 64, 64, 64,
                   0.125, 0, fa.FA_DTYPE_BF16, torch.cuda.current_stream().cuda_stream)
    assert st == fa.FA_OK
    torch.cuda.synchronize()
    o2, _ = fa.attention(q, k, v)
    assert torch.equal(o, o2)
    with pytest.raises(NotImplementedError):
        fa.attention(q[..., :32].contiguous(), k[..., :32].contiguous(), v[..., :32].contiguous())
    with pytest.raises(ValueError):
        fa.attention(q, k, v, causal=True, scale=-1.0)


def _random_prefill_cases(n=12, seed=31):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        d = int(rng.choice([64, 128]))
        Hkv = int(rng.choice([1, 2, 4]))
        Hq = Hkv * int(rng.choice([1, 2, 4]))
        B = int(rng.integers(1, 3))
        Nk = int(rng.integers(1, 1100))
        causal = bool(rng.random() < 0.6)
        Nq = int(rng.integers(1, Nk + 1)) if causal else int(rng.integers(1, 1100))
        dt = ai.BF16 if rng.random() < 0.5 else ai.FP16
        cases.append((300 + i, B, Hq, Hkv, Nq, Nk, d, dt, causal))
    return cases


@pytest.mark.parametrize("case", _random_prefill_cases(),
                         ids=lambda c: f"s{c[0]}B{c[1]}Hq{c[2]}Hkv{c[3]}Nq{c[4]}Nk{c[5]}d{c[6]}{c[7]}{'c' if c[8] else 'n'}")
def test_random_shapes(fa, case):
    # Seeded shapes with ragged query and key tails at both head widths,
    # GQA groups, causal with Nq <= Nk (bottom-right aligned).
    full_case(fa, *case)
