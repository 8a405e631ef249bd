"""The online softmax's reference-point move on the GPU, against the oracle.

With i.i.d. N(0,1) inputs at scale 1/sqrt(d) no tile after a row's first one
ever makes the kernels move their reference point, so the rescale by
exp2(m_old - m_new) of the running sum and of the output accumulator (the
merge identity of "The math of Flash Attention", unite.ai; running M and L of
"Implementation details") would go untested. These cases plant scores that
force the move (``rescale_cases``) in every kernel that uses the rule:
prefill (both head widths, causal and not), packed prefill, contiguous and
paged decode (32-key blocks) and FP8 prefill (limit 448 on 2^4 P). Each case
first asserts on the CPU that its inputs cross the limit, so it cannot
silently stop exercising the branch. The tolerances are the usual ones.

The last two cases pin the 16-bit limit itself: an fp16 P of 2^16 would
round to infinity, so the fp16 kernels must keep every P below 65504.
"""
import math

import numpy as np
import pytest

import attn_inputs as ai
import oracle
import rescale_cases as rc
from gpu_util import announce, compare, from_dev, to_dev

pytestmark = pytest.mark.gpu

LIM16 = 2.0 ** 16   # reference-move limit of the 16-bit kernels (an upper bound for fp16)
LIM8 = 448.0 / 16   # FP8: sums of 2^4 P above 448


def _tile(d):
    return 64 if d == 128 else 128


@pytest.mark.parametrize("d,dt,causal", [(128, ai.BF16, False), (128, ai.BF16, True), (64, ai.FP16, False),
                                         (64, ai.FP16, True)])
def test_prefill_outlier_key(fa, d, dt, causal):
    """~10^5 flat keys and one key 17 log2 units above them at position
    60000: the keys before it keep about a quarter of the weight after the
    rescale, V is +1 before it and -1 after it."""
    import torch
    Nq, Nk, j_out, Hq = 40, 100001, 60000, 2
    scale = 1.0 / math.sqrt(d)
    announce(f"rescale prefill outlier d={d} {dt} causal={causal}")
    q, k, v = rc.outlier(1, Nq, Nk, d, j_out, 17.0, scale, H=Hq)
    (qb, q64), (kb, k64), (vb, v64) = rc.rounded(q, dt), rc.rounded(k[:1], dt), rc.rounded(v[:1], dt)
    for h in range(Hq):
        assert rc.jump_rows(q64[h], k64[0], scale, _tile(d), LIM16, causal) == Nq
    o, lse = fa.attention(to_dev(qb[None], dt), to_dev(kb[None], dt), to_dev(vb[None], dt), causal=causal)
    torch.cuda.synchronize()
    O_ref, L_ref = oracle.attention(q64[None], k64[None], v64[None], scale, causal)
    compare(from_dev(o, dt), O_ref, lse.cpu().numpy(), L_ref, f"outlier d={d} {dt} causal={causal}")


@pytest.mark.parametrize("d,dt,causal", [(128, ai.BF16, False), (128, ai.BF16, True), (64, ai.FP16, True)])
def test_prefill_q_times_8(fa, d, dt, causal):
    """The workload's N(0,1) draws with Q scaled by 8 (exact in bf16/fp16):
    sharper rows, some of whose later tiles cross the limit."""
    import torch
    B, Hq, Hkv, N = 1, 8, 2, 2048
    announce(f"rescale prefill Q*8 d={d} {dt} causal={causal}")
    x = ai.prefill_inputs(900 + d, B, Hq, Hkv, N, d, dt)
    q64 = ai.bits_to_f64(x["q"], dt) * 8.0
    qb = ai.round_to_bits(q64.astype(np.float32), dt)
    assert np.array_equal(ai.bits_to_f64(qb, dt), q64)
    k64, v64 = ai.bits_to_f64(x["k"], dt), ai.bits_to_f64(x["v"], dt)
    scale = 1.0 / math.sqrt(d)
    crossing = sum(rc.jump_rows(q64[0, h], k64[0, h // (Hq // Hkv)], scale, _tile(d), LIM16, causal)
                   for h in range(Hq))
    assert crossing > 0
    o, lse = fa.attention(to_dev(qb, dt), to_dev(x["k"], dt), to_dev(x["v"], dt), causal=causal)
    torch.cuda.synchronize()
    O_ref, L_ref = oracle.attention(q64, k64, v64, scale, causal)
    compare(from_dev(o, dt), O_ref, lse.cpu().numpy(), L_ref, f"Q*8 d={d} {dt} causal={causal} ({crossing} rows)")


@pytest.mark.parametrize("d,dt", [(128, ai.BF16), (64, ai.FP16)])
def test_prefill_ramp(fa, d, dt):
    """Tiny scores first, larger ones later: each 32-key block 17 log2 units
    above the previous one, so the reference moves at every tile."""
    import torch
    Nq, Nk = 70, 300
    scale = 1.0 / math.sqrt(d)
    announce(f"rescale prefill ramp d={d} {dt}")
    q, k, v = rc.ramp(2, Nq, Nk, d, 17.0, scale, H=2)
    (qb, q64), (kb, k64), (vb, v64) = rc.rounded(q, dt), rc.rounded(k, dt), rc.rounded(v, dt)
    assert rc.jump_rows(q64[0], k64[0], scale, _tile(d), LIM16) == Nq
    for causal in (False, True):
        o, lse = fa.attention(to_dev(qb[None], dt), to_dev(kb[None], dt), to_dev(vb[None], dt), causal=causal)
        torch.cuda.synchronize()
        O_ref, L_ref = oracle.attention(q64[None], k64[None], v64[None], scale, causal)
        compare(from_dev(o, dt), O_ref, lse.cpu().numpy(), L_ref, f"ramp d={d} {dt} causal={causal}")


def test_varlen_outlier_sequence(fa):
    """A packed batch whose long sequence holds the outlier key and whose
    short ones are plain draws."""
    import torch
    d, dt = 128, ai.BF16
    scale = 1.0 / math.sqrt(d)
    announce("rescale varlen outlier")
    Hq, Hkv = 4, 2
    q0, k0, v0 = rc.outlier(3, 37, 70001, d, 40000, 17.0, scale, H=Hq)
    rng = np.random.default_rng(4)
    lens_q, lens_k = [37, 100, 5], [70001, 300, 64]
    qs = [q0] + [rng.standard_normal((Hq, n, d)).astype(np.float32) for n in lens_q[1:]]
    ks = [k0[:Hkv]] + [rng.standard_normal((Hkv, n, d)).astype(np.float32) for n in lens_k[1:]]
    vs = [v0[:Hkv]] + [rng.standard_normal((Hkv, n, d)).astype(np.float32) for n in lens_k[1:]]
    (qb, q64), (kb, k64), (vb, v64) = (rc.rounded(np.concatenate(t, axis=1), dt) for t in (qs, ks, vs))
    cu_q = np.concatenate([[0], np.cumsum(lens_q)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(lens_k)]).astype(np.int32)
    assert rc.jump_rows(q64[0, :37], k64[0, :70001], scale, 64, LIM16, True) == 37
    for causal in (False, True):
        o, lse = fa.attention_varlen(to_dev(qb, dt), to_dev(kb, dt), to_dev(vb, dt),
                                     torch.from_numpy(cu_q).cuda(), torch.from_numpy(cu_k).cuda(), max(lens_q),
                                     causal=causal)
        torch.cuda.synchronize()
        O_ref, L_ref = oracle.attention_varlen(q64, k64, v64, cu_q, cu_k, scale, causal)
        compare(from_dev(o, dt), O_ref, lse.cpu().numpy(), L_ref, f"varlen outlier causal={causal}")


def _decode_outlier(dt, d, Lcap, lens, j_outs, Hq=8, Hkv=2):
    """q [B,Hq,d] and caches [B,Hkv,Lcap,d] (NaN past each length) with one
    outlier key per sequence; returns bits, float64 values and the scale."""
    scale = 1.0 / math.sqrt(d)
    B = len(lens)
    qb = np.empty((B, Hq, d), np.uint16)
    nan = ai.BF16_NAN_BITS if dt == ai.BF16 else ai.FP16_NAN_BITS
    kc = np.full((B, Hkv, Lcap, d), nan, np.uint16)
    vc = np.full((B, Hkv, Lcap, d), nan, np.uint16)
    for b, (L, j) in enumerate(zip(lens, j_outs)):
        for g in range(Hkv):
            q, k, v = rc.outlier(20 + 3 * b + g, Hq // Hkv, L, d, j, 17.0, scale, H=1)
            qb[b, g * (Hq // Hkv):(g + 1) * (Hq // Hkv)] = rc.rounded(q[0], dt)[0]
            kc[b, g, :L] = rc.rounded(k[0], dt)[0]
            vc[b, g, :L] = rc.rounded(v[0], dt)[0]
    f = lambda a: ai.bits_to_f64(a, dt)
    for b, L in enumerate(lens):
        for h in range(Hq):
            g = h // (Hq // Hkv)
            assert rc.jump_rows(f(qb[b, h:h + 1]), f(kc[b, g, :L]), scale, 32, LIM16) == 1
    return qb, kc, vc, scale


@pytest.mark.parametrize("dt,d", [(ai.BF16, 128), (ai.FP16, 64)])
def test_decode_outlier(fa, dt, d):
    import torch
    lens, j_outs, Lcap = [100001, 5000], [60000, 4000], 100096
    announce(f"rescale decode outlier {dt} d={d}")
    qb, kc, vc, scale = _decode_outlier(dt, d, Lcap, lens, j_outs)
    sl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    o, lse = fa.decode(to_dev(qb, dt), to_dev(kc, dt), to_dev(vc, dt), sl)
    torch.cuda.synchronize()
    f = lambda a: ai.bits_to_f64(a, dt)
    O_ref, L_ref = oracle.decode(f(qb), f(kc), f(vc), lens, scale)
    compare(from_dev(o, dt), O_ref, lse.cpu().numpy(), L_ref, f"decode outlier {dt} d={d}")


def test_decode_paged_outlier(fa):
    import torch
    dt, d, P = ai.BF16, 128, 256
    lens, j_outs, Lcap = [100001, 5000], [60000, 4000], 100096
    announce("rescale paged decode outlier")
    qb, kc, vc, scale = _decode_outlier(dt, d, Lcap, lens, j_outs)
    pl = ai.paged_layout(kc, vc, P, 5, dt, spare_pages=2)
    o, lse = fa.decode_paged(to_dev(qb, dt), to_dev(pl["k_pages"], dt), to_dev(pl["v_pages"], dt),
                             torch.from_numpy(np.ascontiguousarray(pl["block_table"], np.int32)).cuda(),
                             torch.tensor(lens, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    f = lambda a: ai.bits_to_f64(a, dt)
    O_ref, L_ref = oracle.decode_paged(f(qb), f(pl["k_pages"]), f(pl["v_pages"]), pl["block_table"], lens, scale)
    compare(from_dev(o, dt), O_ref, lse.cpu().numpy(), L_ref, "paged decode outlier")


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_outlier(fa, causal):
    """FP8 prefill moves its reference when a lane's sum of 2^4 P exceeds
    448; the outlier is 17 log2 units up, 200 keys before the end. (After
    the move the flat keys have P = 2^-17, and 2^4 P is below E4M3's
    smallest subnormal: in the P V product they count as 0. With the outlier
    late, the keys after it carry about 0.1% of the weight; the keys before
    it, rescaled in fp32, about 40%.) Tolerances of the FP8 tests."""
    import torch
    from test_gpu_fp8 import check
    d, Nq, Nk, Hq = 128, 40, 100001, 2
    scale = 1.0 / math.sqrt(d)
    announce(f"rescale fp8 outlier causal={causal}")
    q, k, v = rc.outlier(6, Nq, Nk, d, Nk - 200, 17.0, scale, H=Hq)
    enc = {}
    for name, x in (("q", q[None]), ("k", k[None, :1]), ("v", v[None, :1])):
        codes = np.empty(x.shape, np.uint8)
        ds = np.empty(x.shape[:2], np.float32)
        for h in range(x.shape[1]):
            codes[0, h], ds[0, h] = ai.fp8_quantize(x[0, h])
        enc[name], enc[name + "_ds"] = codes, ds
    f = {n: ai.fp8_to_f64(enc[n], enc[n + "_ds"]) for n in "qkv"}
    for h in range(Hq):
        assert rc.jump_rows(f["q"][0, h], f["k"][0, 0], scale, 64, LIM8, causal) == Nq
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    o, lse = fa.attention_fp8(dev(enc["q"]), dev(enc["k"]), dev(enc["v"]), dev(enc["q_ds"]), dev(enc["k_ds"]),
                              dev(enc["v_ds"]), causal=causal)
    torch.cuda.synchronize()
    O_ref, L_ref = oracle.attention(f["q"], f["k"], f["v"], scale, causal)
    check(o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64), O_ref, L_ref,
          f"fp8 outlier causal={causal}")


def _unit_scale():
    """A float32 scale whose factor to log2 units rounds to just below 1."""
    s = np.float32(1.0 / rc.LOG2E)
    for _ in range(64):
        c = np.float32(s * np.float32(rc.LOG2E))
        if c < 1.0:
            return float(s), float(c)
        s = np.nextafter(s, np.float32(0))
    raise AssertionError("no scale found")


def _fp16_limit_keys(Nk, first_block, j1, d):
    """K rows: 0 before ``first_block`` (score 0), 4 e_0 at j1 (score 16 with
    q = 4 e_0), -25 e_0 elsewhere (score -100). V: N(0,1)."""
    k = np.zeros((Nk, d), np.float32)
    k[first_block:, 0] = -25.0
    k[j1, 0] = 4.0
    v = np.random.default_rng(7).standard_normal((Nk, d)).astype(np.float32)
    return k, v


def test_fp16_p_below_half_max_prefill(fa):
    """A tile whose only non-negligible score is 16 log2 units above the
    reference (factor c just below 1, so 2^(16c) < 2^16): the tile's sum
    stays within 2^16, and rounding that P to fp16 must not give infinity."""
    import torch
    d, dt, Nq, Nk = 64, ai.FP16, 8, 400
    scale, c = _unit_scale()
    announce("fp16 P at the limit (prefill)")
    assert 2.0 ** (16 * c) > 65520  # would round to fp16 infinity
    q = np.zeros((Nq, d), np.float32)
    q[:, 0] = 4.0
    k, v = _fp16_limit_keys(Nk, 128, 200, d)
    (qb, q64), (kb, k64), (vb, v64) = rc.rounded(q, dt), rc.rounded(k, dt), rc.rounded(v, dt)
    o, lse = fa.attention(to_dev(qb[None, None], dt), to_dev(kb[None, None], dt), to_dev(vb[None, None], dt),
                          scale=scale)
    torch.cuda.synchronize()
    O_ref, L_ref = oracle.attention(q64[None, None], k64[None, None], v64[None, None], scale, False)
    compare(from_dev(o, dt), O_ref, lse.cpu().numpy(), L_ref, "fp16 P at the limit, prefill")


def test_fp16_p_below_half_max_decode(fa):
    """The same edge in the decode kernel (32-key blocks)."""
    import torch
    d, dt, L = 64, ai.FP16, 100
    scale, c = _unit_scale()
    announce("fp16 P at the limit (decode)")
    q = np.zeros((1, 4, d), np.float32)
    q[..., 0] = 4.0
    k, v = _fp16_limit_keys(L, 32, 40, d)
    qb, q64 = rc.rounded(q, dt)
    kb, k64 = rc.rounded(np.broadcast_to(k, (1, 1, L, d)).copy(), dt)
    vb, v64 = rc.rounded(np.broadcast_to(v, (1, 1, L, d)).copy(), dt)
    o, lse = fa.decode(to_dev(qb, dt), to_dev(kb, dt), to_dev(vb, dt),
                       torch.tensor([L], dtype=torch.int32, device="cuda"), scale=scale)
    torch.cuda.synchronize()
    O_ref, L_ref = oracle.decode(q64, k64, v64, [L], scale)
    compare(from_dev(o, dt), O_ref, lse.cpu().numpy(), L_ref, "fp16 P at the limit, decode")
