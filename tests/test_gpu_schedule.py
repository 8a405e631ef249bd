"""Both causal prefill schedules against the oracle.

fa_set_prefill_schedule picks how causal query tiles are spread over
workgroups: 256-row tiles heaviest first, or split mode, where a workgroup
takes the 128-row blocks nb-1-p and p of a head and its two wave groups take
the two halves of every key tile, joined at the end by the merge identity of
"The math of Flash Attention" (unite.ai). The automatic choice sends small
causal grids to split mode and large ones to tiles, so each shape below is run
under both forced modes: odd and even block counts, a ragged last block, a
second block of one row, Nq < Nk, multi-query, head widths 64 and 128, both
16-bit types, the reference-point move inside one key half, and the two
full-size workloads in the mode the automatic choice does not take for them.
"""
import contextlib
import math

import numpy as np
import pytest

import attn_inputs as ai
import oracle
import rescale_cases as rc
from gpu_util import announce, compare, from_dev, to_dev
from test_gpu_fwd import full_case, sampled_case

pytestmark = pytest.mark.gpu

MODES = {"tiles": 1, "split": 2}


@contextlib.contextmanager
def schedule(fa, mode):
    prev = fa.fa_set_prefill_schedule(mode)
    assert prev >= 0
    try:
        yield
    finally:
        fa.fa_set_prefill_schedule(prev)


CAUSAL = [
    # B, Hq, Hkv, Nq, Nk, d, dtype
    (1, 2, 1, 1, 1, 128, ai.BF16),        # one row: one block
    (2, 4, 2, 100, 100, 64, ai.BF16),     # one ragged block
    (1, 4, 2, 129, 129, 64, ai.FP16),     # second block of one row
    (1, 4, 2, 256, 256, 128, ai.BF16),    # two full blocks
    (1, 4, 1, 300, 300, 128, ai.BF16),    # three blocks: the middle one alone
    (1, 2, 1, 384, 384, 128, ai.FP16),
    (1, 8, 1, 200, 200, 128, ai.FP16),    # multi-query
    (1, 4, 2, 77, 300, 128, ai.BF16),     # Nq < Nk (bottom-right)
    (1, 2, 1, 513, 700, 64, ai.BF16),
    (2, 4, 4, 640, 1111, 64, ai.BF16),
    (1, 2, 2, 1000, 1000, 64, ai.FP16),
]
IDS = [f"B{c[0]}Hq{c[1]}Hkv{c[2]}Nq{c[3]}Nk{c[4]}d{c[5]}{c[6]}" for c in CAUSAL]


@pytest.mark.parametrize("mode", list(MODES))
@pytest.mark.parametrize("case", CAUSAL, ids=IDS)
def test_causal_shapes(fa, case, mode):
    with schedule(fa, MODES[mode]):
        announce(f"schedule {mode}")
        full_case(fa, 500 + CAUSAL.index(case), *case, True)


@pytest.mark.parametrize("case", [CAUSAL[4], CAUSAL[9]], ids=[IDS[4], IDS[9]])
def test_split_agrees_with_tiles(fa, case):
    import torch
    B, Hq, Hkv, Nq, Nk, d, dt = case
    announce(f"split vs tiles {case}")
    x = ai.prefill_inputs(520, B, Hq, Hkv, Nq, d, dt, Nk=Nk)
    q, k, v = to_dev(x["q"], dt), to_dev(x["k"], dt), to_dev(x["v"], dt)
    outs = {}
    for mode, code in MODES.items():
        with schedule(fa, code):
            outs[mode] = fa.attention(q, k, v, causal=True)
    torch.cuda.synchronize()
    # both are within the oracle bar; between themselves they differ only by
    # the order of the fp32 sums and one rounding of O
    o_t, o_s = (from_dev(outs[m][0], dt) for m in MODES)
    assert np.abs(o_t - o_s).max() <= 2e-2
    assert np.linalg.norm(o_t - o_s) / np.linalg.norm(o_t) <= 4e-3
    assert torch.allclose(outs["tiles"][1], outs["split"][1], atol=1e-4, rtol=0)


@pytest.mark.parametrize("d,dt", [(128, ai.BF16), (64, ai.FP16)])
def test_split_outlier_key(fa, d, dt):
    """~10^5 flat keys and one key 17 log2 units above them: in split mode
    only the group holding the outlier's half tile moves its reference
    point, so the final merge has to rescale one half against the other."""
    import torch
    Nq, Nk, j_out, Hq = 40, 100001, 60000, 2
    scale = 1.0 / math.sqrt(d)
    announce(f"split outlier d={d} {dt}")
    q, k, v = rc.outlier(1, Nq, Nk, d, j_out, 17.0, scale, H=Hq)
    (qb, q64), (kb, k64), (vb, v64) = rc.rounded(q, dt), rc.rounded(k[:1], dt), rc.rounded(v[:1], dt)
    with schedule(fa, MODES["split"]):
        o, lse = fa.attention(to_dev(qb[None], dt), to_dev(kb[None], dt), to_dev(vb[None], dt), causal=True)
    torch.cuda.synchronize()
    O_ref, L_ref = oracle.attention(q64[None], k64[None], v64[None], scale, True)
    compare(from_dev(o, dt), O_ref, lse.cpu().numpy(), L_ref, f"split outlier d={d} {dt}")


def test_tiles_q_times_8(fa):
    """Sharper rows whose later tiles move the reference point, on the
    256-row schedule (the automatic choice splits this grid)."""
    import torch
    B, Hq, Hkv, N, d, dt = 1, 8, 2, 2048, 64, ai.FP16
    announce("tiles Q*8")
    x = ai.prefill_inputs(964, B, Hq, Hkv, N, d, dt)
    q64 = ai.bits_to_f64(x["q"], dt) * 8.0
    qb = ai.round_to_bits(q64.astype(np.float32), dt)
    k64, v64 = ai.bits_to_f64(x["k"], dt), ai.bits_to_f64(x["v"], dt)
    with schedule(fa, MODES["tiles"]):
        o, lse = fa.attention(to_dev(qb, dt), to_dev(x["k"], dt), to_dev(x["v"], dt), causal=True)
    torch.cuda.synchronize()
    O_ref, L_ref = oracle.attention(q64, k64, v64, 1.0 / math.sqrt(d), True)
    compare(from_dev(o, dt), O_ref, lse.cpu().numpy(), L_ref, "tiles Q*8")


def test_mha_n4096_fp16_causal_tiles(fa):
    c = ai.CONFIGS["mha_n4096_fp16"]
    with schedule(fa, MODES["tiles"]):
        full_case(fa, c["seed"], c["B"], c["Hq"], c["Hkv"], c["N"], c["N"], c["d"], c["dtype"], True)


def test_llama3_gqa_n8192_split_sampled(fa):
    with schedule(fa, MODES["split"]):
        sampled_case(fa, "llama3_8b_gqa_n8192", True, 96)
