"""Strided layouts on the GPU (through fa_fwd_strided / fa_fwd_varlen_strided):
the (batch, seq, heads, dim) layout that flash_attn_func takes ("FlashAttention
complete guide for beginners", section 5), padded rows, a packed QKV tensor,
and the packed (total, heads, dim) varlen layout. The addressing changes, the
arithmetic does not: each result is checked against the float64 oracle and
must equal, bit for bit, what fa_fwd / fa_fwd_varlen return on contiguous
copies of the same values."""
import math

import numpy as np
import pytest

import attn_inputs as ai
import oracle
from gpu_util import announce, compare, from_dev, to_dev

pytestmark = pytest.mark.gpu


def contiguous_run(fa, x, causal):
    import torch
    dt = x["dtype"]
    q, k, v = (to_dev(x[n], dt) for n in "qkv")
    o, lse = fa.attention(q, k, v, causal=causal)
    torch.cuda.synchronize()
    return o, lse


def bshd(t):
    """[B,H,N,d] device tensor -> the same values in a (B,N,H,d) tensor."""
    return t.transpose(1, 2).contiguous()


CASES = [
    # B, Hq, Hkv, Nq, Nk, d, dtype, causal
    (2, 8, 2, 333, 333, 128, ai.BF16, True),
    (1, 8, 8, 300, 520, 64, ai.FP16, False),
    (2, 4, 1, 200, 700, 128, ai.FP16, True),   # chunked prefill: Nq < Nk against a longer cache
    (1, 32, 8, 1024, 1024, 128, ai.BF16, True),
]


@pytest.mark.parametrize("case", CASES, ids=[f"c{i}" for i in range(len(CASES))])
def test_bshd_vs_oracle_and_bitwise(fa, case):
    import torch
    B, Hq, Hkv, Nq, Nk, d, dt, causal = case
    announce(f"flash_attn_func BSHD B={B} Hq={Hq} Hkv={Hkv} Nq={Nq} Nk={Nk} d={d} {dt} causal={causal}")
    x = ai.prefill_inputs(500 + CASES.index(case), B, Hq, Hkv, Nq, d, dt, Nk=Nk)
    o_ref_dev, l_ref_dev = contiguous_run(fa, x, causal)
    q, k, v = (bshd(to_dev(x[n], dt)) for n in "qkv")
    o, lse = fa.flash_attn_func(q, k, v, causal=causal, return_lse=True)
    torch.cuda.synchronize()
    assert tuple(o.shape) == (B, Nq, Hq, d) and o.is_contiguous()
    assert torch.equal(o.transpose(1, 2).contiguous().view(torch.int16), o_ref_dev.view(torch.int16))
    assert torch.equal(lse, l_ref_dev)
    f = lambda a: ai.bits_to_f64(a, dt)
    scale = 1.0 / math.sqrt(d)
    rows = np.unique(np.r_[0, Nq - 1, np.random.default_rng(7).integers(0, Nq, 48)])
    fq, fk, fv = f(x["q"]), f(x["k"]), f(x["v"])
    O_ref = np.empty((B, Hq, len(rows), d))
    L_ref = np.empty((B, Hq, len(rows)))
    for b in range(B):
        for h in range(Hq):
            g = h // (Hq // Hkv)
            O_ref[b, h], L_ref[b, h] = oracle.attention_rows(fq[b, h, rows], rows, fk[b, g], fv[b, g], scale,
                                                             causal, Nq)
    o_h = from_dev(o.transpose(1, 2), dt)[:, :, rows]
    compare(o_h, O_ref, lse.cpu().numpy()[:, :, rows], L_ref, f"BSHD {case}")


def test_padded_rows_and_untouched_padding(fa):
    """Rows padded to 192 elements (d=128): inputs are slices of wider
    buffers, the output goes into the first 128 columns of a wider buffer
    whose padding must keep its sentinel."""
    import torch
    B, Hq, Hkv, N, d, dt = 1, 4, 2, 700, 128, ai.BF16
    announce("padded rows d=128 pitch 192")
    x = ai.prefill_inputs(520, B, Hq, Hkv, N, d, dt)
    o_ref, l_ref = contiguous_run(fa, x, True)

    def padded(bits):
        t = to_dev(bits, dt)
        wide = torch.full((*t.shape[:3], 192), float("nan"), dtype=t.dtype, device="cuda")
        wide[..., :d] = t
        return wide[..., :d]

    q, k, v = padded(x["q"]), padded(x["k"]), padded(x["v"])
    assert q.stride(2) == 192 and not q.is_contiguous()
    o_wide = torch.full((B, Hq, N, 192), 7.0, dtype=q.dtype, device="cuda")
    o, lse = fa.attention(q, k, v, causal=True, out=o_wide[..., :d])
    torch.cuda.synchronize()
    assert torch.equal(o.contiguous().view(torch.int16), o_ref.view(torch.int16))
    assert torch.equal(lse, l_ref)
    assert bool((o_wide[..., d:] == 7.0).all())


def test_packed_qkv_views(fa):
    """q, k, v as views into one (B, N, 3, H, d) tensor, as a fused QKV
    projection produces them."""
    import torch
    B, H, N, d, dt = 2, 8, 410, 64, ai.FP16
    announce("packed QKV views")
    x = ai.prefill_inputs(521, B, H, H, N, d, dt)
    o_ref, l_ref = contiguous_run(fa, x, False)
    qkv = torch.stack([bshd(to_dev(x[n], dt)) for n in "qkv"], dim=2)  # [B, N, 3, H, d]
    q, k, v = qkv[:, :, 0], qkv[:, :, 1], qkv[:, :, 2]
    assert q.stride() == (N * 3 * H * d, 3 * H * d, d, 1)
    o, lse = fa.flash_attn_func(q, k, v, causal=False, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(o.transpose(1, 2).contiguous().view(torch.int16), o_ref.view(torch.int16))
    assert torch.equal(lse, l_ref)


def test_varlen_thd_layout(fa):
    """flash_attn_varlen_func's (total, heads, dim) layout against the packed
    [heads, total, dim] call and the oracle."""
    import torch
    lens_q, lens_k = [1, 255, 600, 77], [1, 300, 600, 200]
    Hq, Hkv, d, dt = 8, 2, 128, ai.BF16
    announce(f"varlen THD lens_q={lens_q} lens_k={lens_k}")
    x = ai.varlen_inputs(522, lens_q, lens_k, Hq, Hkv, d, dt)
    q, k, v = (to_dev(x[n], dt) for n in "qkv")   # [H, total, d]
    cq = torch.from_numpy(np.asarray(x["cu_q"], np.int32)).cuda()
    ck = torch.from_numpy(np.asarray(x["cu_k"], np.int32)).cuda()
    o1, l1 = fa.attention_varlen(q, k, v, cq, ck, max(lens_q), causal=True)
    o2, l2 = fa.flash_attn_varlen_func(q.transpose(0, 1).contiguous(), k.transpose(0, 1).contiguous(),
                                       v.transpose(0, 1).contiguous(), cq, ck, max(lens_q), max(lens_k),
                                       causal=True, return_lse=True)
    torch.cuda.synchronize()
    assert tuple(o2.shape) == (sum(lens_q), Hq, d)
    assert torch.equal(o2.transpose(0, 1).contiguous().view(torch.int16), o1.view(torch.int16))
    assert torch.equal(l1, l2)
    f = lambda a: ai.bits_to_f64(a, dt)
    O_ref, L_ref = oracle.attention_varlen(f(x["q"]), f(x["k"]), f(x["v"]), x["cu_q"], x["cu_k"],
                                           1.0 / math.sqrt(d), True)
    compare(from_dev(o2.transpose(0, 1), dt), O_ref, l2.cpu().numpy(), L_ref, "varlen THD")


def test_bshd_llama3_layer_bitwise(fa):
    """The Llama-3-8B GQA layer (B=1, Hq=32, Hkv=8, N=8192, d=128, causal) in
    the (batch, seq, heads, dim) layout returns exactly the contiguous result."""
    import torch
    c = ai.CONFIGS["llama3_8b_gqa_n8192"]
    announce("BSHD Llama-3-8B layer N=8192")
    x = ai.prefill_inputs(c["seed"], c["B"], c["Hq"], c["Hkv"], c["N"], c["d"], c["dtype"])
    o_ref, l_ref = contiguous_run(fa, x, True)
    q, k, v = (bshd(to_dev(x[n], c["dtype"])) for n in "qkv")
    o, lse = fa.flash_attn_func(q, k, v, causal=True, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(o.transpose(1, 2).contiguous().view(torch.int16), o_ref.view(torch.int16))
    assert torch.equal(lse, l_ref)
