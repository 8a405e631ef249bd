"""Attention backward on the GPU (fa_bwd through the C ABI) against the float64
gradient oracle. The forward output and LSE fed to fa_bwd come from fa_fwd on
the GPU, as in training; the oracle differentiates the exact definition.

Tolerance (the pages state none for gradients): the kernels round P and dS to
the input type as MFMA operands (relative error up to 2^-9 for bf16) and the
gradients themselves to the input type, and delta uses the rounded O; over the
sums of products that make a gradient element these roundings add up like a
random walk, so the relative L2 error stays a small multiple of 2^-9. The
bar: relative L2 <= 1e-2 per gradient (about five bf16 half-ulps) and every
element within 2e-2 of the largest reference magnitude."""
import math

import numpy as np
import pytest

import attn_inputs as ai
import oracle
from gpu_util import announce, from_dev, to_dev

pytestmark = pytest.mark.gpu

REL_L2 = 1e-2
MAX_ABS_FRAC = 2e-2
ZERO_REF_ABS = 1e-4


def run_gpu(fa, x, do_bits, causal):
    import torch
    dt = x["dtype"]
    q, k, v = (to_dev(x[n], dt) for n in "qkv")
    do = to_dev(do_bits, dt)
    o, lse = fa.attention(q, k, v, causal=causal)
    dq, dk, dv = fa.attention_bwd(q, k, v, o, lse, do, causal=causal)
    torch.cuda.synchronize()
    return dq, dk, dv


def check_grads(got, ref, what):
    import sys
    bad = []
    for name, g, r in zip(("dQ", "dK", "dV"), got, ref):
        if not np.all(np.isfinite(g)):
            bad.append(f"{name}: non-finite")
            continue
        err = g - r
        nrm = float(np.linalg.norm(r))
        rel = float(np.linalg.norm(err) / nrm) if nrm > 0 else float(np.linalg.norm(err))
        mx = float(np.abs(err).max())
        top = float(np.abs(r).max())
        print(f"[parity] {what} {name}: rel_l2={rel:.3e} max_abs={mx:.3e} max_ref={top:.3e}", file=sys.stderr,
              flush=True)
        if top == 0.0:
            # An exactly zero gradient (one visible key: P = 1, so dS = dP -
            # delta = 0) has no relative scale. What is left is the fp32
            # difference of two summation orders of one d-term dot product
            # (dO . V in the MFMA against dO . O in the delta kernel, O = V):
            # below d 2^-24 sum |dO V|, under 1e-4 for N(0,1) inputs.
            if mx > ZERO_REF_ABS:
                bad.append(f"{name}: max-abs {mx} against an exactly zero reference")
            continue
        if rel > REL_L2:
            bad.append(f"{name}: rel-L2 {rel}")
        if mx > MAX_ABS_FRAC * top:
            bad.append(f"{name}: max-abs {mx} vs max |ref| {top}")
    assert not bad, f"{what}: " + "; ".join(bad)


CASES = [
    # B, Hq, Hkv, Nq, Nk, d, dtype, causal
    (1, 8, 8, 128, 128, 64, ai.BF16, False),
    (1, 4, 2, 200, 200, 128, ai.BF16, True),
    (2, 2, 2, 300, 450, 64, ai.FP16, False),
    (1, 8, 2, 150, 400, 128, ai.BF16, True),     # causal Nq < Nk (chunked prefill)
    (1, 4, 4, 513, 513, 64, ai.BF16, True),
    (1, 4, 1, 257, 1000, 128, ai.FP16, False),
    # dK/dV splits each key group's accumulation between two waves and hands
    # P / dS over through LDS; a row half above the diagonal counts as zero
    (1, 2, 1, 1, 1, 64, ai.FP16, True),          # one row, one key
    (2, 6, 2, 77, 77, 128, ai.BF16, True),       # three q-heads per kv-head, one ragged tile
    (1, 4, 2, 640, 1100, 64, ai.FP16, True),     # causal Nq < Nk, ragged key blocks
    (1, 2, 2, 1000, 1000, 128, ai.FP16, True),   # key blocks walking down and up
]


@pytest.mark.parametrize("case", CASES, ids=[f"c{i}" for i in range(len(CASES))])
def test_bwd_vs_oracle(fa, case):
    B, Hq, Hkv, Nq, Nk, d, dt, causal = case
    announce(f"fa_bwd B={B} Hq={Hq} Hkv={Hkv} Nq={Nq} Nk={Nk} d={d} {dt} causal={causal}")
    seed = 600 + CASES.index(case)
    x = ai.prefill_inputs(seed, B, Hq, Hkv, Nq, d, dt, Nk=Nk)
    do_bits = ai.grad_output(seed, B, Hq, Nq, d, dt)
    dq, dk, dv = run_gpu(fa, x, do_bits, causal)
    f = lambda a: ai.bits_to_f64(a, dt)
    ref = oracle.attention_bwd(f(x["q"]), f(x["k"]), f(x["v"]), f(do_bits), 1.0 / math.sqrt(d), causal)
    check_grads([from_dev(t, dt) for t in (dq, dk, dv)], ref, f"bwd {case}")


def _random_bwd_cases(n=10, seed=47):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        d = int(rng.choice([64, 128]))
        Hkv = int(rng.choice([1, 2, 4]))
        Hq = Hkv * int(rng.choice([1, 2, 3, 4]))
        Nk = int(rng.integers(1, 900))
        causal = bool(rng.random() < 0.6)
        Nq = int(rng.integers(1, Nk + 1)) if causal else int(rng.integers(1, 900))
        dt = ai.BF16 if rng.random() < 0.5 else ai.FP16
        cases.append((640 + i, int(rng.integers(1, 3)), Hq, Hkv, Nq, Nk, d, dt, causal))
    return cases


@pytest.mark.parametrize("case", _random_bwd_cases(),
                         ids=lambda c: f"s{c[0]}B{c[1]}Hq{c[2]}Hkv{c[3]}Nq{c[4]}Nk{c[5]}d{c[6]}{c[7]}{'c' if c[8] else 'n'}")
def test_bwd_random_shapes(fa, case):
    # Seeded shapes: ragged query and key tails, GQA groups of 1-4 (3 too),
    # causal with Nq <= Nk, both head widths and 16-bit types.
    seed, B, Hq, Hkv, Nq, Nk, d, dt, causal = case
    announce(f"fa_bwd random {case}")
    x = ai.prefill_inputs(seed, B, Hq, Hkv, Nq, d, dt, Nk=Nk)
    do_bits = ai.grad_output(seed, B, Hq, Nq, d, dt)
    dq, dk, dv = run_gpu(fa, x, do_bits, causal)
    f = lambda a: ai.bits_to_f64(a, dt)
    ref = oracle.attention_bwd(f(x["q"]), f(x["k"]), f(x["v"]), f(do_bits), 1.0 / math.sqrt(d), causal)
    check_grads([from_dev(t, dt) for t in (dq, dk, dv)], ref, f"bwd random {case}")


def test_bwd_deterministic(fa):
    """No atomics: two calls give the same bits."""
    import torch
    announce("fa_bwd determinism")
    x = ai.prefill_inputs(620, 1, 8, 2, 700, 128, ai.BF16)
    do_bits = ai.grad_output(620, 1, 8, 700, 128, ai.BF16)
    a = run_gpu(fa, x, do_bits, True)
    b = run_gpu(fa, x, do_bits, True)
    for u, w in zip(a, b):
        assert torch.equal(u.view(torch.int16), w.view(torch.int16))


def test_bwd_llama3_layer_sampled(fa):
    """The Llama-3-8B GQA layer (B=1, Hq=32, Hkv=8, N=8192, d=128, causal):
    all of dQ, dK, dV finite, and for the last kv-head (with its 4 q-heads)
    the gradients of sampled rows against the oracle over the full sequence."""
    import torch
    c = ai.CONFIGS["llama3_8b_gqa_n8192"]
    B, Hq, Hkv, N, d, dt = c["B"], c["Hq"], c["Hkv"], c["N"], c["d"], c["dtype"]
    announce("fa_bwd Llama-3-8B layer N=8192")
    x = ai.prefill_inputs(c["seed"], B, Hq, Hkv, N, d, dt)
    do_bits = ai.grad_output(c["seed"], B, Hq, N, d, dt)
    dq, dk, dv = run_gpu(fa, x, do_bits, True)
    for t in (dq, dk, dv):
        assert bool(torch.isfinite(t.float()).all())
    f = lambda a: ai.bits_to_f64(a, dt)
    grp = Hq // Hkv
    rows = np.unique(np.r_[0, 1, N - 1, np.random.default_rng(11).integers(0, N, 24)])
    for g in (Hkv - 1,):
        hs = range(g * grp, (g + 1) * grp)
        # one kv-head with its q-heads as a small grouped problem of its own
        ref = oracle.attention_bwd(f(x["q"][:, hs]), f(x["k"][:, g:g + 1]), f(x["v"][:, g:g + 1]),
                                   f(do_bits[:, hs]), 1.0 / math.sqrt(d), True)
        got = (from_dev(dq[:, hs.start:hs.stop], dt), from_dev(dk[:, g:g + 1], dt), from_dev(dv[:, g:g + 1], dt))
        check_grads([got[0][:, :, rows], got[1][:, :, rows], got[2][:, :, rows]],
                    [ref[0][:, :, rows], ref[1][:, :, rows], ref[2][:, :, rows]], f"bwd llama3 kv-head {g}")


def test_flash_attn_func_autograd(fa):
    """flash_attn_func on tensors that require grad: loss.backward() runs
    fa_bwd, and the gradients match the float64 oracle (BSHD layout, GQA,
    causal)."""
    import torch
    B, Hq, Hkv, N, d, dt = 1, 8, 2, 300, 128, ai.BF16
    announce("flash_attn_func autograd")
    x = ai.prefill_inputs(640, B, Hq, Hkv, N, d, dt)
    do_bits = ai.grad_output(640, B, Hq, N, d, dt)
    q, k, v = (to_dev(x[n], dt).transpose(1, 2).contiguous().requires_grad_(True) for n in "qkv")
    do = to_dev(do_bits, dt).transpose(1, 2).contiguous()
    out = fa.flash_attn_func(q, k, v, causal=True)
    assert out.requires_grad and tuple(out.shape) == (B, N, Hq, d)
    out.backward(do)
    torch.cuda.synchronize()
    f = lambda a: ai.bits_to_f64(a, dt)
    ref = oracle.attention_bwd(f(x["q"]), f(x["k"]), f(x["v"]), f(do_bits), 1.0 / math.sqrt(d), True)
    got = [from_dev(t.grad.transpose(1, 2), dt) for t in (q, k, v)]
    check_grads(got, ref, "flash_attn_func autograd")
