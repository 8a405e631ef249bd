"""fa_decode_noalloc (decode on the library's static workspace) against
fa_decode (decode on a caller-owned workspace), through the C ABI.

Two calls in a row on the same GPU, the second with a smaller input, then the
32-sequence decode workload: each must give bit-identical O and LSE to
fa_decode with the same split plan (same kernels, same work split), and both
must meet the oracle's tolerances. A size whose workspace exceeds the static
array is refused with nothing written.
"""
import math

import numpy as np
import pytest

import attn_inputs as ai
import oracle
from gpu_util import announce, compare, from_dev, to_dev

pytestmark = pytest.mark.gpu


def _both(fa, x, num_splits=0):
    import torch
    dt = x["dtype"]
    q, kc, vc = to_dev(x["q"], dt), to_dev(x["k_cache"], dt), to_dev(x["v_cache"], dt)
    sl = torch.from_numpy(np.asarray(x["seqlens"], np.int32)).cuda()
    B, Hq, d = q.shape
    Hkv, Lcap = kc.shape[1], kc.shape[2]
    o1, l1 = fa.decode(q, kc, vc, sl, num_splits=num_splits)
    o2 = torch.full_like(q, float("nan"))
    l2 = torch.full((B, Hq), float("nan"), device="cuda")
    st = fa.fa_decode_noalloc(q.data_ptr(), kc.data_ptr(), vc.data_ptr(), sl.data_ptr(), o2.data_ptr(),
                              l2.data_ptr(), B, Hq, Hkv, Lcap, d, 1.0 / math.sqrt(d), num_splits, fa.dtype_code(q.dtype),
                              torch.cuda.current_stream().cuda_stream)
    assert st == fa.FA_OK, fa.fa_last_error()
    torch.cuda.synchronize()
    return o1, l1, o2, l2


def _oracle(x):
    dt = x["dtype"]
    f = lambda a: ai.bits_to_f64(a, dt)
    d = x["q"].shape[2]
    B = x["q"].shape[0]
    O = np.zeros(x["q"].shape)
    L = np.zeros(x["q"].shape[:2])
    for b in range(B):
        n = int(x["seqlens"][b])
        O[b:b + 1], L[b:b + 1] = oracle.decode(f(x["q"][b:b + 1]), f(x["k_cache"][b:b + 1, :, :n]),
                                              f(x["v_cache"][b:b + 1, :, :n]), [n], 1.0 / math.sqrt(d))
    return O, L


@pytest.mark.parametrize("case", [
    # seed, B, Hq, Hkv, Lcap, d, dtype, lens, num_splits
    (51, 4, 8, 2, 2048, 128, ai.BF16, [2048, 1, 700, 1500], 0),
    (52, 2, 4, 4, 700, 64, ai.FP16, [699, 33], 3),  # the second call: smaller
], ids=["first", "second_smaller"])
def test_noalloc_matches_decode(fa, case):
    import torch
    seed, B, Hq, Hkv, Lcap, d, dt, lens, ns = case
    announce(f"decode_noalloc B={B} Hq={Hq} Hkv={Hkv} Lcap={Lcap} d={d} {dt} splits={ns}")
    x = ai.decode_inputs(seed, B, Hq, Hkv, Lcap, d, dt, np.asarray(lens, np.int32))
    o1, l1, o2, l2 = _both(fa, x, ns)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    O_ref, L_ref = _oracle(x)
    compare(from_dev(o2, dt), O_ref, l2.cpu().numpy(), L_ref, f"decode_noalloc {case[:7]}")


def test_noalloc_decode_workload(fa):
    """The 32-sequence decode workload (a 34 MB workspace) on the static array."""
    import torch
    c = ai.CONFIGS["decode_32seq_gqa"]
    announce("decode_noalloc on the 32-sequence workload")
    lens = ai.decode_lengths(c["seed"], c["B"], c["len_lo"], c["len_hi"])
    x = ai.decode_inputs(c["seed"], c["B"], c["Hq"], c["Hkv"], c["Lcap"], c["d"], c["dtype"], lens)
    o1, l1, o2, l2 = _both(fa, x)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_noalloc_refuses_oversize(fa):
    import torch
    announce("decode_noalloc refuses a workspace above the static array")
    B, Hq, Hkv, Lcap, d = 64, 32, 8, 32768, 128
    q = torch.zeros((B, Hq, d), dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros((1, 16), dtype=torch.bfloat16, device="cuda")  # never read: refused first
    sl = torch.zeros(B, dtype=torch.int32, device="cuda")
    o = torch.full_like(q, 7.0)
    st = fa.fa_decode_noalloc(q.data_ptr(), kc.data_ptr(), kc.data_ptr(), sl.data_ptr(), o.data_ptr(), None, B, Hq,
                              Hkv, Lcap, d, 0.1, 0, fa.FA_DTYPE_BF16, torch.cuda.current_stream().cuda_stream)
    assert st == fa.FA_ERR_INVALID_ARG and "static" in fa.fa_last_error()
    torch.cuda.synchronize()
    assert bool(torch.all(o == 7.0).item())
