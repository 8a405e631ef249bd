"""Caller-supplied outputs and workspaces are refused before any launch.

The C entry points only receive pointers, so the binding checks every tensor
a caller passes for the results: exact shape and dtype, the device of the
inputs, contiguity (or a unit last stride where the entry point takes
strides), and, for a workspace, its size. A refused call raises ValueError
and leaves the tensors it was given untouched.
"""
import numpy as np
import pytest

import attn_inputs as ai
from gpu_util import announce, to_dev

pytestmark = pytest.mark.gpu


def _untouched(t, fill):
    import torch
    torch.cuda.synchronize()
    return bool(torch.all(t == fill).item())


def test_prefill_outputs_checked(fa):
    import torch
    announce("binding checks: prefill out / lse")
    x = ai.prefill_inputs(41, 1, 4, 2, 100, 64, ai.BF16)
    q, k, v = (to_dev(x[n], ai.BF16) for n in "qkv")
    for out, lse in ((torch.full((1, 4, 99, 64), 7.0, dtype=torch.bfloat16, device="cuda"), None),
                     (torch.full((1, 4, 100, 64), 7.0, dtype=torch.float16, device="cuda"), None),
                     (None, torch.full((1, 4, 100), 7.0, dtype=torch.float16, device="cuda")),
                     (None, torch.full((1, 4, 99), 7.0, device="cuda")),
                     (None, torch.full((1, 4, 100), 7.0))):
        with pytest.raises(ValueError):
            fa.attention(q, k, v, out=out, lse=lse)
        assert _untouched(out if out is not None else lse, 7.0)


def test_decode_outputs_checked(fa):
    import torch
    announce("binding checks: decode out / lse / workspace")
    lens = np.array([300, 77], np.int32)
    y = ai.decode_inputs(42, 2, 8, 2, 512, 128, ai.BF16, lens)
    q, kc, vc = to_dev(y["q"], ai.BF16), to_dev(y["k_cache"], ai.BF16), to_dev(y["v_cache"], ai.BF16)
    sl = torch.from_numpy(lens).cuda()
    need = fa.fa_decode_workspace_bytes(2, 8, 2, 512, 128, 0)
    bad = [dict(out=torch.full((2, 8, 127), 7.0, dtype=torch.bfloat16, device="cuda")),
           dict(out=torch.full((2, 8, 128), 7.0, device="cuda")),
           dict(lse=torch.full((2, 7), 7.0, device="cuda")),
           dict(lse=torch.full((2, 8), 7.0, dtype=torch.bfloat16, device="cuda")),
           dict(workspace=torch.full((need - 1,), 7, dtype=torch.uint8, device="cuda")),
           dict(workspace=torch.full((need,), 7, dtype=torch.uint8))]
    for kw in bad:
        with pytest.raises(ValueError):
            fa.decode(q, kc, vc, sl, **kw)
        (t,) = kw.values()
        assert _untouched(t, 7)
    # the paged entry point: the same checks
    pl = ai.paged_layout(y["k_cache"], y["v_cache"], 128, 42, ai.BF16)
    kp, vp = to_dev(pl["k_pages"], ai.BF16), to_dev(pl["v_pages"], ai.BF16)
    table = torch.from_numpy(np.ascontiguousarray(pl["block_table"], np.int32)).cuda()
    for kw in bad[:4]:
        with pytest.raises(ValueError):
            fa.decode_paged(q, kp, vp, table, sl, **kw)


def test_fp8_outputs_checked(fa):
    import torch
    announce("binding checks: fp8 out / lse")
    x = ai.prefill_inputs_fp8(43, 1, 4, 2, 64, 128)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    args = [dev(x["q"]), dev(x["k"]), dev(x["v"]), dev(x["q_descale"]), dev(x["k_descale"]), dev(x["v_descale"])]
    for kw in (dict(out=torch.full((1, 4, 64, 128), 7.0, dtype=torch.float16, device="cuda")),
               dict(out=torch.full((1, 4, 63, 128), 7.0, dtype=torch.bfloat16, device="cuda")),
               dict(lse=torch.full((1, 4, 64), 7.0, dtype=torch.bfloat16, device="cuda"))):
        with pytest.raises(ValueError):
            fa.attention_fp8(*args, **kw)
        (t,) = kw.values()
        assert _untouched(t, 7.0)
