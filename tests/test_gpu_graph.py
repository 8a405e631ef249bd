"""Prefill and decode captured in a HIP graph (torch.cuda.CUDAGraph) and
replayed: the kernels allocate nothing, synchronise nothing and take every
buffer from the caller, so a replay must give exactly the eager result. Each
replay follows eager work that overwrites the outputs, and is checked on its
own."""
import numpy as np
import pytest

import attn_inputs as ai
from gpu_util import announce, to_dev

pytestmark = pytest.mark.gpu


def test_graph_replay_prefill_and_decode(fa):
    import torch
    announce("graph capture: prefill B=1 Hq=8 Hkv=2 N=700 d=128 causal + decode B=6 Hq=8 Hkv=2 Lcap=900")
    x = ai.prefill_inputs(41, 1, 8, 2, 700, 128, ai.BF16)
    q, k, v = (to_dev(x[n], ai.BF16) for n in "qkv")
    lens = np.array([900, 1, 0, 333, 640, 77], np.int32)
    xd = ai.decode_inputs(42, 6, 8, 2, 900, 128, ai.BF16, lens)
    qd, kc, vc = (to_dev(xd[n], ai.BF16) for n in ("q", "k_cache", "v_cache"))
    sl = torch.from_numpy(lens).cuda()

    o_e, l_e = fa.attention(q, k, v, causal=True)
    od_e, ld_e = fa.decode(qd, kc, vc, sl)
    torch.cuda.synchronize()

    o_g, l_g = torch.empty_like(o_e), torch.empty_like(l_e)
    od_g, ld_g = torch.empty_like(od_e), torch.empty_like(ld_e)
    ws = torch.empty(fa.fa_decode_workspace_bytes(6, 8, 2, 900, 128, 0), dtype=torch.uint8, device="cuda")

    def step():
        fa.attention(q, k, v, causal=True, out=o_g, lse=l_g)
        fa.decode(qd, kc, vc, sl, workspace=ws, out=od_g, lse=ld_g)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        for t in (o_g, l_g, od_g, ld_g):
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o_g, o_e) and torch.equal(l_g, l_e), f"prefill replay {rep}"
        assert torch.equal(od_g, od_e) and torch.equal(ld_g, ld_e), f"decode replay {rep}"
