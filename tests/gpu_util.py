"""Helpers for GPU parity tests: move generator bits to the device and back,
and compare against the oracle with the stated tolerances."""
from __future__ import annotations

import sys

import numpy as np

import attn_inputs as ai

# Tolerances against the float64 oracle on O (in the output dtype) and LSE (fp32).
O_MAX_ABS = 2e-2
O_REL_L2 = 5e-3
LSE_MAX_ABS = 1e-3


def torch_dtype(dtype):
    import torch
    return torch.bfloat16 if dtype == ai.BF16 else torch.float16


def to_dev(bits: np.ndarray, dtype: str):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch_dtype(dtype))
    return t.cuda()


def from_dev(t, dtype: str) -> np.ndarray:
    import torch
    return ai.bits_to_f64(t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16), dtype)


def compare(o_gpu, o_ref, lse_gpu=None, lse_ref=None, what=""):
    """Assert parity; return the error metrics."""
    o_gpu = np.asarray(o_gpu, np.float64)
    o_ref = np.asarray(o_ref, np.float64)
    assert np.all(np.isfinite(o_gpu)), f"{what}: non-finite O"
    err = o_gpu - o_ref
    max_abs = float(np.abs(err).max()) if err.size else 0.0
    nrm = float(np.linalg.norm(o_ref))
    rel = float(np.linalg.norm(err) / nrm) if nrm > 0 else float(np.linalg.norm(err))
    m = dict(o_max_abs=max_abs, o_rel_l2=rel)
    if lse_gpu is not None:
        lse_gpu = np.asarray(lse_gpu, np.float64)
        fin = np.isfinite(lse_ref)
        assert np.array_equal(np.isfinite(lse_gpu), fin), f"{what}: LSE finiteness differs"
        m["lse_max_abs"] = float(np.abs(lse_gpu[fin] - lse_ref[fin]).max()) if fin.any() else 0.0
    print(f"[parity] {what}: {m}", file=sys.stderr, flush=True)
    assert max_abs <= O_MAX_ABS, f"{what}: O max-abs {max_abs}"
    assert rel <= O_REL_L2, f"{what}: O rel-L2 {rel}"
    if lse_gpu is not None:
        assert m["lse_max_abs"] <= LSE_MAX_ABS, f"{what}: LSE max-abs {m['lse_max_abs']}"
    return m


def announce(msg):
    print(f"[gpu-step] {msg}", file=sys.stderr, flush=True)
