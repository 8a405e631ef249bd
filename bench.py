#!/usr/bin/env python3
"""Benchmark: exact attention forward (prefill) and split-KV decode on one MI355X.

One step = one pass of the whole path over one batch of synthetic input:
  * prefill fa_fwd on the Llama-3-8B-shaped layer (B=1, Hq=32, Hkv=8,
    N=8192, d=128, causal, bf16), the configuration the metric is quoted on;
  * decode fa_decode (split + combine) for 32 sequences x 1 token, Hq=32,
    Hkv=8, d=128, bf16, cache lengths uniform in [1024, 32768].
Inputs are generated once, copied to HBM, and stay resident; the timed region
holds only the library calls. Each call is bracketed by HIP events on the
stream it is launched on. Before the W warmup steps, untimed steps run back to
back for --settle seconds (0.5 by default) so that the GPU has left its idle
clocks; the K timed steps are then exactly K passes of the whole path.

Prints ONE JSON line on stdout. `value` is prefill TFLOP/s counting
4*B*Hq*Nq*Nk*d FLOPs halved for causal; `decode` carries decode GB/s counting
the K/V rows actually read plus q, o and lse. `roofline` is the prefill
kernel against the bf16 dense MFMA peak; `decode.roofline` the decode split
kernel against HBM peak. `cpu_baseline` times the float64 oracle on a bounded
sample of the same workload on the host cores.

Other modes (used to take rocprofv3 counter readings):
  --calibrate-copy   time a plain device copy of known size (counter scale)
  --config NAME      a single configuration (tiny_mha_n128, mha_n4096_fp16,
                     mha_n4096_fp16_causal, llama3_8b_gqa_n8192, llama3_8b_gqa_n131072,
                     decode_32seq_gqa, decode_32seq_gqa_paged: the same decode with
                     the cache in 128-row pages in a shuffled page order,
                     llama3_8b_gqa_varlen: packed causal prefill of 16
                     sequences with lengths U[512, 8192])
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import attn_inputs as ai  # noqa: E402

MFMA_PEAK_TFLOPS = 2516.6   # MI355X dense bf16/fp16 MFMA: 256 CU x 2.4 GHz x 4096 FLOP/clk
MFMA_PEAK_FP8_TFLOPS = 5033.2  # dense FP8 MFMA: twice the 16-bit rate
HBM_PEAK_GBS = 8000.0       # MI355X HBM3E
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "exact_tiled_attention_fwd_amd", "csrc")
KERNEL_SOURCES = [os.path.join(CSRC, f)
                  for f in ("fa_tile.h", "fa_fwd.hip", "fa_decode.hip", "fa_launch.h", "fa_api.cpp")]
# The device code behind each measured kernel (its counter summary records these).
FWD_SOURCES = ("fa_fwd.hip", "fa_tile.h", "fa_launch.h")
DECODE_SOURCES = ("fa_decode.hip", "fa_tile.h", "fa_launch.h")
BWD_SOURCES = ("fa_bwd.hip", "fa_bwd_launch.h", "fa_tile.h", "fa_launch.h")
FP8_SOURCES = ("fa_fwd_fp8.hip", "fa_fp8_launch.h", "fa_tile.h", "fa_launch.h")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ------------------------------------------------------------------ accounting
def prefill_flops(B, Hq, Nq, Nk, d, causal):
    f = 4.0 * B * Hq * Nq * Nk * d
    return f / 2 if causal else f


def prefill_bytes(B, Hq, Hkv, Nq, Nk, d, elem=2):
    """Q, K, V read once; O and LSE written once."""
    return elem * (2 * B * Hq * Nq * d + 2 * B * Hkv * Nk * d) + 4 * B * Hq * Nq


def decode_bytes(lens, Hq, Hkv, d, elem=2):
    """K/V rows actually read, plus q read, o and lse written."""
    B = len(lens)
    kv = sum(int(L) for L in lens) * Hkv * d * 2 * elem
    return kv + 2 * elem * B * Hq * d + 4 * B * Hq


def kv_cache_bytes(seq_len, layers, hidden, bytes_per_value):
    """Per-sequence cache size: 2 (K and V) x layers x hidden x bytes per token."""
    return seq_len * 2 * layers * hidden * bytes_per_value


def kernel_source_hash(files=None):
    """sha256 prefix over the named csrc files (default: all kernel sources)."""
    h = hashlib.sha256()
    paths = KERNEL_SOURCES if files is None else [os.path.join(CSRC, f) for f in files]
    for p in paths:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def counter_traffic(name):
    """HBM bytes per launch from a committed counter summary, if the kernel
    sources it names still hash to the recorded value; else None."""
    path = os.path.join(PROFILES, name)
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_files = re.search(r"kernel_sources:\s*(.+)", text)
    m_src = re.search(r"kernel_source_sha256:\s*([0-9a-f]+)", text)
    m_b = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_files or not m_src or not m_b:
        return None
    try:
        if m_src.group(1) != kernel_source_hash(m_files.group(1).split()):
            return None
    except OSError:  # a source the summary names no longer exists
        return None
    return float(m_b.group(1))


def counter_clock_ghz(name):
    """Shader clock (GHz) measured during the kernel, from a committed counter
    summary whose kernel sources still hash to the recorded value; else None."""
    path = os.path.join(PROFILES, name)
    if counter_traffic(name) is None:
        return None
    m = re.search(r"dispatch time:\s*([0-9.]+) GHz", open(path).read())
    return float(m.group(1)) if m else None


# ------------------------------------------------------------------ device data
def to_dev(bits, dtype):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16 if dtype == ai.BF16 else torch.float16).cuda()


class Prefill:
    """One prefill layer; layout "bhnd" holds q, k, v, o as [B, H, N, d],
    "bshd" as (batch, seq, heads, dim) tensors read and written in place
    through their strides."""

    def __init__(self, fa, name, causal, layout="bhnd"):
        import torch
        c = ai.CONFIGS[name]
        self.fa, self.name, self.causal = fa, name, causal
        self.B, self.Hq, self.Hkv, self.N, self.d, self.dtype = c["B"], c["Hq"], c["Hkv"], c["N"], c["d"], c["dtype"]
        t0 = time.time()
        x = ai.prefill_inputs(c["seed"], self.B, self.Hq, self.Hkv, self.N, self.d, self.dtype)
        self.q, self.k, self.v = to_dev(x["q"], self.dtype), to_dev(x["k"], self.dtype), to_dev(x["v"], self.dtype)
        del x
        self.o = torch.empty_like(self.q)
        if layout == "bshd":
            # the (B, N, H, d) storage, seen as [B, H, N, d] views
            self.q, self.k, self.v, self.o = (t.transpose(1, 2).contiguous().transpose(1, 2)
                                              for t in (self.q, self.k, self.v, self.o))
        self.lse = torch.empty((self.B, self.Hq, self.N), dtype=torch.float32, device="cuda")
        self.flops = prefill_flops(self.B, self.Hq, self.N, self.N, self.d, causal)
        self.bytes = prefill_bytes(self.B, self.Hq, self.Hkv, self.N, self.N, self.d)
        log(f"[bench] {name} causal={causal}: inputs ready in {time.time() - t0:.1f}s")

    def __call__(self):
        self.fa.attention(self.q, self.k, self.v, causal=self.causal, out=self.o, lse=self.lse)


class PrefillFp8:
    """The Llama-3 layer with E4M3 inputs (per-slab power-of-two descales);
    output bf16. Same FLOP count as the 16-bit layer; the FP8 matrix-core
    peak is twice the 16-bit one."""

    def __init__(self, fa, name, causal):
        import torch
        c = ai.CONFIGS[name]
        self.fa, self.causal = fa, causal
        B, Hq, Hkv, N, d = c["B"], c["Hq"], c["Hkv"], c["N"], c["d"]
        t0 = time.time()
        x = ai.prefill_inputs_fp8(c["seed"], B, Hq, Hkv, N, d)
        self.q, self.k, self.v = (torch.from_numpy(x[n]).cuda() for n in "qkv")
        self.ds = [torch.from_numpy(x[n + "_descale"]).cuda() for n in "qkv"]
        del x
        self.o = torch.empty((B, Hq, N, d), dtype=torch.bfloat16, device="cuda")
        self.lse = torch.empty((B, Hq, N), dtype=torch.float32, device="cuda")
        self.flops = prefill_flops(B, Hq, N, N, d, causal)
        # q, k, v one byte per element; o bf16; lse fp32
        self.bytes = (B * Hq * N * d + 2 * B * Hkv * N * d) + 2 * B * Hq * N * d + 4 * B * Hq * N
        log(f"[bench] {name} fp8 causal={causal}: inputs ready in {time.time() - t0:.1f}s")

    def __call__(self):
        self.fa.attention_fp8(self.q, self.k, self.v, *self.ds, causal=self.causal, out=self.o, lse=self.lse)


class Backward:
    """dQ, dK, dV of one prefill layer (fa_bwd: delta, dK/dV and dQ kernels),
    with O and LSE from the forward and a seeded N(0,1) upstream gradient.
    FLOPs count the five products of the gradient (2.5x the forward's)."""

    def __init__(self, fa, name, causal):
        import torch
        c = ai.CONFIGS[name]
        self.fa, self.causal = fa, causal
        B, Hq, Hkv, N, d, dt = c["B"], c["Hq"], c["Hkv"], c["N"], c["d"], c["dtype"]
        t0 = time.time()
        x = ai.prefill_inputs(c["seed"], B, Hq, Hkv, N, d, dt)
        self.q, self.k, self.v = to_dev(x["q"], dt), to_dev(x["k"], dt), to_dev(x["v"], dt)
        del x
        self.do = to_dev(ai.grad_output(c["seed"], B, Hq, N, d, dt), dt)
        self.o, self.lse = fa.attention(self.q, self.k, self.v, causal=causal)
        self.dq, self.dk, self.dv = (torch.empty_like(t) for t in (self.q, self.k, self.v))
        self.ws = torch.empty(fa.fa_bwd_workspace_bytes(B, Hq, N), dtype=torch.uint8, device="cuda")
        self.flops = 2.5 * prefill_flops(B, Hq, N, N, d, causal)
        # reads q, k, v, o, dO, lse; writes dq, dk, dv
        self.bytes = 2 * (4 * B * Hq * N * d + 4 * B * Hkv * N * d) + 4 * B * Hq * N
        log(f"[bench] {name} backward causal={causal}: inputs ready in {time.time() - t0:.1f}s")

    def __call__(self):
        self.fa.attention_bwd(self.q, self.k, self.v, self.o, self.lse, self.do, causal=self.causal,
                              dq=self.dq, dk=self.dk, dv=self.dv, workspace=self.ws)


class PrefillVarlen:
    """Packed causal prefill: 16 Llama-3-shaped sequences of seeded lengths,
    one slab per head, no padding. FLOPs sum the per-sequence counts."""

    def __init__(self, fa, name="llama3_8b_gqa_varlen"):
        import torch
        c = ai.CONFIGS[name]
        self.fa = fa
        t0 = time.time()
        self.lens = ai.decode_lengths(c["seed"], c["B"], c["len_lo"], c["len_hi"])
        x = ai.varlen_inputs(c["seed"], self.lens, self.lens, c["Hq"], c["Hkv"], c["d"], c["dtype"])
        self.q, self.k, self.v = to_dev(x["q"], c["dtype"]), to_dev(x["k"], c["dtype"]), to_dev(x["v"], c["dtype"])
        self.cu_q = torch.from_numpy(x["cu_q"]).cuda()
        self.cu_k = torch.from_numpy(x["cu_k"]).cuda()
        del x
        self.max_q = int(self.lens.max())
        self.o = torch.empty_like(self.q)
        self.lse = torch.empty((c["Hq"], self.q.shape[1]), dtype=torch.float32, device="cuda")
        self.flops = sum(prefill_flops(1, c["Hq"], int(n), int(n), c["d"], True) for n in self.lens)
        self.bytes = sum(prefill_bytes(1, c["Hq"], c["Hkv"], int(n), int(n), c["d"]) for n in self.lens)
        log(f"[bench] {name}: {len(self.lens)} sequences, {int(self.lens.sum())} tokens, "
            f"inputs ready in {time.time() - t0:.1f}s")

    def __call__(self):
        self.fa.attention_varlen(self.q, self.k, self.v, self.cu_q, self.cu_k, self.max_q, causal=True,
                                 out=self.o, lse=self.lse)


class Decode:
    def __init__(self, fa, name="decode_32seq_gqa", num_splits=0):
        import torch
        c = ai.CONFIGS[name]
        self.fa = fa
        self.B, self.Hq, self.Hkv, self.Lcap, self.d, self.dtype = c["B"], c["Hq"], c["Hkv"], c["Lcap"], c["d"], c["dtype"]
        t0 = time.time()
        self.lens = ai.decode_lengths(c["seed"], self.B, c["len_lo"], c["len_hi"])
        x = ai.decode_inputs(c["seed"], self.B, self.Hq, self.Hkv, self.Lcap, self.d, self.dtype, self.lens)
        self.q = to_dev(x["q"], self.dtype)
        self.kc = to_dev(x["k_cache"], self.dtype)
        self.vc = to_dev(x["v_cache"], self.dtype)
        del x
        self.seqlens = torch.from_numpy(self.lens).cuda()
        self.num_splits = num_splits
        ws = fa.fa_decode_workspace_bytes(self.B, self.Hq, self.Hkv, self.Lcap, self.d, num_splits)
        self.ws = torch.empty(ws, dtype=torch.uint8, device="cuda")
        self.o = torch.empty_like(self.q)
        self.lse = torch.empty((self.B, self.Hq), dtype=torch.float32, device="cuda")
        self.bytes = decode_bytes(self.lens, self.Hq, self.Hkv, self.d)
        self.flops = 4.0 * float(self.lens.sum()) * self.Hq * self.d
        log(f"[bench] decode: inputs ready in {time.time() - t0:.1f}s, sum(len)={int(self.lens.sum())}, "
            f"workspace {ws / 2**20:.1f} MiB")

    def __call__(self):
        self.fa.decode(self.q, self.kc, self.vc, self.seqlens, num_splits=self.num_splits,
                       workspace=self.ws, out=self.o, lse=self.lse)


class DecodePaged(Decode):
    """The 32-sequence decode with each cache scattered over 128-row pages in
    a seeded shuffled order (the same logical caches and byte count)."""

    def __init__(self, fa, name="decode_32seq_gqa", num_splits=0, page_size=128):
        import torch
        c = ai.CONFIGS[name]
        self.fa = fa
        self.B, self.Hq, self.Hkv, self.Lcap, self.d, self.dtype = c["B"], c["Hq"], c["Hkv"], c["Lcap"], c["d"], c["dtype"]
        self.page_size = page_size
        t0 = time.time()
        self.lens = ai.decode_lengths(c["seed"], self.B, c["len_lo"], c["len_hi"])
        x = ai.decode_inputs(c["seed"], self.B, self.Hq, self.Hkv, self.Lcap, self.d, self.dtype, self.lens)
        self.q = to_dev(x["q"], self.dtype)
        pl = ai.paged_layout(x["k_cache"], x["v_cache"], page_size, c["seed"], self.dtype)
        del x
        self.kp = to_dev(pl["k_pages"], self.dtype)
        self.vp = to_dev(pl["v_pages"], self.dtype)
        self.table = torch.from_numpy(np.ascontiguousarray(pl["block_table"], np.int32)).cuda()
        del pl
        self.seqlens = torch.from_numpy(self.lens).cuda()
        self.num_splits = num_splits
        ws = fa.fa_decode_workspace_bytes(self.B, self.Hq, self.Hkv, self.Lcap, self.d, num_splits)
        self.ws = torch.empty(ws, dtype=torch.uint8, device="cuda")
        self.o = torch.empty_like(self.q)
        self.lse = torch.empty((self.B, self.Hq), dtype=torch.float32, device="cuda")
        self.bytes = decode_bytes(self.lens, self.Hq, self.Hkv, self.d)
        log(f"[bench] paged decode (page {page_size}): inputs ready in {time.time() - t0:.1f}s")

    def __call__(self):
        self.fa.decode_paged(self.q, self.kp, self.vp, self.table, self.seqlens, num_splits=self.num_splits,
                             workspace=self.ws, out=self.o, lse=self.lse)


def settle(parts, seconds, max_steps=20000):
    """Run untimed steps back to back for `seconds` of wall time.

    Coming out of idle, the GPU raises its clocks over the first tens of
    milliseconds of sustained work: on one MI355X the Llama-3 prefill took
    0.60 ms per call at first and 0.475 ms from about the 40th call on. A few
    warmup steps end inside that ramp, so the timed steps would measure it
    instead of the kernels. Steps go out in batches of 8 between
    synchronisations, so the GPU stays busy. Returns the steps run."""
    import torch
    n = 0
    t_end = time.perf_counter() + seconds
    while n < max_steps and time.perf_counter() < t_end:
        for _ in range(8):
            for p in parts:
                p()
        n += 8
        torch.cuda.synchronize()
    return n


def time_steps(parts, steps, warmup):
    """Warm up, then time exactly `steps` steps; per-part event timings."""
    import torch
    for _ in range(warmup):
        for p in parts:
            p()
    torch.cuda.synchronize()
    evs = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in parts]
           for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(steps):
        for i, p in enumerate(parts):
            evs[s][i][0].record()
            p()
            evs[s][i][1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = [[evs[s][i][0].elapsed_time(evs[s][i][1]) for s in range(steps)] for i in range(len(parts))]
    return wall, per


# ------------------------------------------------------------------ CPU baseline
def cpu_cores_used():
    cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        blas = [i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"]
        if blas:
            return min(cores, max(blas))
    except Exception:
        pass
    return cores


def cpu_baseline_prefill(name="llama3_8b_gqa_n8192", heads=32, fp8=False):
    """The oracle on `heads` full heads of the prefill workload (all query rows,
    all keys, causal): TFLOP/s by the same FLOP convention as the GPU. With
    fp8, the inputs are the values the E4M3 workload's codes stand for."""
    import oracle
    c = ai.CONFIGS[name]
    N, d, dt, grp = c["N"], c["d"], c["dtype"], c["Hq"] // c["Hkv"]
    scale = 1.0 / math.sqrt(d)
    x8 = ai.prefill_inputs_fp8(c["seed"], 1, c["Hq"], c["Hkv"], N, d) if fp8 else None
    elapsed = 0.0
    for h in range(heads):
        g = h // grp
        if fp8:
            q = ai.fp8_decode(x8["q"][0, h]) * float(x8["q_descale"][0, h])
            k = ai.fp8_decode(x8["k"][0, g]) * float(x8["k_descale"][0, g])
            v = ai.fp8_decode(x8["v"][0, g]) * float(x8["v_descale"][0, g])
        else:
            q = ai.bits_to_f64(ai.slab(c["seed"], ai.Q_ID, 0, h, N, d, dt), dt)
            k = ai.bits_to_f64(ai.slab(c["seed"], ai.K_ID, 0, g, N, d, dt), dt)
            v = ai.bits_to_f64(ai.slab(c["seed"], ai.V_ID, 0, g, N, d, dt), dt)
        t0 = time.perf_counter()
        oracle.attention_head(q, k, v, scale, causal=True)
        elapsed += time.perf_counter() - t0
    flops = prefill_flops(1, heads, N, N, d, True)
    return {"value": flops / elapsed / 1e12, "unit": "TFLOP/s", "cores": cpu_cores_used(), "kind": "oracle",
            "sample": f"{heads} of 32 q-heads of the N=8192 causal layer{' (E4M3 inputs, dequantized)' if fp8 else ''}, "
                      f"all 8192 query rows each (float64 NumPy, score matrix materialised); {elapsed:.1f}s"}


def cpu_baseline_full(name, causal):
    """The oracle on every (batch, q-head) of a small prefill workload (all
    rows, all keys): TFLOP/s by the GPU's FLOP convention."""
    import oracle
    c = ai.CONFIGS[name]
    B, Hq, N, d, dt, grp = c["B"], c["Hq"], c["N"], c["d"], c["dtype"], c["Hq"] // c["Hkv"]
    scale = 1.0 / math.sqrt(d)
    elapsed = 0.0
    for b in range(B):
        for h in range(Hq):
            q = ai.bits_to_f64(ai.slab(c["seed"], ai.Q_ID, b, h, N, d, dt), dt)
            k = ai.bits_to_f64(ai.slab(c["seed"], ai.K_ID, b, h // grp, N, d, dt), dt)
            v = ai.bits_to_f64(ai.slab(c["seed"], ai.V_ID, b, h // grp, N, d, dt), dt)
            t0 = time.perf_counter()
            oracle.attention_head(q, k, v, scale, causal=causal)
            elapsed += time.perf_counter() - t0
    flops = prefill_flops(B, Hq, N, N, d, causal)
    return {"value": flops / elapsed / 1e12, "unit": "TFLOP/s", "cores": cpu_cores_used(), "kind": "oracle",
            "sample": f"the whole workload ({B} x {Hq} heads, N={N}, causal={causal}; float64 NumPy, score matrix "
                      f"materialised); {elapsed:.1f}s"}


def cpu_baseline_sampled(name="llama3_8b_gqa_n131072"):
    """The oracle on the sampled query rows of every q-head of the long-context
    workload (each row against all of its visible keys): TFLOP/s by the GPU's
    FLOP convention over the sampled rows, and the full layer's time at that
    rate."""
    import oracle
    c = ai.CONFIGS[name]
    Hq, N, d, dt, grp, count = c["Hq"], c["N"], c["d"], c["dtype"], c["Hq"] // c["Hkv"], c["sample_rows"]
    scale = 1.0 / math.sqrt(d)
    elapsed = 0.0
    flops = 0.0
    kv = {}
    for h in range(Hq):
        g = h // grp
        if g not in kv:
            kv = {g: (ai.bits_to_f64(ai.slab(c["seed"], ai.K_ID, 0, g, N, d, dt), dt),
                      ai.bits_to_f64(ai.slab(c["seed"], ai.V_ID, 0, g, N, d, dt), dt))}
        k, v = kv[g]
        rows = ai.sample_rows(c["seed"], h, N, count)
        q = ai.bits_to_f64(ai.slab(c["seed"], ai.Q_ID, 0, h, N, d, dt)[rows], dt)
        t0 = time.perf_counter()
        oracle.attention_rows(q, rows, k, v, scale, True, N)
        elapsed += time.perf_counter() - t0
        flops += 4.0 * d * float(np.sum(rows + 1))  # row r sees keys 0..r
    rate = flops / elapsed
    full_s = prefill_flops(1, Hq, N, N, d, True) / rate
    return {"value": rate / 1e12, "unit": "TFLOP/s", "cores": cpu_cores_used(), "kind": "oracle",
            "sample": f"{count} sampled query rows of each of the {Hq} q-heads against all their visible keys "
                      f"(float64 NumPy); {elapsed:.1f}s; the whole N={N} layer would take about {full_s:.0f}s "
                      "at this rate (extrapolated)"}


def cpu_baseline_backward(name="llama3_8b_gqa_n8192", heads=4):
    """The gradient oracle on `heads` q-heads (one kv-head group) of the
    backward workload, all rows and keys, causal: TFLOP/s by the GPU's FLOP
    convention (2.5x the forward's)."""
    import oracle
    c = ai.CONFIGS[name]
    N, d, dt = c["N"], c["d"], c["dtype"]
    f = lambda a: ai.bits_to_f64(a, dt)
    q = np.stack([f(ai.slab(c["seed"], ai.Q_ID, 0, h, N, d, dt)) for h in range(heads)])[None]
    do = np.stack([f(ai.slab(c["seed"], ai.DO_ID, 0, h, N, d, dt)) for h in range(heads)])[None]
    k = f(ai.slab(c["seed"], ai.K_ID, 0, 0, N, d, dt))[None, None]
    v = f(ai.slab(c["seed"], ai.V_ID, 0, 0, N, d, dt))[None, None]
    t0 = time.perf_counter()
    oracle.attention_bwd(q, k, v, do, 1.0 / math.sqrt(d), True)
    elapsed = time.perf_counter() - t0
    flops = 2.5 * prefill_flops(1, heads, N, N, d, True)
    return {"value": flops / elapsed / 1e12, "unit": "TFLOP/s", "cores": cpu_cores_used(), "kind": "oracle",
            "sample": f"{heads} of 32 q-heads (kv-head 0's group) of the N=8192 causal layer, all rows and keys "
                      f"(float64 NumPy gradients, score matrix materialised); {elapsed:.1f}s"}


def cpu_baseline_varlen(name="llama3_8b_gqa_varlen", seqs=16, heads=4):
    """The oracle's packed prefill on the first `seqs` sequences, `heads`
    q-heads each (all rows, causal): TFLOP/s by the GPU's FLOP convention."""
    import oracle
    c = ai.CONFIGS[name]
    lens = ai.decode_lengths(c["seed"], c["B"], c["len_lo"], c["len_hi"])[:seqs]
    x = ai.varlen_inputs(c["seed"], lens, lens, heads, max(1, heads // (c["Hq"] // c["Hkv"])), c["d"], c["dtype"])
    f = lambda a: ai.bits_to_f64(a, c["dtype"])
    q, k, v = f(x["q"]), f(x["k"]), f(x["v"])
    t0 = time.perf_counter()
    oracle.attention_varlen(q, k, v, x["cu_q"], x["cu_k"], 1.0 / math.sqrt(c["d"]), causal=True)
    elapsed = time.perf_counter() - t0
    flops = sum(prefill_flops(1, heads, int(n), int(n), c["d"], True) for n in lens)
    return {"value": flops / elapsed / 1e12, "unit": "TFLOP/s", "cores": cpu_cores_used(), "kind": "oracle",
            "sample": f"first {seqs} of {c['B']} sequences (lengths {lens.tolist()}), {heads} of 32 q-heads, "
                      f"all rows, causal (float64 NumPy); {elapsed:.1f}s"}


def cpu_baseline_decode(name="decode_32seq_gqa", seqs=32, page_size=0, min_seconds=10.0):
    """The oracle's decode (paged decode when page_size > 0, through a
    shuffled page table) on the first `seqs` sequences: GB/s by the same byte
    count as the GPU. One pass takes well under a second, so each sequence's
    call is repeated until its share (by length) of `min_seconds` is spent."""
    import oracle
    c = ai.CONFIGS[name]
    lens = ai.decode_lengths(c["seed"], c["B"], c["len_lo"], c["len_hi"])[:seqs]
    Hq, Hkv, d, dt = c["Hq"], c["Hkv"], c["d"], c["dtype"]
    elapsed = 0.0
    nbytes = 0
    passes = []
    total_len = float(sum(int(n) for n in lens))
    for b in range(seqs):
        L = int(lens[b])
        budget = min_seconds * L / total_len
        q = np.stack([ai.bits_to_f64(ai.slab(c["seed"], ai.Q_ID, b, h, 1, d, dt), dt)[0] for h in range(Hq)])[None]
        kc = np.stack([ai.bits_to_f64(ai.slab(c["seed"], ai.K_ID, b, g, L, d, dt), dt) for g in range(Hkv)])[None]
        vc = np.stack([ai.bits_to_f64(ai.slab(c["seed"], ai.V_ID, b, g, L, d, dt), dt) for g in range(Hkv)])[None]
        if page_size:
            n_pg = (L + page_size - 1) // page_size
            pad = n_pg * page_size - L
            kpad = np.concatenate([kc, np.zeros((1, Hkv, pad, d))], axis=2)
            vpad = np.concatenate([vc, np.zeros((1, Hkv, pad, d))], axis=2)
            order = np.random.default_rng([c["seed"], 7, b]).permutation(n_pg)
            kp = np.empty((n_pg, Hkv, page_size, d))
            vp = np.empty((n_pg, Hkv, page_size, d))
            kp[order] = kpad[0].reshape(Hkv, n_pg, page_size, d).transpose(1, 0, 2, 3)
            vp[order] = vpad[0].reshape(Hkv, n_pg, page_size, d).transpose(1, 0, 2, 3)
            call = lambda: oracle.decode_paged(q, kp, vp, order[None, :], [L], 1.0 / math.sqrt(d))
        else:
            call = lambda: oracle.decode(q, kc, vc, [L], 1.0 / math.sqrt(d))
        spent, n = 0.0, 0
        while n == 0 or spent < budget:
            t0 = time.perf_counter()
            call()
            spent += time.perf_counter() - t0
            n += 1
        elapsed += spent
        nbytes += n * decode_bytes([L], Hq, Hkv, d)
        passes.append(n)
    what = f"paged ({page_size}-row pages), " if page_size else ""
    return {"value": nbytes / elapsed / 1e9, "unit": "GB/s", "cores": cpu_cores_used(), "kind": "oracle",
            "sample": f"{what}first {seqs} of 32 sequences (lengths {lens.tolist()}), all 32 q-heads, each sequence "
                      f"repeated {min(passes)}-{max(passes)} times; {elapsed:.1f}s"}


# ------------------------------------------------------------------ modes
def calibrate_copy(nbytes=1 << 30, reps=5):
    """A plain device-to-device copy of known size, for counter calibration."""
    import torch
    x = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    y = torch.empty_like(x)
    for _ in range(reps):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"mode": "calibrate_copy", "bytes_read_per_copy": nbytes, "bytes_written_per_copy": nbytes,
                      "reps": reps}))


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--settle", type=float, default=0.5,
                    help="seconds of untimed steps before the warmup steps (GPU clock ramp-up)")
    ap.add_argument("--config", default="default")
    ap.add_argument("--num-splits", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): this path has no multi-GPU mode; "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    if args.calibrate_copy:
        calibrate_copy()
        return

    import exact_tiled_attention_fwd_amd as fa
    fa.load_library()

    cfg = args.config
    run_prefill = cfg in ("default", "tiny_mha_n128", "mha_n4096_fp16", "mha_n4096_fp16_causal", "llama3_8b_gqa_n8192",
                          "llama3_8b_gqa_n131072", "llama3_8b_gqa_varlen", "llama3_8b_gqa_n8192_bshd",
                          "llama3_8b_gqa_n8192_bwd", "llama3_8b_gqa_n8192_fp8")
    run_decode = cfg in ("default", "decode_32seq_gqa", "decode_32seq_gqa_paged")
    paged = cfg == "decode_32seq_gqa_paged"
    if not (run_prefill or run_decode):
        raise SystemExit(f"unknown --config {cfg}")
    pname = ("llama3_8b_gqa_n8192" if cfg in ("default", "llama3_8b_gqa_n8192_bshd", "llama3_8b_gqa_n8192_bwd",
                                              "llama3_8b_gqa_n8192_fp8")
             else cfg.replace("_causal", ""))
    causal = cfg in ("default", "llama3_8b_gqa_n8192", "llama3_8b_gqa_n131072", "mha_n4096_fp16_causal",
                     "llama3_8b_gqa_varlen", "llama3_8b_gqa_n8192_bshd", "llama3_8b_gqa_n8192_bwd",
                     "llama3_8b_gqa_n8192_fp8")
    parts = []
    pre = dec = None
    if run_prefill:
        if cfg == "llama3_8b_gqa_varlen":
            pre = PrefillVarlen(fa)
        elif cfg.endswith("_bwd"):
            pre = Backward(fa, pname, causal)
        elif cfg.endswith("_fp8"):
            pre = PrefillFp8(fa, pname, causal)
        else:
            pre = Prefill(fa, pname, causal, layout="bshd" if cfg.endswith("_bshd") else "bhnd")
        parts.append(pre)
    if run_decode:
        dec = DecodePaged(fa, num_splits=args.num_splits) if paged else Decode(fa, num_splits=args.num_splits)
        parts.append(dec)

    n_settle = settle(parts, args.settle) if args.settle > 0 else 0
    wall, per = time_steps(parts, args.steps, args.warmup)
    ms_per_step = wall * 1e3 / args.steps
    out = {"metric": "attn fwd TFLOP/s & % MFMA peak, Llama-3-8B GQA causal N=8192; decode GB/s"}
    i = 0
    if pre is not None:
        t_ms = float(np.mean(per[i]))
        tflops = pre.flops / (t_ms * 1e-3) / 1e12
        out.update(value=round(tflops, 2), unit="TFLOP/s")
        wl = cfg if cfg in ("llama3_8b_gqa_varlen", "llama3_8b_gqa_n8192_bshd", "llama3_8b_gqa_n8192_bwd",
                            "llama3_8b_gqa_n8192_fp8") else pname
        peak = MFMA_PEAK_FP8_TFLOPS if cfg.endswith("_fp8") else MFMA_PEAK_TFLOPS
        out["prefill"] = {"workload": f"{wl} causal={causal}", "ms_mean": round(t_ms, 4),
                          "ms_median": round(float(np.median(per[i])), 4),
                          "ms_min": round(float(np.min(per[i])), 4), "tflops": round(tflops, 2),
                          "frac_mfma_peak": round(tflops / peak, 4)}
        prof = cfg if cfg in ("llama3_8b_gqa_varlen", "llama3_8b_gqa_n8192_bshd", "llama3_8b_gqa_n8192_fp8",
                              "mha_n4096_fp16_causal") else pname
        kind = "bwd" if cfg.endswith("_bwd") else "fwd"
        traffic = counter_traffic(f"fa_{kind}_{prof}_counters.md")
        out["roofline"] = {"bound": "mfma", "achieved": round(tflops, 2), "peak": peak,
                           "unit": "TFLOP/s", "frac": round(tflops / peak, 4), "traffic": traffic,
                           "algorithmic_bytes": pre.bytes, "flops_per_launch": pre.flops}
        # The published peak assumes 2.4 GHz; the committed profile records the
        # clock the kernel actually ran at, and the fraction of the peak at it.
        ghz = counter_clock_ghz(f"fa_{kind}_{prof}_counters.md")
        if ghz:
            out["roofline"]["clock_ghz"] = ghz
            out["roofline"]["frac_at_clock"] = round(tflops / (peak * ghz / 2.4), 4)
        i += 1
    if dec is not None:
        t_ms = float(np.mean(per[i]))
        gbs = dec.bytes / (t_ms * 1e-3) / 1e9
        droof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                 "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": counter_traffic(f"fa_{cfg if paged else 'decode_32seq_gqa'}_counters.md"),
                 "algorithmic_bytes": dec.bytes}
        out["decode"] = {"workload": cfg if paged else "decode_32seq_gqa", "ms_mean": round(t_ms, 4),
                         "ms_median": round(float(np.median(per[i])), 4), "ms_min": round(float(np.min(per[i])), 4),
                         "value": round(gbs, 1), "unit": "GB/s", "roofline": droof}
        if pre is None:
            out.update(value=round(gbs, 1), unit="GB/s", roofline=droof)
    out.update({
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "settle": {"seconds": args.settle, "steps": n_settle}, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": ("fp8e4m3" if cfg.endswith("_fp8") else "bf16" if cfg not in ("mha_n4096_fp16", "mha_n4096_fp16_causal")
                  else "fp16"),
        "data": ("synthetic: seeded N(0,1) quantized to E4M3 per (batch, head) slab" if cfg.endswith("_fp8")
                 else "synthetic: seeded N(0,1) rounded to bf16/fp16"),
        "config": {"workload": "llama3_8b_gqa_n8192 prefill (B=1,Hq=32,Hkv=8,N=8192,d=128,causal,bf16) + decode_32seq_gqa (32 seq x 1 token, Hq=32,Hkv=8,d=128,bf16, L~U[1024,32768])"
                   if cfg == "default" else cfg,
                   "kernel_source_sha256": kernel_source_hash()},
    })
    if not args.no_cpu_baseline:
        if cfg == "llama3_8b_gqa_varlen":
            out["cpu_baseline"] = cpu_baseline_varlen()
        elif cfg == "llama3_8b_gqa_n8192_bwd":
            out["cpu_baseline"] = cpu_baseline_backward()
        elif cfg == "llama3_8b_gqa_n8192_fp8":
            out["cpu_baseline"] = cpu_baseline_prefill(fp8=True)
        elif pre is not None and pname == "llama3_8b_gqa_n131072":
            out["cpu_baseline"] = cpu_baseline_sampled()
        elif pre is not None and pname in ("mha_n4096_fp16", "tiny_mha_n128"):
            out["cpu_baseline"] = cpu_baseline_full(pname, causal)
        elif pre is not None and pname == "llama3_8b_gqa_n8192":
            out["cpu_baseline"] = cpu_baseline_prefill()
            if dec is not None:
                out["decode"]["cpu_baseline"] = cpu_baseline_decode()
        elif dec is not None:
            out["cpu_baseline"] = cpu_baseline_decode(page_size=128 if paged else 0)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
