"""Seeded synthetic inputs for exact attention forward and KV-cache decode.

This module is shared by the CPU oracle and the GPU path. It holds no part of
the attention arithmetic: it only draws random numbers, rounds them to the
16-bit storage formats, and converts stored bit patterns back to float64.

Workloads follow the shapes the pages use. The SDPA page ("Flash Attention 2 ...
PyTorch native", devhandbook.co.kr, Example 1 and Example 5) draws
``torch.randn`` tensors in (B, H, L, D) layout, including grouped K/V with fewer
heads; the KV-cache page ("Advanced techniques for enhancing LLM throughput",
cabseo.com, section "Memory requirements") gives the per-sequence cache that
decode reads.

Seeding: every (tensor, batch, head) slab has its own NumPy substream
``default_rng([seed, tensor_id, b, head])`` with tensor_id Q=0, K=1, V=2 and
the upstream gradient dO=9 (backward workloads), so a
slab can be regenerated alone (long-context row samples, per-head oracles).
Values are float32 ``standard_normal`` draws in row-major (row, dim) order,
rounded to nearest-even into bf16 or fp16.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

__all__ = [
    "BF16", "FP16", "FP8", "Q_ID", "K_ID", "V_ID", "DO_ID", "grad_output", "fp8_decode", "fp8_encode",
    "fp8_quantize", "prefill_inputs_fp8", "fp8_to_f64",
    "round_to_bits", "bits_to_f64", "slab", "prefill_inputs",
    "decode_lengths", "decode_inputs", "paged_layout", "varlen_inputs", "sample_rows", "CONFIGS",
]

BF16 = "bf16"
FP16 = "fp16"
Q_ID, K_ID, V_ID = 0, 1, 2
DO_ID = 9  # upstream gradient of O
BF16_NAN_BITS = 0x7FC0
FP16_NAN_BITS = 0x7E00

# The workloads: shapes, dtype, mask. Seed of config k is k.
CONFIGS = {
    "tiny_mha_n128": dict(seed=1, B=1, Hq=8, Hkv=8, N=128, d=64, dtype=BF16, causal=(False,)),
    "mha_n4096_fp16": dict(seed=2, B=2, Hq=8, Hkv=8, N=4096, d=64, dtype=FP16, causal=(False, True)),
    "llama3_8b_gqa_n8192": dict(seed=3, B=1, Hq=32, Hkv=8, N=8192, d=128, dtype=BF16, causal=(True,)),
    "llama3_8b_gqa_n131072": dict(seed=4, B=1, Hq=32, Hkv=8, N=131072, d=128, dtype=BF16, causal=(True,),
                            sample_rows=256),
    "decode_32seq_gqa": dict(seed=5, B=32, Hq=32, Hkv=8, Lcap=32768, d=128, dtype=BF16,
                      len_lo=1024, len_hi=32768),
    # Packed prefill of 16 Llama-3-shaped sequences, lengths U[512, 8192]
    # (drawn like the decode lengths), causal, no padding.
    "llama3_8b_gqa_varlen": dict(seed=6, B=16, Hq=32, Hkv=8, d=128, dtype=BF16, causal=(True,),
                          len_lo=512, len_hi=8192),
}


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def round_to_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float32 values to nearest-even bf16/fp16; return uint16 bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == FP16:
        return x.astype(np.float16).view(np.uint16)
    if dtype != BF16:
        raise ValueError(f"unknown dtype {dtype!r}")
    u = x.view(np.uint32)
    # round-to-nearest-even on the upper 16 bits; inputs here are finite
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    out = ((u + bias) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = BF16_NAN_BITS
    return out


def bits_to_f64(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Exact widening of stored bf16/fp16 bit patterns to float64."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    if dtype == FP16:
        return bits.view(np.float16).astype(np.float64)
    if dtype != BF16:
        raise ValueError(f"unknown dtype {dtype!r}")
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


# ------------------------------------------------------------------ FP8 (e4m3)
# OCP 8-bit float E4M3 ("fn": no infinities): 1 sign, 4 exponent (bias 7), 3
# mantissa bits; exponent field 0 is subnormal (m * 2^-9); 0x7F / 0xFF is NaN;
# the largest finite value is 448 (0x7E).
FP8 = "fp8e4m3"
FP8_MAX = 448.0


def fp8_decode(codes: np.ndarray) -> np.ndarray:
    """E4M3 codes (uint8) -> float64, exactly."""
    c = np.asarray(codes, np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    out = sign * mag
    return np.where((c & 0x7F) == 0x7F, np.nan, out)


_FP8_POS = fp8_decode(np.arange(0x7F, dtype=np.uint8))  # codes 0..0x7E, increasing


def fp8_encode(x: np.ndarray) -> np.ndarray:
    """float -> nearest E4M3 code, ties to the even code; |x| > 448 saturates
    to 448 (inputs are scaled into range first, so this does not occur)."""
    x = np.asarray(x, np.float64)
    a = np.minimum(np.abs(x), FP8_MAX)
    hi = np.clip(np.searchsorted(_FP8_POS, a, side="left"), 0, 0x7E)
    lo = np.clip(hi - 1, 0, 0x7E)
    dlo, dhi = a - _FP8_POS[lo], _FP8_POS[hi] - a
    pick = np.where(dlo < dhi, lo, np.where(dhi < dlo, hi, np.where(lo % 2 == 0, lo, hi)))
    code = pick.astype(np.uint8)
    return np.where((x < 0) & (code != 0), code | 0x80, code).astype(np.uint8)


def fp8_quantize(x: np.ndarray):
    """One slab -> (codes, descale): descale is the power of two that brings
    max|x| to at most 448, so x / descale is exact before rounding and the
    value a code stands for is fp8_decode(code) * descale."""
    amax = float(np.max(np.abs(x))) if x.size else 0.0
    e = int(np.ceil(np.log2(amax / FP8_MAX))) if amax > 0 else 0
    descale = float(2.0 ** e)
    return fp8_encode(np.asarray(x, np.float64) / descale), descale


def prefill_inputs_fp8(seed: int, B: int, Hq: int, Hkv: int, N: int, d: int, Nk: int | None = None) -> dict:
    """Q [B,Hq,N,d], K/V [B,Hkv,Nk,d] as E4M3 codes (uint8) with one float32
    descale per (batch, head) slab ([B,Hq] for q, [B,Hkv] for k and v). The
    underlying draws are the float32 N(0,1) values of ``slab`` (before any
    16-bit rounding), quantized slab by slab."""
    Nk = N if Nk is None else Nk
    out = {}
    for name, tid, H, n in (("q", Q_ID, Hq, N), ("k", K_ID, Hkv, Nk), ("v", V_ID, Hkv, Nk)):
        codes = np.empty((B, H, n, d), np.uint8)
        ds = np.empty((B, H), np.float32)
        for b in range(B):
            for h in range(H):
                raw = np.random.default_rng([seed, tid, b, h]).standard_normal(size=(n, d), dtype=np.float32)
                codes[b, h], ds[b, h] = fp8_quantize(raw)
        out[name], out[name + "_descale"] = codes, ds
    out["dtype"] = FP8
    return out


def fp8_to_f64(codes: np.ndarray, descale: np.ndarray) -> np.ndarray:
    """Codes [B,H,N,d] and descales [B,H] -> the float64 values they stand for."""
    return fp8_decode(codes) * np.asarray(descale, np.float64)[:, :, None, None]


def slab(seed: int, tensor_id: int, b: int, head: int, n: int, d: int, dtype: str) -> np.ndarray:
    """One (n, d) slab of N(0,1) values rounded to ``dtype``, as uint16 bits."""
    rng = np.random.default_rng([seed, tensor_id, b, head])
    return round_to_bits(rng.standard_normal(size=(n, d), dtype=np.float32), dtype)


def _fill(out: np.ndarray, seed: int, tensor_id: int, n: int, d: int, dtype: str) -> None:
    B, H = out.shape[0], out.shape[1]

    def job(bh):
        b, h = divmod(bh, H)
        out[b, h, :n] = slab(seed, tensor_id, b, h, n, d, dtype)

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(job, range(B * H)))


def prefill_inputs(seed: int, B: int, Hq: int, Hkv: int, N: int, d: int, dtype: str,
                   Nk: int | None = None) -> dict:
    """Q [B,Hq,N,d], K/V [B,Hkv,Nk,d] as uint16 bit arrays (contiguous)."""
    Nk = N if Nk is None else Nk
    q = np.empty((B, Hq, N, d), np.uint16)
    k = np.empty((B, Hkv, Nk, d), np.uint16)
    v = np.empty((B, Hkv, Nk, d), np.uint16)
    _fill(q, seed, Q_ID, N, d, dtype)
    _fill(k, seed, K_ID, Nk, d, dtype)
    _fill(v, seed, V_ID, Nk, d, dtype)
    return dict(q=q, k=k, v=v, dtype=dtype)


def grad_output(seed: int, B: int, Hq: int, N: int, d: int, dtype: str) -> np.ndarray:
    """dO [B,Hq,N,d] as uint16 bits: the upstream gradient of O for backward
    workloads, N(0,1) like the inputs."""
    do = np.empty((B, Hq, N, d), np.uint16)
    _fill(do, seed, DO_ID, N, d, dtype)
    return do


def decode_lengths(seed: int, B: int, lo: int, hi: int) -> np.ndarray:
    """Per-sequence cache lengths, uniform on [lo, hi] inclusive, int32."""
    rng = np.random.default_rng([seed, 3])
    return rng.integers(lo, hi, size=B, endpoint=True).astype(np.int32)


def decode_inputs(seed: int, B: int, Hq: int, Hkv: int, Lcap: int, d: int, dtype: str,
                  lengths: np.ndarray) -> dict:
    """q [B,Hq,d]; k/v caches [B,Hkv,Lcap,d]; rows >= lengths[b] hold NaN bits."""
    lengths = np.asarray(lengths, np.int32)
    nan_bits = BF16_NAN_BITS if dtype == BF16 else FP16_NAN_BITS
    q = np.empty((B, Hq, d), np.uint16)
    for b in range(B):
        for h in range(Hq):
            q[b, h] = slab(seed, Q_ID, b, h, 1, d, dtype)[0]
    kc = np.empty((B, Hkv, Lcap, d), np.uint16)
    vc = np.empty((B, Hkv, Lcap, d), np.uint16)

    def job(args):
        cache, tid, b, g = args
        L = int(min(max(lengths[b], 0), Lcap))
        cache[b, g, :L] = slab(seed, tid, b, g, L, d, dtype)
        cache[b, g, L:] = nan_bits

    work = [(c, t, b, g) for (c, t) in ((kc, K_ID), (vc, V_ID)) for b in range(B) for g in range(Hkv)]
    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(job, work))
    return dict(q=q, k_cache=kc, v_cache=vc, seqlens=lengths, dtype=dtype)


def paged_layout(k_cache: np.ndarray, v_cache: np.ndarray, page_size: int, seed: int, dtype: str,
                 spare_pages: int = 0) -> dict:
    """Scatter contiguous caches [B,Hkv,Lcap,d] into pages [num_pages,Hkv,page_size,d].

    Page j of sequence b (rows j*page_size ..) goes to page id
    block_table[b, j], taken from a seeded permutation
    (``default_rng([seed, 6])``) of all num_pages = B*max_pages + spare_pages
    ids; spare pages hold NaN bits. Pure data movement: the logical cache of
    every sequence is unchanged.
    """
    B, Hkv, Lcap, d = k_cache.shape
    assert Lcap % page_size == 0
    max_pages = Lcap // page_size
    num_pages = B * max_pages + spare_pages
    perm = np.random.default_rng([seed, 6]).permutation(num_pages).astype(np.int32)
    table = perm[: B * max_pages].reshape(B, max_pages)
    nan_bits = BF16_NAN_BITS if dtype == BF16 else FP16_NAN_BITS
    out = {}
    for name, cache in (("k_pages", k_cache), ("v_pages", v_cache)):
        pages = np.full((num_pages, Hkv, page_size, d), nan_bits, np.uint16)
        pages[table.reshape(-1)] = (cache.reshape(B, Hkv, max_pages, page_size, d)
                                    .transpose(0, 2, 1, 3, 4).reshape(-1, Hkv, page_size, d))
        out[name] = pages
    out.update(block_table=table, page_size=page_size)
    return out


def varlen_inputs(seed: int, lens_q, lens_k, Hq: int, Hkv: int, d: int, dtype: str) -> dict:
    """A packed batch: q [Hq, total_q, d], k/v [Hkv, total_k, d] with sequence
    b's rows drawn as the slabs of batch index b (the same values
    ``prefill_inputs`` gives sequence b), plus cu_seqlens [B+1] int32."""
    lens_q = np.asarray(lens_q, np.int64)
    lens_k = np.asarray(lens_k, np.int64)
    cu_q = np.concatenate([[0], np.cumsum(lens_q)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(lens_k)]).astype(np.int32)
    q = np.empty((Hq, int(cu_q[-1]), d), np.uint16)
    k = np.empty((Hkv, int(cu_k[-1]), d), np.uint16)
    v = np.empty((Hkv, int(cu_k[-1]), d), np.uint16)
    for b in range(len(lens_q)):
        for h in range(Hq):
            q[h, cu_q[b]:cu_q[b + 1]] = slab(seed, Q_ID, b, h, int(lens_q[b]), d, dtype)
        for g in range(Hkv):
            k[g, cu_k[b]:cu_k[b + 1]] = slab(seed, K_ID, b, g, int(lens_k[b]), d, dtype)
            v[g, cu_k[b]:cu_k[b + 1]] = slab(seed, V_ID, b, g, int(lens_k[b]), d, dtype)
    return dict(q=q, k=k, v=v, cu_q=cu_q, cu_k=cu_k, dtype=dtype)


def sample_rows(seed: int, head: int, N: int, count: int = 256) -> np.ndarray:
    """Sorted distinct query rows for a per-head spot check: 0, N-1 and count-2 others."""
    if N <= count:
        return np.arange(N, dtype=np.int64)
    rng = np.random.default_rng([seed, 4, head])
    mid = rng.choice(np.arange(1, N - 1), size=count - 2, replace=False)
    return np.sort(np.concatenate([[0, N - 1], mid]).astype(np.int64))
