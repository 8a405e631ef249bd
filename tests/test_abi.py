"""The C-ABI library loads, exports what include/fa.h declares, and rejects bad
arguments before touching a device (these calls run without a GPU)."""
import ctypes
import math
import os
import re

import pytest

import exact_tiled_attention_fwd_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

FAKE = 0x10000  # 16-byte aligned, never dereferenced: validation fails first


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z0-9_]+)\s*\(", text)))


def test_library_built_and_loads():
    assert os.path.exists(fa.lib_path()), "run exact_tiled_attention_fwd_amd.build first"
    lib = fa.load_library()
    assert lib.fa_abi_version() == 1


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert {"fa_fwd", "fa_fwd_strided", "fa_fwd_varlen", "fa_fwd_varlen_strided", "fa_fwd_fp8", "fa_bwd",
            "fa_bwd_workspace_bytes",
            "fa_decode", "fa_decode_paged", "fa_decode_workspace_bytes", "fa_status_string",
            "fa_last_error"} <= set(names)
    raw = ctypes.CDLL(fa.lib_path())
    for n in names:
        assert hasattr(raw, n), f"{n} declared in fa.h but not exported"


def test_status_strings():
    assert fa.fa_status_string(0) == "FA_OK"
    assert fa.fa_status_string(1) == "FA_ERR_INVALID_ARG"
    assert fa.fa_status_string(2) == "FA_ERR_UNSUPPORTED"
    assert fa.fa_status_string(3) == "FA_ERR_HIP"
    assert fa.fa_status_string(99) == "FA_UNKNOWN_STATUS"


def test_prefill_schedule_knob():
    # a host-side setting: no device is touched
    prev = fa.fa_set_prefill_schedule(fa.FA_SCHEDULE_SPLIT)
    try:
        assert prev == fa.FA_SCHEDULE_AUTO
        assert fa.fa_set_prefill_schedule(fa.FA_SCHEDULE_TILES) == fa.FA_SCHEDULE_SPLIT
        for bad in (-1, 3, 99):
            assert fa.fa_set_prefill_schedule(bad) == -1
        assert fa.fa_set_prefill_schedule(fa.FA_SCHEDULE_AUTO) == fa.FA_SCHEDULE_TILES
    finally:
        fa.fa_set_prefill_schedule(fa.FA_SCHEDULE_AUTO)


def fwd(**kw):
    a = dict(q=FAKE, k=FAKE + 0x100000, v=FAKE + 0x200000, o=FAKE + 0x300000, lse=None,
             B=1, Hq=8, Hkv=8, Nq=128, Nk=128, d=64, scale=0.125, causal=0, dtype=0, stream=None)
    a.update(kw)
    return fa.fa_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"], a["Nq"], a["Nk"],
                     a["d"], a["scale"], a["causal"], a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), fa.FA_ERR_INVALID_ARG),
    (dict(o=None), fa.FA_ERR_INVALID_ARG),
    (dict(k=FAKE + 8), fa.FA_ERR_INVALID_ARG),            # misaligned
    (dict(lse=FAKE + 0x400002), fa.FA_ERR_INVALID_ARG),   # misaligned lse
    (dict(B=0), fa.FA_ERR_INVALID_ARG),
    (dict(Nq=-1), fa.FA_ERR_INVALID_ARG),
    (dict(Nk=0), fa.FA_ERR_INVALID_ARG),
    (dict(Hq=6, Hkv=4), fa.FA_ERR_INVALID_ARG),
    (dict(causal=1, Nq=129, Nk=128), fa.FA_ERR_INVALID_ARG),
    (dict(causal=2), fa.FA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), fa.FA_ERR_INVALID_ARG),
    (dict(scale=float("inf")), fa.FA_ERR_INVALID_ARG),
    (dict(scale=0.0), fa.FA_ERR_INVALID_ARG),
    (dict(scale=-0.1), fa.FA_ERR_INVALID_ARG),
    (dict(d=96), fa.FA_ERR_UNSUPPORTED),
    (dict(d=256), fa.FA_ERR_UNSUPPORTED),
    (dict(dtype=2), fa.FA_ERR_UNSUPPORTED),
    (dict(o=FAKE + 0x1000), fa.FA_ERR_INVALID_ARG),       # o overlaps q
    (dict(lse=FAKE + 0x200100), fa.FA_ERR_INVALID_ARG),   # lse overlaps v
])
def test_fwd_rejects_before_launch(kw, status):
    st = fwd(**kw)
    assert st == status, (st, fa.fa_last_error())
    assert fa.fa_last_error() != ""


def dec(**kw):
    a = dict(q=FAKE, k=FAKE + 0x1000000, v=FAKE + 0x2000000, seqlens=FAKE + 0x3000000, o=FAKE + 0x3100000,
             lse=None, ws=FAKE + 0x4000000, ws_bytes=1 << 30, B=2, Hq=8, Hkv=2, Lcap=1024, d=128,
             scale=0.088, num_splits=0, dtype=0, stream=None)
    a.update(kw)
    return fa.fa_decode(a["q"], a["k"], a["v"], a["seqlens"], a["o"], a["lse"], a["ws"], a["ws_bytes"],
                        a["B"], a["Hq"], a["Hkv"], a["Lcap"], a["d"], a["scale"], a["num_splits"],
                        a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), fa.FA_ERR_INVALID_ARG),
    (dict(B=65535, Hq=64, Hkv=64, Lcap=1 << 20), fa.FA_ERR_UNSUPPORTED),   # block stream exceeds int32
    (dict(seqlens=None), fa.FA_ERR_INVALID_ARG),
    (dict(ws=None), fa.FA_ERR_INVALID_ARG),
    (dict(ws=FAKE + 0x4000010), fa.FA_ERR_INVALID_ARG),   # workspace not 256-aligned
    (dict(seqlens=FAKE + 0x3000002), fa.FA_ERR_INVALID_ARG),
    (dict(ws_bytes=16), fa.FA_ERR_INVALID_ARG),           # too small
    (dict(Lcap=0), fa.FA_ERR_INVALID_ARG),
    (dict(Hq=6, Hkv=4), fa.FA_ERR_INVALID_ARG),
    (dict(num_splits=-1), fa.FA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), fa.FA_ERR_INVALID_ARG),
    (dict(d=80), fa.FA_ERR_UNSUPPORTED),
    (dict(dtype=7), fa.FA_ERR_UNSUPPORTED),
    (dict(Hq=64, Hkv=1), fa.FA_ERR_UNSUPPORTED),          # > 32 q-heads per kv-head
    (dict(o=FAKE + 0x10), fa.FA_ERR_INVALID_ARG),         # o overlaps q
    (dict(o=FAKE + 0x2fff800), fa.FA_ERR_INVALID_ARG),    # o runs over seqlens
    (dict(lse=FAKE + 0x100), fa.FA_ERR_INVALID_ARG),      # lse inside q
    (dict(lse=FAKE + 0x3100020), fa.FA_ERR_INVALID_ARG),  # lse inside o
    (dict(lse=FAKE + 0x4000100), fa.FA_ERR_INVALID_ARG),  # lse inside the workspace
    (dict(ws=FAKE + 0x3000000), fa.FA_ERR_INVALID_ARG),   # workspace over seqlens
])
def test_decode_rejects_before_launch(kw, status):
    st = dec(**kw)
    assert st == status, (st, fa.fa_last_error())


def fwd_varlen(**kw):
    a = dict(q=FAKE, k=FAKE + 0x1000000, v=FAKE + 0x2000000, o=FAKE + 0x3000000, lse=None,
             cu_q=FAKE + 0x4000000, cu_k=FAKE + 0x4100000, B=3, Hq=8, Hkv=2, total_q=1000, total_k=1200,
             max_q=600, d=128, scale=0.088, causal=1, dtype=0, stream=None)
    a.update(kw)
    return fa.fa_fwd_varlen(a["q"], a["k"], a["v"], a["o"], a["lse"], a["cu_q"], a["cu_k"], a["B"], a["Hq"],
                            a["Hkv"], a["total_q"], a["total_k"], a["max_q"], a["d"], a["scale"], a["causal"],
                            a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(cu_q=None), fa.FA_ERR_INVALID_ARG),
    (dict(cu_k=FAKE + 0x4100002), fa.FA_ERR_INVALID_ARG),
    (dict(total_q=0), fa.FA_ERR_INVALID_ARG),
    (dict(max_q=0), fa.FA_ERR_INVALID_ARG),
    (dict(max_q=1001), fa.FA_ERR_INVALID_ARG),             # more than total_q
    (dict(causal=2), fa.FA_ERR_INVALID_ARG),
    (dict(Hq=6, Hkv=4), fa.FA_ERR_INVALID_ARG),
    (dict(d=96), fa.FA_ERR_UNSUPPORTED),
    (dict(o=FAKE + 0x100), fa.FA_ERR_INVALID_ARG),          # o overlaps q
    (dict(o=FAKE + 0x3fff000), fa.FA_ERR_INVALID_ARG),      # o runs over cu_seqlens_q
    (dict(lse=FAKE + 0x4100000), fa.FA_ERR_INVALID_ARG),    # lse over cu_seqlens_k
])
def test_fwd_varlen_rejects_before_launch(kw, status):
    st = fwd_varlen(**kw)
    assert st == status, (st, fa.fa_last_error())


# (batch, seq, heads, dim) strides of q/o [B=2, N=256, Hq=8, d=64] and k/v [B=2, N=256, Hkv=2, d=64]
BSHD = [256 * 8 * 64, 64, 8 * 64, 256 * 2 * 64, 64, 2 * 64, 256 * 2 * 64, 64, 2 * 64, 256 * 8 * 64, 64, 8 * 64]


def fwd_strided(strides=BSHD, **kw):
    a = dict(q=FAKE, k=FAKE + 0x1000000, v=FAKE + 0x2000000, o=FAKE + 0x3000000, lse=None,
             B=2, Hq=8, Hkv=2, Nq=256, Nk=256, d=64, scale=0.125, causal=1, dtype=0, stream=None)
    a.update(kw)
    if strides is None:
        lib = fa.load_library()
        return lib.fa_fwd_strided(a["q"], a["k"], a["v"], a["o"], a["lse"], None, a["B"], a["Hq"], a["Hkv"],
                                  a["Nq"], a["Nk"], a["d"], a["scale"], a["causal"], a["dtype"], a["stream"])
    return fa.fa_fwd_strided(a["q"], a["k"], a["v"], a["o"], a["lse"], strides, a["B"], a["Hq"], a["Hkv"],
                             a["Nq"], a["Nk"], a["d"], a["scale"], a["causal"], a["dtype"], a["stream"])


def _with(i, x):
    s = list(BSHD)
    s[i] = x
    return s


@pytest.mark.parametrize("strides,kw,status", [
    (None, {}, fa.FA_ERR_INVALID_ARG),                        # no stride array
    (_with(2, -512), {}, fa.FA_ERR_INVALID_ARG),              # negative row stride of q
    (_with(4, 60), {}, fa.FA_ERR_INVALID_ARG),                # k head stride not a multiple of 8
    (_with(8, 1 << 24), {}, fa.FA_ERR_INVALID_ARG),           # v row stride too large
    (_with(11, 32), {}, fa.FA_ERR_INVALID_ARG),               # o rows overlap each other (32 < d)
    (_with(10, 0), {}, fa.FA_ERR_INVALID_ARG),                # every o head writes the same rows
    (_with(9, 1 << 40), {}, fa.FA_ERR_INVALID_ARG),           # o batch stride too large
    (BSHD, dict(o=FAKE + 0x400), fa.FA_ERR_INVALID_ARG),      # o inside the span of q
    (BSHD, dict(lse=FAKE + 0x2000100), fa.FA_ERR_INVALID_ARG),  # lse inside the span of v
    (BSHD, dict(causal=1, Nq=257), fa.FA_ERR_INVALID_ARG),    # causal needs Nq <= Nk
    (BSHD, dict(d=96), fa.FA_ERR_UNSUPPORTED),
])
def test_fwd_strided_rejects_before_launch(strides, kw, status):
    st = fwd_strided(strides, **kw)
    assert st == status, (st, fa.fa_last_error())
    assert fa.fa_last_error() != ""


def fwd_varlen_strided(strides, **kw):
    a = dict(q=FAKE, k=FAKE + 0x1000000, v=FAKE + 0x2000000, o=FAKE + 0x3000000, lse=None,
             cu_q=FAKE + 0x4000000, cu_k=FAKE + 0x4100000, B=3, Hq=8, Hkv=2, total_q=1000, total_k=1200,
             max_q=600, d=128, scale=0.088, causal=1, dtype=0, stream=None)
    a.update(kw)
    return fa.fa_fwd_varlen_strided(a["q"], a["k"], a["v"], a["o"], a["lse"], strides, a["cu_q"], a["cu_k"], a["B"],
                                    a["Hq"], a["Hkv"], a["total_q"], a["total_k"], a["max_q"], a["d"], a["scale"],
                                    a["causal"], a["dtype"], a["stream"])


THD = [128, 8 * 128, 128, 2 * 128, 128, 2 * 128, 128, 8 * 128]  # (total, heads, dim)


@pytest.mark.parametrize("strides,kw,status", [
    ([THD[0], -THD[1]] + THD[2:], {}, fa.FA_ERR_INVALID_ARG),
    (THD[:7] + [64], {}, fa.FA_ERR_INVALID_ARG),              # o tokens overlap
    (THD[:6] + [0, THD[7]], {}, fa.FA_ERR_INVALID_ARG),       # o heads alias
    (THD, dict(cu_q=None), fa.FA_ERR_INVALID_ARG),
    (THD, dict(o=FAKE + 0x800), fa.FA_ERR_INVALID_ARG),       # o inside q
    (THD, dict(max_q=1001), fa.FA_ERR_INVALID_ARG),
])
def test_fwd_varlen_strided_rejects_before_launch(strides, kw, status):
    st = fwd_varlen_strided(strides, **kw)
    assert st == status, (st, fa.fa_last_error())


def test_fwd_strided_needs_its_stride_count():
    with pytest.raises(ValueError):
        fa.fa_fwd_strided(FAKE, FAKE, FAKE, FAKE, None, [64] * 11, 1, 1, 1, 8, 8, 64, 0.1, 0, 0, None)
    with pytest.raises(ValueError):
        fa.fa_fwd_varlen_strided(FAKE, FAKE, FAKE, FAKE, None, [64] * 7, FAKE, FAKE, 1, 1, 1, 8, 8, 8, 64, 0.1, 0,
                                 0, None)


def bwd(**kw):
    a = dict(q=FAKE, k=FAKE + 0x100000, v=FAKE + 0x200000, o=FAKE + 0x300000, lse=FAKE + 0x400000,
             do=FAKE + 0x500000, dq=FAKE + 0x600000, dk=FAKE + 0x700000, dv=FAKE + 0x800000,
             ws=FAKE + 0x900000, ws_bytes=1 << 20, B=1, Hq=8, Hkv=2, Nq=128, Nk=128, d=64, scale=0.125,
             causal=1, dtype=0, stream=None)
    a.update(kw)
    return fa.fa_bwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["do"], a["dq"], a["dk"], a["dv"], a["ws"],
                     a["ws_bytes"], a["B"], a["Hq"], a["Hkv"], a["Nq"], a["Nk"], a["d"], a["scale"], a["causal"],
                     a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(lse=None), fa.FA_ERR_INVALID_ARG),
    (dict(do=None), fa.FA_ERR_INVALID_ARG),
    (dict(dv=FAKE + 0x800008), fa.FA_ERR_INVALID_ARG),     # misaligned
    (dict(ws=FAKE + 0x900010), fa.FA_ERR_INVALID_ARG),     # workspace not 256-byte aligned
    (dict(ws_bytes=128 * 8 * 4 - 4), fa.FA_ERR_INVALID_ARG),  # workspace too small
    (dict(Nq=0), fa.FA_ERR_INVALID_ARG),
    (dict(causal=1, Nq=200, Nk=128), fa.FA_ERR_INVALID_ARG),
    (dict(Hq=6, Hkv=4), fa.FA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), fa.FA_ERR_INVALID_ARG),
    (dict(d=96), fa.FA_ERR_UNSUPPORTED),
    (dict(dtype=3), fa.FA_ERR_UNSUPPORTED),
    (dict(dq=FAKE + 0x1000), fa.FA_ERR_INVALID_ARG),        # dq inside q
    (dict(dk=FAKE + 0x800000), fa.FA_ERR_INVALID_ARG),      # dk == dv
    (dict(ws=FAKE + 0x600000), fa.FA_ERR_INVALID_ARG),      # workspace inside dq
    (dict(dv=FAKE + 0x400000), fa.FA_ERR_INVALID_ARG),      # dv over lse
])
def test_bwd_rejects_before_launch(kw, status):
    st = bwd(**kw)
    assert st == status, (st, fa.fa_last_error())
    assert fa.fa_last_error() != ""


def test_bwd_workspace_bytes():
    assert fa.fa_bwd_workspace_bytes(1, 32, 8192) == 32 * 8192 * 4
    assert fa.fa_bwd_workspace_bytes(2, 3, 5) == 256
    assert fa.fa_bwd_workspace_bytes(0, 3, 5) == 0


def fwd_fp8(**kw):
    a = dict(q=FAKE, k=FAKE + 0x100000, v=FAKE + 0x200000, o=FAKE + 0x300000, lse=None, qd=FAKE + 0x500000,
             kd=FAKE + 0x500100, vd=FAKE + 0x500200, B=1, Hq=8, Hkv=2, Nq=128, Nk=128, d=128, scale=0.088, causal=1,
             stream=None)
    a.update(kw)
    return fa.fa_fwd_fp8(a["q"], a["k"], a["v"], a["o"], a["lse"], a["qd"], a["kd"], a["vd"], a["B"], a["Hq"],
                         a["Hkv"], a["Nq"], a["Nk"], a["d"], a["scale"], a["causal"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(qd=None), fa.FA_ERR_INVALID_ARG),
    (dict(k=FAKE + 0x100008), fa.FA_ERR_INVALID_ARG),       # misaligned
    (dict(vd=FAKE + 0x500202), fa.FA_ERR_INVALID_ARG),      # misaligned descale
    (dict(d=64), fa.FA_ERR_UNSUPPORTED),
    (dict(Nq=0), fa.FA_ERR_INVALID_ARG),
    (dict(causal=1, Nq=200, Nk=128), fa.FA_ERR_INVALID_ARG),
    (dict(Hq=6, Hkv=4), fa.FA_ERR_INVALID_ARG),
    (dict(scale=float("inf")), fa.FA_ERR_INVALID_ARG),
    (dict(o=FAKE + 0x1000), fa.FA_ERR_INVALID_ARG),         # o inside q
    (dict(o=FAKE + 0x4fff00), fa.FA_ERR_INVALID_ARG),       # o over the q descales
    (dict(lse=FAKE + 0x200010), fa.FA_ERR_INVALID_ARG),     # lse inside v
    (dict(lse=FAKE + 0x500100), fa.FA_ERR_INVALID_ARG),     # lse over the k descales
])
def test_fwd_fp8_rejects_before_launch(kw, status):
    st = fwd_fp8(**kw)
    assert st == status, (st, fa.fa_last_error())


def dec_paged(**kw):
    a = dict(q=FAKE, k=FAKE + 0x1000000, v=FAKE + 0x2000000, table=FAKE + 0x2800000, seqlens=FAKE + 0x3000000,
             o=FAKE + 0x3100000, lse=None, ws=FAKE + 0x4000000, ws_bytes=1 << 30, B=2, Hq=8, Hkv=2,
             num_pages=64, page_size=128, max_pages=8, d=128, scale=0.088, num_splits=0, dtype=0, stream=None)
    a.update(kw)
    return fa.fa_decode_paged(a["q"], a["k"], a["v"], a["table"], a["seqlens"], a["o"], a["lse"], a["ws"],
                              a["ws_bytes"], a["B"], a["Hq"], a["Hkv"], a["num_pages"], a["page_size"],
                              a["max_pages"], a["d"], a["scale"], a["num_splits"], a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(table=None), fa.FA_ERR_INVALID_ARG),
    (dict(table=FAKE + 0x2800002), fa.FA_ERR_INVALID_ARG),  # table not 4-byte aligned
    (dict(num_pages=0), fa.FA_ERR_INVALID_ARG),
    (dict(max_pages=0), fa.FA_ERR_INVALID_ARG),
    (dict(page_size=48), fa.FA_ERR_UNSUPPORTED),            # not a multiple of 32
    (dict(page_size=1 << 20, max_pages=1 << 12), fa.FA_ERR_INVALID_ARG),  # capacity overflows int
    (dict(ws_bytes=16), fa.FA_ERR_INVALID_ARG),
    (dict(d=80), fa.FA_ERR_UNSUPPORTED),
    (dict(o=FAKE + 0x1000010), fa.FA_ERR_INVALID_ARG),      # o inside k_pages
    (dict(o=FAKE + 0x27ff800), fa.FA_ERR_INVALID_ARG),      # o runs over the block table
    (dict(lse=FAKE + 0x2800010), fa.FA_ERR_INVALID_ARG),    # lse inside the block table
])
def test_decode_paged_rejects_before_launch(kw, status):
    st = dec_paged(**kw)
    assert st == status, (st, fa.fa_last_error())


def test_decode_workspace_bytes():
    # Layout: O partials [B, Hq, slots, d] fp32, LSE partials [B, Hq, slots]
    # fp32, split header (B + 1) int32, each rounded up to 256 bytes; slots =
    # splits + 1 (a wave's equal share of the rows may start inside a chunk).
    r256 = lambda x: (x + 255) // 256 * 256
    # auto plan for the 32-sequence, 32K-cache shape: 512-key chunks, 64 splits
    n = fa.fa_decode_workspace_bytes(32, 32, 8, 32768, 128, 0)
    rows = 32 * 32 * 65
    assert n == r256(rows * 128 * 4) + r256(rows * 4) + r256(33 * 4)
    # explicit splits: chunk rounded up to a multiple of 128 keys
    n1 = fa.fa_decode_workspace_bytes(1, 4, 1, 1000, 64, 3)   # chunk 334 -> 384, 3 splits
    assert n1 == r256(4 * 4 * 64 * 4) + r256(4 * 4 * 4) + r256(2 * 4)
    assert fa.fa_decode_workspace_bytes(1, 4, 1, 1000, 64, 1) == r256(4 * 2 * 64 * 4) + 256 + 256
    assert fa.fa_decode_workspace_bytes(0, 4, 1, 1000, 64, 0) == 0
    assert fa.fa_decode_workspace_bytes(1, 4, 1, 1000, 96, 0) == 0
    assert fa.fa_decode_workspace_bytes(1, 4, 1, 1000, 64, -1) == 0


def test_python_helpers_validate_tensors():
    import torch
    with pytest.raises(ValueError):
        fa.attention(torch.zeros(1, 1, 4, 64), torch.zeros(1, 1, 4, 64), torch.zeros(1, 1, 4, 64))
    with pytest.raises(NotImplementedError):
        fa.dtype_code(torch.float32)
    with pytest.raises(NotImplementedError):   # dropout is not part of the forward path
        fa.flash_attn_func(torch.zeros(1, 4, 1, 64), torch.zeros(1, 4, 1, 64), torch.zeros(1, 4, 1, 64),
                           dropout_p=0.1)
    with pytest.raises(ValueError):            # host tensors are refused
        fa.flash_attn_func(torch.zeros(1, 4, 1, 64), torch.zeros(1, 4, 1, 64), torch.zeros(1, 4, 1, 64))


@pytest.mark.parametrize("case,msg", [
    ("shape", "shape"),
    ("dtype", "float32"),
    ("noncontig", "contiguous"),
    ("device", "expected"),
    ("notensor", "torch.Tensor"),
])
def test_caller_outputs_are_checked(case, msg):
    """Caller-supplied out / lse tensors are refused unless they are exactly
    what the kernel writes (the C layer only sees a pointer)."""
    import torch
    cpu = torch.device("cpu")
    t, dev = torch.empty((2, 4, 8)), cpu
    if case == "shape":
        t = torch.empty((2, 4, 7))
    elif case == "dtype":
        t = torch.empty((2, 4, 8), dtype=torch.float16)
    elif case == "noncontig":
        t = torch.empty((2, 8, 4)).transpose(1, 2)
    elif case == "device":
        dev = torch.device("cuda:0")
    elif case == "notensor":
        t = [0.0] * 64
    with pytest.raises(ValueError, match=msg):
        fa._check_out("lse", t, (2, 4, 8), torch.float32, dev)
    fa._check_out("lse", torch.empty((2, 4, 8)), (2, 4, 8), torch.float32, cpu)  # the right one passes


def test_caller_workspace_is_checked():
    import torch
    cpu = torch.device("cpu")
    with pytest.raises(ValueError, match="bytes"):
        fa._check_workspace(torch.empty(100, dtype=torch.uint8), 101, cpu)
    with pytest.raises(ValueError, match="expected"):
        fa._check_workspace(torch.empty(200, dtype=torch.uint8), 101, torch.device("cuda:0"))
    with pytest.raises(ValueError, match="contiguous"):
        fa._check_workspace(torch.empty(40, 10, dtype=torch.uint8).t(), 101, cpu)
    fa._check_workspace(torch.empty(26, dtype=torch.float32), 101, cpu)  # 104 bytes: enough


def test_decode_noalloc_rejects_before_launch():
    """The static-workspace decode validates like fa_decode, and refuses
    sizes whose workspace exceeds the static array, before any HIP call."""
    base = dict(q=FAKE, k_cache=FAKE, v_cache=FAKE, seqlens=FAKE, o=FAKE * 2, lse=None, B=2, Hq=8, Hkv=2, Lcap=512,
                d=128, scale=0.1, num_splits=0, dtype=fa.FA_DTYPE_BF16, stream=None)
    for kw, status in ((dict(q=None), fa.FA_ERR_INVALID_ARG), (dict(o=FAKE + 4), fa.FA_ERR_INVALID_ARG),
                       (dict(d=96), fa.FA_ERR_UNSUPPORTED), (dict(Hq=7), fa.FA_ERR_INVALID_ARG),
                       (dict(num_splits=-1), fa.FA_ERR_INVALID_ARG), (dict(scale=0.0), fa.FA_ERR_INVALID_ARG)):
        assert fa.fa_decode_noalloc(**{**base, **kw}) == status, kw
    # 64 sequences x 32 q-heads at Lcap 32768: a 68 MB workspace, above the 64 MiB array
    big = dict(base, B=64, Hq=32, Hkv=8, Lcap=32768)
    assert fa.fa_decode_workspace_bytes(64, 32, 8, 32768, 128, 0) > (64 << 20)
    assert fa.fa_decode_noalloc(**big) == fa.FA_ERR_INVALID_ARG
    assert "static" in fa.fa_last_error()
