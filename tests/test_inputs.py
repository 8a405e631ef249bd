"""The seeded input generator: determinism, rounding, layout, regression hashes."""
import hashlib
import json
import os

import numpy as np
import pytest

import attn_inputs as ai

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_bf16_round_to_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -7, -(1.0 + 2 ** -8),
                  1.0 + 2 ** -8 + 2 ** -20, 3.0e38, 1e-40], np.float32)
    b = ai.round_to_bits(x, ai.BF16)
    # ties go to the even mantissa, anything above a tie rounds up
    assert b.tolist() == [0x3F80, 0x3F80, 0x3F82, 0x3F81, 0xBF80, 0x3F81, 0x7F62, 0x0001]
    back = ai.bits_to_f64(b, ai.BF16)
    assert back[0] == 1.0 and back[2] == 1.0 + 2 ** -6


def test_fp16_round_to_nearest_even():
    x = np.array([1.0 + 2 ** -11, 1.0 + 3 * 2 ** -11, 65504.0], np.float32)
    b = ai.round_to_bits(x, ai.FP16)
    assert b.tolist() == [0x3C00, 0x3C02, 0x7BFF]
    assert ai.bits_to_f64(b, ai.FP16).tolist() == [1.0, 1.0 + 2 ** -9, 65504.0]


def test_slab_is_deterministic_and_independent():
    a = ai.slab(3, ai.Q_ID, 0, 5, 16, 8, ai.BF16)
    b = ai.slab(3, ai.Q_ID, 0, 5, 16, 8, ai.BF16)
    c = ai.slab(3, ai.K_ID, 0, 5, 16, 8, ai.BF16)
    assert np.array_equal(a, b) and not np.array_equal(a, c)
    # a prefix of a longer slab is the shorter slab (row-major draws)
    long = ai.slab(3, ai.Q_ID, 0, 5, 32, 8, ai.BF16)
    assert np.array_equal(long[:16], a)


def test_prefill_layout_matches_slabs():
    x = ai.prefill_inputs(7, 2, 4, 2, 20, 8, ai.FP16)
    assert x["q"].shape == (2, 4, 20, 8) and x["k"].shape == (2, 2, 20, 8)
    assert np.array_equal(x["q"][1, 3], ai.slab(7, ai.Q_ID, 1, 3, 20, 8, ai.FP16))
    assert np.array_equal(x["v"][0, 1], ai.slab(7, ai.V_ID, 0, 1, 20, 8, ai.FP16))
    vals = ai.bits_to_f64(x["q"], ai.FP16)
    assert abs(vals.mean()) < 0.1 and 0.8 < vals.std() < 1.2


def test_decode_inputs_nan_tail():
    lens = ai.decode_lengths(5, 3, 4, 9)
    assert lens.dtype == np.int32 and np.all((lens >= 4) & (lens <= 9))
    x = ai.decode_inputs(5, 3, 4, 2, 12, 8, ai.BF16, lens)
    for b in range(3):
        L = lens[b]
        assert np.all(x["k_cache"][b, :, L:] == ai.BF16_NAN_BITS)
        assert np.all(x["v_cache"][b, :, L:] == ai.BF16_NAN_BITS)
        assert np.all(np.isfinite(ai.bits_to_f64(x["k_cache"][b, :, :L], ai.BF16)))


def test_sample_rows():
    r = ai.sample_rows(4, 3, 131072, 256)
    assert len(r) == 256 and r[0] == 0 and r[-1] == 131071 and len(set(r.tolist())) == 256
    assert np.array_equal(r, np.sort(r))
    assert np.array_equal(ai.sample_rows(4, 3, 100, 256), np.arange(100))


def test_generator_hashes():
    """Regression pin: the byte streams recorded by tests/golden/make_generator_hashes.py."""
    with open(os.path.join(GOLDEN, "generator_sha256.json")) as f:
        want = json.load(f)
    from golden.make_generator_hashes import CASES, digest
    for name, args in CASES.items():
        assert digest(*args) == want[name], name


def test_decode_lengths_in_range():
    cfg = ai.CONFIGS["decode_32seq_gqa"]
    lens = ai.decode_lengths(cfg["seed"], cfg["B"], cfg["len_lo"], cfg["len_hi"])
    assert lens.min() >= 1024 and lens.max() <= 32768 and len(lens) == 32


def test_fp8_e4m3_codec():
    """OCP E4M3: known codes, every finite code round-trips, ties go to the
    even code, the largest finite value is 448 and NaN is 0x7F / 0xFF."""
    import math
    d = ai.fp8_decode(np.arange(256, dtype=np.uint8))
    assert d[0x38] == 1.0 and d[0xB8] == -1.0 and d[0x7E] == 448.0
    assert d[0x08] == 2.0 ** -6 and d[0x01] == 2.0 ** -9 and d[0x07] == 7 * 2.0 ** -9
    assert d[0x39] == 1.125 and d[0x40] == 2.0 and d[0x00] == 0.0
    assert math.isnan(d[0x7F]) and math.isnan(d[0xFF]) and np.sum(np.isnan(d)) == 2
    codes = np.arange(256, dtype=np.uint8)
    fin = ~np.isnan(d) & (codes != 0x80)
    assert np.array_equal(ai.fp8_encode(d[fin]), codes[fin])
    # midpoints: 1.0625 between 0x38 and 0x39 -> 0x38 (even); 1.1875 -> 0x3A
    assert ai.fp8_encode(np.array([1.0625, 1.1875, -1.0625]))[:3].tolist() == [0x38, 0x3A, 0xB8]
    assert ai.fp8_encode(np.array([1000.0]))[0] == 0x7E


def test_fp8_quantize_is_exact_scaling():
    x = np.random.default_rng(3).standard_normal((64, 128)).astype(np.float32)
    codes, ds = ai.fp8_quantize(x)
    assert ds == 2.0 ** np.ceil(np.log2(np.abs(x).max() / 448.0))
    back = ai.fp8_decode(codes) * ds
    assert np.abs(back).max() <= 448 * ds
    # relative rounding error of normal values within half an E4M3 ulp (2^-4)
    big = np.abs(x) > 2.0 ** -6 * ds * 2
    assert np.max(np.abs(back[big] - x[big]) / np.abs(x[big])) <= 2.0 ** -4
    y = ai.prefill_inputs_fp8(5, 1, 2, 1, 16, 128)
    assert y["q"].dtype == np.uint8 and y["q_descale"].shape == (1, 2) and y["k_descale"].shape == (1, 1)
