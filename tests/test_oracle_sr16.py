"""Pins of the oracle's SR16 rule and its counter-based entropy.

The rule ("Nemotron 3 Ultra: replaying a rounded state", section "Stochastic
rounding and the mean state"): a value between two grid points goes to the
upper one when the entropy residue is smaller than the discarded remainder, so
it is unbiased and its error is below one grid step.  The grid is binary16.

Pins: SplitMix64's published seed-0 outputs; the result is always one of the
two binary16 neighbours that numpy's float16 type gives; representable values
are unchanged; 1027.25 (binary16 spacing 1) reproduces the page's 3.25 example
(up with probability 1/4, errors +0.75/-0.25, square excess 3/16); unbiasedness
over many keys; special values; uniformity of the entropy words.
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_splitmix64_published_vectors():
    gold = json.load(open(os.path.join(GOLD, "splitmix64_seed0.json")))
    for k, hx in enumerate(gold["outputs_hex"]):
        assert oracle.splitmix64_output(gold["seed"], k) == int(hx, 16)


def test_hash_is_keyed_by_all_three_counters():
    base = oracle.hash32(7, 3, 100)
    assert base == oracle.hash32(7, 3, 100)
    assert base != oracle.hash32(8, 3, 100)
    assert base != oracle.hash32(7, 4, 100)
    assert base != oracle.hash32(7, 3, 101)
    # definition: output e // 2 of the stream seeded by output j, high word for even e,
    # low word for odd e (one output serves two elements)
    sub = oracle.splitmix64_output(7, 3)
    out = oracle.splitmix64_output(sub, 50)
    assert base == out >> 32
    assert oracle.hash32(7, 3, 101) == out & 0xFFFFFFFF
    assert oracle.hash32(7, 3, 102) == oracle.splitmix64_output(sub, 51) >> 32


def test_hash_uniform_top_byte():
    n = 1 << 16
    bins = np.zeros(256)
    for e in range(n):
        bins[oracle.hash32(12345, 2, e) >> 24] += 1
    exp = n / 256
    chi2 = float(((bins - exp) ** 2 / exp).sum())
    # 255 dof: mean 255, sd ~22.6; 400 is > 6 sd
    assert chi2 < 400, chi2


def _neighbours16(v):
    """Binary16 values bracketing |v| (lo <= |v| <= hi), via numpy float16."""
    m = abs(float(v))
    h = np.float16(m)
    if float(h) > m:
        hi, lo = h, np.nextafter(h, np.float16(0))
    else:
        lo, hi = h, np.nextafter(h, np.float16(np.inf))
    return float(lo), float(hi)


def test_results_are_binary16_neighbours_and_exact_values_fixed():
    r = np.random.default_rng(3)
    vals = np.concatenate([
        r.standard_normal(4000).astype(np.float32) * np.float32(10.0) ** r.integers(-6, 5, 4000),
        np.float32(r.uniform(-6e-8, 6e-8, 500)),  # subnormal binary16 range
    ]).astype(np.float32)
    bits = oracle.sr16(vals, seed=99, ckpt=5)
    back = bits.view(np.float16).astype(np.float64)
    for v, b in zip(vals, back):
        lo, hi = _neighbours16(v)
        assert abs(b) in (lo, hi), (v, b, lo, hi)
        assert math.copysign(1.0, b) == math.copysign(1.0, v) or b == 0.0
        if float(np.float16(v)) == float(v):
            assert b == float(v)
    # every representable binary16 value is a fixed point for every key
    allh = np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float32)
    for ck in range(3):
        assert np.array_equal(oracle.sr16(allh, seed=1, ckpt=ck),
                              allh.astype(np.float16).view(np.uint16))


def test_page_example_three_and_a_quarter():
    gold = json.load(open(os.path.join(GOLD, "stochastic_rounding_example.json")))
    v = gold["fp16_value"]
    n = 1 << 16
    res = oracle.sr16(np.full(n, v, np.float32), seed=2024, ckpt=0).view(np.float16)
    res = res.astype(np.float64)
    assert set(np.unique(res)) == {gold["fp16_down"], gold["fp16_up"]}
    p_up = float(np.mean(res == gold["fp16_up"]))
    sd = math.sqrt(0.25 * 0.75 / n)
    assert abs(p_up - 0.25) < 5 * sd
    err = res - v
    assert set(np.unique(err)) == {-0.25, 0.75}
    assert abs(err.mean()) < 5 * math.sqrt(3 / 16 / n)
    # the square's mean exceeds the squared mean by the variance 3/16
    assert abs((res ** 2).mean() - res.mean() ** 2 - 3 / 16) < 0.01


def test_unbiased_over_keys():
    r = np.random.default_rng(5)
    vals = (r.standard_normal(40) * 3).astype(np.float32)
    n = 1 << 14
    for i, v in enumerate(vals):
        res = oracle.sr16(np.full(n, v, np.float32), seed=77, ckpt=i).view(np.float16)
        res = res.astype(np.float64)
        lo, hi = _neighbours16(v)
        q = hi - lo
        sd = q * 0.5 / math.sqrt(n)
        assert abs(res.mean() - float(v)) < 5 * sd + 1e-300


def test_special_values():
    f32 = np.float32
    cases = [f32(0.0), f32(-0.0), f32(np.inf), f32(-np.inf), f32(np.nan), f32(-np.nan),
             f32(65504.0), f32(-65504.0), f32(65536.0), f32(1e30)]
    bits = [oracle.sr16_one(float(c), u) for c in cases for u in (0, 0xFFFFFFFF)]
    exp = [0x0000, 0x0000, 0x8000, 0x8000, 0x7C00, 0x7C00, 0xFC00, 0xFC00, 0x7E00, 0x7E00,
           0xFE00, 0xFE00, 0x7BFF, 0x7BFF, 0xFBFF, 0xFBFF, 0x7C00, 0x7C00, 0x7C00, 0x7C00]
    assert bits == exp
    # between 65504 and 65536: 65504 or infinity, up with probability (v-65504)/32
    v = 65512.0  # remainder 1/4
    assert oracle.sr16_one(v, 0) == 0x7C00
    assert oracle.sr16_one(v, (1 << 30) - 1) == 0x7C00
    assert oracle.sr16_one(v, 1 << 30) == 0x7BFF
    # half the smallest subnormal: 0 or 2^-24, threshold at 2^31
    v = 2.0 ** -25
    assert oracle.sr16_one(v, (1 << 31) - 1) == 0x0001
    assert oracle.sr16_one(v, 1 << 31) == 0x0000
    # the largest subnormal rounds up into the smallest normal
    v = (1023.5) * 2.0 ** -24
    assert oracle.sr16_one(v, 0) == 0x0400
    assert oracle.sr16_one(v, 0xFFFFFFFF) == 0x03FF
    # top of a binade rounds up into the next binade
    v = float(np.float32(2047.5))
    assert oracle.sr16_one(v, 0) == int(np.float16(2048.0).view(np.uint16))


def test_threshold_is_strict():
    """u < R rounds up; u == R does not (R = floor(remainder * 2^32))."""
    v = 1.0 + 2.0 ** -12  # remainder 1/4 of the spacing 2^-10 -> R = 2^30
    assert oracle.sr16_one(v, (1 << 30) - 1) == int(np.float16(1.0 + 2 ** -10).view(np.uint16))
    assert oracle.sr16_one(v, 1 << 30) == int(np.float16(1.0).view(np.uint16))


def test_element_offset_keys():
    r = np.random.default_rng(1)
    v = r.standard_normal(1000).astype(np.float32)
    full = oracle.sr16(v, seed=5, ckpt=9)
    part = oracle.sr16(v[300:], seed=5, ckpt=9, elem_offset=300)
    assert np.array_equal(full[300:], part)
    for i in (0, 17, 999):
        assert full[i] == oracle.sr16_one(float(v[i]), oracle.hash32(5, 9, i))


def test_half_widening_exact():
    allbits = np.arange(0, 1 << 16, dtype=np.uint16)
    ours = oracle.half_bits_to_double(allbits)
    ref = allbits.view(np.float16).astype(np.float64)
    fin = np.isfinite(ref)
    assert np.array_equal(ours[fin], ref[fin])
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
