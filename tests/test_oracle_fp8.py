"""Pins of the oracle's E4M3 codec against the format definition, a library routine and
brute force (no GPU)."""
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import e4m3_decode, e4m3_encode, e4m3_table


def test_table_known_values():
    t = e4m3_table()
    assert t[0x00] == 0.0 and not np.signbit(t[0x00])
    assert t[0x80] == 0.0 and np.signbit(t[0x80])
    assert t[0x01] == 2.0 ** -9                 # smallest subnormal
    assert t[0x07] == 7 * 2.0 ** -9             # largest subnormal
    assert t[0x08] == 2.0 ** -6                 # smallest normal
    assert t[0x38] == 1.0
    assert t[0x39] == 1.125
    assert t[0x7E] == 448.0 and t[0xFE] == -448.0
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    assert np.sum(np.isnan(t)) == 2
    # codes 0x00..0x7E increase strictly
    assert np.all(np.diff(t[:0x7F]) > 0)
    # the bottom 16 codes are linear: code c has value c * 2^-9 (subnormals, then the
    # first binade), the fact the decode kernel's offset encoding relies on
    assert np.array_equal(t[:16], np.arange(16) * 2.0 ** -9)


def test_table_matches_torch_float8_e4m3fn():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    t = e4m3_table()
    nan = np.isnan(t)
    assert np.array_equal(nan, np.isnan(ref))
    assert np.array_equal(t[~nan], ref[~nan])


def test_roundtrip_every_finite_code():
    t = e4m3_table()
    codes = np.array([c for c in range(256) if not np.isnan(t[c])], dtype=np.uint8)
    assert np.array_equal(e4m3_encode(t[codes]), codes)


def _all_bf16_finite():
    bits = np.arange(65536, dtype=np.uint32)
    v = (bits << 16).view(np.float32)
    return v[np.isfinite(v)]


@pytest.mark.parametrize("scale", [1.0, 0.0123, 3.7e-3, 7.25])
def test_encode_matches_torch_cast_exhaustive_bf16(scale):
    """For |v| <= 448 torch's fp32 -> float8_e4m3fn cast rounds to nearest even; it is an
    independent implementation of the same rounding."""
    with np.errstate(over="ignore"):
        v = (_all_bf16_finite() / np.float32(scale)).astype(np.float32)
    v = v[np.abs(v) <= 448.0]
    ours = e4m3_encode(v)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    # torch may produce +0 for tiny negatives; compare values, and signs on nonzero
    same = (ours == ref) | ((ours & 0x7F) == 0) & ((ref & 0x7F) == 0)
    assert np.all(same)


def _brute_force_code(x: float) -> int:
    """Nearest finite code by scanning all 254 finite codes; tie -> even code."""
    t = e4m3_table()
    if abs(x) >= 448.0:
        return 0x7E | (0x80 if x < 0 else 0)
    best, bd = None, None
    for c in range(256):
        if np.isnan(t[c]):
            continue
        d = abs(Fraction(float(t[c])) - Fraction(x))
        if best is None or d < bd or (d == bd and c % 2 == 0 and best % 2 == 1):
            best, bd = c, d
    if t[best] == 0.0:
        best = 0x80 if np.signbit(x) else 0x00
    return best


def test_encode_brute_force_random_and_midpoints():
    rng = np.random.default_rng(7)
    t = e4m3_table()
    mags = t[:0x7F]
    mids = (mags[:-1] + mags[1:]) / 2                      # exact ties
    vals = np.concatenate([
        rng.standard_normal(300) * 50, rng.uniform(-460, 460, 200),
        mids, -mids, np.nextafter(mids, 0), np.nextafter(mids, 1000),
        [0.0, -0.0, 1e-30, -1e-30, 448.0, 449.0, 470.0, 1e9, -1e9],
    ]).astype(np.float32)
    got = e4m3_encode(vals)
    for v, g in zip(vals, got):
        assert g == _brute_force_code(float(v)), (float(v), hex(g))


def test_ties_to_even_examples():
    # 1.0625 lies halfway between 1.0 (0x38) and 1.125 (0x39): the even code wins
    assert e4m3_encode(1.0625) == 0x38
    # 1.1875 between 1.125 (0x39) and 1.25 (0x3A): even 0x3A
    assert e4m3_encode(1.1875) == 0x3A
    # halfway between 0 and the smallest subnormal rounds to zero
    assert e4m3_encode(2.0 ** -10) == 0x00
    assert e4m3_encode(-2.0 ** -10) == 0x80


def test_saturation_and_signed_zero():
    assert e4m3_encode(448.0) == 0x7E
    assert e4m3_encode(1e6) == 0x7E
    assert e4m3_encode(-1e6) == 0xFE
    assert e4m3_encode(-0.0) == 0x80
    assert e4m3_encode(0.0) == 0x00
    assert e4m3_encode(float("inf")) == 0x7E and e4m3_encode(float("-inf")) == 0xFE
    with pytest.raises(ValueError):
        e4m3_encode(float("nan"))


def test_int4_values_exact_in_e4m3(golden_dir):
    rows = [l.split() for l in open(os.path.join(golden_dir, "int4_e4m3_codes.txt"))
            if l.strip() and not l.startswith("#")]
    vals = np.array([int(r[0]) for r in rows])
    codes = np.array([int(r[1], 16) for r in rows], dtype=np.uint8)
    assert np.array_equal(vals, np.arange(-8, 8))
    assert np.array_equal(e4m3_encode(vals.astype(np.float64)), codes)
    assert np.array_equal(e4m3_decode(codes), vals.astype(np.float64))
