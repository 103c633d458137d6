"""Pins of the oracle's bf16 rounding and int4 quantization / packing (no GPU)."""
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import synth
from oracle import (bf16_to_f32, bf16_to_f64, f64_to_bf16_bits, w4_dequant, w4_pack,
                    w4_pack_codes, w4_quantize, w4_unpack_codes)


# ---------------------------------------------------------------- bf16

def test_bf16_decode_known():
    assert bf16_to_f32(np.uint16(0x3F80)) == 1.0
    assert bf16_to_f32(np.uint16(0xC000)) == -2.0
    assert bf16_to_f32(np.uint16(0x0001)) == 2.0 ** -133


def test_bf16_roundtrip_all_finite():
    bits = np.arange(65536, dtype=np.uint16)
    v = bf16_to_f64(bits)
    ok = np.isfinite(v)
    assert np.array_equal(f64_to_bf16_bits(v[ok]), bits[ok])


def test_bf16_rounding_matches_torch_on_fp32_values():
    rng = np.random.default_rng(3)
    v = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-8, 8, 20000),
                        rng.standard_normal(1000)]).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(f64_to_bf16_bits(v.astype(np.float64)), ref)


def test_bf16_ties_and_double_rounding():
    # exactly halfway between 1.0 (0x3F80) and the next bf16 (1 + 2^-7): even wins
    assert f64_to_bf16_bits(1.0 + 2.0 ** -8) == 0x3F80
    assert f64_to_bf16_bits(1.0 + 3 * 2.0 ** -8) == 0x3F82
    # just above the tie in fp64, but the tie itself in fp32: direct rounding goes up
    assert f64_to_bf16_bits(1.0 + 2.0 ** -8 + 2.0 ** -40) == 0x3F81


def test_synth_bf16_rounding_is_rne():
    v = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -3.14159, 1e-3], dtype=np.float32)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(synth.f32_to_bf16_bits(v), ref)


# ---------------------------------------------------------------- int4

def _rows(seed, n, k, sigma=0.02):
    rng = np.random.default_rng(seed)
    return synth.f32_to_bf16_bits((rng.standard_normal((n, k)) * sigma).astype(np.float32))


def test_quantize_invariants():
    w = _rows(1, 64, 512)
    q, s = w4_quantize(w)
    wf = bf16_to_f64(w)
    assert q.dtype == np.int8 and q.min() >= -7 and q.max() <= 7
    amax = np.max(np.abs(wf), axis=1)
    # the max-|w| element of every row maps to +-7 exactly
    arg = np.argmax(np.abs(wf), axis=1)
    assert np.array_equal(np.abs(q[np.arange(64), arg]), np.full(64, 7))
    # dequantization error at most half a step (plus fp32 rounding of the quotient)
    err = np.abs(wf - q * s.astype(np.float64)[:, None])
    assert np.all(err <= s[:, None] * (0.5 + 1e-6))
    # s is the correctly rounded fp32 of amax / 7
    for a, sv in zip(amax[:16], s[:16]):
        exact = Fraction(float(a)) / 7
        cand = [np.float32(sv), np.nextafter(np.float32(sv), np.float32(0)),
                np.nextafter(np.float32(sv), np.float32(1))]
        dists = [abs(Fraction(float(c)) - exact) for c in cand]
        assert dists[0] == min(dists)


def test_quantize_integer_rows_are_exact():
    rng = np.random.default_rng(2)
    qi = rng.integers(-7, 8, size=(8, 64))
    qi[:, 5] = 7                                    # every row has amax 7 -> s = 1
    w = synth.f32_to_bf16_bits(qi.astype(np.float32))
    q, s = w4_quantize(w)
    assert np.all(s == 1.0)
    assert np.array_equal(q, qi)


def test_quantize_rounding_half_even_and_zero_row():
    vals = np.array([[7.0, 2.5, 3.5, -2.5, -3.5, 0.5, -0.5, 1.5]], dtype=np.float32)
    q, s = w4_quantize(synth.f32_to_bf16_bits(vals))
    assert s[0] == 1.0
    assert q[0].tolist() == [7, 2, 4, -2, -4, 0, 0, 2]
    q0, s0 = w4_quantize(np.zeros((2, 16), np.uint16))
    assert np.all(s0 == 0) and np.all(q0 == 0)


def test_pack_layout_golden(golden_dir):
    for line in open(os.path.join(golden_dir, "int4_pack_layout.txt")):
        if not line.strip() or line.startswith("#"):
            continue
        parts = line.split()
        codes = np.array([int(p) for p in parts[:8]])
        word = np.uint32(int(parts[8], 16))
        got = w4_pack_codes(codes[None, :])[0, 0]
        assert np.uint32(got.view(np.uint32)) == word
        assert np.array_equal(w4_unpack_codes(np.array([[word]], np.uint32).view(np.int32))[0], codes)


def test_pack_unpack_roundtrip_brute_force():
    rng = np.random.default_rng(5)
    codes = rng.integers(-8, 8, size=(7, 96))
    assert np.array_equal(w4_unpack_codes(w4_pack_codes(codes)), codes)
    words = rng.integers(-2 ** 31, 2 ** 31, size=(5, 40), dtype=np.int64).astype(np.int32)
    assert np.array_equal(w4_pack_codes(w4_unpack_codes(words)), words)
    # one nibble at a time: element k lands in word k//8, nibble 2*(k%4) + (k%8)//4
    for k in range(16):
        c = np.zeros((1, 16), np.int64)
        c[0, k] = 1
        w = w4_pack_codes(c).view(np.uint32)[0]
        nib = 2 * (k % 4) + (k % 8) // 4
        expect = np.zeros(2, np.uint32)
        expect[k // 8] = np.uint32(1) << np.uint32(4 * nib)
        assert np.array_equal(w, expect)


def test_pack_matches_quantize_and_dequant():
    w = _rows(9, 32, 256)
    words, s = w4_pack(w)
    q, s2 = w4_quantize(w)
    assert np.array_equal(s, s2)
    assert words.shape == (32, 32)
    assert np.array_equal(w4_unpack_codes(words), q)
    assert np.allclose(w4_dequant(words, s), q * s[:, None].astype(np.float64))
