"""Pins of the oracle's per-tensor FP8 (W8A8) dense linear and its quantizers (no GPU)."""
from fractions import Fraction

import numpy as np

import synth
from oracle import (E4M3_MAX, bf16_to_f64, e4m3_decode, e4m3_encode, fp8_linear, fp8_linear_bruteforce,
                    fp8_quantize_activations, fp8_tensor_quantize, f64_to_bf16_bits, static_scale)


def _codes_without_nan(rng, shape):
    c = rng.integers(0, 256, size=shape).astype(np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x00
    return c


def test_integer_case_is_an_integer_matmul():
    """Integer x with s_x = 1 is its own code (|x| <= 8 is exact in E4M3) and s_w = 1:
    y is the plain matrix product of x and the decoded weights, exactly."""
    rng = np.random.default_rng(81)
    M, N, K = 3, 40, 256
    xi = rng.integers(-8, 9, size=(M, K)).astype(np.float32)
    x = synth.f32_to_bf16_bits(xi)
    codes = _codes_without_nan(rng, (N, K))
    y, ybits, xq = fp8_linear(x, np.float32(1.0), codes, np.float32(1.0))
    assert np.array_equal(e4m3_decode(xq), xi.astype(np.float64))
    ref = xi.astype(np.float64) @ e4m3_decode(codes).T
    assert np.array_equal(y, ref)
    assert np.array_equal(ybits, f64_to_bf16_bits(ref))


def test_vectorised_equals_brute_force_loops():
    cfg = synth.custom_block("lb", M=2, N=24, K=96, cfg=82)
    w = synth.block_weights(cfg)
    x = synth.block_activations(cfg)
    codes, s_w = fp8_tensor_quantize(w)
    s_x = static_scale(np.max(np.abs(bf16_to_f64(x))))
    y, _, _ = fp8_linear(x, s_x, codes, s_w)
    yb = fp8_linear_bruteforce(x, s_x, codes, s_w)
    assert np.allclose(y, yb, rtol=1e-13, atol=1e-13 * np.abs(yb).max())


def test_tensor_quantizer_invariants():
    """One scale fp32(amax / 448) (checked with exact rationals), every code within
    +-448, the largest element maps to +-448, and each weight is within half an E4M3
    step (times s_w) of its decoded code."""
    cfg = synth.custom_block("lq", M=1, N=64, K=384, cfg=83)
    w = synth.block_weights(cfg)
    codes, s_w = fp8_tensor_quantize(w)
    wf = bf16_to_f64(w)
    amax = np.max(np.abs(wf))
    exact = Fraction(float(amax)) / 448
    # s_w is the float32 nearest to amax / 448
    lo = np.nextafter(s_w, np.float32(0)); hi = np.nextafter(s_w, np.float32(np.inf))
    assert abs(Fraction(float(s_w)) - exact) <= abs(Fraction(float(lo)) - exact)
    assert abs(Fraction(float(s_w)) - exact) <= abs(Fraction(float(hi)) - exact)
    dec = e4m3_decode(codes)
    assert np.all(np.abs(dec) <= E4M3_MAX)
    i = np.unravel_index(np.argmax(np.abs(wf)), wf.shape)
    assert abs(dec[i]) == E4M3_MAX and np.sign(dec[i]) == np.sign(wf[i])
    # E4M3 step at |v|: 2^(floor(log2 |v|) - 3) for normals, 2^-9 below 2^-6
    v = np.abs(wf / float(s_w))
    step = np.where(v >= 2.0 ** -6, 2.0 ** (np.floor(np.log2(np.maximum(v, 2.0 ** -6))) - 3), 2.0 ** -9)
    assert np.all(np.abs(wf - dec * float(s_w)) <= 0.5 * step * float(s_w) * (1 + 1e-6) + 1e-30)


def test_zero_weights_and_activation_codes():
    codes, s_w = fp8_tensor_quantize(np.zeros((16, 128), np.uint16))
    assert s_w == 0 and not codes.any()
    # activation codes are the static quantizer's: e4m3(fp32(x / s))
    x = synth.f32_to_bf16_bits(np.array([[0.0, 1.0, -3.5, 1000.0, 1e-9]], np.float32))
    s = np.float32(0.5)
    q = fp8_quantize_activations(x, s)
    assert np.array_equal(q, e4m3_encode(np.array([[0.0, 2.0, -7.0, 2000.0, 2e-9]], np.float32)))
    assert e4m3_decode(q)[0, 3] == 448.0                    # saturates


def test_against_unquantized_linear_within_the_quantization_bound():
    """|y - x W^T| <= sum_k |x - s_x dec(xq)| |W| + |s_x dec(xq)| |W - s_w dec(Wq)| per
    element (triangle inequality), and the relative error is that of 8-bit codes."""
    cfg = synth.custom_block("lu", M=4, N=96, K=512, cfg=84)
    w = synth.block_weights(cfg)
    x = synth.block_activations(cfg)
    codes, s_w = fp8_tensor_quantize(w)
    s_x = static_scale(np.max(np.abs(bf16_to_f64(x))))
    y, _, xq = fp8_linear(x, s_x, codes, s_w)
    xf, wf = bf16_to_f64(x), bf16_to_f64(w)
    xd = e4m3_decode(xq) * float(s_x)
    wd = e4m3_decode(codes) * float(s_w)
    ref = xf @ wf.T
    bound = np.abs(xf - xd) @ np.abs(wf).T + np.abs(xd) @ np.abs(wf - wd).T
    assert np.all(np.abs(y - ref) <= bound * (1 + 1e-12) + 1e-12)
    rel = np.linalg.norm(y - ref) / np.linalg.norm(ref)
    assert rel < 0.08, rel


def test_page_shapes():
    """Grok-1 attention: hidden 6144 = 48 heads x 128; 8 key/value heads x 128 = 1024."""
    assert synth.FP8_QKV_M1.N == 48 * 128 + 2 * 8 * 128 and synth.FP8_QKV_M1.K == 6144
    assert synth.FP8_O_M1.N == 6144 and synth.FP8_O_M1.K == 48 * 128
