"""Pins of the oracle's FP8 KV cache store (no GPU)."""
import numpy as np

import synth
from oracle import E4M3_MAX, MIN_KV_SCALE, bf16_to_f64, e4m3_decode, kv_cache_store, kv_scale


def _rows(T, D, seed, sigma=1.0):
    rng = np.random.default_rng(seed)
    return synth.f32_to_bf16_bits((rng.standard_normal((T, D)) * sigma).astype(np.float32))


def test_scale_floor_and_exact_cases():
    assert MIN_KV_SCALE == 1.0                                  # page A: min_kv_scale 1.0
    assert kv_scale(10.0) == np.float32(1.0)                    # 10 / 448 < 1: the floor
    assert kv_scale(448.0 * 3) == np.float32(3.0)               # exact quotient
    assert kv_scale(0.0) == np.float32(1.0)
    assert kv_scale(1000.0) == np.float32(np.float32(1000.0) / np.float32(448.0))


def test_integer_rows_are_stored_exactly_under_the_floor():
    """With s = 1 an integer of magnitude <= 16 is an E4M3 value: the code decodes to it."""
    T, D = 6, 32
    ki = np.random.default_rng(1).integers(-16, 17, size=(T, D)).astype(np.float32)
    k = synth.f32_to_bf16_bits(ki)
    kc, vc = kv_cache_store(k, k, np.arange(T), 1.0, 1.0, np.zeros((T, D), np.uint8), np.zeros((T, D), np.uint8))
    assert np.array_equal(e4m3_decode(kc), ki.astype(np.float64))
    assert np.array_equal(kc, vc)


def test_slots_padding_and_untouched_rows():
    """Token t lands in row slots[t] (brute force, row by row); a negative slot stores
    nothing; rows not written keep their bytes."""
    T, D, S = 9, 64, 20
    k, v = _rows(T, D, 2, 3.0), _rows(T, D, 3, 0.5)
    slots = np.array([7, -1, 0, 19, 3, -1, 12, 5, 8])
    k0 = np.random.default_rng(4).integers(0, 256, size=(S, D)).astype(np.uint8)
    v0 = np.random.default_rng(5).integers(0, 256, size=(S, D)).astype(np.uint8)
    s_k, s_v = np.float32(1.25), np.float32(1.0)
    kc, vc = kv_cache_store(k, v, slots, s_k, s_v, k0, v0)
    kf, vf = bf16_to_f64(k), bf16_to_f64(v)
    written = set(int(s) for s in slots if s >= 0)
    for row in range(S):
        if row not in written:
            assert np.array_equal(kc[row], k0[row]) and np.array_equal(vc[row], v0[row])
    for t, s in enumerate(slots):
        if s < 0:
            continue
        # every stored code decodes to within half an E4M3 step (times the scale) of the value
        for val, code, sc in ((kf[t], kc[s], s_k), (vf[t], vc[s], s_v)):
            q = val / float(sc)
            dec = e4m3_decode(code)
            a = np.abs(q)
            step = np.where(a >= 2.0 ** -6, 2.0 ** (np.floor(np.log2(np.maximum(a, 2.0 ** -6))) - 3), 2.0 ** -9)
            assert np.all((np.abs(dec - q) <= 0.5 * step * (1 + 1e-9)) | (np.abs(q) > E4M3_MAX))


def test_saturation():
    k = synth.f32_to_bf16_bits(np.array([[1000.0, -5000.0, 448.0, 0.0]], np.float32))
    kc, _ = kv_cache_store(k, k, [0], 1.0, 1.0, np.zeros((1, 4), np.uint8), np.zeros((1, 4), np.uint8))
    assert e4m3_decode(kc).tolist() == [[448.0, -448.0, 448.0, 0.0]]
