"""GPU parity of the FP8 KV cache store against the oracle, through the C ABI: stored
codes bit-exact, padding and out-of-range slots not stored, untouched rows kept."""
import numpy as np
import pytest

import oracle
import synth
import w4a8_moe_amd as W
from tests.gpu_util import bf16_dev, host, same_codes, torch

pytestmark = pytest.mark.gpu


def _rows(T, D, seed, sigma):
    rng = np.random.default_rng(seed)
    return synth.f32_to_bf16_bits((rng.standard_normal((T, D)) * sigma).astype(np.float32))


# Grok-1: 8 key/value heads of 128 (D = 1024), one GPU's 8-way share holds one head (D = 128);
# sigma 200 puts the calibrated scale above the min_kv_scale floor, 0.5 below it
@pytest.mark.parametrize("T,D,S,sigma", [(32, 1024, 4096, 0.5), (32, 128, 512, 200.0), (1, 8, 4, 3.0),
                                         (300, 1024, 1000, 50.0)])
def test_kv_cache_store_bit_exact(T, D, S, sigma):
    t = torch()
    k, v = _rows(T, D, T + D, sigma), _rows(T, D, T + D + 1, sigma * 0.7)
    s_k = oracle.kv_scale(np.max(np.abs(oracle.bf16_to_f32(k))))
    s_v = oracle.kv_scale(np.max(np.abs(oracle.bf16_to_f32(v))))
    rng = np.random.default_rng(S)
    slots = rng.choice(S, size=T, replace=False).astype(np.int32)
    slots[rng.random(T) < 0.1] = -1                                   # padding tokens
    k0 = rng.integers(0, 256, size=(S, D)).astype(np.uint8)
    v0 = rng.integers(0, 256, size=(S, D)).astype(np.uint8)
    kc, vc = t.from_numpy(k0).cuda(), t.from_numpy(v0).cuda()
    W.fp8_kv_cache_store(bf16_dev(k), bf16_dev(v), t.from_numpy(slots).cuda(), s_k, s_v, kc, vc)
    rk, rv = oracle.kv_cache_store(k, v, slots, s_k, s_v, k0, v0)
    assert same_codes(host(kc), rk).all() and same_codes(host(vc), rv).all()
    written = np.zeros(S, bool)
    written[slots[slots >= 0]] = True
    assert np.array_equal(host(kc)[~written], k0[~written])          # untouched rows: same bytes


def test_kv_cache_store_out_of_range_slot():
    t = torch()
    T, D, S = 4, 64, 8
    k = _rows(T, D, 7, 1.0)
    slots = np.array([0, 8, 100, 3], np.int32)                          # 8 and 100 are past the cache
    k0 = np.full((S, D), 0x5A, np.uint8)
    kc, vc = t.from_numpy(k0.copy()).cuda(), t.from_numpy(k0.copy()).cuda()
    W.fp8_kv_cache_store(bf16_dev(k), bf16_dev(k), t.from_numpy(slots).cuda(), 1.0, 1.0, kc, vc)
    rk, _ = oracle.kv_cache_store(k, k, np.array([0, -1, -1, 3]), 1.0, 1.0, k0, k0)
    assert same_codes(host(kc), rk).all() and same_codes(host(vc), rk).all()
