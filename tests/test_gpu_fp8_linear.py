"""GPU parity of the per-tensor FP8 (W8A8) dense linear and its tensor-wise quantizer
against the oracle, through the C ABI: codes and scale bit-exact; outputs to the final
bar (|d| <= 1e-2 max|ref|, <= 0.1% of elements above 1e-3 max|ref|, against the oracle's
bf16 rounding), bit-exact in the integer case; deterministic."""
import numpy as np
import pytest

import oracle
import synth
import w4a8_moe_amd as W
from tests.gpu_util import assert_final_close, bf16_bits_to_f64, bf16_dev, host, same_codes, static_scales, torch

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("N,K", [(1, 8), (3, 40), (16, 128), (257, 384), (64, 2560 + 8)])
def test_tensor_quant_bit_exact(N, K):
    cfg = synth.custom_block("tq", M=1, N=N, K=K, cfg=91, sub=N)
    w = synth.block_weights(cfg)
    q, s = W.fp8_tensor_quant(bf16_dev(w))
    qo, so = oracle.fp8_tensor_quantize(w)
    assert host(s)[0] == so
    assert same_codes(host(q), qo).all()


def test_tensor_quant_zeros():
    q, s = W.fp8_tensor_quant(bf16_dev(np.zeros((16, 256), np.uint16)))
    assert host(s)[0] == 0.0 and not host(q).any()


def test_integer_case_bit_exact():
    """Integer x with s_x = 1 and s_w = 1: every product and partial sum is an integer
    below 2^24, so the fp32 sums are exact in any order and y equals the oracle's bits."""
    rng = np.random.default_rng(92)
    M, N, K = 5, 96, 256
    xi = rng.integers(-8, 9, size=(M, K)).astype(np.float32)
    codes = rng.integers(0, 256, size=(N, K)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0
    x = synth.f32_to_bf16_bits(xi)
    y = W.fp8_linear_w8a8(bf16_dev(x), 1.0, torch().from_numpy(codes).cuda(), 1.0)
    _, ybits, _ = oracle.fp8_linear(x, np.float32(1.0), codes, np.float32(1.0))
    assert np.array_equal(host(y), ybits)


# larger N: up to 2 rows the activations are quantized inside the kernel (2 row blocks per
# workgroup), above that in a launch of their own (4 row blocks per workgroup)
@pytest.mark.parametrize("M,N,K", [(1, 256, 384), (8, 400, 256), (16, 128, 4096), (3, 1024, 6144), (10, 48, 6144),
                                   (2, 16, 128), (4, 16384, 256), (2, 8192, 384), (8, 8192, 256),
                                   # activations staged in chunks of K: more than 16 rows (up to 64, ragged
                                   # tiles), or M * K past 64 KB, or a ragged last K-quarter
                                   (32, 1024, 6144), (32, 6144, 768), (64, 512, 2560), (20, 256, 6144),
                                   (17, 128, 128), (16, 256, 8192), (2, 64, 33024), (48, 96, 1152),
                                   # two blocks in flight per lane: K-quarters of 2, 2, 1 and 0 blocks, of 4, 4,
                                   # 4 and 1
                                   (5, 64, 640), (12, 48, 1664)])
def test_fp8_linear_parity(M, N, K):
    cfg = synth.custom_block("fl", M=M, N=N, K=K, cfg=93, sub=N)
    w = synth.block_weights(cfg)
    x = synth.block_activations(cfg)
    s_x = oracle.static_scale(np.max(np.abs(bf16_to_f32(x)))) * np.float32(0.75)    # some codes saturate
    qo, so = oracle.fp8_tensor_quantize(w)
    q, s = W.fp8_tensor_quant(bf16_dev(w))
    assert same_codes(host(q), qo).all() and host(s)[0] == so
    y = W.fp8_linear_w8a8(bf16_dev(x), s_x, q, float(so))
    _, ybits, xq = oracle.fp8_linear(x, s_x, qo, so)
    # the activation codes the kernel stages follow fp8_quant_static's arithmetic
    assert same_codes(host(W.fp8_quant_static(bf16_dev(x), s_x)), xq).all()
    assert_final_close(bf16_bits_to_f64(host(y)), bf16_bits_to_f64(ybits))
    y2 = W.fp8_linear_w8a8(bf16_dev(x), s_x, q, float(so))
    assert torch().equal(y, y2)                                          # deterministic


def bf16_to_f32(bits):
    return oracle.bf16_to_f32(bits)


@pytest.mark.parametrize("name", sorted(synth.LINEAR_CONFIGS))
def test_fp8_linear_page_shapes(name):
    """The Grok-1 attention projections at decode rows 1 and 8, every output."""
    cfg = synth.LINEAR_CONFIGS[name]
    s_x = static_scales_linear(name)
    w = synth.block_weights(cfg)
    x = synth.block_activations(cfg)
    q, s = W.fp8_tensor_quant(bf16_dev(w))
    qo, so = oracle.fp8_tensor_quantize(w)
    assert host(s)[0] == so and same_codes(host(q), qo).all()
    y = W.fp8_linear_w8a8(bf16_dev(x), s_x, q, float(host(s)[0]))
    _, ybits, _ = oracle.fp8_linear(x, s_x, qo, so)
    assert_final_close(bf16_bits_to_f64(host(y)), bf16_bits_to_f64(ybits))


def static_scales_linear(name):
    import json
    import os
    from tests.gpu_util import GOLDEN
    d = json.load(open(os.path.join(GOLDEN, "static_scales.json")))[name]
    return np.float32(float.fromhex(d["s_x_hex"]))
