"""Pins of the oracle's block-FP8 weight-only linear and its harness quantizer (no GPU)."""
import json
import os

import numpy as np

import synth
from oracle import (bf16_to_f64, e4m3_decode, fp8_block_linear, fp8_block_linear_bruteforce,
                    fp8_block_quantize, f64_to_bf16_bits)


def test_vectorised_equals_brute_force_loops():
    cfg = synth.custom_block("bb", M=2, N=144, K=256, cfg=71)     # a partial 128-row block
    w = synth.block_weights(cfg)
    x = synth.block_activations(cfg)
    codes, S = fp8_block_quantize(w)
    assert S.shape == (2, 2)
    y, _ = fp8_block_linear(x, codes, S)
    yb = fp8_block_linear_bruteforce(x, codes, S)
    assert np.allclose(y, yb, rtol=1e-12, atol=1e-12 * np.abs(yb).max())


def test_unit_scales_integer_x_reduce_to_matmul():
    rng = np.random.default_rng(72)
    M, N, K = 3, 256, 384
    codes = rng.integers(0, 256, size=(N, K)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x00                    # no NaN codes
    S = np.ones((2, 3), np.float32)
    xi = rng.integers(-4, 5, size=(M, K)).astype(np.float32)
    x = synth.f32_to_bf16_bits(xi)
    y, _ = fp8_block_linear(x, codes, S)
    assert np.array_equal(y, xi.astype(np.float64) @ e4m3_decode(codes).T)


def test_quantizer_invariants_and_dense_bound():
    cfg = synth.custom_block("bq", M=4, N=256, K=384, cfg=73)
    w = synth.block_weights(cfg)
    x = synth.block_activations(cfg)
    codes, S = fp8_block_quantize(w)
    wf = bf16_to_f64(w)
    deq = e4m3_decode(codes) * np.repeat(np.repeat(S.astype(np.float64), 128, 0), 128, 1)[:256, :384]
    for nb in range(2):
        for kb in range(3):
            blk = np.abs(wf[nb * 128:(nb + 1) * 128, kb * 128:(kb + 1) * 128])
            c = codes[nb * 128:(nb + 1) * 128, kb * 128:(kb + 1) * 128]
            assert np.abs(e4m3_decode(c)).max() == 448.0              # block max -> 448
            assert S[nb, kb] == np.float32(np.float32(blk.max()) / np.float32(448.0))
    # e4m3 relative half-step is 2^-4 for normals; subnormal steps are 2^-9 * S
    err = np.abs(wf - deq)
    step = np.maximum(np.abs(wf) * 2.0 ** -4, 2.0 ** -10 * np.repeat(np.repeat(S, 128, 0), 128, 1)[:256, :384])
    assert np.all(err <= step * (1 + 1e-6))
    y, ybits = fp8_block_linear(x, codes, S)
    ref = bf16_to_f64(x) @ wf.T
    assert np.all(np.abs(y - ref) <= np.abs(bf16_to_f64(x)) @ err.T + 1e-9)
    assert np.array_equal(ybits, f64_to_bf16_bits(y))


def test_zero_block():
    w = np.zeros((128, 256), np.uint16)
    w[:, 128:] = synth.f32_to_bf16_bits(np.full((128, 128), 0.5, np.float32))
    codes, S = fp8_block_quantize(w)
    assert S[0, 0] == 0 and np.all(codes[:, :128] == 0)
    assert S[0, 1] == np.float32(0.5) / np.float32(448)


def test_page_shapes(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "page_shapes.json")))
    for item in g["block_fp8"]:
        N, K = item["weight"]
        assert [(N + 127) // 128, (K + 127) // 128] == item["scale"]
    b = g["block_fp8_bytes"]
    # 2 bytes per bf16 element -> 1 byte per e4m3 element, within the pages' rounding
    assert abs(b["elements"] * 2 / 2 ** 30 - b["bf16_gib"]) < 0.02
    assert abs(b["elements"] * 1 / 2 ** 30 - b["fp8_gib"]) < 0.02
    gk = g["grok1"]
    assert (synth.GROK_DECODE.H, synth.GROK_DECODE.I, synth.GROK_DECODE.E) == \
        (gk["hidden_size"], gk["intermediate_size"], gk["num_local_experts"])
    assert synth.GROK_PREFILL.T == g["prefill"]["batch"] * g["prefill"]["input_len"]
    for c in synth.BLOCK_CONFIGS.values():
        assert [c.N, c.K] in [item["weight"] for item in g["block_fp8"]]


def test_fused_groups_concatenate_exactly():
    """Page C: every fp8 fusion group is a whole number of 128-row blocks (10240 / 6144 for
    in_proj_qkvz, 12288 / 512 / 512 for qkv), so quantizing the groups apart and
    concatenating rows and block scales gives the fused tensor's quantization, and the
    fused projection's outputs are the groups' outputs side by side."""
    for sizes, sub in (((10240, 6144), 0), ((12288, 512, 512), 1)):
        K = 256
        parts = [synth.block_weights(synth.custom_block(f"grp{sub}_{i}", M=1, N=n, K=K, cfg=75, sub=10 * sub + i))
                 for i, n in enumerate(sizes)]
        fused = np.concatenate(parts, axis=0)
        qf, Sf = fp8_block_quantize(fused)
        qs = [fp8_block_quantize(p) for p in parts]
        assert np.array_equal(qf, np.concatenate([q for q, _ in qs], axis=0))
        assert np.array_equal(Sf, np.concatenate([S for _, S in qs], axis=0))
        assert Sf.shape == (sum(sizes) // 128, K // 128)
        x = synth.block_activations(synth.custom_block("grpx", M=2, N=16, K=K, cfg=76))
        yf, _ = fp8_block_linear(x, qf, Sf)
        ys = np.concatenate([fp8_block_linear(x, q, S)[0] for q, S in qs], axis=1)
        assert np.array_equal(yf, ys)
