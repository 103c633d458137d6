"""Parity of the HIP library (through the C ABI) with the CPU oracle on seeded inputs.

Bit-exact: packing, the tiled weight layout, scales, fp8 activation codes, routing ids, counts, offsets,
sorted_pair, pair_pos, block-FP8 codes and scales. Tolerances: topk_w 1e-6; gate|up
1e-4 x row max; final outputs 1e-2 x max|ref| with at most 0.1% of elements above
1e-3 x max|ref| (bf16 outputs against the oracle's bf16-rounded result).
"""
import numpy as np
import pytest

import oracle
import synth
import w4a8_moe_amd as W
from tests.gpu_util import (assert_codes_consistent, assert_final_close, assert_gateup_close, bf16_bits_to_f64,
                            bf16_dev, f32_dev, host, same_codes, tile_words, torch, u8_dev)

pytestmark = pytest.mark.gpu


def _all_bf16_finite():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = bf16_bits_to_f64(bits)
    return bits[np.isfinite(v)]


# ----------------------------------------------------------------- fp8 activation quant

@pytest.mark.parametrize("scale", [1.0, 0.0123, 3.7e-3, 7.25, 2.0 ** -20])
def test_fp8_quant_exhaustive_bf16(scale):
    bits = _all_bf16_finite()
    got = host(W.fp8_quant_static(bf16_dev(bits), np.float32(scale)))
    ref = oracle.quantize_static(oracle.bf16_to_f32(bits), np.float32(scale))
    assert same_codes(got, ref).all()


@pytest.mark.parametrize("n", [1, 7, 8, 9, 1000, 4099])
def test_fp8_quant_tails(n):
    rng = np.random.default_rng(n)
    bits = synth.f32_to_bf16_bits(rng.standard_normal(n).astype(np.float32) * 3)
    got = host(W.fp8_quant_static(bf16_dev(bits), np.float32(0.01)))
    assert same_codes(got, oracle.quantize_static(oracle.bf16_to_f32(bits), np.float32(0.01))).all()


# ----------------------------------------------------------------------------- w4_pack

@pytest.mark.parametrize("E,N,K", [(1, 1, 8), (2, 48, 64), (3, 17, 264), (2, 5, 4096 + 8)])
def test_w4_pack_bit_exact(E, N, K):
    rng = np.random.default_rng(E * 1000 + N + K)
    w = synth.f32_to_bf16_bits((rng.standard_normal((E, N, K)) * 0.02).astype(np.float32))
    w[0, 0, :] = 0                                           # an all-zero row
    if N > 2:
        w[-1, 2, :] = synth.f32_to_bf16_bits(rng.integers(-7, 8, K).astype(np.float32))
    packed, scale = W.w4_pack(bf16_dev(w))
    ref_p, ref_s = oracle.w4_pack(w)
    assert np.array_equal(host(scale), ref_s)
    assert np.array_equal(host(packed), ref_p)


def test_w4_pack_tiny_layer():
    cfg = synth.TINY
    for which in ("w13", "w2"):
        w = synth.moe_weights(cfg, which)
        packed, scale = W.w4_pack(bf16_dev(w))
        ref_p, ref_s = oracle.w4_pack(w)
        assert np.array_equal(host(scale), ref_s) and np.array_equal(host(packed), ref_p)


@pytest.mark.parametrize("E,N,K", [(1, 16, 128), (3, 48, 384), (2, 272, 1152)])
def test_w4_tile_bit_exact(E, N, K):
    rng = np.random.default_rng(E * 7 + N + K)
    packed = rng.integers(-2**31, 2**31, (E, N, K // 8), dtype=np.int64).astype(np.int32)
    tiled = W.w4_tile(torch().from_numpy(packed).to("cuda"))
    assert np.array_equal(host(tiled), tile_words(packed))
    t2 = W.w4_pack(bf16_dev(synth.f32_to_bf16_bits(rng.standard_normal((E, N, K)).astype(np.float32))), tiled=True)
    assert tuple(t2[0].shape) == (E, N // 16, K // 128, 256)


# ------------------------------------------------------------------------ route + sort

def _check_route(logits):
    T, E = logits.shape
    r = W.moe_route_sort(f32_dev(logits))
    ids, w = oracle.route_top2(logits)
    counts, offsets, sp, pos = oracle.route_sort(ids, E)
    if T:
        assert np.array_equal(host(r["ids"]), ids)
        assert np.max(np.abs(host(r["weights"]) - w)) <= 1e-6
        assert np.array_equal(host(r["sorted_pair"]), sp)
        assert np.array_equal(host(r["pair_pos"]), pos)
    assert np.array_equal(host(r["counts"]), counts)
    assert np.array_equal(host(r["offsets"]), offsets)
    return r


@pytest.mark.parametrize("T,E,sigma", [(16, 4, 1.0), (32, 8, 1.5), (1, 2, 1.0), (255, 8, 1.5), (256, 8, 1.5),
                                       (257, 8, 1.5), (5000, 8, 1.5), (1000, 64, 1.0), (300, 256, 1.0),
                                       (4097, 3, 2.0), (20000, 8, 1.5), (33000, 256, 1.0), (40000, 3, 2.0),
                                       (70000, 100, 1.0)])
def test_route_sort_bit_exact(T, E, sigma):
    rng = np.random.default_rng(T * 7 + E)
    _check_route((rng.standard_normal((T, E)) * sigma).astype(np.float32))


@pytest.mark.parametrize("T,E", [(1 << 22, 8), ((1 << 17) + 5, 256)], ids=["max_tokens", "max_experts"])
def test_route_sort_largest(T, E):
    """The largest token count the calls accept (2^22: 16384 blocks of 256 tokens in the scan,
    512 per segment) and the largest expert count (one segment of 513 blocks per expert)."""
    rng = np.random.default_rng(E)
    _check_route((rng.standard_normal((T, E)) * 1.5).astype(np.float32))


@pytest.mark.parametrize("T,E,H", [(32, 8, 4096), (1, 2, 136), (256, 8, 520), (257, 8, 264), (3, 16, 9), (0, 8, 64)])
def test_route_sort_quant_matches_separate_calls(T, E, H):
    """One launch (T <= 256) or the multi-kernel routing then the quantization: the same
    bytes as moe_route_sort and fp8_quant_static called apart (ragged T*H % 8 tails too)."""
    rng = np.random.default_rng(T * 3 + E + H)
    logits = f32_dev((rng.standard_normal((T, E)) * 1.5).astype(np.float32))
    x = bf16_dev(synth.f32_to_bf16_bits((rng.standard_normal((T, H)) * 2).astype(np.float32)))
    s_x = np.float32(0.0123)
    got = W.moe_route_sort_quant(logits, x, s_x)
    ref = W.moe_route_sort(logits)
    for k in ("ids", "weights", "counts", "offsets", "sorted_pair", "pair_pos"):
        assert torch().equal(got[k], ref[k]), k
    assert torch().equal(got["xq"], W.fp8_quant_static(x, s_x))
    if T:
        assert same_codes(host(got["xq"]).reshape(-1),
                          oracle.quantize_static(oracle.bf16_to_f32(host(x).reshape(-1)), s_x)).all()


def test_route_sort_empty_and_ties():
    _check_route(np.zeros((0, 8), np.float32))
    l = np.array([[1, 2, 2, 0.5], [0, 0, 0, 0], [3, 1, 3, 3], [-1, 5, -1, -1], [7, 7, 7, 7]], np.float32)
    _check_route(l)
    rng = np.random.default_rng(5)
    skew = rng.standard_normal((3000, 8)).astype(np.float32)
    skew[:, 5] += 4.0                                          # one expert takes almost every token
    _check_route(skew)
    q = np.round(rng.standard_normal((600, 16)) * 2).astype(np.float32) / 2   # many equal logits
    _check_route(q)


def test_route_sort_deterministic():
    rng = np.random.default_rng(9)
    l = f32_dev(rng.standard_normal((4000, 8)).astype(np.float32))
    a, b = W.moe_route_sort(l), W.moe_route_sort(l)
    for k in ("ids", "weights", "counts", "offsets", "sorted_pair", "pair_pos"):
        assert torch().equal(a[k], b[k])


# ------------------------------------------------------------------------- MoE layer

def _oracle_scales(cfg, x, logits, p13, p2):
    s_x = oracle.static_scale(np.max(np.abs(oracle.bf16_to_f32(x))))
    pre = oracle.moe_forward(x, logits, s_x, p13, p2, cfg.act, np.float32(1.0), cfg.out_f32)
    return s_x, oracle.static_scale(np.max(np.abs(pre["a"])))


def _check_final(cfg, x, logits, s_x, p13, p2, s_a, ref, a, out):
    """The layer's output against the oracle's end-to-end result (its own gate|up, its own
    requantized codes, its own down projection and combine): the full bar, 1e-2 x max|ref|
    everywhere and at most 0.1% of the elements above 1e-3 x max|ref|. As a separate check
    of the down call alone, the output also meets the full bar against the oracle's down
    projection and combine of the kernel's own codes."""
    same = oracle.moe_forward(x, logits, s_x, p13, p2, cfg.act, s_a, cfg.out_f32, a_codes_given=host(a))
    if cfg.out_f32:
        got, want, e2e = host(out), same["out"].astype(np.float32), ref["out"].astype(np.float32)
    else:
        got = bf16_bits_to_f64(host(out))
        want, e2e = bf16_bits_to_f64(same["out_rounded"]), bf16_bits_to_f64(ref["out_rounded"])
    print("end to end:", end=" ")
    assert_final_close(got, e2e)
    print("down call on the kernel's codes:", end=" ")
    assert_final_close(got, want)


LAYER_CASES = [
    synth.TINY,
    synth.custom_moe("ragged_k", T=32, H=640, I=4736, E=8, act=synth.ACT_GELU_ERF, out_f32=False, w_cfg=201,
                     x_cfg=201, logit_sigma=1.5),
    synth.custom_moe("chunked", T=52, H=1152, I=1280, E=2, act=synth.ACT_SILU, w_cfg=202, x_cfg=202),
    # the most tokens the streaming kernel takes: every expert holds 64 rows, two passes of 32
    synth.custom_moe("two_passes", T=64, H=384, I=640, E=2, act=synth.ACT_GELU_TANH, w_cfg=207, x_cfg=207,
                     out_f32=False),
    synth.custom_moe("three_tiles", T=40, H=512, I=512, E=3, act=synth.ACT_GELU_TANH, w_cfg=203, x_cfg=203),
    synth.custom_moe("one_token", T=1, H=256, I=256, E=8, w_cfg=204, x_cfg=204),
    synth.custom_moe("many_experts", T=24, H=256, I=384, E=32, w_cfg=205, x_cfg=205, out_f32=False),
    # the largest expert count the calls accept: 256 experts, at most 48 of them routed to
    synth.custom_moe("max_experts", T=24, H=128, I=128, E=256, w_cfg=206, x_cfg=206, out_f32=False,
                     logit_sigma=2.0),
]


@pytest.mark.parametrize("cfg", LAYER_CASES, ids=[c.name for c in LAYER_CASES])
def test_moe_layer_parity(cfg):
    x = synth.activations(cfg)
    logits = synth.router_logits(cfg)
    w13 = synth.moe_weights(cfg, "w13")
    w2 = synth.moe_weights(cfg, "w2")
    p13, p2 = oracle.w4_pack(w13), oracle.w4_pack(w2)
    s_x, s_a = _oracle_scales(cfg, x, logits, p13, p2)
    ref = oracle.moe_forward(x, logits, s_x, p13, p2, cfg.act, s_a, cfg.out_f32)

    gw13, gs13 = W.w4_pack(bf16_dev(w13))
    gw2, gs2 = W.w4_pack(bf16_dev(w2))
    assert np.array_equal(host(gw13), p13[0]) and np.array_equal(host(gs13), p13[1])
    assert np.array_equal(host(gw2), p2[0]) and np.array_equal(host(gs2), p2[1])
    gw13, gw2 = W.w4_tile(gw13), W.w4_tile(gw2)
    r = W.moe_route_sort(f32_dev(logits))
    assert np.array_equal(host(r["sorted_pair"]), ref["sorted_pair"])
    xd = bf16_dev(x)
    a, h = W.moe_gemm1_w4a8(xd, s_x, gw13, gs13, r["offsets"], r["sorted_pair"], cfg.act, s_a, debug=True)
    assert_gateup_close(host(h), ref["h"])
    assert_codes_consistent(host(a), ref["a_codes"], host(h), cfg.act, s_a, cfg.I, a_ref=ref["a"])
    # the pre-quantized x path gives identical bytes
    xq = W.fp8_quant_static(xd, s_x)
    a2 = W.moe_gemm1_w4a8(xq, s_x, gw13, gs13, r["offsets"], r["sorted_pair"], cfg.act, s_a)
    assert torch().equal(a, a2)
    out = W.moe_gemm2_w4a8(a, s_a, gw2, gs2, r["offsets"], r["pair_pos"], r["weights"],
                           "f32" if cfg.out_f32 else "bf16")
    _check_final(cfg, x, logits, s_x, p13, p2, s_a, ref, a, out)
    # determinism: a second run is byte-identical
    a3 = W.moe_gemm1_w4a8(xd, s_x, gw13, gs13, r["offsets"], r["sorted_pair"], cfg.act, s_a)
    out3 = W.moe_gemm2_w4a8(a3, s_a, gw2, gs2, r["offsets"], r["pair_pos"], r["weights"],
                            "f32" if cfg.out_f32 else "bf16")
    assert torch().equal(a, a3) and torch().equal(out, out3)


# Token counts above 80 take the tiled kernel: tiles of 32, 64 or 256 rows (by the mean rows
# per expert) over each expert's segment (ragged last tiles, empty experts), 128-channel gate|up
# tiles, 256-channel down tiles.
PREFILL_CASES = [
    synth.custom_moe("pf_small", T=96, H=256, I=512, E=4, w_cfg=301, x_cfg=301),
    # the fewest tokens that take the tiled kernel (80 take the streaming one)
    synth.custom_moe("pf_first_tiled", T=81, H=384, I=256, E=8, act=synth.ACT_GELU_ERF, out_f32=False, w_cfg=307,
                     x_cfg=307, logit_sigma=1.5),
    synth.custom_moe("pf_ragged", T=300, H=640, I=384, E=8, act=synth.ACT_GELU_ERF, out_f32=False, w_cfg=302,
                     x_cfg=302, logit_sigma=1.5),
    synth.custom_moe("pf_multi_tile", T=700, H=1152, I=1280, E=2, w_cfg=303, x_cfg=303),
    synth.custom_moe("pf_skewed", T=520, H=512, I=256, E=8, act=synth.ACT_GELU_TANH, w_cfg=304, x_cfg=304,
                     expert_bias=True, logit_sigma=2.0),
    synth.custom_moe("pf_many_experts", T=200, H=384, I=256, E=32, w_cfg=305, x_cfg=305, out_f32=False),
    # 9 of 16 experts empty, several with a single row
    synth.custom_moe("pf_empty_experts", T=130, H=256, I=256, E=16, w_cfg=306, x_cfg=306, expert_bias=True,
                     logit_sigma=0.5),
    # the largest expert count the calls accept: 600 rows over 256 experts, tiles of one to a few rows
    synth.custom_moe("pf_max_experts", T=300, H=128, I=128, E=256, w_cfg=308, x_cfg=308, out_f32=False,
                     logit_sigma=2.0),
    # batches between decode and prefill (8 experts: 32 and 64 rows per expert on average)
    synth.custom_moe("pf_mid_128", T=128, H=512, I=1024, E=8, act=synth.ACT_SILU, w_cfg=309, x_cfg=309,
                     out_f32=False, logit_sigma=1.5),
    synth.custom_moe("pf_mid_256", T=256, H=512, I=1024, E=8, act=synth.ACT_GELU_ERF, w_cfg=310, x_cfg=310,
                     out_f32=False, logit_sigma=1.5),
    # a small grid with a long reduction: the down projection split into 4 K-slices
    synth.custom_moe("pf_split_k", T=96, H=256, I=4096, E=8, act=synth.ACT_SILU, w_cfg=311, x_cfg=311,
                     out_f32=False, logit_sigma=1.5),
    # odd k-step counts (3 for gate|up, 9 for down) through the two-step register ring of the
    # 32-row tiles: the ring's last pass is half empty
    synth.custom_moe("pf_odd_steps", T=80, H=384, I=1152, E=8, act=synth.ACT_GELU_ERF, w_cfg=312, x_cfg=312,
                     out_f32=False, logit_sigma=1.5),
    # enough rows per expert (about 1600) for the 256-row tiles
    synth.custom_moe("pf_big_tiles", T=3200, H=256, I=512, E=4, act=synth.ACT_SILU, w_cfg=313, x_cfg=313,
                     out_f32=False, logit_sigma=1.5),
]


@pytest.mark.parametrize("cfg", PREFILL_CASES, ids=[c.name for c in PREFILL_CASES])
def test_moe_prefill_parity(cfg):
    """The tiled path: gate|up to the 1e-4 bar, codes and final output as in the layer test."""
    x = synth.activations(cfg)
    logits = synth.router_logits(cfg)
    w13 = synth.moe_weights(cfg, "w13")
    w2 = synth.moe_weights(cfg, "w2")
    p13, p2 = oracle.w4_pack(w13), oracle.w4_pack(w2)
    s_x, s_a = _oracle_scales(cfg, x, logits, p13, p2)
    ref = oracle.moe_forward(x, logits, s_x, p13, p2, cfg.act, s_a, cfg.out_f32)
    gw13, gs13 = W.w4_pack(bf16_dev(w13), tiled=True)
    gw2, gs2 = W.w4_pack(bf16_dev(w2), tiled=True)
    r = W.moe_route_sort(f32_dev(logits))
    assert np.array_equal(host(r["offsets"]), ref["offsets"])
    print(f"{cfg.name}: rows per expert {np.diff(ref['offsets']).tolist()}", flush=True)
    xd = bf16_dev(x)
    a, h = W.moe_gemm1_w4a8(xd, s_x, gw13, gs13, r["offsets"], r["sorted_pair"], cfg.act, s_a, debug=True)
    assert_gateup_close(host(h), ref["h"])
    assert_codes_consistent(host(a), ref["a_codes"], host(h), cfg.act, s_a, cfg.I, a_ref=ref["a"])
    a2 = W.moe_gemm1_w4a8(W.fp8_quant_static(xd, s_x), s_x, gw13, gs13, r["offsets"], r["sorted_pair"], cfg.act,
                          s_a)
    assert torch().equal(a, a2)
    od = "f32" if cfg.out_f32 else "bf16"
    out = W.moe_gemm2_w4a8(a, s_a, gw2, gs2, r["offsets"], r["pair_pos"], r["weights"], od)
    _check_final(cfg, x, logits, s_x, p13, p2, s_a, ref, a, out)
    a3 = W.moe_gemm1_w4a8(xd, s_x, gw13, gs13, r["offsets"], r["sorted_pair"], cfg.act, s_a)
    out3 = W.moe_gemm2_w4a8(a3, s_a, gw2, gs2, r["offsets"], r["pair_pos"], r["weights"], od)
    assert torch().equal(a, a3) and torch().equal(out, out3)


@pytest.mark.parametrize("T,E", [(20, 4), (66, 8), (100, 4), (600, 4), (3200, 2)])
def test_integer_case_gate_up_bit_exact(T, E):
    """Integer x and w, max |w| = 7 per row, s_x = 1: fp32 accumulation is exact in any
    order, so gate|up must equal the integer product exactly (20 tokens: the streaming
    kernel; then the tiled kernel with 32-, 64- (two cases) and 256-row tiles)."""
    rng = np.random.default_rng(77 + T)
    H, I = 384, 256
    xi = rng.integers(-16, 17, size=(T, H))
    w13i = rng.integers(-7, 8, size=(E, 2 * I, H))
    w13i[:, :, 3] = 7
    x = synth.f32_to_bf16_bits(xi.astype(np.float32))
    w13 = synth.f32_to_bf16_bits(w13i.astype(np.float32))
    logits = rng.standard_normal((T, E)).astype(np.float32)
    gw13, gs13 = W.w4_pack(bf16_dev(w13), tiled=True)
    assert np.all(host(gs13) == 1.0)
    r = W.moe_route_sort(f32_dev(logits))
    a, h = W.moe_gemm1_w4a8(bf16_dev(x), 1.0, gw13, gs13, r["offsets"], r["sorted_pair"], W.ACT_SILU, 1.0,
                            debug=True)
    h = host(h)
    sp, off = host(r["sorted_pair"]), host(r["offsets"])
    for row in range(2 * T):
        e = int(np.searchsorted(off, row, side="right") - 1)
        assert np.array_equal(h[row], (w13i[e] @ xi[sp[row] // 2]).astype(np.float32)), row


# -------------------------------------------------------------------------- block FP8

@pytest.mark.parametrize("N,K", [(200, 400), (128, 128), (16, 2560)])
def test_fp8_block_quant_bit_exact(N, K):
    cfg = synth.custom_block("bq", M=1, N=N, K=K, cfg=300 + N)
    w = synth.block_weights(cfg)
    w[:3, :] = 0
    if N >= 128 and K >= 128:
        w[:128, :128] = 0                                    # a zero block
    q, S = W.fp8_block_quant(bf16_dev(w))
    rq, rS = oracle.fp8_block_quantize(w)
    assert np.array_equal(host(S), rS)
    assert same_codes(host(q), rq).all()


@pytest.mark.parametrize("M,N,K", [(1, 256, 384), (8, 400, 256), (16, 128, 2048), (3, 1024, 2560), (12, 64, 2560),
                                   (2, 48, 384), (5, 80, 1152), (1, 16, 128),
                                   # activations staged in chunks of K: more than 16 rows (up to 64, ragged
                                   # tiles), or more than 64 KB of them, or a ragged last K-quarter
                                   (32, 256, 2560), (64, 128, 1024), (20, 512, 2560), (16, 256, 4096),
                                   (48, 80, 1152), (2, 64, 16512), (17, 144, 128)])
def test_fp8_block_linear_parity(M, N, K):
    cfg = synth.custom_block("bl", M=M, N=N, K=K, cfg=400 + M)
    w = synth.block_weights(cfg)
    x = synth.block_activations(cfg)
    codes, S = oracle.fp8_block_quantize(w)
    y_ref, y_bits = oracle.fp8_block_linear(x, codes, S)
    y = W.fp8_block_linear(bf16_dev(x), u8_dev(codes), f32_dev(S))
    assert_final_close(bf16_bits_to_f64(host(y)), bf16_bits_to_f64(y_bits))
    y2 = W.fp8_block_linear(bf16_dev(x), u8_dev(codes), f32_dev(S))
    assert torch().equal(y, y2)


def test_empty_batch():
    """No tokens: every call returns OK and enqueues nothing; the layer's output is empty."""
    t = torch()
    cfg = synth.custom_moe("empty", T=1, H=256, I=256, E=8, w_cfg=208, x_cfg=208, out_f32=False)
    w13, s13 = W.w4_pack(bf16_dev(synth.moe_weights(cfg, "w13")), tiled=True)
    w2, s2 = W.w4_pack(bf16_dev(synth.moe_weights(cfg, "w2")), tiled=True)
    x = t.empty((0, cfg.H), dtype=t.bfloat16, device="cuda")
    logits = t.empty((0, cfg.E), dtype=t.float32, device="cuda")
    out = W.moe_layer(x, 0.01, logits, w13, s13, w2, s2, cfg.act, 0.05)
    t.cuda.synchronize()
    assert tuple(out.shape) == (0, cfg.H)


@pytest.mark.parametrize("sizes", [(10240, 6144), (12288, 512, 512)])
def test_fp8_block_fused_groups(sizes):
    """The fusion groups of the block-FP8 projections (whole numbers of 128-row blocks):
    quantizing the fused weight equals quantizing the groups and concatenating rows and
    scales, and the fused GEMV's outputs equal the groups' GEMVs side by side, bit for bit
    (each 16-row block is reduced on its own, in the same order)."""
    K, M = 512, 8
    parts = [synth.block_weights(synth.custom_block(f"gg{i}", M=1, N=n, K=K, cfg=77, sub=i))
             for i, n in enumerate(sizes)]
    qf, Sf = W.fp8_block_quant(bf16_dev(np.concatenate(parts, axis=0)))
    qs = [W.fp8_block_quant(bf16_dev(p)) for p in parts]
    assert torch().equal(qf, torch().cat([q for q, _ in qs], 0))
    assert torch().equal(Sf, torch().cat([S for _, S in qs], 0))
    x = bf16_dev(synth.block_activations(synth.custom_block("ggx", M=M, N=16, K=K, cfg=78)))
    yf = W.fp8_block_linear(x, qf, Sf)
    ys = torch().cat([W.fp8_block_linear(x, q, S) for q, S in qs], 1)
    assert torch().equal(yf, ys)
