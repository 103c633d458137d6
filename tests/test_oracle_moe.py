"""Pins of the oracle's W4A8 MoE layer against closed forms, exact integer cases, a
plain dense two-expert computation, and the unquantized layer within a rigorous
error bound (no GPU)."""
import math

import numpy as np
import pytest
from scipy.special import expit
from scipy.stats import norm

import synth
from oracle import (ACT_GELU_ERF, ACT_GELU_TANH, ACT_SILU, activation, act_lipschitz,
                    bf16_to_f32, bf16_to_f64, e4m3_decode, moe_error_bound, moe_forward,
                    moe_reference_unquantized, quantize_static, static_scale, w4_pack,
                    w4_quantize, w4_unpack_codes, route_top2)


def test_activation_closed_forms():
    g = np.linspace(-12, 12, 2001)
    assert np.allclose(activation(g, ACT_SILU), g * expit(g), rtol=1e-13, atol=1e-15)
    assert np.allclose(activation(g, ACT_GELU_ERF), g * norm.cdf(g), rtol=1e-12, atol=1e-15)
    for a in (ACT_SILU, ACT_GELU_ERF, ACT_GELU_TANH):
        assert activation(0.0, a) == 0.0
        assert abs(activation(40.0, a) - 40.0) < 1e-9
        assert abs(activation(-40.0, a)) < 1e-9
    # the tanh form stays within 1e-3 of the erf form
    assert np.max(np.abs(activation(g, ACT_GELU_TANH) - activation(g, ACT_GELU_ERF))) < 1e-3


def test_activations_against_torch():
    """Each activation against torch's own implementation of the same function (an
    independent library routine), in float64 to 1e-12: silu, gelu (erf form) and gelu with
    approximate="tanh" (the cubic coefficient 0.044715 and sqrt(2/pi) of the tanh form)."""
    import torch
    g = np.concatenate([np.linspace(-12, 12, 4001), [-3.0, -2.0, -1.0, -0.5, 0.5, 1.0, 2.0, 3.0]])
    t = torch.from_numpy(g)
    F = torch.nn.functional
    for act, ref in ((ACT_SILU, F.silu(t)), (ACT_GELU_ERF, F.gelu(t)), (ACT_GELU_TANH, F.gelu(t, approximate="tanh"))):
        ref = ref.numpy()
        got = activation(g, act)
        assert np.all(np.abs(got - ref) <= 1e-12 * np.maximum(1.0, np.abs(ref))), act


def test_gelu_tanh_identities():
    """The tanh form through an independent algebraic path: 1/2 (1 + tanh y) = sigma(2 y), so
    gelu_tanh(g) = g * expit(2 sqrt(2/pi) (g + 0.044715 g^3)); and it meets gelu_tanh(g) -
    gelu_tanh(-g) = g."""
    g = np.linspace(-9, 9, 3601)
    y = math.sqrt(2.0 / math.pi) * (g + 0.044715 * g * g * g)
    assert np.allclose(activation(g, ACT_GELU_TANH), g * expit(2.0 * y), rtol=1e-12, atol=1e-14)
    assert np.allclose(activation(g, ACT_GELU_TANH) - activation(-g, ACT_GELU_TANH), g, rtol=1e-13, atol=1e-13)


def test_lipschitz_constants():
    # silu' peaks at about 1.0998 near g = 2.4; gelu_erf' = Phi(g) + g phi(g) peaks at g = sqrt 2
    assert abs(act_lipschitz(ACT_SILU) - 1.0998) < 1e-3
    peak = norm.cdf(math.sqrt(2)) + math.sqrt(2) * norm.pdf(math.sqrt(2))
    assert act_lipschitz(ACT_GELU_ERF) >= peak and act_lipschitz(ACT_GELU_ERF) - peak < 1e-4


def test_static_scale_and_quantize():
    assert static_scale(448.0) == np.float32(1.0)
    assert static_scale(4.48) == np.float32(np.float32(4.48) / np.float32(448.0))
    v = np.array([1.0, -2.0, 448.0, 500.0, 1e-9], np.float32)
    assert quantize_static(v, 1.0).tolist() == [0x38, 0xC0, 0x7E, 0x7E, 0x00]
    with pytest.raises(ValueError):
        quantize_static(v, 0.0)


def _layer_inputs(cfg):
    x = synth.activations(cfg)
    logits = synth.router_logits(cfg)
    w13 = synth.moe_weights(cfg, "w13")
    w2 = synth.moe_weights(cfg, "w2")
    return x, logits, w13, w2


def _calibrate(cfg, x, logits, p13, p2):
    s_x = static_scale(np.max(np.abs(bf16_to_f32(x))))
    pre = moe_forward(x, logits, s_x, p13, p2, cfg.act, np.float32(1.0), cfg.out_f32)
    s_a = static_scale(np.max(np.abs(pre["a"])))
    return s_x, s_a


def test_integer_case_gate_up_exact():
    """x and w integer-valued, every row's max |w| = 7 and s_x = 1: the gate|up values
    equal an integer matrix product exactly."""
    rng = np.random.default_rng(21)
    T, H, I, E = 6, 64, 32, 3
    xi = rng.integers(-16, 17, size=(T, H))
    w13i = rng.integers(-7, 8, size=(E, 2 * I, H))
    w13i[:, :, 0] = 7
    w2i = rng.integers(-7, 8, size=(E, H, I))
    w2i[:, :, 0] = -7
    x = synth.f32_to_bf16_bits(xi.astype(np.float32))
    p13 = w4_pack(synth.f32_to_bf16_bits(w13i.astype(np.float32)))
    p2 = w4_pack(synth.f32_to_bf16_bits(w2i.astype(np.float32)))
    assert np.all(p13[1] == 1.0) and np.all(p2[1] == 1.0)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    r = moe_forward(x, logits, np.float32(1.0), p13, p2, ACT_SILU, np.float32(0.5), True)
    for i, row in enumerate(r["rows"]):
        e = int(np.searchsorted(r["offsets"], row, side="right") - 1)
        t = r["sorted_pair"][row] // 2
        assert np.array_equal(r["h"][i], w13i[e] @ xi[t])
    assert np.array_equal(r["x_codes"], quantize_static(xi[r["x_codes_tokens"]].astype(np.float32), 1.0))


def test_two_experts_dense_textbook():
    """E = 2: every token uses both experts, so the layer is w0 FFN_a(x) + w1 FFN_b(x)
    computed densely without any sorting."""
    cfg = synth.custom_moe("e2", T=12, H=128, I=256, E=2, act=ACT_GELU_ERF, w_cfg=31, x_cfg=31)
    x, logits, w13, w2 = _layer_inputs(cfg)
    p13, p2 = w4_pack(w13), w4_pack(w2)
    s_x, s_a = _calibrate(cfg, x, logits, p13, p2)
    r = moe_forward(x, logits, s_x, p13, p2, cfg.act, s_a, True)
    xt = e4m3_decode(quantize_static(bf16_to_f32(x), s_x)) * np.float64(s_x)
    ids, w = route_top2(logits)
    out = np.zeros((cfg.T, cfg.H))
    for e in range(2):
        W13 = w4_unpack_codes(p13[0][e]).astype(np.float64) * p13[1][e].astype(np.float64)[:, None]
        W2 = w4_unpack_codes(p2[0][e]).astype(np.float64) * p2[1][e].astype(np.float64)[:, None]
        h = xt @ W13.T
        a = activation(h[:, :cfg.I], cfg.act) * h[:, cfg.I:]
        at = e4m3_decode(quantize_static(a.astype(np.float32), s_a)) * np.float64(s_a)
        y = at @ W2.T
        we = np.where(ids[:, 0] == e, w[:, 0], w[:, 1])
        out += we[:, None] * y
    assert np.allclose(r["out"], out, rtol=1e-12, atol=1e-12 * np.abs(out).max())


@pytest.mark.parametrize("cfg", [synth.TINY,
                                 synth.custom_moe("tiny_gelu", 16, 256, 512, 4, act=ACT_GELU_ERF,
                                                  w_sigma=0.015, logit_sigma=1.5, w_cfg=41, x_cfg=41)])
def test_quantized_layer_within_rigorous_bound_of_unquantized(cfg):
    x, logits, w13, w2 = _layer_inputs(cfg)
    p13, p2 = w4_pack(w13), w4_pack(w2)
    s_x, s_a = _calibrate(cfg, x, logits, p13, p2)
    r = moe_forward(x, logits, s_x, p13, p2, cfg.act, s_a, cfg.out_f32)
    ref = moe_reference_unquantized(x, logits, w13, w2, cfg.act)
    bound = moe_error_bound(x, logits, w13, w2, cfg.act, s_x, s_a)
    err = np.abs(r["out"] - ref)
    assert np.all(err <= bound * (1 + 1e-9) + 1e-12)
    rel = np.linalg.norm(r["out"] - ref) / np.linalg.norm(ref)
    assert 0.01 < rel < 0.35, rel


def test_token_subset_matches_full_run():
    cfg = synth.custom_moe("sub", T=40, H=128, I=256, E=8, w_cfg=51, x_cfg=51)
    x, logits, w13, w2 = _layer_inputs(cfg)
    p13, p2 = w4_pack(w13), w4_pack(w2)
    full = moe_forward(x, logits, np.float32(0.01), p13, p2, cfg.act, np.float32(0.001), True)
    toks = np.array([3, 17, 39, 0])
    sub = moe_forward(x, logits, np.float32(0.01), p13, p2, cfg.act, np.float32(0.001), True,
                      tokens=toks)
    assert np.array_equal(sub["out"], full["out"][toks])
    provider = lambda e: (p13[0][e], p13[1][e])
    sub2 = moe_forward(x, logits, np.float32(0.01), provider, p2, cfg.act, np.float32(0.001), True,
                       tokens=toks)
    assert np.array_equal(sub2["out"], sub["out"])


def test_pair_rows_and_combine_plumbing():
    """The output of token t only combines the rows of its own two pairs, in slot order."""
    cfg = synth.custom_moe("plumb", T=9, H=128, I=128, E=4, w_cfg=61, x_cfg=61)
    x, logits, w13, w2 = _layer_inputs(cfg)
    p13, p2 = w4_pack(w13), w4_pack(w2)
    r = moe_forward(x, logits, np.float32(0.01), p13, p2, cfg.act, np.float32(0.001), True)
    for t in range(cfg.T):
        r0 = np.nonzero(r["rows"] == r["pair_pos"][2 * t])[0][0]
        r1 = np.nonzero(r["rows"] == r["pair_pos"][2 * t + 1])[0][0]
        assert r["sorted_pair"][r["rows"][r0]] == 2 * t
        expect = r["weights"][t, 0] * r["y"][r0] + r["weights"][t, 1] * r["y"][r1]
        assert np.array_equal(r["out"][t], expect)


def test_given_codes_feed_the_down_projection():
    """Codes passed in replace the requantized ones row by row: the oracle's own codes
    give the same result, and changing one code of sorted row r, channel i moves y[r]
    by exactly (new - old) * s_a * s_w2[e, n] * q2[e, n, i] and leaves other rows alone."""
    cfg = synth.custom_moe("given", T=12, H=128, I=256, E=4, w_cfg=71, x_cfg=71)
    x, logits, w13, w2 = _layer_inputs(cfg)
    p13, p2 = w4_pack(w13), w4_pack(w2)
    s_x, s_a = np.float32(0.01), np.float32(0.002)
    base = moe_forward(x, logits, s_x, p13, p2, cfg.act, s_a, True)
    assert np.array_equal(base["rows"], np.arange(2 * cfg.T))
    same = moe_forward(x, logits, s_x, p13, p2, cfg.act, s_a, True, a_codes_given=base["a_codes"])
    assert np.array_equal(same["y"], base["y"]) and np.array_equal(same["out"], base["out"])
    codes = base["a_codes"].copy()
    r, i = 7, 100
    e = int(np.searchsorted(base["offsets"], r, side="right") - 1)
    old = codes[r, i]
    new = np.uint8(0x38 if old != 0x38 else 0x40)      # 1.0 or 2.0
    codes[r, i] = new
    got = moe_forward(x, logits, s_x, p13, p2, cfg.act, s_a, True, a_codes_given=codes)
    q2 = w4_unpack_codes(p2[0][e], cfg.I).astype(np.float64)      # [H, I]
    delta = (e4m3_decode(np.array([new]))[0] - e4m3_decode(np.array([old]))[0]) * np.float64(s_a)
    expect = base["y"][r] + delta * np.asarray(p2[1][e], np.float64) * q2[:, i]
    assert np.allclose(got["y"][r], expect, rtol=1e-13, atol=1e-12)
    others = np.arange(2 * cfg.T) != r
    assert np.array_equal(got["y"][others], base["y"][others])
    assert np.array_equal(got["h"], base["h"])


def test_weight_row_subsets_match_full_tensor():
    """The sampled full-size checks pack only some weight rows: quantization is per row, so
    the rows regenerated by synth and packed alone equal those rows of the full packing,
    and the per-expert steps on a row subset equal those columns of the full result."""
    from oracle import expert_down, expert_gate_up
    cfg = synth.custom_moe("rows", T=6, H=256, I=384, E=3, w_cfg=81, x_cfg=81)
    x, logits, w13, w2 = _layer_inputs(cfg)
    p13, p2 = w4_pack(w13), w4_pack(w2)
    rows13 = np.array([0, 5, 127, 128, 383, 384, 600, 767])
    rows2 = np.array([0, 1, 200, 255])
    for e in range(cfg.E):
        sub13 = w4_pack(synth.moe_weight_rows(cfg, "w13", e, rows13))
        assert np.array_equal(sub13[0], p13[0][e][rows13]) and np.array_equal(sub13[1], p13[1][e][rows13])
        sub2 = w4_pack(synth.moe_weight_rows(cfg, "w2", e, rows2))
        assert np.array_equal(sub2[0], p2[0][e][rows2]) and np.array_equal(sub2[1], p2[1][e][rows2])
    xc = quantize_static(bf16_to_f32(x), np.float32(0.01))
    full = expert_gate_up(xc, p13[0][1], p13[1][1], np.float32(0.01))
    part = expert_gate_up(xc, p13[0][1][rows13], p13[1][1][rows13], np.float32(0.01))
    assert np.array_equal(part, full[:, rows13])
    ac = quantize_static(np.random.default_rng(1).standard_normal((4, cfg.I)).astype(np.float32), np.float32(0.02))
    full2 = expert_down(ac, p2[0][2], p2[1][2], np.float32(0.02))
    assert np.array_equal(expert_down(ac, p2[0][2][rows2], p2[1][2][rows2], np.float32(0.02)), full2[:, rows2])
