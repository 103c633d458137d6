"""The one-call layer, moe_layer_w4a8: its output is byte for byte the output of the three
calls (moe_route_sort_quant, moe_gemm1_w4a8, moe_gemm2_w4a8) on the same inputs, which the
layer and prefill parity tests hold to the oracle, and it meets the end-to-end bar against
the oracle itself. The cases cover one and two 16-row column tiles per expert, experts with
more than 32 rows (taken in passes of 32, up to three), a split
down reduction, empty experts, the largest expert count, the tiled kernel above 80 tokens,
and one workspace reused by calls of different sizes."""
import numpy as np
import pytest

import oracle
import synth
import w4a8_moe_amd as W
from tests.gpu_util import assert_final_close, bf16_bits_to_f64, bf16_dev, f32_dev, host, torch

pytestmark = pytest.mark.gpu

CASES = [
    synth.TINY,
    synth.custom_moe("fl_one_token", T=1, H=256, I=512, E=8, w_cfg=501, x_cfg=501),
    # I = 37 x 128: a ragged split of the down reduction
    synth.custom_moe("fl_ragged_k", T=32, H=640, I=4736, E=8, act=synth.ACT_GELU_ERF, out_f32=False, w_cfg=502,
                     x_cfg=502, logit_sigma=1.5),
    # two experts: every expert holds every token (two 16-row column tiles; 52 and 64 rows take
    # two passes of 32)
    synth.custom_moe("fl_two_experts_24", T=24, H=384, I=640, E=2, act=synth.ACT_GELU_TANH, w_cfg=503, x_cfg=503),
    synth.custom_moe("fl_two_experts_52", T=52, H=512, I=1024, E=2, w_cfg=504, x_cfg=504, out_f32=False),
    synth.custom_moe("fl_two_experts_64", T=64, H=384, I=768, E=2, act=synth.ACT_GELU_ERF, w_cfg=514, x_cfg=514),
    synth.custom_moe("fl_52", T=52, H=512, I=1024, E=8, w_cfg=505, x_cfg=505, logit_sigma=1.5),
    synth.custom_moe("fl_64", T=64, H=512, I=1024, E=8, w_cfg=513, x_cfg=513, logit_sigma=1.5, out_f32=False),
    # two experts of 72 rows, and the most tokens the streaming kernel takes (80 rows each):
    # three passes
    synth.custom_moe("fl_two_experts_72", T=72, H=256, I=640, E=2, act=synth.ACT_SILU, w_cfg=515, x_cfg=515,
                     out_f32=False),
    synth.custom_moe("fl_two_experts_80", T=80, H=384, I=512, E=2, act=synth.ACT_GELU_ERF, w_cfg=516, x_cfg=516),
    # long down reduction: the down projection split into K-slices
    synth.custom_moe("fl_split_k", T=32, H=256, I=16384, E=8, w_cfg=506, x_cfg=506, out_f32=False),
    synth.custom_moe("fl_empty_experts", T=20, H=256, I=384, E=16, w_cfg=507, x_cfg=507, expert_bias=True,
                     logit_sigma=0.5),
    synth.custom_moe("fl_max_experts", T=24, H=128, I=128, E=256, w_cfg=508, x_cfg=508, out_f32=False,
                     logit_sigma=2.0),
    # the fewest tokens that can need a second pass, and 52 tokens over 256 experts
    synth.custom_moe("fl_33", T=33, H=384, I=768, E=4, act=synth.ACT_GELU_ERF, w_cfg=511, x_cfg=511, out_f32=False),
    synth.custom_moe("fl_max_experts_52", T=52, H=128, I=256, E=256, w_cfg=512, x_cfg=512, logit_sigma=2.0),
    # above 80 tokens: the routing, the tiled gate|up and down launches in sequence
    synth.custom_moe("fl_sequential", T=100, H=256, I=512, E=8, act=synth.ACT_GELU_ERF, w_cfg=509, x_cfg=509,
                     out_f32=False),
]


def _scales(cfg, x, logits, p13, p2):
    s_x = oracle.static_scale(np.max(np.abs(oracle.bf16_to_f32(x))))
    pre = oracle.moe_forward(x, logits, s_x, p13, p2, cfg.act, np.float32(1.0), cfg.out_f32)
    return s_x, oracle.static_scale(np.max(np.abs(pre["a"])))


@pytest.mark.parametrize("cfg", CASES, ids=[c.name for c in CASES])
def test_layer_matches_three_calls_and_oracle(cfg):
    t = torch()
    T, H, I, E = cfg.T, cfg.H, cfg.I, cfg.E
    print(f"{cfg.name}: T={T} H={H} I={I} E={E}", flush=True)
    x = synth.activations(cfg)
    logits = synth.router_logits(cfg)
    w13 = synth.moe_weights(cfg, "w13")
    w2 = synth.moe_weights(cfg, "w2")
    p13, p2 = oracle.w4_pack(w13), oracle.w4_pack(w2)
    s_x, s_a = _scales(cfg, x, logits, p13, p2)
    ref = oracle.moe_forward(x, logits, s_x, p13, p2, cfg.act, s_a, cfg.out_f32)
    gw13, gs13 = W.w4_pack(bf16_dev(w13), tiled=True)
    gw2, gs2 = W.w4_pack(bf16_dev(w2), tiled=True)
    xd, ld = bf16_dev(x), f32_dev(logits)
    od = "f32" if cfg.out_f32 else "bf16"

    r = W.moe_route_sort_quant(ld, xd, s_x)
    a = W.moe_gemm1_w4a8(r["xq"], s_x, gw13, gs13, r["offsets"], r["sorted_pair"], cfg.act, s_a)
    out3 = W.moe_gemm2_w4a8(a, s_a, gw2, gs2, r["offsets"], r["pair_pos"], r["weights"], od)

    nws = W.workspace_bytes(W.OP_LAYER, T, H, I, E)
    ws = t.full((nws,), 0x5A, dtype=t.uint8, device="cuda")   # stale bytes: the call writes all it reads
    out = W.moe_layer_w4a8(ld, xd, s_x, gw13, gs13, gw2, gs2, cfg.act, s_a, od, ws=ws)
    t.cuda.synchronize()
    assert t.equal(out, out3), "the one-call layer differs from the three calls"

    if cfg.out_f32:
        got, e2e = host(out).astype(np.float64), ref["out"].astype(np.float32).astype(np.float64)
    else:
        got, e2e = bf16_bits_to_f64(host(out)), bf16_bits_to_f64(ref["out_rounded"])
    print("end to end:", end=" ")
    assert_final_close(got, e2e)

    # again on the same workspace, and deterministic
    out2 = W.moe_layer_w4a8(ld, xd, s_x, gw13, gs13, gw2, gs2, cfg.act, s_a, od, ws=ws)
    t.cuda.synchronize()
    assert t.equal(out2, out)


def test_layer_back_to_back_shapes():
    """One workspace, calls of different sizes in a row on one stream, each equal to its own
    three-call result."""
    t = torch()
    cfgs = [synth.custom_moe(f"fl_seq_{T}", T=T, H=256, I=1024, E=8, w_cfg=510, x_cfg=510 + T, out_f32=False)
            for T in (48, 5, 32, 1)]
    w13, s13 = W.w4_pack(bf16_dev(synth.moe_weights(cfgs[0], "w13")), tiled=True)
    w2, s2 = W.w4_pack(bf16_dev(synth.moe_weights(cfgs[0], "w2")), tiled=True)
    ws = t.empty(max(W.workspace_bytes(W.OP_LAYER, c.T, 256, 1024, 8) for c in cfgs), dtype=t.uint8, device="cuda")
    s_x, s_a = 0.02, 0.05
    outs, refs = [], []
    for c in cfgs:
        xd, ld = bf16_dev(synth.activations(c)), f32_dev(synth.router_logits(c))
        outs.append(W.moe_layer_w4a8(ld, xd, s_x, w13, s13, w2, s2, c.act, s_a, "bf16", ws=ws))
        r = W.moe_route_sort_quant(ld, xd, s_x)
        a = W.moe_gemm1_w4a8(r["xq"], s_x, w13, s13, r["offsets"], r["sorted_pair"], c.act, s_a)
        refs.append(W.moe_gemm2_w4a8(a, s_a, w2, s2, r["offsets"], r["pair_pos"], r["weights"], "bf16"))
    t.cuda.synchronize()
    for c, o, ref in zip(cfgs, outs, refs):
        assert t.equal(o, ref), c.name
