"""The layer and the dense linear inside captured HIP graphs: every replay (with the
program's own eager work and synchronizations between replays) gives the bytes of the
eager calls. Calls write their outputs with kernels only (the library records no memset
or copy nodes), and a replay must not depend on what an earlier replay left in the
workspaces."""
import numpy as np
import pytest

import synth
import w4a8_moe_amd as W
from tests.gpu_util import bf16_dev, f32_dev, torch

pytestmark = pytest.mark.gpu

LAYERS = [
    synth.custom_moe("graph_decode", T=32, H=1024, I=2048, E=8, act=synth.ACT_SILU, out_f32=False, w_cfg=401,
                     x_cfg=401, logit_sigma=1.5),
    synth.custom_moe("graph_tiled", T=300, H=512, I=512, E=8, act=synth.ACT_GELU_ERF, out_f32=False, w_cfg=402,
                     x_cfg=402, expert_bias=True),
]


@pytest.mark.parametrize("cfg", LAYERS, ids=[c.name for c in LAYERS])
def test_layer_graph_replays_match_eager(cfg):
    t = torch()
    dev = t.device("cuda:0")
    T, H, I, E = cfg.T, cfg.H, cfg.I, cfg.E
    w13, s13 = W.w4_pack(bf16_dev(synth.moe_weights(cfg, "w13")), tiled=True)
    w2, s2 = W.w4_pack(bf16_dev(synth.moe_weights(cfg, "w2")), tiled=True)
    x = bf16_dev(synth.activations(cfg))
    logits = f32_dev(synth.router_logits(cfg))
    s_x, s_a = 0.01, 0.05
    xq = t.empty((T, H), dtype=t.uint8, device=dev)
    a = t.empty((2 * T, I), dtype=t.uint8, device=dev)
    out = t.empty((T, H), dtype=t.bfloat16, device=dev)
    ws1 = t.empty(max(256, W.workspace_bytes(W.OP_GEMM1, T, H, I, E)), dtype=t.uint8, device=dev)
    ws2 = t.empty(max(256, W.workspace_bytes(W.OP_GEMM2, T, H, I, E)), dtype=t.uint8, device=dev)
    ro = W.route_outputs(T, E, dev)

    def step():
        W.moe_route_sort_quant(logits, x, s_x, out=ro, xq=xq)
        W.moe_gemm1_w4a8(xq, s_x, w13, s13, ro["offsets"], ro["sorted_pair"], cfg.act, s_a, ws=ws1, out=a)
        W.moe_gemm2_w4a8(a, s_a, w2, s2, ro["offsets"], ro["pair_pos"], ro["weights"], "bf16", ws=ws2, out=out)

    step()
    t.cuda.synchronize()
    ref_out, ref_a = out.clone(), a.clone()
    g = t.cuda.CUDAGraph()
    with t.cuda.graph(g):
        step()
    for r in range(4):
        # eager work between replays: clobber outputs and workspaces, run an eager step
        out.fill_(float(r + 1)); a.fill_(r + 7); ws2.fill_(r + 3); xq.fill_(0)
        for k in ("ws", "counts", "sorted_pair"):
            if ro.get(k) is not None and ro[k].numel() > 0:
                ro[k].fill_(r + 5)
        if r == 2:
            step()
        t.cuda.synchronize()
        g.replay()
        t.cuda.synchronize()
        assert t.equal(out, ref_out), f"replay {r}: output differs from the eager step"
        assert t.equal(a, ref_a), f"replay {r}: intermediate differs from the eager step"


@pytest.mark.parametrize("cfg", LAYERS, ids=[c.name for c in LAYERS])
def test_one_call_layer_graph_replays_match_eager(cfg):
    """moe_layer_w4a8 captured: replays over a workspace full of stale bytes give the eager
    bytes."""
    t = torch()
    T, H, I, E = cfg.T, cfg.H, cfg.I, cfg.E
    w13, s13 = W.w4_pack(bf16_dev(synth.moe_weights(cfg, "w13")), tiled=True)
    w2, s2 = W.w4_pack(bf16_dev(synth.moe_weights(cfg, "w2")), tiled=True)
    x = bf16_dev(synth.activations(cfg))
    logits = f32_dev(synth.router_logits(cfg))
    out = t.empty((T, H), dtype=t.bfloat16, device="cuda")
    ws = t.empty(W.workspace_bytes(W.OP_LAYER, T, H, I, E), dtype=t.uint8, device="cuda")

    def step():
        W.moe_layer_w4a8(logits, x, 0.01, w13, s13, w2, s2, cfg.act, 0.05, "bf16", ws=ws, out=out)

    step()
    t.cuda.synchronize()
    ref_out = out.clone()
    g = t.cuda.CUDAGraph()
    with t.cuda.graph(g):
        step()
    for r in range(4):
        out.fill_(float(r + 1)); ws.fill_(r + 3)
        if r == 2:
            step()
        t.cuda.synchronize()
        g.replay()
        t.cuda.synchronize()
        assert t.equal(out, ref_out), f"replay {r}: output differs from the eager call"


@pytest.mark.parametrize("M", [1, 8])
def test_fp8_linear_graph_replays_match_eager(M):
    t = torch()
    cfg = synth.custom_block("graph_lin", M=M, N=1024, K=2048, cfg=403, sub=M)
    q, s = W.fp8_tensor_quant(bf16_dev(synth.block_weights(cfg)))
    s_w = float(s.item())
    x = bf16_dev(synth.block_activations(cfg))
    y = t.empty((M, cfg.N), dtype=t.bfloat16, device="cuda")
    nws = W.workspace_bytes(W.OP_FP8_LINEAR, M, cfg.N, cfg.K, 0)
    ws = t.empty(max(256, nws), dtype=t.uint8, device="cuda")
    W.fp8_linear_w8a8(x, 0.01, q, s_w, out=y, ws=ws)
    t.cuda.synchronize()
    ref = y.clone()
    g = t.cuda.CUDAGraph()
    with t.cuda.graph(g):
        W.fp8_linear_w8a8(x, 0.01, q, s_w, out=y, ws=ws)
    for r in range(4):
        y.fill_(float(r)); ws.fill_(r + 1)
        t.cuda.synchronize()
        g.replay()
        t.cuda.synchronize()
        assert t.equal(y, ref), f"replay {r}"
