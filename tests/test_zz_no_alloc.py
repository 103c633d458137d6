"""The allocation-free down call (moe_gemm2_w4a8_noalloc) against the workspace call
(moe_gemm2_w4a8) through the C ABI: byte-identical outputs on two calls in a row, the
second with a smaller batch, on the streaming kernel with split-K partials and on the
tiled kernel."""
import numpy as np
import pytest

import synth
import w4a8_moe_amd as W
from tests.gpu_util import bf16_dev, f32_dev, torch

pytestmark = pytest.mark.gpu


def _layer(cfg, T):
    t = torch()
    x = bf16_dev(synth.activations(cfg)[:T])
    logits = f32_dev(synth.router_logits(cfg)[:T])
    w13, s13 = W.w4_pack(bf16_dev(synth.moe_weights(cfg, "w13")), tiled=True)
    w2, s2 = W.w4_pack(bf16_dev(synth.moe_weights(cfg, "w2")), tiled=True)
    r = W.moe_route_sort(logits)
    a = W.moe_gemm1_w4a8(x, 0.01, w13, s13, r["offsets"], r["sorted_pair"], cfg.act, 0.05)
    t.cuda.synchronize()
    return a, w2, s2, r


@pytest.mark.parametrize("name,T1,T2,H,I,E", [
    # streaming kernel, I = 8192: two split-K slices of the down projection
    ("decode_split", 32, 5, 512, 8192, 8),
    # the tiled kernel (more than 80 tokens), then a decode batch
    ("tiled", 100, 20, 256, 512, 4),
])
def test_noalloc_matches_workspace_call(name, T1, T2, H, I, E):
    t = torch()
    cfg = synth.custom_moe("noalloc_" + name, T=T1, H=H, I=I, E=E, w_cfg=900 + E, x_cfg=900 + E, out_f32=False)
    for T in (T1, T2):                     # two calls in a row, the second smaller
        print(f"{name}: T={T} H={H} I={I} E={E}", flush=True)
        a, w2, s2, r = _layer(cfg, T)
        ref = W.moe_gemm2_w4a8(a, 0.05, w2, s2, r["offsets"], r["pair_pos"], r["weights"], "bf16")
        got = W.moe_gemm2_w4a8_noalloc(a, 0.05, w2, s2, r["offsets"], r["pair_pos"], r["weights"], "bf16")
        t.cuda.synchronize()
        assert t.equal(got, ref)
        assert bool(t.isfinite(got.float()).all())
