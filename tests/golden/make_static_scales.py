"""Write tests/golden/static_scales.json: the static per-tensor fp8 scales of the
synthetic MoE workloads, from a calibration pass of the CPU oracle.

The pages fix that activation scales are static (page "ROCm: enable trillion-parameter
MoE models with INT4-FP8 single node", quantization_config: activation_scheme static)
but print no values. Reading: s_x = fp32(max|x| / 448) over the layer's input and
s_a = fp32(max|a| / 448) over the gated intermediate of an oracle pass (for the prefill
workload: over the oracle's sampled token subset); for the per-tensor FP8 dense linear
workloads, s_x = fp32(max|x| / 448) over their rows. Calls only oracle/ and synth/.

    python tests/golden/make_static_scales.py [config ...]
"""
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import synth  # noqa: E402
import oracle  # noqa: E402
from oracle.sample import prefill_token_subset  # noqa: E402

OUT = os.path.join(ROOT, "tests", "golden", "static_scales.json")


def packed_provider(cfg, which):
    """Oracle-packed weights of one expert, generated on demand and cached."""
    cache = {}

    def get(e):
        if e not in cache:
            cache.clear()
            cache[e] = oracle.w4_pack(synth.moe_expert_weights(cfg, which, e))
        return cache[e]
    return get


def calibrate(cfg):
    t0 = time.time()
    x = synth.activations(cfg)
    logits = synth.router_logits(cfg)
    s_x = oracle.static_scale(np.max(np.abs(oracle.bf16_to_f32(x))))
    tokens = None
    if cfg.T > 4096:
        ids, _ = oracle.route_top2(logits)
        _, offsets, sp, _ = oracle.route_sort(ids, cfg.E)
        tokens = prefill_token_subset(offsets, sp, cfg.T)
    r = oracle.moe_forward(x, logits, s_x, packed_provider(cfg, "w13"), packed_provider(cfg, "w2"),
                           cfg.act, np.float32(1.0), cfg.out_f32, tokens=tokens, E=cfg.E)
    s_a = oracle.static_scale(np.max(np.abs(r["a"])))
    print(f"{cfg.name}: s_x={float(s_x)!r} s_a={float(s_a)!r} ({time.time() - t0:.1f}s)", flush=True)
    return {"s_x": float(s_x), "s_a": float(s_a), "s_x_hex": float(s_x).hex(),
            "s_a_hex": float(s_a).hex(), "calibration_tokens": "all" if tokens is None else int(tokens.size)}


def calibrate_linear(cfg):
    """Per-tensor FP8 dense linear: the static activation scale over the workload's rows."""
    x = synth.block_activations(cfg)
    s_x = oracle.static_scale(np.max(np.abs(oracle.bf16_to_f32(x))))
    print(f"{cfg.name}: s_x={float(s_x)!r}", flush=True)
    return {"s_x": float(s_x), "s_x_hex": float(s_x).hex(), "calibration_tokens": "all"}


def main(names):
    data = json.load(open(OUT)) if os.path.exists(OUT) else {}
    data["_written_by"] = "tests/golden/make_static_scales.py (oracle calibration pass)"
    for name in names:
        if name in synth.LINEAR_CONFIGS:
            data[name] = calibrate_linear(synth.LINEAR_CONFIGS[name])
        else:
            data[name] = calibrate(synth.MOE_CONFIGS[name])
        json.dump(data, open(OUT, "w"), indent=1, sort_keys=True)


if __name__ == "__main__":
    main(sys.argv[1:] or list(synth.MOE_CONFIGS) + list(synth.LINEAR_CONFIGS))
