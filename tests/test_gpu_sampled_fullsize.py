"""Parity at the full workload sizes, in the launch configuration the benchmark times.

The layer runs whole on the GPU (Mixtral- and Grok-1-shaped decode, Grok-1-shaped
prefill with 32768 tokens, and one GPU's 8-way tensor-parallel share of the Grok-1
layer, I = 4096, decode and prefill); the oracle then computes the outputs of sampled
tokens one by one: routing and sort in full (bit-exact), packed words and scales of
every expert (bit-exact), the oracle's own gate|up and requantized codes over all I
channels of the sampled tokens' rows, its own down projection and combine on those
codes for sampled output channels. The layer's output is held to the full bar against
that end-to-end result. Sampled tokens include those whose rows sit at the first and
last rows of every expert segment and at tile edges; sampled output channels include
the first and last ones and those at tile edges. As a separate check of the down call
alone, the output also meets the bar against the oracle's down projection of the
kernel's own codes. The one-call layer, moe_layer_w4a8, gives the same output bytes as
the three calls.
"""
import concurrent.futures as cf
import dataclasses

import numpy as np
import pytest

import oracle
import synth
import w4a8_moe_amd as W
from oracle.sample import prefill_token_subset
from tests.gpu_util import (assert_final_close, bf16_bits_to_f64, bf16_dev, f32_dev, host, rows_of_tiled,
                            same_codes, static_scales, torch)

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


def _channels(n, count, edges, seed):
    rng = np.random.default_rng(seed)
    fixed = [c for c in edges if 0 <= c < n]
    rest = np.setdiff1d(np.arange(n), fixed)
    pick = rng.choice(rest, max(0, count - len(fixed)), replace=False)
    return np.unique(np.concatenate([np.array(fixed, dtype=np.int64), pick]))


def _code_key(c):
    """E4M3 codes in value order (+0 and -0 the same key)."""
    c = np.asarray(c, np.int64)
    return np.where(c & 0x80, -(c & 0x7F), c & 0x7F)


def _reachable_codes(g, u, d, act, s_a):
    """Order keys of the lowest and highest codes that an activation of gate|up values
    within d of (g, u) rounds to: min and max over a 3 x 3 grid of the (tiny) box."""
    lo = hi = None
    for dg in (-d, 0.0, d):
        for du in (-d, 0.0, d):
            v = oracle.activation(g + dg, act) * (u + du)
            lo = v if lo is None else np.minimum(lo, v)
            hi = v if hi is None else np.maximum(hi, v)
    return (_code_key(oracle.quantize_static(lo.astype(np.float32), s_a)),
            _code_key(oracle.quantize_static(hi.astype(np.float32), s_a)))


_PACKED = {}


def _model_weights(cfg):
    """bf16 weights of the workload (host) and the oracle's packing of every expert, kept
    for the next workload of the same model (decode and prefill share their weights)."""
    key = (cfg.w_cfg, cfg.E, cfg.H, cfg.I, cfg.w_sigma)
    if key not in _PACKED:
        _PACKED.clear()
        bf = {which: synth.moe_weights(cfg, which) for which in ("w13", "w2")}
        print("weights drawn; the oracle packs them", flush=True)
        packed = {}
        with cf.ThreadPoolExecutor(4) as ex:
            for which in ("w13", "w2"):
                parts = list(ex.map(lambda e: oracle.w4_pack(bf[which][e]), range(cfg.E)))
                packed[which] = (np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]))
        _PACKED[key] = (bf, packed)
    return _PACKED[key]


def _run_sampled(cfg, n_tokens, n_out_ch=512):
    T, H, I, E = cfg.T, cfg.H, cfg.I, cfg.E
    s_x, s_a = static_scales(cfg.name)
    print(f"{cfg.name}: T={T} H={H} I={I} E={E}", flush=True)
    x = synth.activations(cfg)
    logits = synth.router_logits(cfg)
    bf, packed = _model_weights(cfg)
    gw = {}
    for which in ("w13", "w2"):
        wb = bf16_dev(bf[which])
        gw[which] = W.w4_pack(wb, tiled=True)
        del wb
        torch().cuda.empty_cache()
    r = W.moe_route_sort(f32_dev(logits))
    a = W.moe_gemm1_w4a8(bf16_dev(x), s_x, gw["w13"][0], gw["w13"][1], r["offsets"], r["sorted_pair"], cfg.act, s_a)
    out = W.moe_gemm2_w4a8(a, s_a, gw["w2"][0], gw["w2"][1], r["offsets"], r["pair_pos"], r["weights"], "bf16")
    # the one-call layer (what the benchmark times) gives the same bytes
    out1 = W.moe_layer_w4a8(f32_dev(logits), bf16_dev(x), s_x, gw["w13"][0], gw["w13"][1], gw["w2"][0],
                            gw["w2"][1], cfg.act, s_a, "bf16")
    torch().cuda.synchronize()
    assert torch().equal(out1, out), "moe_layer_w4a8 differs from the three calls"
    del out1
    torch().cuda.empty_cache()

    ids, wts = oracle.route_top2(logits)
    counts, offsets, sp, pos = oracle.route_sort(ids, E)
    assert np.array_equal(host(r["ids"]), ids) and np.array_equal(host(r["offsets"]), offsets)
    assert np.array_equal(host(r["sorted_pair"]), sp) and np.array_equal(host(r["pair_pos"]), pos)
    assert np.max(np.abs(host(r["weights"]) - wts)) <= 1e-6

    toks = np.arange(T) if T <= n_tokens else prefill_token_subset(offsets, sp, T, n_tokens=n_tokens, seed=5)
    rows = np.unique(np.concatenate([pos[2 * toks], pos[2 * toks + 1]]))
    # output channels: enough that the 0.1% rule is a fraction of many thousand elements
    ch2 = _channels(H, n_out_ch, [0, 1, 127, 128, 255, 256, H - 1], seed=2)
    a_rows = host(a[torch().from_numpy(rows).to(a.device)])                 # [rows, I] kernel codes
    expert_of = np.searchsorted(offsets, rows, side="right") - 1
    c_ref = np.zeros((rows.size, I), np.uint8)
    y_ref = np.zeros((rows.size, ch2.size))
    y_kc = np.zeros((rows.size, ch2.size))
    within = 0
    for e in np.unique(expert_of):
        e = int(e)
        sel = np.nonzero(expert_of == e)[0]
        w13w, w13s = packed["w13"][0][e], packed["w13"][1][e]
        w2w, w2s = packed["w2"][0][e], packed["w2"][1][e]
        # the GPU's packing of this expert: scales in full, words of sampled rows
        pick = _channels(2 * I, 64, [0, 15, 16, I - 1, I, 2 * I - 1], seed=e)
        assert np.array_equal(host(gw["w13"][1][e]), w13s) and np.array_equal(host(gw["w2"][1][e]), w2s)
        assert np.array_equal(rows_of_tiled(gw["w13"][0][e], pick), w13w[pick])
        assert np.array_equal(rows_of_tiled(gw["w2"][0][e], ch2), w2w[ch2])
        # the oracle's own gate|up and codes over all I channels of these rows
        xc = oracle.quantize_static(oracle.bf16_to_f32(x[sp[rows[sel]] // 2]), s_x)
        h = oracle.expert_gate_up(xc, w13w, w13s, s_x)                      # [sel, 2I]
        g, u = h[:, :I], h[:, I:]
        c_ref[sel] = oracle.quantize_static((oracle.activation(g, cfg.act) * u).astype(np.float32), s_a)
        # every kernel code is one that gate|up within the 1e-4 row bar rounds to
        lo, hi = _reachable_codes(g, u, 1e-4 * np.max(np.abs(h), axis=1, keepdims=True), cfg.act, s_a)
        got = _code_key(a_rows[sel])
        within += int(np.sum((got >= lo) & (got <= hi)))
        y_ref[sel] = oracle.expert_down(c_ref[sel], w2w[ch2], w2s[ch2], s_a)
        y_kc[sel] = oracle.expert_down(a_rows[sel], w2w[ch2], w2s[ch2], s_a)
        print(f"expert {e}: {sel.size} rows checked", flush=True)
    eq = same_codes(a_rows, c_ref)
    print(f"codes: {eq.mean():.6%} of {eq.size} equal the oracle's ({int((~eq).sum())} differ), "
          f"{within / eq.size:.4%} within reach of the 1e-4 row bar", flush=True)
    assert within == eq.size

    row_of = {int(rr): i for i, rr in enumerate(rows)}

    def combine(y):
        return np.stack([wts[t, 0] * y[row_of[int(pos[2 * t])]] + wts[t, 1] * y[row_of[int(pos[2 * t + 1])]]
                         for t in toks])

    got_out = bf16_bits_to_f64(host(out[torch().from_numpy(toks).to(out.device)])[:, ch2])
    print("end to end:", end=" ")
    assert_final_close(got_out, bf16_bits_to_f64(oracle.f64_to_bf16_bits(combine(y_ref))))
    print("down call on the kernel's codes:", end=" ")
    assert_final_close(got_out, bf16_bits_to_f64(oracle.f64_to_bf16_bits(combine(y_kc))))
    del gw, a, out
    torch().cuda.empty_cache()


# Grouped by model, so that one packing of the weights serves its decode and prefill workloads.
# The second case is the Mixtral-shaped decode at 64 tokens with unequal expert loads (a
# per-expert router bias): experts 0 and 3 hold 36 and 38 rows, which the streaming kernel
# takes in two passes of at most 32.
SKEWED_64 = dict(T=64, expert_bias=True)


@pytest.mark.parametrize("name,change,n_tokens", [("mixtral_decode", None, 32), ("mixtral_decode", SKEWED_64, 64),
                                                  ("grok_decode", None, 32), ("grok_prefill", None, 48),
                                                  ("grok_tp8_decode", None, 32), ("grok_tp8_prefill", None, 48)],
                         ids=["mixtral_decode", "mixtral_decode_64_skewed", "grok_decode", "grok_prefill",
                              "grok_tp8_decode", "grok_tp8_prefill"])
def test_fullsize_sampled(name, change, n_tokens):
    cfg = synth.MOE_CONFIGS[name]
    _run_sampled(cfg if change is None else dataclasses.replace(cfg, **change), n_tokens)
    if name == "grok_tp8_prefill":
        _PACKED.clear()


@pytest.mark.parametrize("name", sorted(synth.BLOCK_CONFIGS))
def test_block_linear_fullsize(name):
    """The block-FP8 GEMV at the page shapes, every output against the oracle."""
    cfg = synth.BLOCK_CONFIGS[name]
    w = synth.block_weights(cfg)
    x = synth.block_activations(cfg)
    q, S = W.fp8_block_quant(bf16_dev(w))
    qo, So = oracle.fp8_block_quantize(w)
    assert np.array_equal(host(S), So) and same_codes(host(q), qo).all()
    y = W.fp8_block_linear(bf16_dev(x), q, S)
    _, y_bits = oracle.fp8_block_linear(x, qo, So)
    assert_final_close(bf16_bits_to_f64(host(y)), bf16_bits_to_f64(y_bits))
