"""Parity at the full workload sizes, in the launch configuration the benchmark times.

The layer runs whole on the GPU (Mixtral- and Grok-1-shaped decode, Grok-1-shaped
prefill with 32768 tokens, and one GPU's 8-way tensor-parallel share of the Grok-1
layer, I = 4096, decode and prefill); the oracle then computes sampled outputs one by one:
routing and sort in full (bit-exact), packed words and scales of the sampled weight
rows (bit-exact), the requantized codes of sampled (row, channel) pairs, and sampled
output channels of sampled tokens. Sampled rows include the first and last rows of
every expert segment and the rows at tile edges; sampled channels include the first
and last ones and those at tile edges. The down projection is evaluated on the GPU's
own requantized codes (the rounding decision taken on the kernel's gate|up), which
the code check ties to the oracle's gate|up within the 1e-4 row bar.
"""
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
    vals = []
    for dg in (-d, 0.0, d):
        for du in (-d, 0.0, d):
            vals.append(oracle.activation(g + dg, act) * (u + du))
    vals = np.stack(vals)
    lo = oracle.quantize_static(vals.min(axis=0).astype(np.float32), s_a)
    hi = oracle.quantize_static(vals.max(axis=0).astype(np.float32), s_a)
    return _code_key(lo), _code_key(hi)


def _run_sampled(cfg, n_tokens, n_ch, n_out_ch=256):
    T, H, I, E = cfg.T, cfg.H, cfg.I, cfg.E
    s_x, s_a = static_scales(cfg.name)
    print(f"{cfg.name}: T={T} H={H} I={I} E={E}", flush=True)
    x = synth.activations(cfg)
    logits = synth.router_logits(cfg)
    gw = {}
    for which in ("w13", "w2"):
        wb = bf16_dev(synth.moe_weights(cfg, which))
        gw[which] = W.w4_pack(wb, tiled=True)
        del wb
        torch().cuda.empty_cache()
    r = W.moe_route_sort(f32_dev(logits))
    a = W.moe_gemm1_w4a8(bf16_dev(x), s_x, gw["w13"][0], gw["w13"][1], r["offsets"], r["sorted_pair"], cfg.act, s_a)
    out = W.moe_gemm2_w4a8(a, s_a, gw["w2"][0], gw["w2"][1], r["offsets"], r["pair_pos"], r["weights"], "bf16")
    torch().cuda.synchronize()

    ids, wts = oracle.route_top2(logits)
    counts, offsets, sp, pos = oracle.route_sort(ids, E)
    assert np.array_equal(host(r["ids"]), ids) and np.array_equal(host(r["offsets"]), offsets)
    assert np.array_equal(host(r["sorted_pair"]), sp) and np.array_equal(host(r["pair_pos"]), pos)
    assert np.max(np.abs(host(r["weights"]) - wts)) <= 1e-6

    toks = np.arange(T) if T <= n_tokens else prefill_token_subset(offsets, sp, T, n_tokens=n_tokens, seed=5)
    rows = np.unique(np.concatenate([pos[2 * toks], pos[2 * toks + 1]]))
    ch = _channels(I, n_ch, [0, 1, 127, 128, 255, 256, I - 1], seed=1)
    # output channels: enough that the 0.1% rule is a fraction of several thousand
    # elements (a bf16 output that lands one step from the oracle's rounding counts
    # against it when |y| is above a quarter of the largest output)
    ch2 = _channels(H, n_out_ch, [0, 1, 127, 128, 255, 256, H - 1], seed=2)
    a_rows = host(a[torch().from_numpy(rows).to(a.device)])                 # [rows, I] codes
    expert_of = np.searchsorted(offsets, rows, side="right") - 1
    y = np.zeros((rows.size, ch2.size))
    exact = within = near = total = 0
    for e in np.unique(expert_of):
        sel = np.nonzero(expert_of == e)[0]
        r13 = np.concatenate([ch, I + ch])
        words13, sc13 = oracle.w4_pack(synth.moe_weight_rows(cfg, "w13", int(e), r13))
        assert np.array_equal(rows_of_tiled(gw["w13"][0][int(e)], r13), words13)
        assert np.array_equal(host(gw["w13"][1][int(e)][torch().from_numpy(r13).to(a.device)]), sc13)
        xc = oracle.quantize_static(oracle.bf16_to_f32(x[sp[rows[sel]] // 2]), s_x)
        h = oracle.expert_gate_up(xc, words13, sc13, s_x)                     # [sel, 2 n_ch]
        g, u = h[:, :ch.size], h[:, ch.size:]
        d = 1e-4 * np.max(np.abs(h), axis=1, keepdims=True)                   # the row bar, sampled max
        lo, hi = _reachable_codes(g, u, d, cfg.act, s_a)
        ref = oracle.quantize_static((oracle.activation(g, cfg.act) * u).astype(np.float32), s_a)
        got_c = a_rows[sel][:, ch]
        got = _code_key(got_c)
        exact += int(np.sum(got == _code_key(ref)))
        ok = (got >= lo) & (got <= hi)
        within += int(ok.sum())
        # one code beyond the reachable range: the fp32 epilogue rounding of a value at a
        # code boundary (at most 1e-3 of the sample)
        near += int(np.sum(~ok & (got >= lo - 1) & (got <= hi + 1)))
        total += got.size
        words2, sc2 = oracle.w4_pack(synth.moe_weight_rows(cfg, "w2", int(e), ch2))
        assert np.array_equal(rows_of_tiled(gw["w2"][0][int(e)], ch2), words2)
        y[sel] = oracle.expert_down(a_rows[sel], words2, sc2, s_a)
    print(f"codes: {exact / total:.4%} equal the oracle's, {within / total:.4%} within reach of the 1e-4 row bar",
          flush=True)
    assert within + near == total and near <= max(1, 1e-3 * total), (within, near, total)

    row_of = {int(rr): i for i, rr in enumerate(rows)}
    ref_out = np.stack([wts[t, 0] * y[row_of[int(pos[2 * t])]] + wts[t, 1] * y[row_of[int(pos[2 * t + 1])]]
                        for t in toks])
    got_out = host(out[torch().from_numpy(toks).to(out.device)])[:, ch2]
    assert_final_close(bf16_bits_to_f64(got_out), bf16_bits_to_f64(oracle.f64_to_bf16_bits(ref_out)))
    del gw, a, out
    torch().cuda.empty_cache()


@pytest.mark.parametrize("name,n_tokens,n_ch", [("mixtral_decode", 32, 48), ("grok_decode", 32, 48),
                                                ("grok_prefill", 48, 40), ("grok_tp8_decode", 32, 48),
                                                ("grok_tp8_prefill", 48, 40)])
def test_fullsize_sampled(name, n_tokens, n_ch):
    _run_sampled(synth.MOE_CONFIGS[name], n_tokens, n_ch)


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
