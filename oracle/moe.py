"""The W4A8 MoE layer forward, step by step, in fp64.

Page A: "INT4 MoE weights, FP8 compute"; ``activation_scheme`` static. Page B: the
int4 MoE weights are upcast to float8 so that the math runs in fp8; activations get
tensor-wise FP8 quantization. The layer is the top-2 routed expert FFN of the
Grok-1 / Mixtral block (``num_experts_per_tok`` 2):

1. route: top-2 of the router logits, renormalised weights (``route.route_top2``);
2. sort: expert-contiguous order of the (token, slot) pairs (``route.route_sort``);
3. x quant: x_hat = e4m3(fp32(x / s_x)) with a static per-tensor scale s_x;
4. gate|up: for pair row r of expert e and token t,
   acc[r, n] = sum_k dec(x_hat[t, k]) * q13[e, n, k] -- exact in fp64 (each product
   is a multiple of 2^-9 of magnitude <= 448*8, sums stay below 2^27 for K <= 32768,
   so fewer than 53 significant bits are ever needed);
   h = acc * s_x * s_w13[e, n];
5. gated activation: a = act(h[:, :I]) * h[:, I:] (rows [0, I) of w13 are the gate,
   rows [I, 2I) the up projection);
6. requant: a_hat = e4m3(fp32(fp32(a) / s_a)) with a static per-tensor scale s_a;
7. down: Y[r, n] = s_a * s_w2[e, n] * sum_j dec(a_hat[r, j]) * q2[e, n, j] (exact sum);
8. combine: out[t] = w0 * Y[pos(2t)] + w1 * Y[pos(2t+1)], then bf16 (or fp32) rounding.

Readings (pages silent): the gating function per model (SwiGLU for Mixtral,
GELU-gated for Grok-1; erf form by default, tanh form selectable); the static scales
are max|.| / 448 from a calibration pass; one scalar per tensor, not per expert.
"""
from __future__ import annotations

import math

import numpy as np
from scipy.special import erf as _erf

from .bf16 import bf16_to_f32, bf16_to_f64, f64_to_bf16_bits
from .fp8 import E4M3_MAX, e4m3_decode, e4m3_encode
from .int4 import w4_quantize, w4_unpack_codes
from .route import route_sort, route_top2

ACT_SILU, ACT_GELU_ERF, ACT_GELU_TANH = 0, 1, 2


def activation(g, act):
    """The gating nonlinearity, fp64: silu(g) = g / (1 + e^-g);
    gelu_erf(g) = g/2 (1 + erf(g/sqrt 2)); gelu_tanh(g) = g/2 (1 + tanh(sqrt(2/pi)(g + 0.044715 g^3)))."""
    g = np.asarray(g, dtype=np.float64)
    if act == ACT_SILU:
        with np.errstate(over="ignore"):
            return g / (1.0 + np.exp(-g))
    if act == ACT_GELU_ERF:
        return 0.5 * g * (1.0 + _erf(g / math.sqrt(2.0)))
    if act == ACT_GELU_TANH:
        return 0.5 * g * (1.0 + np.tanh(math.sqrt(2.0 / math.pi) * (g + 0.044715 * g ** 3)))
    raise ValueError(f"unknown activation {act}")


def act_lipschitz(act) -> float:
    """An upper bound of sup |act'| (numerical maximum on a fine grid plus a margin
    that covers the grid spacing; the derivative is smooth with |act'''| < 2)."""
    x = np.linspace(-30.0, 30.0, 600001)
    h = 1e-6
    d = (activation(x + h, act) - activation(x - h, act)) / (2 * h)
    return float(np.max(np.abs(d))) + 1e-5


def static_scale(max_abs) -> np.float32:
    """Static per-tensor fp8 scale: fp32(fp32(max|v|) / 448), division correctly rounded."""
    return np.float32(np.float32(max_abs) / np.float32(E4M3_MAX))


def quantize_static(v, s) -> np.ndarray:
    """Tensor-wise FP8 quantization: e4m3(fp32(fp32(v) / s)); s > 0 (fp32)."""
    s = np.float32(s)
    if not s > 0:
        raise ValueError("static scale must be positive")
    with np.errstate(over="ignore"):                            # overflow -> inf -> saturates
        q = (np.asarray(v, dtype=np.float32) / s).astype(np.float32)   # correctly rounded
    return e4m3_encode(q)


def _provider(w):
    """Weights as (words [E, N, K/8], scales [E, N]) or a callable e -> (words, scales)."""
    if callable(w):
        return w
    words, scales = w
    return lambda e: (words[e], scales[e])


def _int4_matmul(a_codes_f64, words, row_chunk=4096):
    """sum_k a[r, k] * q[n, k] for all n, exact in fp64; q unpacked in row chunks."""
    N = words.shape[0]
    out = np.empty((a_codes_f64.shape[0], N), dtype=np.float64)
    for n0 in range(0, N, row_chunk):
        q = w4_unpack_codes(words[n0:n0 + row_chunk]).astype(np.float64)
        out[:, n0:n0 + row_chunk] = a_codes_f64 @ q.T
    return out


def expert_gate_up(x_codes, words13, scales13, s_x):
    """Step 4 for the rows of one expert: h = s_x * s_w13[n] * sum_k dec(x_hat[k]) q13[n, k].

    x_codes: E4M3 codes [rows, H] of the tokens of these rows; words13 / scales13: any
    subset of the expert's weight rows (the sums are independent per weight row).
    """
    acc = _int4_matmul(e4m3_decode(x_codes), words13)                     # exact
    return acc * np.float64(s_x) * np.asarray(scales13, dtype=np.float64)[None, :]


def expert_down(a_codes, words2, scales2, s_a):
    """Step 7 for the rows of one expert: Y = s_a * s_w2[n] * sum_j dec(a_hat[j]) q2[n, j].

    a_codes: E4M3 codes [rows, I]; words2 / scales2: any subset of the expert's rows.
    """
    acc2 = _int4_matmul(e4m3_decode(a_codes), words2)                      # exact
    return acc2 * np.float64(s_a) * np.asarray(scales2, dtype=np.float64)[None, :]


def moe_forward(x_bits, logits, s_x, w13, w2, act, s_a, out_f32=False, tokens=None,
                E=None, a_codes_given=None):
    """Run the quantized layer (steps 1-8 of the module docstring).

    x_bits: bf16 bits [T, H]; logits: float32 [T, E]; s_x, s_a: fp32 static scales;
    w13: (words [E, 2I, H/8], scales [E, 2I]) or callable e -> that pair for one expert;
    w2: (words [E, H, I/8], scales [E, H]) or callable; tokens: optional subset of
    token ids whose outputs are computed (routing and sort always cover all tokens);
    a_codes_given: optional uint8 [2T, I] E4M3 codes indexed by sorted row. When given,
    the down projection (step 7) reads these codes instead of requantizing this
    oracle's own gate|up: the requantization is a rounding decision, and a caller that
    took it from another evaluation of gate|up passes the codes it took (steps 1-6 are
    still computed and returned as usual).

    Returns a dict: ids, weights, counts, offsets, sorted_pair, pair_pos (all tokens);
    rows (sorted row ids computed), h [rows, 2I] fp64, a [rows, I] fp64,
    a_codes [rows, I] uint8, y [rows, H] fp64 (per sorted row), tokens, out [tokens, H]
    fp64, out_rounded (bf16 bits, or float32 when out_f32).
    """
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    logits = np.asarray(logits, dtype=np.float32)
    T, H = x_bits.shape
    E = logits.shape[1] if E is None else E
    ids, wts = route_top2(logits)
    counts, offsets, sorted_pair, pair_pos = route_sort(ids, E)
    tokens = np.arange(T) if tokens is None else np.asarray(tokens, dtype=np.int64)
    get13, get2 = _provider(w13), _provider(w2)

    # sorted rows needed for the requested tokens
    rows = np.unique(np.concatenate([pair_pos[2 * tokens], pair_pos[2 * tokens + 1]]).astype(np.int64))
    row_index = {int(r): i for i, r in enumerate(rows)}
    expert_of_row = np.searchsorted(offsets, rows, side="right") - 1
    token_of_row = sorted_pair[rows].astype(np.int64) // 2

    x_codes = quantize_static(bf16_to_f32(x_bits[np.unique(token_of_row)]), s_x)
    code_of_token = {int(t): i for i, t in enumerate(np.unique(token_of_row))}

    h = a = a_codes = y = None
    for e in range(E):
        sel = np.nonzero(expert_of_row == e)[0]
        if sel.size == 0:
            continue
        words13, sc13 = get13(e)
        words2, sc2 = get2(e)
        I = words13.shape[0] // 2
        if h is None:
            h = np.empty((rows.size, 2 * I))
            a = np.empty((rows.size, I))
            a_codes = np.empty((rows.size, I), dtype=np.uint8)
            y = np.empty((rows.size, H))
        he = expert_gate_up(x_codes[[code_of_token[int(t)] for t in token_of_row[sel]]], words13, sc13, s_x)
        ae = activation(he[:, :I], act) * he[:, I:]
        ce = quantize_static(ae.astype(np.float32), s_a)
        cd = ce if a_codes_given is None else np.asarray(a_codes_given, np.uint8)[rows[sel]]
        ye = expert_down(cd, words2, sc2, s_a)
        h[sel], a[sel], a_codes[sel], y[sel] = he, ae, ce, ye

    out = np.empty((tokens.size, H))
    for i, t in enumerate(tokens):
        r0 = row_index[int(pair_pos[2 * t])]
        r1 = row_index[int(pair_pos[2 * t + 1])]
        out[i] = wts[t, 0] * y[r0] + wts[t, 1] * y[r1]
    out_rounded = out.astype(np.float32) if out_f32 else f64_to_bf16_bits(out)
    return dict(ids=ids, weights=wts, counts=counts, offsets=offsets, sorted_pair=sorted_pair,
                pair_pos=pair_pos, rows=rows, h=h, a=a, a_codes=a_codes, y=y, tokens=tokens,
                out=out, out_rounded=out_rounded, x_codes_tokens=np.unique(token_of_row),
                x_codes=x_codes)


def moe_reference_unquantized(x_bits, logits, w13_bits, w2_bits, act):
    """The same routed layer with bf16 weights and activations, no quantization, fp64."""
    x = bf16_to_f64(x_bits)
    ids, wts = route_top2(logits)
    T, H = x.shape
    I = w13_bits.shape[1] // 2
    out = np.zeros((T, H))
    for t in range(T):
        for slot in range(2):
            e = ids[t, slot]
            hh = bf16_to_f64(w13_bits[e]) @ x[t]
            aa = activation(hh[:I], act) * hh[I:]
            out[t] += wts[t, slot] * (bf16_to_f64(w2_bits[e]) @ aa)
    return out


def moe_error_bound(x_bits, logits, w13_bits, w2_bits, act, s_x, s_a):
    """Elementwise bound on |quantized layer - unquantized layer| (fp64, before rounding).

    Triangle inequality through the steps, with Wq = q*s the dequantized weights,
    xt = dec(x_hat)*s_x, at = dec(a_hat)*s_a, and L = sup |act'|:
      |dh| <= |x - xt| |W13|^T + |xt| |W13 - W13q|^T
      |da| <= L |dg| |u| + |act(g_q)| |du| + |a_q - at|
      |dy| <= |da| |W2|^T + |at| |W2 - W2q|^T
      |dout| <= w0 |dy0| + w1 |dy1|
    """
    x = bf16_to_f64(x_bits)
    ids, wts = route_top2(logits)
    T, H = x.shape
    I = w13_bits.shape[1] // 2
    L = act_lipschitz(act)
    q13, s13 = w4_quantize(w13_bits)
    q2, s2 = w4_quantize(w2_bits)
    xt = e4m3_decode(quantize_static(bf16_to_f32(x_bits), s_x)) * np.float64(s_x)
    bound = np.zeros((T, H))
    for t in range(T):
        for slot in range(2):
            e = ids[t, slot]
            W = bf16_to_f64(w13_bits[e])
            Wq = q13[e].astype(np.float64) * s13[e].astype(np.float64)[:, None]
            h_ref = W @ x[t]
            h_q = Wq @ xt[t]
            dh = np.abs(W) @ np.abs(x[t] - xt[t]) + np.abs(W - Wq) @ np.abs(xt[t])
            g_q, u_q = h_q[:I], h_q[I:]
            a_q = activation(g_q, act) * u_q
            at = e4m3_decode(quantize_static(a_q.astype(np.float32), s_a)) * np.float64(s_a)
            da = L * dh[:I] * np.abs(h_ref[I:]) + np.abs(activation(g_q, act)) * dh[I:] + np.abs(a_q - at)
            W2 = bf16_to_f64(w2_bits[e])
            W2q = q2[e].astype(np.float64) * s2[e].astype(np.float64)[:, None]
            dy = np.abs(W2) @ da + np.abs(W2 - W2q) @ np.abs(at)
            bound[t] += wts[t, slot] * dy
    return bound
