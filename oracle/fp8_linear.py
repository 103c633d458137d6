"""Per-tensor static FP8 dense linear (W8A8): the attention projections of the W4A8 model.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Page A: the Grok-1 W4A8KV8 checkpoint is quantized with ``quant_method`` "fp8" and a
static ``activation_scheme``; only the MoE router gates and ``lm_head`` are left out
(``ignored_layers``), and the experts are the int4 part (``int4_experts``). So the dense
attention projections (q, k, v, o of 48 query and 8 key/value heads of 128 over hidden
6144) are FP8 weights against statically scaled FP8 activations. Page B lists
"tensor-wise FP8 quantization" among its core quantization utilities and a linear method
(QuarkInt4Fp8LinearMethod) beside the MoE one.

Readings (the pages do not spell out the arithmetic):

* per-tensor weight scale, the tensor-wise rule of page B: s_w = fp32(fp32(max|W|) / 448),
  Wq = e4m3(fp32(W / s_w)) (nearest even, saturating); an all-zero W gives s_w = 0, Wq = 0;
* static per-tensor activation scale s_x (a calibrated constant, like the MoE layer's):
  xq = e4m3(fp32(x / s_x));
* y[m, n] = s_x * s_w * sum_k dec(xq[m, k]) * dec(Wq[n, k]) in fp64, then bf16 (nearest
  even). The sum is exact in fp64: every product of two E4M3 values is a multiple of
  2^-18 below 448^2 (36 significant bits), and K <= 65536 adds at most 16 more.
"""
import numpy as np

from .bf16 import bf16_to_f32, f64_to_bf16_bits
from .fp8 import E4M3_MAX, e4m3_decode, e4m3_encode


def fp8_tensor_quantize(w_bits):
    """bf16 bits [N, K] -> (codes uint8 [N, K], s_w float32): one scale for the tensor."""
    w = bf16_to_f32(w_bits)
    amax = np.float32(np.max(np.abs(w))) if w.size else np.float32(0.0)
    s = np.float32(amax / np.float32(E4M3_MAX))                   # correctly rounded fp32 quotient
    if not s > 0:
        return np.zeros(w.shape, np.uint8), np.float32(0.0)
    with np.errstate(over="ignore"):
        q = (w / s).astype(np.float32)                            # correctly rounded, saturates below
    return e4m3_encode(q), s


def fp8_quantize_activations(x_bits, s_x):
    """Static activation quantization: e4m3(fp32(x / s_x)), s_x > 0."""
    s = np.float32(s_x)
    if not s > 0:
        raise ValueError("static scale must be positive")
    with np.errstate(over="ignore"):
        q = (bf16_to_f32(x_bits) / s).astype(np.float32)
    return e4m3_encode(q)


def fp8_linear(x_bits, s_x, codes, s_w):
    """bf16 x [M, K], static s_x, e4m3 weight codes [N, K] and s_w ->
    (y fp64 [M, N], y bf16 bits [M, N], x codes uint8 [M, K])."""
    xq = fp8_quantize_activations(x_bits, s_x)
    acc = e4m3_decode(xq) @ e4m3_decode(codes).T                  # exact (module docstring)
    y = float(np.float32(s_x)) * float(np.float32(s_w)) * acc
    return y, f64_to_bf16_bits(y), xq


def fp8_linear_bruteforce(x_bits, s_x, codes, s_w):
    """The same result with plain Python loops, element by element (tiny inputs only)."""
    xq = fp8_quantize_activations(x_bits, s_x)
    table = e4m3_decode(np.arange(256))
    M, K = xq.shape
    N = codes.shape[0]
    y = np.zeros((M, N))
    for m in range(M):
        for n in range(N):
            total = 0.0
            for k in range(K):
                total += table[xq[m, k]] * table[codes[n, k]]
            y[m, n] = float(np.float32(s_x)) * float(np.float32(s_w)) * total
    return y
