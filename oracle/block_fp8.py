"""Block-FP8 weight-only dense linear (the FP8_PB_WO projections).

Page C: the block-FP8 dense projections are kept quantized and consumed by the
existing block-FP8 linears: an e4m3 weight [N, K] plus a scale tensor
``weight_scale_inv`` with one fp32 value per 128 x 128 block, shapes [16384, 2560]
with scales [128, 20] and [13312, 2560] with scales [104, 20]; the fused groups are
whole numbers of 128-row blocks, so block scales concatenate with their rows.

Readings (page C does not spell out the arithmetic):

* weight-only: the activation x stays bf16, it is not quantized;
* the stored scale multiplies the decoded weight (it is a dequantization factor
  despite the "_inv" in its name): W[n, k] ~= S[n // 128, k // 128] * dec(Wq[n, k]);
* y[m, n] = sum over K-blocks kb of S[n//128, kb] * sum_{k in kb} x[m, k] * dec(Wq[n, k]),
  in fp64, then rounded to bf16 (nearest, ties to even);
* the harness quantizer that makes Wq and S from bf16 weights: per block,
  S = fp32(fp32(max|w|) / 448) and Wq = e4m3(fp32(w / S)); a block of zeros gets
  S = 0 and Wq = 0. Partial edge blocks use the elements they contain.
"""
import numpy as np

from .bf16 import bf16_to_f32, bf16_to_f64, f64_to_bf16_bits
from .fp8 import E4M3_MAX, e4m3_decode, e4m3_encode

BLOCK = 128


def _nblocks(n):
    return (n + BLOCK - 1) // BLOCK


def fp8_block_quantize(w_bits):
    """bf16 bits [N, K] -> (codes uint8 [N, K], scales float32 [ceil(N/128), ceil(K/128)])."""
    w = bf16_to_f32(w_bits)
    N, K = w.shape
    codes = np.zeros((N, K), dtype=np.uint8)
    S = np.zeros((_nblocks(N), _nblocks(K)), dtype=np.float32)
    for nb in range(_nblocks(N)):
        for kb in range(_nblocks(K)):
            blk = w[nb * BLOCK:(nb + 1) * BLOCK, kb * BLOCK:(kb + 1) * BLOCK]
            amax = np.float32(np.max(np.abs(blk)))
            s = np.float32(amax / np.float32(E4M3_MAX))
            S[nb, kb] = s
            if s > 0:
                codes[nb * BLOCK:(nb + 1) * BLOCK, kb * BLOCK:(kb + 1) * BLOCK] = \
                    e4m3_encode((blk / s).astype(np.float32))
    return codes, S


def fp8_block_linear(x_bits, codes, S):
    """bf16 x [M, K], e4m3 codes [N, K], scales [ceil(N/128), ceil(K/128)] -> (y fp64 [M, N], y bf16 bits)."""
    x = bf16_to_f64(x_bits)
    M, K = x.shape
    N = codes.shape[0]
    Wd = e4m3_decode(codes)
    y = np.zeros((M, N))
    for kb in range(_nblocks(K)):
        ks = slice(kb * BLOCK, (kb + 1) * BLOCK)
        part = x[:, ks] @ Wd[:, ks].T                     # [M, N]
        scale_n = np.repeat(S[:, kb].astype(np.float64), BLOCK)[:N]
        y += part * scale_n[None, :]
    return y, f64_to_bf16_bits(y)


def fp8_block_linear_bruteforce(x_bits, codes, S):
    """The same sum with plain Python loops, element by element (tiny inputs only)."""
    x = bf16_to_f64(x_bits)
    M, K = x.shape
    N = codes.shape[0]
    table = e4m3_decode(np.arange(256))
    y = np.zeros((M, N))
    for m in range(M):
        for n in range(N):
            total = 0.0
            for k in range(K):
                total += float(S[n // BLOCK, k // BLOCK]) * x[m, k] * table[codes[n, k]]
            y[m, n] = total
    return y
