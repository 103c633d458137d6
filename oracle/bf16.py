"""bfloat16 <-> float conversions.

Inputs are carried as uint16 bit patterns. bf16 is the upper half of an IEEE fp32,
so decoding is exact. The model's weights and activations are bf16 (page A,
``config.json``: ``torch_dtype`` bfloat16). Output rounding reading (pages silent):
round to nearest, ties to even, directly from the fp64 result.
"""
import numpy as np


def bf16_to_f32(bits) -> np.ndarray:
    """uint16 bf16 bits -> exact float32 values."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


def bf16_to_f64(bits) -> np.ndarray:
    with np.errstate(invalid="ignore"):                      # NaN patterns stay NaN
        return bf16_to_f32(bits).astype(np.float64)


def _f32_bits_to_f64(u32) -> np.ndarray:
    return np.asarray(u32, dtype=np.uint32).view(np.float32).astype(np.float64)


def f64_to_bf16_bits(v) -> np.ndarray:
    """Round fp64 values to the nearest bf16 (ties to even); uint16 bits.

    Three candidates around the bf16 truncation of fp32(v) are compared exactly in
    fp64; the nearest wins, an exact tie goes to the even bit pattern. Finite,
    in-range inputs only.
    """
    v = np.asarray(v, dtype=np.float64)
    if not np.all(np.isfinite(v)):
        raise ValueError("f64_to_bf16_bits: non-finite input")
    f = v.astype(np.float32)
    t = (f.view(np.uint32) >> np.uint32(16)).astype(np.int64)   # truncation, with sign
    sign = t & 0x8000
    mag = t & 0x7FFF
    cands = []
    for d in (-1, 0, 1):
        m = np.clip(mag + d, 0, 0x7F7F)                          # stay finite
        cands.append(sign | m)
    vals = [_f32_bits_to_f64((c.astype(np.uint32) << np.uint32(16))) for c in cands]
    dist = [np.abs(x - v) for x in vals]
    best = cands[1].copy()
    best_d = dist[1].copy()
    for c, d in ((cands[0], dist[0]), (cands[2], dist[2])):
        better = (d < best_d) | ((d == best_d) & (c % 2 == 0) & (best % 2 == 1))
        best = np.where(better, c, best)
        best_d = np.where(better, d, best_d)
    # the sign of zero follows the input
    zero = (best & 0x7FFF) == 0
    best = np.where(zero, np.where(np.signbit(v), 0x8000, 0), best)
    return best.astype(np.uint16)
