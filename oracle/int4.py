"""Column-wise symmetric int4 quantization of expert weights and int32 packing.

Page A, ``config.json`` -> ``quantization_config.int4_experts``: ``bits`` 4,
``sym`` true, ``group`` "column"; ``export.pack_method`` "reorder". Page B, the
highlight "Core Quantization Utilities": column-wise INT4 quantization and packing
of INT4 values into INT32.

Readings taken where the pages are silent:

* "column" = one scale per output channel, i.e. per row of a ``[out, in]`` weight
  (torch Linear layout), the maximum taken over the input dimension K.
* scale s = fp32(max_k |w| / 7), the division correctly rounded in fp32;
  q = clamp(round_half_even(fp32(w / s)), -8, 7), the quotient correctly rounded
  in fp32. A row of zeros gets s = 0 and q = 0.
* the int4 container is two's complement [-8, 7]; quantization only produces
  [-7, 7] and the max-|w| element maps to +-7.
* "reorder" packing: in int32 word j of a row, byte b (b = 0..3) holds element
  8j + b in its low nibble and element 8j + 4 + b in its high nibble. Spelled
  per nibble: nibble i (bits 4i..4i+3) holds element 8j + i//2 + 4*(i%2).
"""
import numpy as np

from .bf16 import bf16_to_f32


def w4_quantize(w_bits):
    """bf16 bits [..., N, K] -> (q int8 [..., N, K] in [-8, 7], scale float32 [..., N])."""
    w = bf16_to_f32(w_bits)
    amax = np.max(np.abs(w), axis=-1)                          # exact in fp32
    s = (amax / np.float32(7.0)).astype(np.float32)            # correctly rounded
    safe = np.where(s == 0, np.float32(1.0), s).astype(np.float32)
    r = (w / safe[..., None]).astype(np.float32)               # correctly rounded
    q = np.clip(np.rint(r), -8, 7)
    q = np.where((s == 0)[..., None], 0, q)
    return q.astype(np.int8), s


# element offset (within a group of 8) held by nibble i of a word
NIBBLE_ELEMENT = np.array([i // 2 + 4 * (i % 2) for i in range(8)], dtype=np.int64)


def w4_pack_codes(q) -> np.ndarray:
    """int4 codes [..., K] (K % 8 == 0) -> int32 words [..., K/8] in the reorder layout."""
    q = np.asarray(q, dtype=np.int64)
    K = q.shape[-1]
    if K % 8:
        raise ValueError("K must be a multiple of 8")
    g = q.reshape(q.shape[:-1] + (K // 8, 8))
    word = np.zeros(g.shape[:-1], dtype=np.uint64)
    for i in range(8):
        nib = (g[..., NIBBLE_ELEMENT[i]] & 0xF).astype(np.uint64)
        word |= nib << np.uint64(4 * i)
    return word.astype(np.uint32).view(np.int32)


def w4_unpack_codes(words, K=None) -> np.ndarray:
    """int32 words [..., K/8] -> int4 codes int8 [..., K], nibbles sign-extended."""
    w = np.asarray(words, dtype=np.int32).view(np.uint32).astype(np.int64)
    out = np.empty(w.shape + (8,), dtype=np.int8)
    for i in range(8):
        nib = (w >> (4 * i)) & 0xF
        out[..., NIBBLE_ELEMENT[i]] = np.where(nib >= 8, nib - 16, nib)
    out = out.reshape(w.shape[:-1] + (w.shape[-1] * 8,))
    if K is not None and out.shape[-1] != K:
        raise ValueError("K mismatch")
    return out


def w4_pack(w_bits):
    """bf16 bits [..., N, K] -> (packed int32 [..., N, K/8], scale float32 [..., N])."""
    q, s = w4_quantize(w_bits)
    return w4_pack_codes(q), s


def w4_dequant(words, scale) -> np.ndarray:
    """Packed words + scales -> fp64 weights q * s."""
    q = w4_unpack_codes(words).astype(np.float64)
    return q * np.asarray(scale, dtype=np.float64)[..., None]
