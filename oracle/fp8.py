"""OCP FP8 E4M3 ("e4m3fn") codec, written from the format's definition.

The pages say "FP8" (page A, "Motivation": FP8 compute; page B: upcast to float8,
tensor-wise FP8 quantization) without naming the variant. Reading: the OCP 8-bit
E4M3 format of the MI355X generation: 1 sign bit, 4 exponent bits with bias 7,
3 mantissa bits, subnormals, no infinities, only S.1111.111 is NaN, largest finite
magnitude 448.

Rounding reading (the pages are silent): round to nearest, ties to the even code,
saturate magnitudes above 448 to 448, keep the sign of the input on a zero result.
The encoder is a brute-force nearest search over the 127 non-negative magnitudes;
it uses no hardware conversion.
"""
import numpy as np

E4M3_MAX = 448.0


def _value_of_code(c: int) -> float:
    """Value of one E4M3 code from the format definition."""
    sign = -1.0 if c & 0x80 else 1.0
    e = (c >> 3) & 0xF
    m = c & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:                                   # subnormal: m/8 * 2^(1-7)
        return sign * (m / 8.0) * 2.0 ** -6
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


_TABLE = np.array([_value_of_code(c) for c in range(256)], dtype=np.float64)
# codes 0x00..0x7E are the non-negative finite values in increasing order
_MAGS = _TABLE[:0x7F].copy()


def e4m3_table() -> np.ndarray:
    """The 256 code values (fp64; NaN at 0x7F and 0xFF)."""
    return _TABLE.copy()


def e4m3_decode(codes) -> np.ndarray:
    """Code(s) -> exact fp64 value(s)."""
    return _TABLE[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(v) -> np.ndarray:
    """Nearest E4M3 code of each value; ties to even code; saturating (an fp32 quotient
    that overflowed to +-inf saturates too). NaN is rejected.

    ``v`` is read exactly as fp64 (pass the fp32 quotient the method forms).
    """
    v = np.asarray(v, dtype=np.float64)
    if np.any(np.isnan(v)):
        raise ValueError("e4m3_encode: NaN input")
    a = np.abs(v)
    hi = np.searchsorted(_MAGS, a, side="left")          # first magnitude >= a
    hi = np.clip(hi, 1, 0x7E)
    lo = hi - 1
    with np.errstate(invalid="ignore"):                    # inf - inf on saturated lanes
        d_lo = a - _MAGS[lo]                               # exact in fp64
        d_hi = _MAGS[hi] - a
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(take_hi, hi, lo)
    code = np.where(a >= E4M3_MAX, 0x7E, code)             # saturate
    sign = np.signbit(v).astype(np.int64) << 7
    return (code | sign).astype(np.uint8)
