"""OCP FP8 E4M3 codec (oracle; test infrastructure only).

Page "生成一个字，为什么要背一整本账", section "再往后：压 KV 的三条路线":
K/V stored in FP8 instead of FP16 halve the cache, with per-channel
calibrated scaling factors narrowing the error.  The pages name no FP8
variant; the OCP 8-bit floating-point format E4M3 is used (1 sign bit,
4 exponent bits with bias 7, 3 mantissa bits, no infinities, NaN only at
S.1111.111, largest finite 448, smallest subnormal 2**-9).

Encoding rule used on both sides: round to nearest, ties to the code with an
even mantissa, magnitudes >= 448 (including infinities) saturate to +-448, NaN
maps to 0x7F.  The sign of zero is kept.

Written from the format definition: the decode table enumerates all 256 codes
and the encoder searches that table, so it shares nothing with a bit-twiddling
encoder.
"""
import numpy as np

E4M3_MAX = 448.0
_EXP_BIAS = 7


def e4m3_decode_table() -> np.ndarray:
    """float64[256]: the value of every E4M3 code (NaN for 0x7F and 0xFF)."""
    out = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        exp = (code >> 3) & 0xF
        man = code & 0x7
        if exp == 0xF and man == 0x7:
            out[code] = np.nan
        elif exp == 0:
            out[code] = sign * (man / 8.0) * 2.0 ** (1 - _EXP_BIAS)
        else:
            out[code] = sign * (1.0 + man / 8.0) * 2.0 ** (exp - _EXP_BIAS)
    return out


_TABLE = e4m3_decode_table()
# Non-negative finite codes 0x00..0x7E in increasing value order.
_POS_VALUES = _TABLE[:0x7F].copy()


def e4m3_encode(x) -> np.ndarray:
    """Encode float values (float32 or float64 array) to uint8 E4M3 codes."""
    a = np.asarray(x, dtype=np.float64)
    mag = np.abs(a)
    sign = np.where(np.signbit(a), 0x80, 0x00).astype(np.uint8)
    finite_mag = np.where(np.isnan(mag), 0.0, np.minimum(mag, E4M3_MAX))
    # Index of the first table value >= mag; the answer is that code or the
    # one below it.
    hi = np.searchsorted(_POS_VALUES, finite_mag, side="left")
    hi = np.minimum(hi, 0x7E)
    lo = np.maximum(hi - 1, 0)
    d_lo = finite_mag - _POS_VALUES[lo]
    d_hi = _POS_VALUES[hi] - finite_mag
    pick = np.where(d_lo < d_hi, lo, hi)
    tie = (d_lo == d_hi) & (hi != lo)
    pick = np.where(tie, np.where((lo & 1) == 0, lo, hi), pick)
    exact = _POS_VALUES[hi] == finite_mag
    pick = np.where(exact, hi, pick)
    codes = (sign | pick.astype(np.uint8)).astype(np.uint8)
    codes = np.where(np.isnan(a), np.uint8(0x7F), codes)
    return codes.astype(np.uint8)


def e4m3_to_f64(codes) -> np.ndarray:
    """Decode uint8 codes to float64 through the table."""
    return _TABLE[np.asarray(codes, dtype=np.uint8)]
