"""OCP FP8 E4M3 ("e4m3fn") codec and the per-page scale quantiser — oracle side.

Format (OCP 8-bit Floating Point Specification, rev. 1.0, E4M3 column):
1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits.
  E in 1..15:  (-1)^S * 2^(E-7) * (1 + M/8)   except S.1111.111, which is NaN
  E = 0:       (-1)^S * 2^(-6) * (M/8)        (subnormals)
No infinities; the largest finite magnitude is 448 = 2^8 * 1.75.

The pages store K/V "in e4m3 FP8 format with per-block scaling factors S_K,
S_V" (atozofsoftwareengineering.blog, section "Custom FP8 Quantized Memory
Block Layout") but give no rule for the scale or the rounding.  Readings used
here:
  * scale granularity: one fp32 scale per (page, KV head), separately for K
    and V, fixed when a page is first written (fresh page);
  * scale value: s = amax / 448 in fp32 (s = 1 when amax == 0), amax taken over
    the tokens that first write fills into that page-head;
  * code: y = x * (1/s) in fp32 (two IEEE-rounded fp32 operations), then
    round-to-nearest-even onto the E4M3 grid with saturation to +-448.
The fp32 steps are done in numpy float32 so the integer codes are exactly the
ones any IEEE-conforming fp32 implementation gets.
"""
import numpy as np

FP8_MAX = 448.0


def decode_table():
    """Value of every one of the 256 codes (fp64), NaN for 0x7F / 0xFF."""
    vals = np.empty(256, dtype=np.float64)
    for code in range(256):
        s = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            vals[code] = np.nan
        elif e == 0:
            vals[code] = s * 2.0 ** -6 * (m / 8.0)
        else:
            vals[code] = s * 2.0 ** (e - 7) * (1.0 + m / 8.0)
    return vals


_TABLE = decode_table()
# Non-negative finite codes 0x00..0x7E in increasing value order.
_POS_VALUES = _TABLE[:0x7F]


def decode(codes):
    """uint8 codes -> fp64 values."""
    return _TABLE[np.asarray(codes, dtype=np.uint8)]


def encode_rne_sat(y):
    """Round values (exactly representable in fp64) to the nearest E4M3 code,
    ties to the even code (even mantissa), saturating magnitudes above 448 to
    448.  NaN -> 0x7F."""
    y = np.asarray(y, dtype=np.float64)
    a = np.abs(y)
    nan = np.isnan(a)
    a = np.where(nan, 0.0, np.minimum(a, FP8_MAX))
    hi = np.searchsorted(_POS_VALUES, a, side="left")      # first value >= a
    hi = np.minimum(hi, 0x7E)
    lo = np.maximum(hi - 1, 0)
    d_hi = _POS_VALUES[hi] - a
    d_lo = a - _POS_VALUES[lo]
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    pick_hi |= _POS_VALUES[lo] > a                          # a below grid start
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    code = np.where(np.signbit(y) & (code != 0), code | 0x80, code).astype(np.uint8)
    code = np.where(np.signbit(y) & (code == 0), np.uint8(0x80), code)
    return np.where(nan, np.uint8(0x7F), code).astype(np.uint8)


def page_scale(x_tokens):
    """fp32 scale for one page-head from the float32 values first written
    into it: amax / 448 in fp32, or 1 when amax is 0."""
    amax = np.float32(np.max(np.abs(np.asarray(x_tokens, dtype=np.float32)))) \
        if np.size(x_tokens) else np.float32(0)
    if amax == 0:
        return np.float32(1.0)
    return np.float32(amax / np.float32(FP8_MAX))


def quantise(x, scale):
    """fp32 values -> codes with a given fp32 scale (y = x * (1/s), fp32)."""
    x = np.asarray(x, dtype=np.float32)
    inv = np.float32(np.float32(1.0) / np.float32(scale))
    y = (x * inv).astype(np.float32)
    return encode_rne_sat(y.astype(np.float64))
