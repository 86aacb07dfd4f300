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
    and V, set when a page is first written (fresh page);
  * scale value: s = amax / 448 in fp32 (s = 1 when amax == 0), amax taken over
    the tokens that first write fills into that page-head;
  * a later append into the page whose values exceed its range
    (amax > 448 s) doubles s until they fit and encodes the page's codes
    again with the new scale (value decode(c) * s_old in fp32, then the
    quantiser below); a power-of-two change leaves every code whose value
    stays in E4M3's normal range exactly representable.  Without it a page
    whose first fill is a few decode tokens clips the later ones;
  * code: y = x * (1/s) in fp32 (two IEEE-rounded fp32 operations), then
    round-to-nearest-even onto the E4M3 grid with saturation to +-448.
The fp32 steps are done in numpy float32 so the integer codes are exactly the
ones any IEEE-conforming fp32 implementation gets.
"""
import math

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


def needs_growth(x_new, scale):
    """True when values appended to a page written before exceed the page's
    range: max |x| > 448 * s (fp32 product and comparison)."""
    if not np.size(x_new):
        return False
    amax = np.float32(np.max(np.abs(np.asarray(x_new, dtype=np.float32))))
    return bool(amax > np.float32(np.float32(FP8_MAX) * np.float32(scale)))


def grown_scale(x_new, scale):
    """The page's scale times the smallest power of two 2^k (k >= 1) with
    max |x_new| <= 448 * s * 2^k (fp32).  Codes re-encoded under a power-of-two
    ratio keep their values except where they fall below the normal range."""
    amax = np.float32(np.max(np.abs(np.asarray(x_new, dtype=np.float32))))
    s = np.float32(scale)
    while True:
        s = np.float32(s * np.float32(2.0))
        if not amax > np.float32(np.float32(FP8_MAX) * s):
            return s


def reencode(codes, old_scale, new_scale):
    """Codes of a page encoded again under a larger scale: the value each code
    stands for, decode(c) * s_old in fp32, quantised with s_new."""
    v = (decode(codes).astype(np.float32) * np.float32(old_scale)).astype(np.float32)
    return quantise(v, new_scale)


def quantise(x, scale):
    """fp32 values -> codes with a given fp32 scale (y = x * (1/s), fp32)."""
    x = np.asarray(x, dtype=np.float32)
    inv = np.float32(np.float32(1.0) / np.float32(scale))
    y = (x * inv).astype(np.float32)
    return encode_rne_sat(y.astype(np.float64))


# ----------------------------------------------------------------------------
# Per-64-element tile scales
# ----------------------------------------------------------------------------
# The same page asks for FP8 block scales to be recomputed per 64-element tile
# (atozofsoftwareengineering.blog, closing checklist, "Precision
# Benchmarking").  Readings used here:
#   * a tile is 64 consecutive channels of one token of one KV head (head_dim
#     128 has two tiles per token), for K and for V separately; every token is
#     quantised on its own when it is appended, so codes never depend on which
#     other tokens share its page;
#   * the scale is a power of two stored as an OCP E8M0 exponent byte
#     (value 2^(e - 127)), as in the OCP microscaling formats: s = 2^k with k
#     the smallest integer for which amax / 2^k <= 448 (k = 0 when amax = 0),
#     k clamped to [-127, 127];
#   * code: y = x * 2^-k (exact in fp32), then the E4M3 encoder above.
# Power-of-two scales make decode(code) * s exact in bf16 as well as fp32.

def tile_exponent(amax):
    """k of the tile scale 2^k for a tile whose largest magnitude is amax."""
    amax = float(amax)
    if amax == 0.0:
        return 0
    m, E = math.frexp(amax)               # amax = m * 2^E, m in [0.5, 1)
    k = E - 9 + (1 if m > 0.875 else 0)   # 448 = 0.875 * 2^9
    return max(-127, min(127, k))


def quantise_tiles(x):
    """x [..., D] fp32 with D a multiple of 64 -> (codes [..., D] uint8,
    E8M0 exponent bytes [..., D/64] uint8)."""
    x = np.asarray(x, dtype=np.float32)
    shp = x.shape
    D = shp[-1]
    tiles = x.reshape(-1, D // 64, 64)
    codes = np.empty(tiles.shape, dtype=np.uint8)
    exps = np.empty(tiles.shape[:2], dtype=np.uint8)
    for i in range(tiles.shape[0]):
        for g in range(tiles.shape[1]):
            t = tiles[i, g]
            k = tile_exponent(np.max(np.abs(t)))
            exps[i, g] = k + 127
            y = (t * np.float32(2.0 ** -k)).astype(np.float32)
            codes[i, g] = encode_rne_sat(y.astype(np.float64))
    return codes.reshape(shp), exps.reshape(shp[:-1] + (D // 64,))


def dequantise_tiles(codes, exps):
    """Inverse of quantise_tiles (fp64): decode(code) * 2^(e - 127)."""
    codes = np.asarray(codes, dtype=np.uint8)
    D = codes.shape[-1]
    s = np.ldexp(1.0, np.asarray(exps, dtype=np.int64) - 127)
    return (decode(codes).reshape(codes.shape[:-1] + (D // 64, 64)) * s[..., None]).reshape(codes.shape)
