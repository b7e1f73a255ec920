"""OCP FP8 E4M3FN encode/decode and per-block quantisation (host reference).

Test infrastructure (see the package docstring).

Follows "FlashAttention-3: Warp Specialization ...", section "FP8 Block
Quantization": Q and K are cut into blocks of 128 rows, each block is divided
by its own fp32 scale = absmax / 448 (448 being the largest E4M3 value) and
cast to float8_e4m3fn; after the fp8 product the scores are multiplied back by
the product of the two blocks' scales.

Readings taken (the section's code and prose disagree):
* The listing takes amax over the last axis (one scale per row) while the
  prose says each tile gets one scale. One fp32 scalar per 128-row block over
  all d columns is used here.
* Scale s = fp32(absmax) / fp32(448) with IEEE fp32 division; y = fp32(x) / s
  (fp32 division); code = y rounded to the nearest E4M3FN value, ties to the
  even code, magnitudes above 448 saturating to 448. A block of zeros gets
  s = 1 and all-zero codes.
* A ragged last block (rows not a multiple of 128) takes the absmax over the
  rows it has.
* "Incoherent" processing is named but not described; no rotation is applied.

E4M3FN (OCP 8-bit floating point, "fn" = finite, no infinities): 1 sign bit,
4 exponent bits with bias 7, 3 mantissa bits. Exponent field 0 encodes
subnormals m/8 * 2^-6; otherwise (1 + m/8) * 2^(e-7). The all-ones pattern
(S.1111.111) is NaN; the largest finite value S.1111.110 is 448.
"""

import numpy as np

E4M3_MAX = 448.0
_NAN_CODE = 0x7F


def e4m3_value(code):
    """Exact value of an E4M3FN byte (array or scalar) as float64; NaN for 0x7F/0xFF."""
    c = np.asarray(code).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 0xF) & (m == 0x7), np.nan, mag)
    return sign * mag


def e4m3_table():
    """Non-negative finite E4M3FN values indexed by code 0x00..0x7E (ascending)."""
    return e4m3_value(np.arange(0x7F))


_TABLE = e4m3_table()


def e4m3_encode(y):
    """Round fp32 values to E4M3FN codes: nearest value, ties to even code,
    saturating at +-448. NaN maps to 0x7F. Returns uint8 array."""
    y = np.asarray(y, dtype=np.float32)
    a = np.abs(y.astype(np.float64))
    nan = np.isnan(a)
    a = np.where(nan, 0.0, np.minimum(a, E4M3_MAX))
    hi = np.searchsorted(_TABLE, a, side="left")          # first table value >= a
    hi = np.minimum(hi, _TABLE.size - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _TABLE[lo]
    d_hi = _TABLE[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(_TABLE[hi] == a, hi, code)            # exact hits
    code = code | np.where(np.signbit(y), 0x80, 0)
    code = np.where(nan, _NAN_CODE, code)
    return code.astype(np.uint8)


def pow2_scale(amax):
    """Smallest power of two s with amax / s <= 448 (exactly: 448 * s / 2 <
    amax <= 448 * s), exponent clamped to >= -127; 1 for amax = 0. Computed on
    the exact binary mantissa of amax: amax = m * 2^e, m in [0.5, 1), and
    448 = 0.875 * 2^9, so the exponent is e - 9 when m <= 0.875, else e - 8."""
    amax = np.asarray(amax, dtype=np.float64)
    m, e = np.frexp(amax)
    k = np.where(m <= 0.875, e - 9, e - 8)
    k = np.maximum(k, -127)
    return np.where(amax == 0, 1.0, np.ldexp(1.0, k)).astype(np.float32)


def quantize_blocks(x, block=128, pow2=False):
    """Per-block fp8 quantisation of x [..., N, d] (fp32).

    Scale per block: absmax / 448 in fp32 ("FlashAttention-3 ...", "FP8 Block
    Quantization"), or with pow2 the power of two just above it, so that the
    scale is an exact power of two a matrix core can apply as an exponent.
    Returns (codes uint8 [..., N, d], scales fp32 [..., ceil(N/block)]).
    """
    x = np.asarray(x, dtype=np.float32)
    n = x.shape[-2]
    nb = -(-n // block)
    codes = np.empty(x.shape, dtype=np.uint8)
    scales = np.empty(x.shape[:-2] + (nb,), dtype=np.float32)
    for b in range(nb):
        blk = x[..., b * block:(b + 1) * block, :]
        amax = np.abs(blk).max(axis=(-2, -1)).astype(np.float32)
        if pow2:
            s = pow2_scale(amax)
        else:
            s = (amax / np.float32(E4M3_MAX)).astype(np.float32)
            s = np.where(amax == 0, np.float32(1.0), s).astype(np.float32)
        y = (blk / s[..., None, None]).astype(np.float32)
        codes[..., b * block:(b + 1) * block, :] = e4m3_encode(y)
        scales[..., b] = s
    return codes, scales


def dequantize_blocks(codes, scales, block=128):
    """x_hat = e4m3_value(code) * scale of its block, exactly, in float64."""
    vals = e4m3_value(codes)
    s = np.repeat(np.asarray(scales, dtype=np.float64), block, axis=-1)[..., :vals.shape[-2]]
    return vals * s[..., None]
