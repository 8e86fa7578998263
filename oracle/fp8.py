"""OCP FP8 E4M3 ("E4M3FN") codec used by the oracle.  Test infrastructure only.

The quantized attention path stores P~ and V as FP8 E4M3 (page "SageAttention2: Efficient
Attention with Thorough Outlier Smoothing and Per-thread INT4 Quantization", mlsanity.com,
section "Abstract (arXiv)"; page pith.science verdict on arXiv 2505.21136, key
"key_machinery", which gives the per-channel V scale max|V|/V_r and the P scale max(P~)/P_r).
The pages do not spell out the bit format or the rounding; the oracle reads them as:

* format: sign bit, 4 exponent bits (bias 7), 3 mantissa bits, subnormals, no infinities, the
  single NaN pattern S.1111.111 per sign, largest finite magnitude 448 (= 1.75 * 2**8);
* rounding: IEEE round-to-nearest, ties to the even code (mantissa LSB 0);
* overflow: saturating, |x| >= 448 encodes as +-448 (the quantizers never produce values
  beyond 448 by more than an fp32 rounding step, so this only matters at the edge);
* the sign of zero is kept: negative values that round to zero encode as 0x80.

Nothing here is shared with, or imported by, the GPU path.
"""

from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
NAN_CODE = 0x7F


def _decode_scalar(code: int) -> float:
    sign = -1.0 if code & 0x80 else 1.0
    exp = (code >> 3) & 0xF
    man = code & 0x7
    if exp == 0xF and man == 0x7:
        return float("nan")
    if exp == 0:
        return sign * man * 2.0 ** -9          # subnormal: m/8 * 2**(1-7)
    return sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)


#: decoded value of every byte, float64 (exact)
DECODE_TABLE = np.array([_decode_scalar(c) for c in range(256)], dtype=np.float64)

# the 127 finite non-negative codes 0x00..0x7E are increasing in value
_POS_VALUES = DECODE_TABLE[:0x7F].copy()
assert np.all(np.diff(_POS_VALUES) > 0)


def decode(codes: np.ndarray) -> np.ndarray:
    """FP8 E4M3 bytes -> float64 values (exact)."""
    return DECODE_TABLE[np.asarray(codes, dtype=np.uint8)]


def encode_sat(x: np.ndarray) -> np.ndarray:
    """float32/float64 values -> FP8 E4M3 bytes, RNE, saturating at +-448.

    The input is taken at its own precision (callers pass values already rounded to fp32
    where the method rounds to fp32 first).
    """
    x = np.asarray(x, dtype=np.float64)
    neg = np.signbit(x)
    a = np.abs(x)
    nan = np.isnan(x)
    a = np.where(nan, 0.0, a)
    # index of the largest representable value <= a
    lo = np.searchsorted(_POS_VALUES, a, side="right") - 1
    lo = np.clip(lo, 0, 0x7E)
    hi = np.minimum(lo + 1, 0x7E)
    vlo = _POS_VALUES[lo]
    vhi = _POS_VALUES[hi]
    dlo = a - vlo
    dhi = vhi - a
    # nearest; on an exact tie pick the even code
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0) & (hi != lo))
    code = np.where(pick_hi, hi, lo)
    code = np.where(a >= E4M3_MAX, 0x7E, code)
    code = code.astype(np.uint8) | np.where(neg, 0x80, 0).astype(np.uint8)
    code = np.where(nan, NAN_CODE, code).astype(np.uint8)
    return code


def round_sat(x: np.ndarray) -> np.ndarray:
    """Value of encode_sat(x), as float64."""
    return decode(encode_sat(x))
