"""FP4 (E2M1) block encoding -- test infrastructure (see package doc).

The page "Hardware-Aware FP4 FlashAttention-4" (gist.science) describes a forward pass
whose probabilities P enter the four-bit tensor-core product directly (Direct-P, for
non-causal inference), and names MXFP4, the block-scaled four-bit format.  The format,
as the pages leave it open, is read here as follows:

  * E2M1 element: 1 sign bit, 2 exponent bits (bias 1), 1 mantissa bit, no infinity or
    NaN.  Exponent field 0 is subnormal (0 or 0.5); the finite magnitudes are
    0, 0.5, 1, 1.5, 2, 3, 4, 6.  Code = sign << 3 | exponent << 1 | mantissa.
  * Encoding of a real value: the nearest E2M1 value, ties to the even code (mantissa
    bit 0), magnitudes above 6 saturated to 6.
  * Block scale: one power of two 2^e per block of 32 values, stored as E8M0 (the byte
    e + 127, e in [-127, 127]).  e is the smallest exponent with max |x| <= 6 * 2^e, so
    the block's largest magnitude is represented without saturation (it lands in
    (3, 6] * 2^e); an all-zero block takes e = -127.  The element codes are those of
    x / 2^e.  (The OCP MX rule, e = floor(log2 max|x|) - 2, would clip the largest
    values of a block to 6 * 2^e, up to a quarter of the largest element; since P's
    largest entries carry most of a row's weight, the non-saturating choice is taken.)
  * Decoding: code value * 2^e, exact in float64.
"""

from __future__ import annotations

import math
from typing import Tuple

import numpy as np

BLOCK = 32
E2M1_MAX = 6.0


def e2m1_values() -> np.ndarray:
    """Value of each of the 16 codes (float64), from the field definitions."""
    vals = np.empty(16)
    for c in range(16):
        s, e, m = c >> 3, (c >> 1) & 3, c & 1
        mag = m * 0.5 if e == 0 else (1 + m / 2) * 2.0 ** (e - 1)
        vals[c] = -mag if s else mag
    return vals


_VALS = e2m1_values()
_POS = _VALS[:8]  # 0, 0.5, 1, 1.5, 2, 3, 4, 6 (ascending; code = index)


def e2m1_encode(x: np.ndarray) -> np.ndarray:
    """Nearest E2M1 code of each value (taken in float64), ties to the even code,
    saturating at 6; the sign bit is the sign bit of x."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), E2M1_MAX)
    hi = np.clip(np.searchsorted(_POS, a, side="left"), 0, 7)
    lo = np.maximum(hi - 1, 0)
    dlo, dhi = a - _POS[lo], _POS[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    return np.where(np.signbit(x), code | np.uint8(8), code).astype(np.uint8)


def e2m1_decode(codes: np.ndarray) -> np.ndarray:
    return _VALS[np.asarray(codes, dtype=np.uint8) & 15]


def block_exponent(amax: float) -> int:
    """Smallest e in [-127, 127] with amax <= 6 * 2^e (-127 for an all-zero block)."""
    if amax <= 0:
        return -127
    m, ex = math.frexp(amax / E2M1_MAX)  # amax / 6 = m * 2^ex, m in [0.5, 1)
    e = ex - 1 if m == 0.5 else ex
    # (amax / 6 is rounded in float64; settle the exact inequality)
    while e > -127 and amax <= E2M1_MAX * 2.0 ** (e - 1):
        e -= 1
    while amax > E2M1_MAX * 2.0 ** e:
        e += 1
    return max(-127, min(127, e))


def encode_blocks(x: np.ndarray, block: int = BLOCK) -> Tuple[np.ndarray, np.ndarray]:
    """Codes (uint8, one per value) and block exponents e (int, one per block of `block`
    consecutive values along the last axis) of x."""
    x = np.asarray(x, dtype=np.float64)
    if x.shape[-1] % block:
        raise ValueError("the last axis must hold whole blocks")
    xb = x.reshape(*x.shape[:-1], x.shape[-1] // block, block)
    amax = np.abs(xb).max(axis=-1)
    e = np.vectorize(block_exponent, otypes=[np.int64])(amax)
    codes = e2m1_encode(xb / np.exp2(e.astype(np.float64))[..., None])
    return codes.reshape(x.shape), e


def decode_blocks(codes: np.ndarray, e: np.ndarray, block: int = BLOCK) -> np.ndarray:
    c = np.asarray(codes)
    v = e2m1_decode(c).reshape(*c.shape[:-1], c.shape[-1] // block, block)
    return (v * np.exp2(np.asarray(e, dtype=np.float64))[..., None]).reshape(c.shape)
