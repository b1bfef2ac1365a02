"""FP8 block quantisation with incoherent processing -- test infrastructure (see
package doc).

The FlashAttention-3 news (ctol-digital.de, section "Analyse") names two ways its
FP8 path keeps accuracy with outlier features: block quantisation, and a
processing step whose name the page garbles ("inkorrekte Verarbeitung"); it is
read here as FlashAttention-3's incoherent processing: Q and K are multiplied by
the same random orthogonal matrix before they are quantised, which leaves Q.K^T
unchanged and spreads a large channel over all channels.  The orthogonal matrix
is R = D H / sqrt(d): D a diagonal of random signs (given as input), H the
Sylvester Walsh-Hadamard matrix of order d.

The definition, for one (batch, head, block of 128 rows), in float64 (the
plain reading of block quantisation: one scale per block, the codes the
nearest e4m3 values of x / scale):
  1. x: the bf16 rows, widened exactly; with rotation y = x R (a matrix product
     in float64), without y = x.
  2. amax = max |y| over the block; s = amax / 448 rounded to fp32 (the stored
     scale), 1 for an all-zero block.
  3. code = the e4m3 value nearest to y / s (float64 quotient), ties to the even
     code, magnitudes above 448 saturated to 448; the sign is the sign of y.
So code * s approximates x R (or x).  No evaluation order of the transform is
part of the definition: an implementation that computes y in lower precision
can differ from these codes only where y / s lies within its rounding error of
an e4m3 tie (by one code), and from these scales by its rounding of amax.
"""

from __future__ import annotations

from typing import Optional, Tuple

import numpy as np

from .decode import decode_bf16, decode_e4m3

E4M3_MAX = 448.0
BLOCK = 128


def hadamard(d: int) -> np.ndarray:
    """Sylvester Walsh-Hadamard matrix of order d (a power of two), float64:
    H_1 = [1], H_2n = [[H_n, H_n], [H_n, -H_n]]."""
    if d < 1 or d & (d - 1):
        raise ValueError("order must be a power of two")
    h = np.ones((1, 1))
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    return h


def signs_from_bits(bits, d: int) -> np.ndarray:
    """+-1 float64 [d]: element j is negated when bit j % 32 of word j // 32 is set."""
    words = np.asarray(bits, dtype=np.uint64)
    j = np.arange(d)
    neg = (words[j // 32] >> (j % 32).astype(np.uint64)) & np.uint64(1)
    return np.where(neg == 1, -1.0, 1.0)


def rotation(bits, d: int) -> np.ndarray:
    """R = D H / sqrt(d), float64 [d][d] (orthogonal)."""
    return signs_from_bits(bits, d)[:, None] * hadamard(d) / np.sqrt(d)


def _e4m3_finite_nonneg() -> Tuple[np.ndarray, np.ndarray]:
    """All finite non-negative e4m3 values, ascending, with their codes (0x00..0x7E)."""
    codes = np.arange(0x7F, dtype=np.uint8)
    return decode_e4m3(codes), codes


_VALS, _CODES = _e4m3_finite_nonneg()


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    """Nearest e4m3 code to each real value (taken in float64), ties to the even code
    (mantissa LSB 0), magnitudes above 448 saturated; the sign bit is the sign bit of v."""
    v = np.asarray(v, dtype=np.float64)
    a = np.minimum(np.abs(v), E4M3_MAX)
    hi = np.clip(np.searchsorted(_VALS, a, side="left"), 0, len(_VALS) - 1)
    lo = np.maximum(hi - 1, 0)
    dlo, dhi = a - _VALS[lo], _VALS[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (_CODES[hi] % 2 == 0))
    code = np.where(pick_hi, _CODES[hi], _CODES[lo]).astype(np.uint8)
    return np.where(np.signbit(v), code | np.uint8(0x80), code).astype(np.uint8)


def quantize_blocks_ref(x_bits: np.ndarray, sign_bits: Optional[np.ndarray] = None,
                        block: int = BLOCK) -> Tuple[np.ndarray, np.ndarray]:
    """Codes uint8 [B][H][N][d] and scales float32 [B][H][ceil(N/block)] of bf16 rows
    x_bits [B][H][N][d] (bit patterns), with incoherent processing when sign_bits (d/32
    words) is given (steps 1-3 of the module doc)."""
    y = decode_bf16(x_bits)
    B, H, N, d = y.shape
    if sign_bits is not None:
        y = y @ rotation(sign_bits, d)
    nblk = (N + block - 1) // block
    codes = np.empty(y.shape, dtype=np.uint8)
    scales = np.empty((B, H, nblk), dtype=np.float32)
    for j in range(nblk):
        r0, r1 = j * block, min(N, (j + 1) * block)
        blk = y[:, :, r0:r1, :]
        amax = np.abs(blk).max(axis=(2, 3))
        s = np.where(amax > 0, amax / E4M3_MAX, 1.0).astype(np.float32)
        codes[:, :, r0:r1, :] = e4m3_encode(blk / s.astype(np.float64)[:, :, None, None])
        scales[:, :, j] = s
    return codes, scales
