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

Steps for one (batch, head, block of 128 rows), in the precision the quantiser
works in (fp32: the codes are integer decisions, so this side takes them in the
same precision as the device):
  1. x: the bf16 rows, widened exactly to fp32; with rotation x <- x * signs.
  2. with rotation: y = x H by the fast Walsh-Hadamard transform in fp32, stages
     of stride 1, 2, 4, ..., d/2, each mapping the pair (x[i], x[i+h]) of every
     2h-aligned group to (x[i] + x[i+h], x[i] - x[i+h]); without: y = x.
  3. amax = max |y| over the block; s = fp32(amax / 448) and g = fp32(448 / amax),
     both 1 for an all-zero block.
  4. code = the e4m3 value nearest to fp32(y * g), ties to the even code,
     magnitudes above 448 saturated to 448 (a multiplication by the block's inverse
     scale, the usual form of block quantisation; y * g and y / s can differ in the
     last fp32 bit, and so, at an e4m3 tie, in the code).
  5. stored scale: s * fp32(1/sqrt(d)) (fp32 product) with rotation, else s, so
     that code * scale approximates x R (or x).
"""

from __future__ import annotations

from typing import Optional, Tuple

import numpy as np

from .decode import decode_bf16, decode_e4m3

E4M3_MAX = np.float32(448.0)
BLOCK = 128


def fwht_f32(x: np.ndarray) -> np.ndarray:
    """Fast Walsh-Hadamard transform along the last axis (length a power of two), in
    float32, stages of stride 1, 2, ..., d/2 (step 2 above).  Returns x H (Sylvester)."""
    y = np.array(x, dtype=np.float32, copy=True)
    d = y.shape[-1]
    if d & (d - 1):
        raise ValueError("length must be a power of two")
    lead = y.shape[:-1]
    h = 1
    while h < d:
        g = y.reshape(*lead, d // (2 * h), 2, h)
        a, b = g[..., 0, :], g[..., 1, :]
        y = np.stack([a + b, a - b], axis=-2).reshape(*lead, d)
        h *= 2
    return y


def signs_from_bits(bits, d: int) -> np.ndarray:
    """+-1 float32 [d]: element j is negated when bit j % 32 of word j // 32 is set."""
    words = np.asarray(bits, dtype=np.uint64)
    j = np.arange(d)
    neg = (words[j // 32] >> (j % 32).astype(np.uint64)) & np.uint64(1)
    return np.where(neg == 1, np.float32(-1.0), np.float32(1.0)).astype(np.float32)


def _e4m3_finite_nonneg() -> Tuple[np.ndarray, np.ndarray]:
    """All finite non-negative e4m3 values, ascending, with their codes (0x00..0x7E)."""
    codes = np.arange(0x7F, dtype=np.uint8)
    return decode_e4m3(codes), codes


_VALS, _CODES = _e4m3_finite_nonneg()


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    """Nearest e4m3 code to each float32 value, ties to the even code (mantissa LSB 0),
    magnitudes above 448 saturated; the sign bit is the sign bit of v (step 4)."""
    v = np.asarray(v, dtype=np.float32)
    a = np.minimum(np.abs(v).astype(np.float64), 448.0)
    hi = np.clip(np.searchsorted(_VALS, a, side="left"), 0, len(_VALS) - 1)
    lo = np.maximum(hi - 1, 0)
    dlo, dhi = a - _VALS[lo], _VALS[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (_CODES[hi] % 2 == 0))
    code = np.where(pick_hi, _CODES[hi], _CODES[lo]).astype(np.uint8)
    neg = np.signbit(v)
    return np.where(neg, code | np.uint8(0x80), code).astype(np.uint8)


def quantize_blocks_ref(x_bits: np.ndarray, sign_bits: Optional[np.ndarray] = None,
                        block: int = BLOCK) -> Tuple[np.ndarray, np.ndarray]:
    """Codes uint8 [B][H][N][d] and stored scales float32 [B][H][ceil(N/block)] of bf16
    rows x_bits [B][H][N][d] (bit patterns), with incoherent processing when sign_bits
    (d/32 words) is given."""
    x = decode_bf16(x_bits).astype(np.float32)
    B, H, N, d = x.shape
    if sign_bits is not None:
        x = fwht_f32(x * signs_from_bits(sign_bits, d))
    nblk = (N + block - 1) // block
    codes = np.empty(x.shape, dtype=np.uint8)
    scales = np.empty((B, H, nblk), dtype=np.float32)
    rnorm = np.float32(1.0 / np.sqrt(np.float64(d)))
    for j in range(nblk):
        r0, r1 = j * block, min(N, (j + 1) * block)
        y = x[:, :, r0:r1, :]
        amax = np.abs(y).max(axis=(2, 3))
        s = np.where(amax > 0, amax / E4M3_MAX, np.float32(1.0)).astype(np.float32)
        with np.errstate(divide="ignore"):
            g = np.where(amax > 0, E4M3_MAX / amax, np.float32(1.0)).astype(np.float32)
        codes[:, :, r0:r1, :] = e4m3_encode(y * g[:, :, None, None])
        scales[:, :, j] = (s * rnorm).astype(np.float32) if sign_bits is not None else s
    return codes, scales
