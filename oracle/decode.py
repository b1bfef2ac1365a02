"""Storage formats -> float64, exactly.  Test infrastructure (see package doc).

bf16 is the upper half of an IEEE-754 binary32, so widening is exact.  The
fp8 inputs are OCP E4M3FN codes (1 sign, 4 exponent bits with bias 7, 3
mantissa bits, subnormals, no infinities, S.1111.111 = NaN) times one fp32
scale per (batch, head, 128-row block) -- the block quantisation named in the
FlashAttention-3 news (ctol-digital.de), section "Analyse".  Code times scale
is exact in float64.
"""

from __future__ import annotations

import numpy as np


def decode_bf16(bits: np.ndarray) -> np.ndarray:
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def _e4m3_table() -> np.ndarray:
    tab = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        exp = (code >> 3) & 0xF
        man = code & 0x7
        if exp == 0xF and man == 0x7:
            tab[code] = np.nan
        elif exp == 0:
            tab[code] = sign * (man / 8.0) * 2.0 ** (1 - 7)
        else:
            tab[code] = sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)
    return tab


_E4M3 = _e4m3_table()


def decode_e4m3(codes: np.ndarray) -> np.ndarray:
    return _E4M3[np.asarray(codes, dtype=np.uint8)]


def dequant_blocks(codes: np.ndarray, scales: np.ndarray, block: int = 128) -> np.ndarray:
    """codes uint8 [B][H][N][d], scales fp32 [B][H][ceil(N/block)] -> float64 values."""
    x = decode_e4m3(codes)
    N = x.shape[2]
    row_scale = np.repeat(np.asarray(scales, dtype=np.float64), block, axis=2)[:, :, :N]
    return x * row_scale[..., None]


def decode_problem(p):
    """(Q, K, V) as float64 [B][H][N][d] for a workload.Problem."""
    if p.dtype == "bf16":
        return decode_bf16(p.q), decode_bf16(p.k), decode_bf16(p.v)
    if p.dtype == "fp8":
        return (dequant_blocks(p.q, p.q_scale), dequant_blocks(p.k, p.k_scale),
                dequant_blocks(p.v, p.v_scale))
    raise ValueError(p.dtype)
