"""Seeded input generator for the attention forward pass.

Workloads are the five synthetic configurations of the exact-attention forward
(see CONFIGS).  The pages name no public dataset; the only statement about the
data that they make is that FP8 attention has to cope with outlier features
(FlashAttention-3 news, ctol-digital.de, section "Analyse"), which config 5
models with four channels scaled by 20.

Recipe, fixed so that both sides of the parity check see identical bytes:
  * RNG: numpy PCG64 via ``np.random.default_rng([119, cfg])`` for preset cfg,
    ``np.random.default_rng([119, 1000, seed])`` for ad-hoc shapes.
  * Draw order: document lengths (if any), outlier channels (if any), then Q, K
    and V, each ``standard_normal(shape, float32)``.
  * bf16 inputs: fp32 -> bf16 with round-to-nearest-even on the bit pattern.
  * fp8 inputs: per (b, h, 128-row block) scale = amax / 448 in fp32 (1.0 for
    an all-zero block), code = OCP E4M3FN round-to-nearest-even of
    x / scale, saturated to +-448.  Dequantised value = code value * scale.
  * fp8 inputs with incoherent processing (``rotate=True``; the FlashAttention-3
    news, section "Analyse", names a processing step against outlier features,
    read as incoherent processing): after V, d/32 sign words are drawn with
    ``rng.integers(0, 2**32)``; Q and K (their fp32 values, in float64) are
    multiplied by R = D H / sqrt(d) (D the signs, bit j % 32 of word j // 32 set
    = -1; H the Sylvester Hadamard matrix) before the block quantisation above,
    whose maximum is then taken in float64 and rounded to fp32 after the
    division by 448.  V is not rotated.  Q.K^T is unchanged by R up to the
    quantisation, so the attention of the rotated codes approximates that of the
    source values.
  * Documents: lengths drawn uniformly from [lo, hi] (inclusive) until they
    cover N; the last one is truncated.  Ids 0, 1, 2, ... in token order.
"""

from __future__ import annotations

import dataclasses
import hashlib
import math
from typing import List, Optional, Sequence, Tuple, Union

import numpy as np

# Mask / score-modifier flag bits.  The same values are part of the C ABI.
ATTN_CAUSAL = 1
ATTN_WINDOW = 2
ATTN_DOCUMENT = 4
ATTN_ALIBI = 8
ATTN_SOFTCAP = 16

QUANT_BLOCK = 128  # rows per fp8 scale block
E4M3_MAX = 448.0

CONFIGS = {
    1: "B=1 H=2 N=256 d=64 bf16, no mask, scale 1/8",
    2: "B=4 H=16 N=2048 d=128 bf16, causal, scale 1/sqrt(128)",
    3: "B=2 H=32 N=8192 d=128 bf16, causal + window 1024 + tanh softcap 50",
    4: "B=1 H=16 N=16384 d=128 bf16, document-causal (doc lengths U[512,4096]) + ALiBi",
    5: "B=1 H=16 N=16384 d=128 fp8 e4m3 (per 128-row block scales, 4 outlier channels x20), no mask",
}


@dataclasses.dataclass
class Problem:
    """One attention-forward problem instance, in storage formats.

    q: uint16 bf16 bit patterns, or uint8 E4M3FN codes, shape [B][H][N][d]; k, v the
    same with H_kv heads ([B][H_kv][N][d]; H_kv = H unless set, H_kv divides H).
    q_scale: float32 [B][H][ceil(N/128)], k_scale/v_scale [B][H_kv][...] for fp8, else None.
    doc_id: int32 [B][N] (non-decreasing per batch row) when the DOCUMENT flag is set.
    alibi_slopes: float32 [H] or None (None = the default geometric slopes).
    """

    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str
    flags: int
    window: int
    softcap: float
    scale: float
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    q_scale: Optional[np.ndarray] = None
    k_scale: Optional[np.ndarray] = None
    v_scale: Optional[np.ndarray] = None
    doc_id: Optional[np.ndarray] = None
    doc_lengths: Optional[List[List[int]]] = None
    outlier_channels: Optional[np.ndarray] = None
    alibi_slopes: Optional[np.ndarray] = None
    H_kv: Optional[int] = None
    cu_seqlens: Optional[np.ndarray] = None  # packed variable-length batch (B = 1): int32 [nseq + 1]
    rotate_signs: Optional[np.ndarray] = None  # uint32 [d/32]: Q and K codes are of x R (incoherent processing)

    @property
    def Hkv(self) -> int:
        """Key/value heads (grouped-query attention when below H)."""
        return self.H if self.H_kv is None else self.H_kv

    def digests(self) -> dict:
        """sha256 of every generated buffer (hex)."""
        out = {}
        for key in ("q", "k", "v", "q_scale", "k_scale", "v_scale", "doc_id", "cu_seqlens", "rotate_signs"):
            arr = getattr(self, key)
            if arr is not None:
                out[key] = hashlib.sha256(np.ascontiguousarray(arr).tobytes()).hexdigest()
        return out

    @property
    def nblk(self) -> int:
        return (self.N + QUANT_BLOCK - 1) // QUANT_BLOCK


# --------------------------------------------------------------------------
# Storage-format encoders
# --------------------------------------------------------------------------

def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest, ties to even (no NaN input)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32).astype(np.uint64)
    bias = np.uint64(0x7FFF) + ((bits >> np.uint64(16)) & np.uint64(1))
    return ((bits + bias) >> np.uint64(16)).astype(np.uint16)


def _e4m3_positive_table() -> np.ndarray:
    """Values of the 127 non-negative finite E4M3FN codes 0x00..0x7E.

    OCP 8-bit floating point, E4M3 flavour: 4 exponent bits (bias 7), 3
    mantissa bits, subnormals at exponent field 0, no infinities, only
    S.1111.111 is NaN.  Largest finite value 1.75 * 2^8 = 448.
    """
    vals = np.empty(127, dtype=np.float64)
    for c in range(127):
        e, m = c >> 3, c & 7
        vals[c] = m * 2.0 ** -9 if e == 0 else (8 + m) * 2.0 ** (e - 10)
    return vals


_E4M3_POS = _e4m3_positive_table()


def e4m3_codes_from_f64(x: np.ndarray) -> np.ndarray:
    """Encode real values as E4M3FN codes: round to nearest, ties to even code,
    saturating to +-448 (never NaN)."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), E4M3_MAX)
    hi = np.searchsorted(_E4M3_POS, a, side="left")  # first value >= a
    hi = np.clip(hi, 0, 126)
    lo = np.clip(hi - 1, 0, 126)
    d_lo = a - _E4M3_POS[lo]
    d_hi = _E4M3_POS[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    sign = (np.signbit(x) & (code > 0)).astype(np.uint8) << 7
    return (code | sign).astype(np.uint8)


def quantize_e4m3_blocks(x: np.ndarray, block: int = QUANT_BLOCK) -> Tuple[np.ndarray, np.ndarray]:
    """Per (b, h, row block) E4M3 quantisation of x[B][H][N][d] (fp32, or float64 values
    such as rotated rows: then the maximum is taken in float64 and amax / 448 rounded to fp32).

    Returns (codes uint8 [B][H][N][d], scales float32 [B][H][ceil(N/block)]).
    """
    wide = np.asarray(x).dtype == np.float64
    x = np.asarray(x, dtype=np.float64 if wide else np.float32)
    B, H, N, d = x.shape
    nblk = (N + block - 1) // block
    scales = np.empty((B, H, nblk), dtype=np.float32)
    codes = np.empty(x.shape, dtype=np.uint8)
    for j in range(nblk):
        r0, r1 = j * block, min(N, (j + 1) * block)
        blk = x[:, :, r0:r1, :]
        if wide:
            amax = np.abs(blk).max(axis=(2, 3))
            s = np.where(amax > 0, amax / E4M3_MAX, 1.0).astype(np.float32)
        else:
            amax = np.abs(blk).max(axis=(2, 3)).astype(np.float32)
            s = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
        scales[:, :, j] = s
        codes[:, :, r0:r1, :] = e4m3_codes_from_f64(
            blk.astype(np.float64) / s.astype(np.float64)[:, :, None, None])
    return codes, scales


def sylvester_hadamard(d: int) -> np.ndarray:
    """Sylvester Hadamard matrix of order d (a power of two) as float64, by Kronecker
    products of [[1, 1], [1, -1]]."""
    h = np.ones((1, 1))
    while h.shape[0] < d:
        h = np.kron(np.array([[1.0, 1.0], [1.0, -1.0]]), h)
    if h.shape[0] != d:
        raise ValueError("order must be a power of two")
    return h


def rotation_matrix(sign_words: np.ndarray, d: int) -> np.ndarray:
    """R = D H / sqrt(d) for sign words (bit j % 32 of word j // 32 set: D[j] = -1)."""
    w = np.asarray(sign_words, dtype=np.uint64)
    j = np.arange(d)
    neg = ((w[j // 32] >> (j % 32).astype(np.uint64)) & np.uint64(1)).astype(bool)
    signs = np.where(neg, -1.0, 1.0)
    return (signs[:, None] * sylvester_hadamard(d)) / math.sqrt(d)


# --------------------------------------------------------------------------
# Documents
# --------------------------------------------------------------------------

def draw_doc_lengths(rng: np.random.Generator, N: int, lo: int, hi: int) -> List[int]:
    """Integer lengths uniform on [lo, hi] until they cover N; last one truncated."""
    lengths: List[int] = []
    total = 0
    while total < N:
        n = int(rng.integers(lo, hi + 1))
        n = min(n, N - total)
        lengths.append(n)
        total += n
    return lengths


def doc_ids_from_lengths(lengths: Sequence[int]) -> np.ndarray:
    return np.repeat(np.arange(len(lengths), dtype=np.int32), np.asarray(lengths, dtype=np.int64))


# --------------------------------------------------------------------------
# Problems
# --------------------------------------------------------------------------

def _f32(x: float) -> float:
    return float(np.float32(x))


def _build(name, rng, B, H, N, d, dtype, flags, window, softcap, scale, doc_lengths, n_outliers,
           outlier_gain, alibi_slopes=None, H_kv=None, rotate=False) -> Problem:
    doc_id = None
    if doc_lengths is not None:
        doc_id = np.stack([doc_ids_from_lengths(doc_lengths[b]) for b in range(B)]).astype(np.int32)
    outl = None
    if n_outliers:
        outl = np.sort(rng.choice(d, n_outliers, replace=False)).astype(np.int64)
    Hkv = H if H_kv is None else H_kv
    if Hkv < 1 or H % Hkv:
        raise ValueError(f"{H} query heads cannot share {Hkv} key/value heads")
    xs = []
    for shape in ((B, H, N, d), (B, Hkv, N, d), (B, Hkv, N, d)):
        x = rng.standard_normal(shape, dtype=np.float32)
        if outl is not None:
            x[..., outl] *= np.float32(outlier_gain)
        xs.append(x)
    kw = dict(name=name, B=B, H=H, N=N, d=d, dtype=dtype, flags=flags, window=window,
              softcap=_f32(softcap), scale=_f32(scale), doc_id=doc_id, outlier_channels=outl,
              doc_lengths=None if doc_lengths is None else [list(map(int, l)) for l in doc_lengths],
              alibi_slopes=alibi_slopes, H_kv=H_kv)
    if dtype == "bf16":
        return Problem(q=bf16_bits_from_f32(xs[0]), k=bf16_bits_from_f32(xs[1]),
                       v=bf16_bits_from_f32(xs[2]), **kw)
    if dtype == "fp8":
        signs = None
        if rotate:
            signs = rng.integers(0, 2 ** 32, size=(d + 31) // 32, dtype=np.uint64).astype(np.uint32)
            R = rotation_matrix(signs, d)
            xs[0] = xs[0].astype(np.float64) @ R
            xs[1] = xs[1].astype(np.float64) @ R
        (qc, qs), (kc, ks), (vc, vs) = (quantize_e4m3_blocks(x) for x in xs)
        return Problem(q=qc, k=kc, v=vc, q_scale=qs, k_scale=ks, v_scale=vs, rotate_signs=signs, **kw)
    if rotate:
        raise ValueError("incoherent processing applies to fp8 inputs")
    raise ValueError(f"unknown dtype {dtype!r}")


def config_problem(cfg: int, rotate: bool = False) -> Problem:
    """The five synthetic workloads, drawn with ``default_rng([119, cfg])``; ``rotate``
    (configuration 5 only) quantises Q and K after the rotation R (incoherent processing),
    the same draws otherwise."""
    if rotate and cfg != 5:
        raise ValueError("only the fp8 configuration has a rotated form")
    rng = np.random.default_rng([119, cfg])
    if cfg == 1:
        return _build("cfg1", rng, 1, 2, 256, 64, "bf16", 0, 0, 0.0, 1.0 / 8.0, None, 0, 1.0)
    if cfg == 2:
        return _build("cfg2", rng, 4, 16, 2048, 128, "bf16", ATTN_CAUSAL, 0, 0.0,
                      1.0 / math.sqrt(128), None, 0, 1.0)
    if cfg == 3:
        return _build("cfg3", rng, 2, 32, 8192, 128, "bf16", ATTN_CAUSAL | ATTN_WINDOW | ATTN_SOFTCAP,
                      1024, 50.0, 1.0 / math.sqrt(128), None, 0, 1.0)
    if cfg == 4:
        lengths = draw_doc_lengths(rng, 16384, 512, 4096)
        return _build("cfg4", rng, 1, 16, 16384, 128, "bf16", ATTN_CAUSAL | ATTN_DOCUMENT | ATTN_ALIBI,
                      0, 0.0, 1.0 / math.sqrt(128), [lengths], 0, 1.0)
    if cfg == 5:
        return _build("cfg5-rot" if rotate else "cfg5", rng, 1, 16, 16384, 128, "fp8", 0, 0, 0.0,
                      1.0 / math.sqrt(128), None, 4, 20.0, rotate=rotate)
    raise ValueError(f"no config {cfg}")


def make_problem(B: int, H: int, N: int, d: int, *, dtype: str = "bf16", flags: int = 0,
                 window: int = 0, softcap: float = 0.0, scale: Optional[float] = None,
                 seed: Union[int, Tuple[int, ...]] = 0,
                 doc_len_range: Optional[Tuple[int, int]] = None, n_outliers: int = 0,
                 outlier_gain: float = 20.0, alibi_slopes: Optional[np.ndarray] = None,
                 H_kv: Optional[int] = None, rotate: bool = False) -> Problem:
    """An ad-hoc problem of any shape, drawn with ``default_rng([119, 1000, *seed])``;
    H_kv key/value heads shared by groups of H / H_kv query heads (default H_kv = H);
    ``rotate`` (fp8): Q and K quantised after the rotation R (incoherent processing)."""
    seed_t = (seed,) if isinstance(seed, int) else tuple(seed)
    rng = np.random.default_rng([119, 1000, *seed_t])
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    doc_lengths = None
    if flags & ATTN_DOCUMENT:
        lo, hi = doc_len_range if doc_len_range is not None else (max(1, N // 8), max(1, N // 3))
        doc_lengths = [draw_doc_lengths(rng, N, lo, hi) for _ in range(B)]
    if alibi_slopes is not None:
        alibi_slopes = np.asarray(alibi_slopes, dtype=np.float32)
    name = f"B{B}H{H}N{N}d{d}" + ("" if H_kv is None else f"Hkv{H_kv}")
    return _build(name + ("-rot" if rotate else ""), rng, B, H, N, d, dtype, flags, window, softcap, scale,
                  doc_lengths, n_outliers, outlier_gain, alibi_slopes, H_kv, rotate)


def make_varlen_problem(lengths: Sequence[int], H: int, d: int, *, dtype: str = "bf16", flags: int = 0,
                        window: int = 0, softcap: float = 0.0, scale: Optional[float] = None,
                        seed: Union[int, Tuple[int, ...]] = 0, n_outliers: int = 0, outlier_gain: float = 20.0,
                        alibi_slopes: Optional[np.ndarray] = None, H_kv: Optional[int] = None) -> Problem:
    """A packed variable-length batch: sequences of the given lengths (zeros allowed)
    back to back in one batch row of N = sum(lengths) tokens, drawn with
    ``default_rng([119, 2000, *seed])``; cu_seqlens = [0, l0, l0 + l1, ...]."""
    if flags & ATTN_DOCUMENT:
        raise ValueError("the sequences of a packed batch are its documents")
    lengths = [int(x) for x in lengths]
    if not lengths or min(lengths) < 0 or sum(lengths) < 1:
        raise ValueError("need at least one token")
    seed_t = (seed,) if isinstance(seed, int) else tuple(seed)
    rng = np.random.default_rng([119, 2000, *seed_t])
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if alibi_slopes is not None:
        alibi_slopes = np.asarray(alibi_slopes, dtype=np.float32)
    N = sum(lengths)
    name = f"varlen{len(lengths)}H{H}N{N}d{d}" + ("" if H_kv is None else f"Hkv{H_kv}")
    p = _build(name, rng, 1, H, N, d, dtype, flags, window, softcap, scale, None, n_outliers, outlier_gain,
               alibi_slopes, H_kv)
    p.cu_seqlens = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    return p


def make_dout(p: Problem, seed: Union[int, Tuple[int, ...]] = 0) -> np.ndarray:
    """bf16 output gradients [B][H][N][d] for a problem's backward pass, drawn N(0, 1) with
    ``default_rng([119, 3000, *seed])``."""
    seed_t = (seed,) if isinstance(seed, int) else tuple(seed)
    rng = np.random.default_rng([119, 3000, *seed_t])
    return bf16_bits_from_f32(rng.standard_normal((p.B, p.H, p.N, p.d), dtype=np.float32))
