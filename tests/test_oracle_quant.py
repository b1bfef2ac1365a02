"""Pins of the oracle's fp8 quantiser with incoherent processing (oracle/quant.py):
the transform against the Hadamard matrix, the e4m3 rounding against torch's cast,
and the block quantisation against its defining properties and the input generator's
own (independent) quantiser."""

import numpy as np
import pytest
import scipy.linalg
import torch

from oracle import quant as Qz
from oracle.decode import decode_bf16, decode_e4m3, dequant_blocks
from workload import gen


@pytest.mark.parametrize("d", [2, 8, 64, 128])
def test_fwht_is_the_sylvester_hadamard_product(d):
    rng = np.random.default_rng(d)
    x = rng.standard_normal((5, d)).astype(np.float32)
    H = scipy.linalg.hadamard(d).astype(np.float64)
    y64 = x.astype(np.float64) @ H
    y = Qz.fwht_f32(x)
    assert y.dtype == np.float32
    bound = np.log2(d) * 2.0 ** -23 * np.abs(x).astype(np.float64).sum(axis=1, keepdims=True)
    assert np.all(np.abs(y - y64) <= bound)
    # unit vectors give the rows of H exactly
    np.testing.assert_array_equal(Qz.fwht_f32(np.eye(d, dtype=np.float32)), H)


def test_fwht_twice_is_d_times_identity_and_keeps_the_norm():
    rng = np.random.default_rng(1)
    x = rng.integers(-8, 9, (7, 128)).astype(np.float32)
    np.testing.assert_array_equal(Qz.fwht_f32(Qz.fwht_f32(x)), 128 * x)
    y = Qz.fwht_f32(x)
    np.testing.assert_allclose((y.astype(np.float64) ** 2).sum(1), 128 * (x.astype(np.float64) ** 2).sum(1))


def test_signs_from_bits():
    s = Qz.signs_from_bits([0b101, 1 << 31], 64)
    neg = np.nonzero(s < 0)[0]
    np.testing.assert_array_equal(neg, [0, 2, 63])
    assert set(np.unique(s)) == {-1.0, 1.0}


def test_e4m3_encode_matches_torch_cast():
    rng = np.random.default_rng(2)
    mags = np.exp(rng.uniform(np.log(2.0 ** -12), np.log(448.0), 200000)).astype(np.float32)
    v = mags * rng.choice([-1.0, 1.0], mags.shape).astype(np.float32)
    exact = decode_e4m3(np.arange(256, dtype=np.uint8))
    finite = exact[np.isfinite(exact)].astype(np.float32)
    srt = np.unique(np.abs(finite).astype(np.float64))
    mids = ((srt[1:] + srt[:-1]) / 2).astype(np.float32)  # exact in fp32: ties
    v = np.concatenate([v, finite, mids, -mids, np.float32([0.0, -0.0])])
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(Qz.e4m3_encode(v), ref)


def test_e4m3_encode_round_trips_and_saturates():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    np.testing.assert_array_equal(Qz.e4m3_encode(decode_e4m3(codes).astype(np.float32)), codes)
    np.testing.assert_array_equal(Qz.e4m3_encode(np.float32([450.0, 463.9, -455.0])), [0x7E, 0x7E, 0xFE])


def _bf16(x):
    return gen.bf16_bits_from_f32(np.asarray(x, dtype=np.float32))


def test_quantize_unrotated_agrees_with_the_generators_quantiser():
    """The input generator quantises with an fp64 division; this side multiplies by the
    fp32 inverse scale.  With bf16 inputs and 448 = 7 * 2^6 the exact quotient often
    lies at or next to an e4m3 tie: only there may the two differ, by one code."""
    rng = np.random.default_rng(3)
    x = rng.standard_normal((2, 3, 300, 64)).astype(np.float32)
    bits = _bf16(x)
    codes, scales = Qz.quantize_blocks_ref(bits)
    gcodes, gscales = gen.quantize_e4m3_blocks(decode_bf16(bits).astype(np.float32))
    np.testing.assert_array_equal(scales, gscales)
    diff = decode_e4m3(codes) != decode_e4m3(gcodes)
    assert diff.mean() < 1e-3
    s = np.repeat(scales, 128, axis=2)[:, :, :300, None]
    v64 = (decode_bf16(bits) / s.astype(np.float64))[diff]
    a, b = decode_e4m3(codes)[diff], decode_e4m3(gcodes)[diff]
    tie = (a + b) / 2
    assert np.all(np.abs(v64 - tie) <= np.abs(tie) * 2.0 ** -21)  # within fp32 rounding of a tie
    assert np.all(np.abs(codes.astype(int)[diff] - gcodes.astype(int)[diff]) == 1)


@pytest.mark.parametrize("rotate", [False, True])
def test_quantize_block_properties(rotate):
    rng = np.random.default_rng(4)
    d = 128
    x = rng.standard_normal((1, 2, 260, d)).astype(np.float32)
    x[0, 1, 128:256] = 0.0  # an all-zero block
    bits = _bf16(x)
    sb = np.array([0x9E3779B9, 0x7F4A7C15, 0x2545F491, 0x4F6CDD1D], dtype=np.uint32) if rotate else None
    codes, scales = Qz.quantize_blocks_ref(bits, sb)
    rnorm = np.float32(1 / np.sqrt(d))
    y = decode_bf16(bits)
    if rotate:
        y = (y * Qz.signs_from_bits(sb, d)) @ scipy.linalg.hadamard(d)
    for b in range(2):
        for j in range(3):
            blk = y[0, b, 128 * j:128 * (j + 1)]
            c = codes[0, b, 128 * j:128 * (j + 1)]
            s = scales[0, b, j] / (rnorm if rotate else 1)
            if not np.any(blk):
                # (+0 or -0: a sign flip of +0 gives -0)
                assert np.all(c & 0x7F == 0) and scales[0, b, j] == (rnorm if rotate else 1.0)
                continue
            # the largest magnitude lands on +-448 (code 0x7E / 0xFE)
            i = np.unravel_index(np.argmax(np.abs(blk)), blk.shape)
            assert c[i] & 0x7F == 0x7E
            # every code is within half an e4m3 step (relative 2^-4, or 2^-10 absolute
            # in the subnormal range) of y * 448 / amax
            v = blk * 448.0 / np.abs(blk).max()
            err = np.abs(decode_e4m3(c) - v)
            assert np.all(err <= np.maximum(np.abs(v) * 2.0 ** -4, 2.0 ** -10) * 1.0001)


def test_rotation_keeps_scores_and_reduces_the_outlier_error():
    """Same signs on Q and K: the dequantised products approximate Q.K^T, and with four
    channels x20 (outlier features) the rotated codes give the smaller score error."""
    rng = np.random.default_rng(5)
    d, N = 128, 256
    q = rng.standard_normal((1, 1, N, d)).astype(np.float32)
    k = rng.standard_normal((1, 1, N, d)).astype(np.float32)
    ch = rng.choice(d, 4, replace=False)
    q[..., ch] *= 20
    k[..., ch] *= 20
    qb, kb = _bf16(q), _bf16(k)
    s_exact = decode_bf16(qb)[0, 0] @ decode_bf16(kb)[0, 0].T
    sb = np.array([0x12345678, 0x9ABCDEF0, 0x0F1E2D3C, 0x4B5A6978], dtype=np.uint32)
    err = {}
    for rot in (None, sb):
        qc, qs = Qz.quantize_blocks_ref(qb, rot)
        kc, ks = Qz.quantize_blocks_ref(kb, rot)
        s = dequant_blocks(qc, qs)[0, 0] @ dequant_blocks(kc, ks)[0, 0].T
        err[rot is not None] = np.abs(s - s_exact).mean()
    assert err[True] < 0.5 * err[False]
    # without quantisation the rotation is exact: (x R)(y R)^T = x y^T
    R = np.diag(Qz.signs_from_bits(sb, d).astype(np.float64)) @ scipy.linalg.hadamard(d) / np.sqrt(d)
    xq, xk = decode_bf16(qb)[0, 0], decode_bf16(kb)[0, 0]
    np.testing.assert_allclose((xq @ R) @ (xk @ R).T, s_exact, rtol=1e-9, atol=1e-9)
