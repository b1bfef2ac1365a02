"""Pins of the oracle's fp8 quantiser with incoherent processing (oracle/quant.py):
the Hadamard matrix against scipy's and its closed form, the e4m3 rounding against
torch's cast, and the block quantisation against its defining properties and the
input generator's own (independently written) quantiser."""

import numpy as np
import pytest
import scipy.linalg
import torch

from oracle import quant as Qz
from oracle.decode import decode_bf16, decode_e4m3, dequant_blocks
from workload import gen


@pytest.mark.parametrize("d", [1, 2, 8, 64, 128])
def test_hadamard_is_sylvesters(d):
    H = Qz.hadamard(d)
    np.testing.assert_array_equal(H, scipy.linalg.hadamard(d))
    # closed form: H[i, j] = (-1)^popcount(i & j)
    i, j = np.meshgrid(np.arange(d), np.arange(d), indexing="ij")
    pc = np.vectorize(lambda x: bin(x).count("1"))(i & j) if d > 1 else np.zeros((1, 1), int)
    np.testing.assert_array_equal(H, (-1.0) ** pc)
    np.testing.assert_array_equal(H @ H.T, d * np.eye(d))


def test_signs_and_rotation():
    s = Qz.signs_from_bits([0b101, 1 << 31], 64)
    np.testing.assert_array_equal(np.nonzero(s < 0)[0], [0, 2, 63])
    assert set(np.unique(s)) == {-1.0, 1.0}
    R = Qz.rotation([0x12345678, 0x9ABCDEF0, 0x0F1E2D3C, 0x4B5A6978], 128)
    np.testing.assert_allclose(R @ R.T, np.eye(128), atol=1e-14)
    # row j of R is sign_j times row j of H over sqrt(d)
    sg = Qz.signs_from_bits([0x12345678, 0x9ABCDEF0, 0x0F1E2D3C, 0x4B5A6978], 128)
    np.testing.assert_allclose(R[5], sg[5] * scipy.linalg.hadamard(128)[5] / np.sqrt(128), rtol=0, atol=0)


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


def test_e4m3_encode_in_float64_resolves_what_fp32_cannot():
    """The definition rounds the float64 quotient: a value 2^-40 above a tie goes up,
    2^-40 below goes down, whatever fp32 would make of it."""
    srt = np.unique(np.abs(decode_e4m3(np.arange(0x7F, dtype=np.uint8))))
    mids = (srt[1:] + srt[:-1]) / 2
    up = Qz.e4m3_encode(mids * (1 + 2.0 ** -40))
    down = Qz.e4m3_encode(mids * (1 - 2.0 ** -40))
    np.testing.assert_array_equal(up.astype(int), np.arange(1, 0x7F))
    np.testing.assert_array_equal(down.astype(int), np.arange(0, 0x7E))


def test_e4m3_encode_round_trips_and_saturates():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    np.testing.assert_array_equal(Qz.e4m3_encode(decode_e4m3(codes)), codes)
    np.testing.assert_array_equal(Qz.e4m3_encode(np.array([450.0, 463.9, -455.0])), [0x7E, 0x7E, 0xFE])


def _bf16(x):
    return gen.bf16_bits_from_f32(np.asarray(x, dtype=np.float32))


def test_quantize_unrotated_equals_the_generators_quantiser():
    """Both sides take round-to-nearest-even of x / s with s = fp32(amax / 448): equal
    scales and equal codes everywhere, exact ties included (bf16 inputs and
    448 = 7 * 2^6 put many quotients exactly on an e4m3 tie)."""
    rng = np.random.default_rng(3)
    x = rng.standard_normal((2, 3, 300, 64)).astype(np.float32)
    bits = _bf16(x)
    codes, scales = Qz.quantize_blocks_ref(bits)
    gcodes, gscales = gen.quantize_e4m3_blocks(decode_bf16(bits).astype(np.float32))
    np.testing.assert_array_equal(scales, gscales)
    # (the generator writes +0 for a negative value that rounds to zero, the oracle -0)
    np.testing.assert_array_equal(decode_e4m3(codes), decode_e4m3(gcodes))
    s = np.repeat(scales, 128, axis=2)[:, :, :300, None].astype(np.float64)
    q = decode_bf16(bits) / s
    srt = np.unique(np.abs(decode_e4m3(np.arange(0x7F, dtype=np.uint8))))
    ties = np.isin(np.abs(q), (srt[1:] + srt[:-1]) / 2)
    assert ties.sum() > 50  # the exact-tie case is exercised, and both sides agree on it


def test_quantize_rotated_equals_the_generators_rotation():
    """The generator rotates with its own Hadamard construction (Kronecker products) and
    its own sign decoding; the oracle's rotated codes and scales are the same."""
    rng = np.random.default_rng(9)
    x = rng.standard_normal((1, 2, 260, 128)).astype(np.float32)
    x[..., [3, 50, 51, 90]] *= 20
    bits = _bf16(x)
    words = np.array([0x9E3779B9, 0x7F4A7C15, 0x2545F491, 0x4F6CDD1D], dtype=np.uint32)
    codes, scales = Qz.quantize_blocks_ref(bits, words)
    gcodes, gscales = gen.quantize_e4m3_blocks(decode_bf16(bits) @ gen.rotation_matrix(words, 128))
    np.testing.assert_array_equal(scales, gscales)
    np.testing.assert_array_equal(decode_e4m3(codes), decode_e4m3(gcodes))


@pytest.mark.parametrize("rotate", [False, True])
def test_quantize_block_properties(rotate):
    rng = np.random.default_rng(4)
    d = 128
    x = rng.standard_normal((1, 2, 260, d)).astype(np.float32)
    x[0, 1, 128:256] = 0.0  # an all-zero block
    bits = _bf16(x)
    sb = np.array([0x9E3779B9, 0x7F4A7C15, 0x2545F491, 0x4F6CDD1D], dtype=np.uint32) if rotate else None
    codes, scales = Qz.quantize_blocks_ref(bits, sb)
    y = decode_bf16(bits)
    if rotate:
        y = (y * Qz.signs_from_bits(sb, d)) @ scipy.linalg.hadamard(d) / np.sqrt(d)
    for b in range(2):
        for j in range(3):
            blk = y[0, b, 128 * j:128 * (j + 1)]
            c = codes[0, b, 128 * j:128 * (j + 1)]
            if not np.any(blk):
                # (+0 or -0: a sign flip of +0 gives -0)
                assert np.all(c & 0x7F == 0) and scales[0, b, j] == 1.0
                continue
            amax = np.abs(blk).max()
            assert abs(scales[0, b, j] - amax / 448) <= 2.0 ** -24 * amax / 448
            # the largest magnitude lands on +-448 (code 0x7E / 0xFE)
            i = np.unravel_index(np.argmax(np.abs(blk)), blk.shape)
            assert c[i] & 0x7F == 0x7E
            # every code is within half an e4m3 step (relative 2^-4, or 2^-10 absolute
            # in the subnormal range) of y / s, and none is nearer
            v = blk / np.float64(scales[0, b, j])
            err = np.abs(decode_e4m3(c) - v)
            assert np.all(err <= np.maximum(np.abs(v) * 2.0 ** -4, 2.0 ** -10) * (1 + 1e-12))
            allv = decode_e4m3(np.arange(0x7F, dtype=np.uint8))
            near = np.abs(np.abs(v)[..., None] - allv).min(axis=-1)
            np.testing.assert_allclose(err, near, rtol=0, atol=1e-12)


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
    R = np.diag(Qz.signs_from_bits(sb, d)) @ scipy.linalg.hadamard(d) / np.sqrt(d)
    xq, xk = decode_bf16(qb)[0, 0], decode_bf16(kb)[0, 0]
    np.testing.assert_allclose((xq @ R) @ (xk @ R).T, s_exact, rtol=1e-9, atol=1e-9)
