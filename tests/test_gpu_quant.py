"""GPU parity for the device fp8 quantiser (attn_fp8_quantize): codes and scales against
the oracle's fp64 definition, with and without incoherent processing (equal except where
the device's fp32 rounding meets an e4m3 tie, counted and bounded), and the device
pipeline's rotation gain on outlier channels."""

import numpy as np
import pytest
import torch

import oracle
import workload as W
from oracle import quant as Qz
from exact_attention_119_amd import lib as L
from _parity import errors

pytestmark = pytest.mark.gpu

SIGNS = {64: [0x9E3779B9, 0x7F4A7C15], 128: [0x9E3779B9, 0x7F4A7C15, 0x2545F491, 0x4F6CDD1D]}


def _announce(*a):
    print("CASE", *a, flush=True)


def _quantize(bits, signs):
    """Device codes and scales of bf16 bit patterns [B][H][N][d] (numpy)."""
    B, H, N, d = bits.shape
    x = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)
    codes = torch.full((B, H, N, d), 0x7F, dtype=torch.uint8, device="cuda")  # NaN codes until written
    scales = torch.full((B, H, (N + 127) // 128), float("nan"), dtype=torch.float32, device="cuda")
    L.attn_fp8_quantize(x, codes, scales, signs)
    torch.cuda.synchronize()
    return codes, scales


def _tie_table():
    vals = np.unique(np.abs(oracle.decode_e4m3(np.arange(0x7F, dtype=np.uint8))))
    return (vals[1:] + vals[:-1]) / 2


TIES = _tie_table()


def compare_with_definition(bits, signs, codes, scales, what):
    """Device codes and scales against the oracle's fp64 definition (RNE of y / s with
    s = fp32(amax / 448), y = x R).  The device computes y in fp32 (a fast transform)
    and multiplies by the fp32 inverse scale, so it may differ from the definition only
    within its rounding error: scales within the transform's error bound on amax plus
    three fp32 roundings (bit-exact without rotation), and a code by one step only where
    y / s lies within that error of an e4m3 tie.  Those exceptions are counted, printed
    and bounded."""
    B, H, N, d = bits.shape
    words = None if signs is None else np.array(signs, np.uint32)
    ref_c, ref_s = Qz.quantize_blocks_ref(bits, words)
    x = oracle.decode_bf16(bits)
    y = x @ Qz.rotation(words, d) if words is not None else x
    got_c, got_s = codes.cpu().numpy(), scales.cpu().numpy()
    nb = (N + 127) // 128
    rows = lambda a: np.repeat(a, 128, axis=2)[:, :, :N]  # noqa: E731
    if words is None:
        np.testing.assert_array_equal(got_s.view(np.uint32), ref_s.view(np.uint32), err_msg=what)
        rel_s = np.zeros((B, H, nb))
        abs_y = np.zeros(x.shape)
    else:
        # fp32 fast transform: |error| <= log2(d) 2^-23 sum|x| per output (unnormalised)
        row_bound = np.log2(d) * 2.0 ** -23 * np.abs(x).sum(axis=-1, keepdims=True) / np.sqrt(d)
        abs_y = np.broadcast_to(row_bound, x.shape)
        blk_bound = np.array([row_bound[:, :, 128 * j:128 * (j + 1)].max(axis=(2, 3)) for j in range(nb)])
        amax = np.array([np.abs(y[:, :, 128 * j:128 * (j + 1)]).max(axis=(2, 3)) for j in range(nb)])
        rel_s = (np.where(amax > 0, blk_bound / np.where(amax > 0, amax, 1), 0) + 4 * 2.0 ** -24)
        rel_s = np.moveaxis(rel_s, 0, -1)
        err_s = np.abs(got_s.astype(np.float64) - ref_s) / ref_s
        assert np.all(err_s <= rel_s), f"{what}: scale error {err_s.max():.3e} beyond its bound"
    s = rows(ref_s.astype(np.float64))[..., None]
    q = y / s
    tol = abs_y / s + np.abs(q) * (rows(rel_s)[..., None] + 4 * 2.0 ** -24)
    dv, rv = oracle.decode_e4m3(got_c), oracle.decode_e4m3(ref_c)
    mism = dv != rv
    n = int(mism.sum())
    print(f"{what}: {n} of {mism.size} codes differ from the definition (near-tie exceptions)", flush=True)
    if words is None:
        # the input itself is y: the device resolves every tie from the exact residual
        np.testing.assert_array_equal(dv, rv, err_msg=f"{what}: codes")
    if n:
        qa = np.abs(q[mism])
        dist = np.abs(qa[:, None] - TIES[None, :]).min(axis=1)
        assert np.all(dist <= tol[mism]), f"{what}: a code differs away from an e4m3 tie"
        gm, rm = got_c[mism].astype(int), ref_c[mism].astype(int)
        same_sign = ((gm ^ rm) & 0x80) == 0
        assert np.all(same_sign & (np.abs((gm & 0x7F) - (rm & 0x7F)) == 1)), f"{what}: not one code apart"
        assert n <= 4 + 1e-5 * mism.size, f"{what}: too many tie exceptions"


@pytest.mark.parametrize("rotate", [False, True])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("shape", [(1, 2, 300), (2, 3, 1), (1, 1, 129), (1, 4, 1000), (1, 5, 16647)])
def test_codes_and_scales_against_the_definition(shape, d, rotate):
    """(1, 5, 16647): 655 blocks, more than the grid's workgroups, so workgroups take
    a second block, and a last block of 7 rows."""
    B, H, N = shape
    p = W.make_problem(B, H, N, d, n_outliers=4, outlier_gain=20.0, seed=(B, H, N, d))
    bits = p.q.copy()
    if N > 256:
        bits[0, 0, 128:256] = 0  # an all-zero block
    signs = SIGNS[d] if rotate else None
    _announce("quant", shape, d, rotate)
    codes, scales = _quantize(bits, signs)
    compare_with_definition(bits, signs, codes, scales, f"quant {shape} d={d} rotate={rotate}")


def test_full_size_rotated_against_the_definition():
    """B1 H16 N16384 d128 (the fp8 workload's shape), four channels x20, rotated."""
    p = W.make_problem(1, 16, 16384, 128, n_outliers=4, outlier_gain=20.0, seed=55)
    _announce("quant full size")
    codes, scales = _quantize(p.q, SIGNS[128])
    compare_with_definition(p.q, SIGNS[128], codes, scales, "quant full size rotated")


@pytest.mark.parametrize("flags", [0, W.ATTN_CAUSAL])
def test_quantised_attention_and_the_rotation_gain(flags):
    """The device pipeline -- Q, K quantised on the device with the same signs, V plain,
    then the fp8 pass -- against the exact bf16 attention of the source values: with
    four channels x20 (outlier features) the rotated codes give the smaller error.  (The
    quantiser's codes and the fp8 pass are each held to the oracle separately; a code
    one step off at a tie moves a score by up to a step of that element, so the two
    pipelines are compared with the exact attention, not with each other.)"""
    p = W.make_problem(1, 4, 1024, 128, n_outliers=4, outlier_gain=20.0, seed=(7, flags), flags=flags)
    _announce("quantised attention", flags)
    exact_o, exact_l = oracle.attention_ref(*oracle.decode_problem(p), scale=p.scale, flags=flags)
    mask = L.make_mask(flags) if flags else None
    mp = None
    if flags:
        mp = torch.empty(L.attn_blockmap_bytes(1, p.N, mask), dtype=torch.uint8, device="cuda")
        L.attn_blockmap_build(1, p.N, mask, mp)
    errs = {}
    for rotate in (False, True):
        sg = SIGNS[128] if rotate else None
        (qc, qs), (kc, ks), (vc, vs) = _quantize(p.q, sg), _quantize(p.k, sg), _quantize(p.v, None)
        o = torch.full((1, 4, p.N, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
        lse = torch.full((1, 4, p.N), float("nan"), dtype=torch.float32, device="cuda")
        L.attn_fwd(qc, kc, vc, o, lse, scale=p.scale, dtype=L.ATTN_FP8_E4M3, mask=mask, blockmap=mp,
                   fp8=L.make_fp8(qs, ks, vs))
        torch.cuda.synchronize()
        o_np, l_np = o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)
        errs[rotate] = errors(o_np, l_np, exact_o, exact_l)
        print(f"rotate={rotate}: vs exact bf16 attention max|dO| {errs[rotate][0]:.3e} "
              f"max|dLSE| {errs[rotate][2]:.3e}", flush=True)
    assert errs[True][2] < errs[False][2]
