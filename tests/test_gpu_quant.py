"""GPU parity for the device fp8 quantiser (attn_fp8_quantize): codes and scales bit for
bit against the oracle's quantiser, with and without incoherent processing, and the
attention pass on the device's codes against the oracle's pass on the oracle's codes."""

import numpy as np
import pytest
import torch

import oracle
import workload as W
from oracle import quant as Qz
from exact_attention_119_amd import lib as L
from _parity import assert_close, errors

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


@pytest.mark.parametrize("rotate", [False, True])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("shape", [(1, 2, 300), (2, 3, 1), (1, 1, 129), (1, 4, 1000)])
def test_codes_and_scales_bit_exact(shape, d, rotate):
    B, H, N = shape
    p = W.make_problem(B, H, N, d, n_outliers=4, outlier_gain=20.0, seed=(B, H, N, d))
    bits = p.q.copy()
    if N > 256:
        bits[0, 0, 128:256] = 0  # an all-zero block
    signs = SIGNS[d] if rotate else None
    _announce("quant", shape, d, rotate)
    codes, scales = _quantize(bits, signs)
    ref_c, ref_s = Qz.quantize_blocks_ref(bits, None if signs is None else np.array(signs, np.uint32))
    np.testing.assert_array_equal(scales.cpu().numpy().view(np.uint32), ref_s.view(np.uint32))
    np.testing.assert_array_equal(codes.cpu().numpy(), ref_c)


def test_full_size_rotated_bit_exact():
    """B1 H16 N16384 d128 (the fp8 workload's shape), four channels x20, rotated."""
    p = W.make_problem(1, 16, 16384, 128, n_outliers=4, outlier_gain=20.0, seed=55)
    _announce("quant full size")
    codes, scales = _quantize(p.q, SIGNS[128])
    ref_c, ref_s = Qz.quantize_blocks_ref(p.q, np.array(SIGNS[128], np.uint32))
    np.testing.assert_array_equal(scales.cpu().numpy().view(np.uint32), ref_s.view(np.uint32))
    np.testing.assert_array_equal(codes.cpu().numpy(), ref_c)


@pytest.mark.parametrize("flags", [0, W.ATTN_CAUSAL])
def test_quantised_attention_and_the_rotation_gain(flags):
    """Q, K rotated with the same signs and V plain, then the fp8 pass: parity against
    the oracle's pass on the oracle's own codes, and a smaller error against the exact
    bf16 attention than the same pipeline without rotation (outlier channels x20)."""
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
        # the oracle's pass on its own codes
        ref = {}
        for name, x, s in (("q", p.q, sg), ("k", p.k, sg), ("v", p.v, None)):
            ref[name] = Qz.quantize_blocks_ref(x, None if s is None else np.array(s, np.uint32))
        pq = W.gen.Problem(name="quantised", B=1, H=4, N=p.N, d=128, dtype="fp8", flags=flags, window=0,
                           softcap=0.0, scale=p.scale, q=ref["q"][0], k=ref["k"][0], v=ref["v"][0],
                           q_scale=ref["q"][1], k_scale=ref["k"][1], v_scale=ref["v"][1])
        o_ref, l_ref = oracle.attention_problem(pq)
        assert_close(pq, o_np, l_np, o_ref, l_ref, f"quantised attention rotate={rotate}")
        errs[rotate] = errors(o_np, l_np, exact_o, exact_l)
        print(f"rotate={rotate}: vs exact bf16 attention max|dO| {errs[rotate][0]:.3e} "
              f"max|dLSE| {errs[rotate][2]:.3e}", flush=True)
    assert errs[True][2] < errs[False][2]
