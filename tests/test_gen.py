"""Pins for the seeded input generator (CPU)."""

import json
import os

import numpy as np
import pytest
import torch

import workload as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_bf16_rounding_matches_torch_rne():
    rng = np.random.default_rng(5)
    x = np.concatenate([
        rng.standard_normal(100000).astype(np.float32) * np.float32(10.0) ** rng.integers(-8, 8, 100000).astype(np.float32),
        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 3.4e38, -3.4e38, 1e-40], dtype=np.float32),
    ]).astype(np.float32)
    ours = W.bf16_bits_from_f32(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_e4m3_codes_match_torch_and_requantize():
    rng = np.random.default_rng(6)
    x = rng.uniform(-448, 448, 200000) * 2.0 ** rng.integers(-12, 1, 200000)
    x = x.astype(np.float32).astype(np.float64)
    ours = W.e4m3_codes_from_f64(x)
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    # torch keeps the sign of values that round to zero (-0 = 0x80); so do we only for nonzero codes
    ref = np.where((ref & 0x7F) == 0, 0, ref).astype(np.uint8)
    assert np.array_equal(ours, ref)
    # every finite code re-quantises to itself
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    vals = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    back = W.e4m3_codes_from_f64(vals)
    back_expected = np.where((codes & 0x7F) == 0, 0, codes)
    assert np.array_equal(back, back_expected)
    # saturation instead of NaN
    assert W.e4m3_codes_from_f64(np.array([1e6, -1e6]))[0] == 0x7E
    assert W.e4m3_codes_from_f64(np.array([1e6, -1e6]))[1] == 0xFE


def test_fp8_block_amax_encodes_to_max():
    p = W.make_problem(1, 2, 300, 16, dtype="fp8", seed=3, n_outliers=2)
    for t, s in ((p.q, p.q_scale), (p.k, p.k_scale), (p.v, p.v_scale)):
        assert s.shape == (1, 2, 3)
        for b in range(1):
            for h in range(2):
                for j in range(3):
                    blk = t[b, h, j * 128:(j + 1) * 128] & 0x7F
                    assert blk.max() == 0x7E


def test_doc_lengths_in_range_and_cover():
    rng = np.random.default_rng(0)
    for _ in range(50):
        L = W.draw_doc_lengths(rng, 16384, 512, 4096)
        assert sum(L) == 16384
        assert all(512 <= n <= 4096 for n in L[:-1])
        assert 1 <= L[-1] <= 4096
        ids = W.doc_ids_from_lengths(L)
        assert ids.shape == (16384,) and np.all(np.diff(ids) >= 0)


def test_config_shapes_and_flags():
    p = W.config_problem(1)
    assert (p.B, p.H, p.N, p.d, p.dtype, p.flags) == (1, 2, 256, 64, "bf16", 0)
    assert p.scale == np.float32(1 / 8)
    p4_lengths = W.draw_doc_lengths(np.random.default_rng([119, 4]), 16384, 512, 4096)
    assert sum(p4_lengths) == 16384


def test_same_seed_same_bytes_golden():
    """sha256 of generated buffers, recorded by tests/golden/make_golden.py."""
    with open(os.path.join(GOLDEN, "input_digests.json")) as f:
        gold = json.load(f)
    for name, digests in gold["small"].items():
        spec = gold["small_specs"][name]
        p = W.make_problem(**spec)
        assert p.digests() == digests, name
    p1 = W.config_problem(1)
    assert p1.digests() == gold["configs"]["1"]
    assert W.config_problem(1).digests() == p1.digests()


@pytest.mark.slow
@pytest.mark.parametrize("cfg", [2, 4])
def test_config_digests_golden(cfg):
    with open(os.path.join(GOLDEN, "input_digests.json")) as f:
        gold = json.load(f)
    assert W.config_problem(cfg).digests() == gold["configs"][str(cfg)]
