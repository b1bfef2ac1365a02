"""GPU parity: the HIP path (through the C ABI) against the fp64 CPU oracle on the
same seeded inputs.  Every case prints what it is before it touches the GPU."""

import numpy as np
import pytest
import torch

import oracle
import workload as W
from workload import device as WD
from exact_attention_119_amd import lib as L
from _parity import assert_close, check_work_order, errors, sample_rows

pytestmark = pytest.mark.gpu

C, WI, DOC, AL, SC = W.ATTN_CAUSAL, W.ATTN_WINDOW, W.ATTN_DOCUMENT, W.ATTN_ALIBI, W.ATTN_SOFTCAP

VARIANTS = {
    "plain": dict(flags=0),
    "causal": dict(flags=C),
    "window": dict(flags=C | WI, window=37),
    "bidir_window": dict(flags=WI, window=50),
    "doc": dict(flags=DOC),
    "doc_causal": dict(flags=C | DOC),
    "alibi_causal": dict(flags=C | AL),
    "alibi": dict(flags=AL),
    "softcap": dict(flags=SC, softcap=2.0),
    # (cap 50: every step on the polynomial; cap 8: scores past 4 send some steps to the
    # exact formula; causal so that masked steps and both paths meet)
    "softcap50": dict(flags=C | SC, softcap=50.0),
    "softcap8": dict(flags=C | SC, softcap=8.0),
    "cfg3like": dict(flags=C | WI | SC, window=100, softcap=3.0),
    "cfg4like": dict(flags=C | DOC | AL),
    "everything": dict(flags=C | WI | DOC | AL | SC, window=70, softcap=2.5),
}


def _announce(*a):
    print("CASE", *a, flush=True)


def _run(p, tau=8.0, pv_mode=L.ATTN_PV_F16, qk_mode=L.ATTN_QK_BF16):
    dp = WD.to_device(p, pv_mode=pv_mode, qk_mode=qk_mode)
    dp.o.fill_(float("nan"))
    dp.lse.fill_(float("nan"))
    WD.step(dp, rescale_tau=tau)
    o, lse = WD.outputs(dp)
    return dp, o, lse


def _check_map(dp, rows=None):
    """The device block map equals the oracle's byte for byte (batch rows `rows`)."""
    p = dp.p
    got = L.read_blockmap(dp.blockmap, p.B, p.N)
    ref = oracle.blockmap_ref(p.B, p.N, p.flags & L.POSITIONAL, p.window, p.doc_id)
    hd = got["header"]
    assert (hd["magic"], hd["B"], hd["N"], hd["flags"], hd["window"]) == \
        (0x39313141, p.B, p.N, p.flags & L.POSITIONAL, p.window if p.flags & L.ATTN_WINDOW else 0)
    np.testing.assert_array_equal(got["status"], ref["status"], err_msg="status")
    # the work order ranks the device's counts of every batch row (an invalid row's
    # counts are unspecified) by the cost the map states
    check_work_order(got["order"], got["counts"], hd, bool(p.flags & L.ATTN_DOCUMENT))
    sel = slice(None) if rows is None else rows
    for key in ("cls", "counts", "idx", "row_lo", "row_hi", "col_lo", "col_hi"):
        np.testing.assert_array_equal(got[key][sel], ref[key][sel], err_msg=key)
    np.testing.assert_array_equal(got["pairs"][sel], ref["qb_pairs"][sel])
    return ref


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [1, 7, 65, 127, 129, 300])
@pytest.mark.parametrize("variant", list(VARIANTS))
def test_small_shapes_bf16(N, d, variant):
    kw = VARIANTS[variant]
    p = W.make_problem(2, 3, N, d, seed=(N, d, sorted(VARIANTS).index(variant)),
                       doc_len_range=(1, max(1, N // 2)), **kw)
    _announce("bf16", variant, N, d)
    dp, o, lse = _run(p)
    if p.flags & L.POSITIONAL:
        _check_map(dp)
    o_ref, lse_ref = oracle.attention_problem(p)
    assert_close(p, o, lse, o_ref, lse_ref, f"bf16 {variant} N={N} d={d}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [7, 129, 300])
@pytest.mark.parametrize("variant", ["plain", "causal", "cfg4like", "cfg3like"])
def test_small_shapes_fp8(N, d, variant):
    kw = VARIANTS[variant]
    p = W.make_problem(1, 2, N, d, dtype="fp8", n_outliers=4, seed=(N, d, 8), **kw)
    _announce("fp8", variant, N, d)
    dp, o, lse = _run(p)
    o_ref, lse_ref = oracle.attention_problem(p)
    assert_close(p, o, lse, o_ref, lse_ref, f"fp8 {variant} N={N} d={d}")


_QK8_CASES = [(v, r) for v in ("plain", "causal", "window", "cfg4like", "cfg3like", "softcap")
              for r in ("map", "derived") if r == "map" or v in ("causal", "window", "cfg3like")]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [7, 300, 1000])
@pytest.mark.parametrize("variant,route", _QK8_CASES)
def test_small_shapes_fp8_qk_on_fp8_mfma_without_outliers(N, d, variant, route):
    """Q.K^T on the e4m3 MFMA (the pipelined kernel's QK8 path).  Its accumulation keeps
    about 14 bits below the largest product; on inputs without outlier channels the scores
    stay O(1) and that error is far inside the fp8 tolerances.  Causal and window masks
    also without a block map (block lists derived in the kernel)."""
    kw = VARIANTS[variant]
    p = W.make_problem(1, 2, N, d, dtype="fp8", n_outliers=0, seed=(N, d, 9), **kw)
    _announce("fp8 qk8", variant, N, d, route)
    dp = WD.to_device(p, qk_mode=L.ATTN_QK_E4M3)
    dp.o.fill_(float("nan"))
    dp.lse.fill_(float("nan"))
    WD.step(dp, use_map=route == "map")
    o, lse = WD.outputs(dp)
    o_ref, lse_ref = oracle.attention_problem(p)
    assert_close(p, o, lse, o_ref, lse_ref, f"fp8-qk8 {variant} N={N} d={d} {route}")


def test_cfg1_full():
    p = W.config_problem(1)
    _announce("cfg1 full")
    dp, o, lse = _run(p)
    o_ref, lse_ref = oracle.attention_problem(p)
    assert_close(p, o, lse, o_ref, lse_ref, "cfg1")


@pytest.mark.parametrize("variant", ["causal", "cfg4like", "softcap"])
def test_tau_zero_and_eight_agree(variant):
    p = W.make_problem(1, 4, 700, 128, seed=5, **VARIANTS[variant])
    _announce("tau", variant)
    _, o8, l8 = _run(p, tau=8.0)
    _, o0, l0 = _run(p, tau=0.0)
    o_ref, lse_ref = oracle.attention_problem(p)
    assert_close(p, o8, l8, o_ref, lse_ref, "tau=8")
    assert_close(p, o0, l0, o_ref, lse_ref, "tau=0")
    e_o, _, e_l = errors(o8, l8, o0, l0)
    assert e_o <= 2e-2 and e_l <= 1e-3


def test_outputs_fully_written_and_deterministic():
    p = W.make_problem(2, 4, 1000, 128, flags=C | DOC | AL, seed=6, doc_len_range=(50, 400))
    _announce("determinism")
    dp = WD.to_device(p)
    dp.o.fill_(float("nan"))
    dp.lse.fill_(float("nan"))
    WD.step(dp)
    torch.cuda.synchronize()
    o1, l1 = dp.o.clone(), dp.lse.clone()
    assert not torch.isnan(o1.float()).any() and not torch.isnan(l1).any()
    for _ in range(3):
        WD.step(dp)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), dp.o.view(torch.int16))
    assert torch.equal(l1.view(torch.int32), dp.lse.view(torch.int32))


def test_decreasing_doc_id_is_reported_and_poisons_its_batch_row():
    p = W.make_problem(2, 2, 300, 64, flags=C | DOC, seed=7)
    p.doc_id[1, 150:] = 0  # batch row 1: ids go back down
    _announce("bad doc ids")
    dp, o, lse = _run(p)
    ref = _check_map(dp, rows=[0])
    assert ref["status"][1].any() and not ref["status"][0].any()
    assert L.attn_blockmap_status(dp.blockmap) == L.ATTN_ERR_BAD_DOC_ID
    assert np.isnan(lse[1]).all() and np.isnan(o[1]).all()
    o_ref, lse_ref = oracle.attention_problem(p, heads=[(0, 0), (0, 1)])
    assert_close(p, o[:1], lse[:1], o_ref[:1], lse_ref[:1], "good batch row")


@pytest.mark.parametrize("cfg", [2, 3, 4, 5])
def test_config_full_size_sampled(cfg):
    p = W.config_problem(cfg)
    _announce("config", cfg)
    dp, o, lse = _run(p)
    if p.flags & L.POSITIONAL:
        ref = _check_map(dp)
        pairs = ref["visible_pairs"]
    else:
        pairs = p.B * p.N * p.N
    print(f"cfg{cfg}: visible pairs per head {pairs // p.B if p.B == 1 else pairs}", flush=True)
    rows = sample_rows(p.N, 48, seed=cfg)
    heads = [(b, h) for b in range(p.B) for h in range(p.H)]
    o_ref, lse_ref = oracle.attention_problem(p, rows=rows, heads=heads, workers=8)
    e = assert_close(p, o[:, :, rows], lse[:, :, rows], o_ref, lse_ref, f"cfg{cfg} sampled")
    if p.dtype == "fp8":
        oc = np.setdiff1d(np.arange(p.d), p.outlier_channels)
        raw_non_outlier = float(np.max(np.abs(o[:, :, rows][..., oc] - o_ref[..., oc])))
        print(f"cfg5 raw max|dO| {e[0]:.3e}, on non-outlier channels {raw_non_outlier:.3e}", flush=True)


_QK8_LSE_REASON = (
    "gfx950's f8f6f4 MFMA truncates a 64-term dot product at about 2^-14 of its largest product "
    "(measured); configuration 5's x20 channels give |LSE| ~ 600 with the dominant scores sums of "
    "a few dozen large products, so the LSE error is ~1e-2 of those products' unit: 6.6e-2 on the "
    "literal codes, 2.7e-3 with incoherent processing, above the 1e-3 gate in both")


def _cfg5_qk8(rotate):
    p = W.config_problem(5, rotate=rotate)
    _announce("cfg5 qk8", "rotated" if rotate else "literal")
    dp, o, lse = _run(p, qk_mode=L.ATTN_QK_E4M3)
    rows = sample_rows(p.N, 32, seed=55)
    heads = [(0, h) for h in range(p.H)]
    o_ref, lse_ref = oracle.attention_problem(p, rows=rows, heads=heads, workers=8)
    e_o, e_ob, e_l = errors(o[:, :, rows], lse[:, :, rows], o_ref, lse_ref)
    print(f"cfg5 qk8 {'rotated' if rotate else 'literal'}: max|dO|={e_o:.3e} beyond-half-ulp={e_ob:.3e} "
          f"max|dLSE|={e_l:.3e} max|LSE|={np.abs(lse_ref).max():.1f}", flush=True)
    return e_ob, e_l


@pytest.mark.parametrize("rotate", [
    pytest.param(False, marks=pytest.mark.xfail(reason="the literal x20 channels: " + _QK8_LSE_REASON, strict=True)),
    True], ids=["literal", "rotated"])
def test_cfg5_qk_on_fp8_mfma_output_within_6e2(rotate):
    """Configuration 5 with Q.K^T on the e4m3 MFMA: O within 6e-2 beyond the bf16 output's own
    rounding.  With incoherent processing (Q and K quantised after the rotation R, the FA3
    page's remedy for outlier features; the oracle runs on the same rotated codes) the
    largest products of a score shrink and O meets the gate; on the literal codes it does
    not."""
    e_ob, _ = _cfg5_qk8(rotate)
    assert e_ob <= 6e-2


@pytest.mark.xfail(reason=_QK8_LSE_REASON, strict=False)
@pytest.mark.parametrize("rotate", [False, True], ids=["literal", "rotated"])
def test_cfg5_qk_on_fp8_mfma_lse_within_1e3(rotate):
    """The LSE gate of the fp8 path (1e-3) for Q.K^T on the e4m3 MFMA at configuration 5."""
    _, e_l = _cfg5_qk8(rotate)
    assert e_l <= 1e-3


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("variant", ["plain", "causal", "cfg3like", "cfg4like"])
def test_fp8_block_scales_spread(d, variant):
    """K and V block scales spread over 2^-3 .. 2^3 between 128-row blocks (the codes are
    kept; the oracle dequantises with the new scales): every key block's K scale must reach
    its own scores and its V scale its own P units, with and without threshold rescaling."""
    kw = VARIANTS[variant]
    p = W.make_problem(1, 2, 1000, d, dtype="fp8", seed=(d, 11, sorted(VARIANTS).index(variant)),
                       doc_len_range=(100, 400), **kw)
    rng = np.random.default_rng([119, 11, d, sorted(VARIANTS).index(variant)])
    p.k_scale = (p.k_scale * 2.0 ** rng.integers(-3, 4, p.k_scale.shape)).astype(np.float32)
    p.v_scale = (p.v_scale * 2.0 ** rng.integers(-3, 4, p.v_scale.shape)).astype(np.float32)
    o_ref, lse_ref = oracle.attention_problem(p)
    for tau in (8.0, 0.0):
        _announce("fp8 spread scales", variant, d, tau)
        _, o, lse = _run(p, tau=tau)
        assert_close(p, o, lse, o_ref, lse_ref, f"fp8 spread scales {variant} d={d} tau={tau}")


def test_work_order_beyond_one_chunk():
    """Document masks with 1152 (batch row, query block) entries: the order kernel streams
    the work values through LDS in chunks of 1024, so the second chunk is exercised.  The
    order sorts the device's counts by the map's stated cost, the counts equal the oracle's, and
    the forward pass that takes its row blocks in that order writes every output and
    matches the oracle on sampled rows."""
    p = W.make_problem(9, 2, 16384, 64, flags=C | DOC, seed=77, doc_len_range=(300, 5000))
    _announce("work order, 1152 entries")
    dp, o, lse = _run(p)
    got = L.read_blockmap(dp.blockmap, p.B, p.N)
    check_work_order(got["order"], got["counts"], got["header"], True)
    for b in (0, 8):
        ref = oracle.blockmap_ref(1, p.N, p.flags & L.POSITIONAL, 0, p.doc_id[b:b + 1])
        np.testing.assert_array_equal(got["counts"][b], ref["counts"][0], err_msg=f"counts of batch row {b}")
    assert not np.isnan(o).any() and not np.isnan(lse).any()
    rows = sample_rows(p.N, 12, seed=77)
    heads = [(b, h) for b in (0, 4, 8) for h in range(p.H)]
    o_ref, lse_ref = oracle.attention_problem(p, rows=rows, heads=heads, workers=8)
    sel_o = np.stack([o[b, h][rows] for b, h in heads]).reshape(3, p.H, len(rows), p.d)
    sel_l = np.stack([lse[b, h][rows] for b, h in heads]).reshape(3, p.H, len(rows))
    ref_o = np.stack([o_ref[b, h] for b, h in heads]).reshape(3, p.H, len(rows), p.d)
    ref_l = np.stack([lse_ref[b, h] for b, h in heads]).reshape(3, p.H, len(rows))
    assert_close(p, sel_o, sel_l, ref_o, ref_l, "work order beyond one chunk")
