"""GPU: causal and window masks without a block map.  The forward kernel then derives
the block lists and row intervals from the flags; the outputs must be bit-identical to
the run that reads the map (itself checked against the oracle elsewhere) and match the
oracle.  Every case prints what it is before it touches the GPU."""

import numpy as np
import pytest
import torch

import oracle
import workload as W
from workload import device as WD
from exact_attention_119_amd import lib as L
from _parity import assert_close, sample_rows

pytestmark = pytest.mark.gpu

C, WI, AL, SC = W.ATTN_CAUSAL, W.ATTN_WINDOW, W.ATTN_ALIBI, W.ATTN_SOFTCAP

VARIANTS = {
    "causal": dict(flags=C),
    "window": dict(flags=C | WI, window=37),
    "window1": dict(flags=C | WI, window=1),
    "window128": dict(flags=C | WI, window=128),
    "window129": dict(flags=C | WI, window=129),
    "window_wide": dict(flags=C | WI, window=5000),
    "bidir_window": dict(flags=WI, window=50),
    "bidir_window200": dict(flags=WI, window=200),
    "alibi_causal": dict(flags=C | AL),
    "alibi_bidir_window": dict(flags=WI | AL, window=90),
    "cfg3like": dict(flags=C | WI | SC, window=100, softcap=3.0),
}


def _announce(*a):
    print("CASE", *a, flush=True)


def _both(p, **kw):
    dp = WD.to_device(p, **kw)
    outs = []
    for use_map in (True, False):
        dp.o.fill_(float("nan"))
        dp.lse.fill_(float("nan"))
        WD.step(dp, use_map=use_map)
        torch.cuda.synchronize()
        outs.append((dp.o.clone(), dp.lse.clone()))
    (o1, l1), (o2, l2) = outs
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)), "O differs between map and derived lists"
    assert torch.equal(l1.view(torch.int32), l2.view(torch.int32)), "LSE differs between map and derived lists"
    return o2.float().cpu().numpy().astype(np.float64), l2.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [1, 7, 127, 128, 129, 300, 1000])
@pytest.mark.parametrize("variant", list(VARIANTS))
def test_derived_lists_bf16(N, d, variant):
    kw = VARIANTS[variant]
    p = W.make_problem(2, 3, N, d, seed=(N, d, 40 + sorted(VARIANTS).index(variant)), **kw)
    _announce("derived bf16", variant, N, d)
    o, lse = _both(p)
    if N <= 300:
        o_ref, lse_ref = oracle.attention_problem(p)
        assert_close(p, o, lse, o_ref, lse_ref, f"derived bf16 {variant} N={N} d={d}")


@pytest.mark.parametrize("variant", ["causal", "cfg3like", "bidir_window"])
def test_derived_lists_fp8(variant):
    p = W.make_problem(1, 2, 300, 128, dtype="fp8", n_outliers=4, seed=(300, 128, 41), **VARIANTS[variant])
    _announce("derived fp8", variant)
    o, lse = _both(p)
    o_ref, lse_ref = oracle.attention_problem(p)
    assert_close(p, o, lse, o_ref, lse_ref, f"derived fp8 {variant}")


def test_derived_lists_gqa():
    p = W.make_problem(1, 8, 700, 128, flags=C | WI, window=200, seed=42, H_kv=2)
    _announce("derived gqa")
    o, lse = _both(p)
    o_ref, lse_ref = oracle.attention_problem(p)
    assert_close(p, o, lse, o_ref, lse_ref, "derived gqa")


@pytest.mark.parametrize("cfg", [2, 3])
def test_derived_lists_full_size(cfg):
    """The benchmarked configurations (causal; causal + window 1024 + softcap 50) at full
    size, in the launch the benchmark times (no map): bit-identical to the map run over every
    output, and equal to the oracle on sampled rows of every head."""
    p = W.config_problem(cfg)
    _announce("derived full size", cfg)
    o, lse = _both(p)
    rows = sample_rows(p.N, 24, seed=100 + cfg)
    heads = [(b, h) for b in range(p.B) for h in range(p.H)]
    o_ref, lse_ref = oracle.attention_problem(p, rows=rows, heads=heads, workers=8)
    assert_close(p, o[:, :, rows], lse[:, :, rows], o_ref, lse_ref, f"derived cfg{cfg} sampled")


def test_document_mask_still_needs_the_map():
    p = W.make_problem(1, 2, 300, 64, flags=C | W.ATTN_DOCUMENT, seed=43)
    _announce("document without map")
    dp = WD.to_device(p)
    with pytest.raises(L.AttnError):
        L.attn_fwd(dp.q, dp.k, dp.v, dp.o, dp.lse, scale=p.scale, mask=dp.mask, blockmap=None)
