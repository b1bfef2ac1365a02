"""GPU parity for grouped-query attention (GQA; MQA when one key/value head serves all
query heads): the HIP path through attn_fwd_gqa against the fp64 oracle, and against
the same library's plain multi-head call on key/value heads repeated per group."""

import dataclasses

import numpy as np
import pytest

import oracle
import workload as W
from workload import device as WD
from exact_attention_119_amd import lib as L
from _parity import assert_close, sample_rows

pytestmark = pytest.mark.gpu

C, WI, DOC, AL, SC = W.ATTN_CAUSAL, W.ATTN_WINDOW, W.ATTN_DOCUMENT, W.ATTN_ALIBI, W.ATTN_SOFTCAP

VARIANTS = {
    "plain": dict(flags=0),
    "causal": dict(flags=C),
    "window": dict(flags=C | WI, window=37),
    "alibi_causal": dict(flags=C | AL),
    "cfg3like": dict(flags=C | WI | SC, window=100, softcap=3.0),
    "cfg4like": dict(flags=C | DOC | AL),
}
HEADS = [(8, 2), (6, 1), (4, 4)]


def _announce(*a):
    print("CASE", *a, flush=True)


def _run_gqa(p, tau=8.0, qk_mode=L.ATTN_QK_BF16):
    """Stage, build the map, and call attn_fwd_gqa (also when H_kv = H)."""
    dp = WD.to_device(p, qk_mode=qk_mode)
    assert tuple(dp.k.shape) == (p.B, p.Hkv, p.N, p.d) and tuple(dp.q.shape) == (p.B, p.H, p.N, p.d)
    dp.o.fill_(float("nan"))
    dp.lse.fill_(float("nan"))
    WD.build_map(dp)
    L.attn_fwd_gqa(dp.q, dp.k, dp.v, dp.o, dp.lse, scale=p.scale, dtype=dp.dtype, mask=dp.mask,
                   blockmap=dp.blockmap, fp8=dp.fp8, rescale_tau=tau)
    o, lse = WD.outputs(dp)
    return dp, o, lse


def _repeat_kv(p):
    """The same problem with every key/value head written out once per query head."""
    g = p.H // p.Hkv
    rep = lambda a: None if a is None else np.ascontiguousarray(np.repeat(a, g, axis=1))
    return dataclasses.replace(p, k=rep(p.k), v=rep(p.v), k_scale=rep(p.k_scale), v_scale=rep(p.v_scale),
                               H_kv=None)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("heads", HEADS, ids=lambda t: f"H{t[0]}kv{t[1]}")
@pytest.mark.parametrize("variant", list(VARIANTS))
def test_grouped_heads_bf16(variant, heads, d):
    H, Hkv = heads
    p = W.make_problem(2, H, 300, d, seed=(H, Hkv, d, sorted(VARIANTS).index(variant)),
                       doc_len_range=(20, 150), H_kv=Hkv, **VARIANTS[variant])
    _announce("gqa bf16", variant, H, Hkv, d)
    _, o, lse = _run_gqa(p)
    o_ref, lse_ref = oracle.attention_problem(p)
    assert_close(p, o, lse, o_ref, lse_ref, f"gqa bf16 {variant} H={H} H_kv={Hkv} d={d}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("heads", [(8, 2), (4, 1)], ids=lambda t: f"H{t[0]}kv{t[1]}")
@pytest.mark.parametrize("variant", ["plain", "causal", "cfg4like"])
def test_grouped_heads_fp8(variant, heads, d):
    H, Hkv = heads
    p = W.make_problem(1, H, 300, d, dtype="fp8", n_outliers=4, seed=(H, Hkv, d, 8), H_kv=Hkv,
                       doc_len_range=(20, 150), **VARIANTS[variant])
    _announce("gqa fp8", variant, H, Hkv, d)
    _, o, lse = _run_gqa(p)
    o_ref, lse_ref = oracle.attention_problem(p)
    assert_close(p, o, lse, o_ref, lse_ref, f"gqa fp8 {variant} H={H} H_kv={Hkv} d={d}")


@pytest.mark.parametrize("variant", ["plain", "causal"])
def test_grouped_heads_fp8_qk_on_fp8_mfma(variant):
    p = W.make_problem(1, 8, 300, 128, dtype="fp8", n_outliers=0, seed=(8, 2, 9), H_kv=2,
                       **VARIANTS[variant])
    _announce("gqa fp8 qk8", variant)
    _, o, lse = _run_gqa(p, qk_mode=L.ATTN_QK_E4M3)
    o_ref, lse_ref = oracle.attention_problem(p)
    assert_close(p, o, lse, o_ref, lse_ref, f"gqa fp8-qk8 {variant}")


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("variant", ["causal", "cfg3like"])
def test_grouped_heads_bit_identical_to_repeated_heads(variant, dtype):
    """Each query head does the same arithmetic on the same key/value values whether its
    key/value head is shared or a private copy, so the outputs agree bit for bit."""
    p = W.make_problem(2, 8, 700, 128, dtype=dtype, seed=(8, 2, 700), H_kv=2, **VARIANTS[variant])
    _announce("gqa vs repeated", variant, dtype)
    _, o, lse = _run_gqa(p)
    pr = _repeat_kv(p)
    dpr = WD.to_device(pr)
    WD.step(dpr)
    o_r, lse_r = WD.outputs(dpr)
    np.testing.assert_array_equal(o, o_r)
    np.testing.assert_array_equal(lse, lse_r)


def _run_gqa_derived(p, tau=8.0):
    """attn_fwd_gqa without a block map: the kernel derives the causal block lists (the
    route the benchmark and map-less callers take)."""
    dp = WD.to_device(p)
    dp.o.fill_(float("nan"))
    dp.lse.fill_(float("nan"))
    L.attn_fwd_gqa(dp.q, dp.k, dp.v, dp.o, dp.lse, scale=p.scale, dtype=dp.dtype, mask=dp.mask,
                   blockmap=None, fp8=dp.fp8, rescale_tau=tau)
    o, lse = WD.outputs(dp)
    return dp, o, lse


@pytest.mark.parametrize("route", ["map", "derived"])
@pytest.mark.parametrize("shape", [(1, 32, 8), (1, 16, 2), (3, 12, 4)], ids=lambda t: f"B{t[0]}H{t[1]}kv{t[2]}")
def test_grouped_heads_full_size_sampled(shape, route):
    """Causal N8192 d128 with grouped key/value heads: every output written, sampled rows
    of every head against the oracle.  B1 H32/8 takes the heaviest-first order (a group's
    heads on one XCD); B1 H16/2 and B3 H12/4 do not meet that order's condition (a group
    would straddle XCDs) and keep the head-major order."""
    B, H, Hkv = shape
    p = W.make_problem(B, H, 8192, 128, flags=C, seed=(32, B, H, Hkv), H_kv=Hkv)
    _announce("gqa full size", p.name, route)
    _, o, lse = _run_gqa(p) if route == "map" else _run_gqa_derived(p)
    assert not np.isnan(o).any() and not np.isnan(lse).any()
    rows = sample_rows(p.N, 12, seed=32)
    heads = [(b, h) for b in range(B) for h in range(p.H)]
    o_ref, lse_ref = oracle.attention_problem(p, rows=rows, heads=heads, workers=8)
    assert_close(p, o[:, :, rows], lse[:, :, rows], o_ref, lse_ref, f"gqa full size sampled {p.name} {route}")
