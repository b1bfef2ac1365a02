"""GPU parity for the backward pass (attn_bwd_gqa): dQ, dK, dV of the HIP path, fed the
HIP forward pass's O and LSE, against the fp64 oracle's gradients of the definition."""

import numpy as np
import pytest
import torch

import oracle
import workload as W
from workload import device as WD
from exact_attention_119_amd import lib as L

pytestmark = pytest.mark.gpu

C, WI, DOC, AL, SC = W.ATTN_CAUSAL, W.ATTN_WINDOW, W.ATTN_DOCUMENT, W.ATTN_ALIBI, W.ATTN_SOFTCAP

VARIANTS = {
    "plain": dict(flags=0),
    "causal": dict(flags=C),
    "window": dict(flags=C | WI, window=37),
    "bidir_window": dict(flags=WI, window=50),
    "doc_causal": dict(flags=C | DOC),
    "alibi_causal": dict(flags=C | AL),
    "softcap": dict(flags=SC, softcap=2.0),
    "cfg3like": dict(flags=C | WI | SC, window=100, softcap=3.0),
    "everything": dict(flags=C | WI | DOC | AL | SC, window=70, softcap=2.5),
}
# gradients: bf16 operands (P, dS, inputs) and bf16 outputs; error relative to the
# largest reference magnitude of each tensor
TOL = 2e-2


def _announce(*a):
    print("CASE", *a, flush=True)


def _bwd(p, dout_bits):
    dp = WD.to_device(p)
    WD.step(dp)
    dout = torch.from_numpy(dout_bits.view(np.int16)).cuda().view(torch.bfloat16)
    dq = torch.full_like(dp.q, float("nan"))
    dk = torch.full_like(dp.k, float("nan"))
    dv = torch.full_like(dp.v, float("nan"))
    delta = torch.empty_like(dp.lse)
    L.attn_bwd_gqa(dp.q, dp.k, dp.v, dp.o, dp.lse, dout, dq, dk, dv, delta, scale=p.scale, mask=dp.mask,
                   blockmap=dp.blockmap)
    torch.cuda.synchronize()
    f = lambda t: t.float().cpu().numpy().astype(np.float64)
    return f(dq), f(dk), f(dv), delta.cpu().numpy().astype(np.float64)


def _check(got, ref, what):
    # a gradient can vanish analytically (dQ, dK of a one-key row are exactly zero) while
    # its rounding noise follows the other gradients: floor the scale at 5% of the largest
    gmax = max(np.abs(r).max() for r in ref[:3])
    for g, r, name in zip(got, ref, ("dQ", "dK", "dV", "D")):
        assert np.isfinite(g).all(), f"{what} {name}: non-finite"
        scale = max(np.abs(r).max(), 0.05 * gmax, 1e-30)
        e = np.abs(g - r).max() / scale
        print(f"{what} {name}: max|err|/max|ref| = {e:.2e}", flush=True)
        assert e <= TOL, f"{what} {name}: {e:.3e} > {TOL}"


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [1, 7, 129, 300])
@pytest.mark.parametrize("variant", list(VARIANTS))
def test_small_shapes(variant, N, d):
    heads = [(2, 2), (4, 2), (3, 1)][(N + d) % 3]
    p = W.make_problem(2, heads[0], N, d, seed=(N, d, sorted(VARIANTS).index(variant)), H_kv=heads[1],
                       doc_len_range=(1, max(1, N // 2)), **VARIANTS[variant])
    dO = W.make_dout(p, seed=(N, d))
    _announce("bwd", variant, N, d, heads)
    got = _bwd(p, dO)
    ref = oracle.attention_bwd_problem(p, dO)
    _check(got, ref, f"bwd {variant} N={N} d={d} H={heads}")


def test_deterministic():
    p = W.make_problem(1, 4, 700, 128, seed=3, H_kv=2, flags=C)
    dO = W.make_dout(p, seed=3)
    _announce("bwd determinism")
    a, b = _bwd(p, dO), _bwd(p, dO)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


@pytest.mark.parametrize("variant", ["causal", "cfg3like", "doc_causal"])
def test_larger(variant):
    p = W.make_problem(1, 4, 1500, 128, seed=(15, sorted(VARIANTS).index(variant)), H_kv=2,
                       doc_len_range=(200, 700), **VARIANTS[variant])
    dO = W.make_dout(p, seed=15)
    _announce("bwd larger", variant)
    got = _bwd(p, dO)
    ref = oracle.attention_bwd_problem(p, dO)
    _check(got, ref, f"bwd {variant} N=1500")


def test_full_size_sampled_heads():
    """B4 H16 N2048 d128 causal (the default forward workload): eight whole heads."""
    p = W.config_problem(2)
    dO = W.make_dout(p, seed=2)
    _announce("bwd full size")
    got = _bwd(p, dO)
    heads = [(b, h) for b, h in ((0, 0), (0, 7), (1, 3), (1, 15), (2, 1), (2, 8), (3, 5), (3, 14))]
    ref = oracle.attention_bwd_problem(p, dO, heads=heads)
    sel = lambda t, hs: np.stack([t[b, h] for b, h in hs])
    _check([sel(g, heads) for g in got], [sel(r, heads) for r in ref], "bwd B4 H16 N2048 causal")


def test_full_size_causal_window_softcap_sampled_heads():
    """B2 H32 N8192 d128 causal + window 1024 + softcap 50 (the default forward workload,
    and the backward bench's second configuration): two whole heads, one per batch row."""
    p = W.config_problem(3)
    dO = W.make_dout(p, seed=3)
    _announce("bwd full size causal+window+softcap")
    got = _bwd(p, dO)
    for b, h in ((0, 5), (1, 30)):
        ref = oracle.attention_bwd_problem(p, dO, heads=[(b, h)])
        _check([g[b, h] for g in got], [r[b, h] for r in ref], f"bwd B2 H32 N8192 cfg3 head ({b}, {h})")


VARLEN_MIXES = {"ragged": [0, 5, 129, 0, 1, 200, 64, 3], "mixed": [37, 300, 128, 1, 211, 90]}


@pytest.mark.parametrize("variant", ["plain", "causal", "cfg3like", "alibi_causal", "bidir_window"])
@pytest.mark.parametrize("mix", list(VARLEN_MIXES))
def test_varlen_against_oracle_and_document_mask(mix, variant):
    """attn_bwd_varlen on a packed batch (the compact workspace of attn_varlen_prepare)
    against the oracle's gradients of the document-masked pass over the sequence ids, and
    bit for bit against attn_bwd_gqa with that document mask and the full block map."""
    lengths = VARLEN_MIXES[mix]
    kw = VARIANTS[variant]
    p = W.make_varlen_problem(lengths, 4, 128, seed=(21, sorted(VARIANTS).index(variant)), H_kv=2, **kw)
    dO = W.make_dout(p, seed=21)
    _announce("bwd varlen", mix, variant, p.N)
    dp = WD.to_device(p)
    WD.step(dp)
    dout = torch.from_numpy(dO.view(np.int16)).cuda().view(torch.bfloat16)
    outs = [torch.full_like(t, float("nan")) for t in (dp.q, dp.k, dp.v)] + [torch.empty_like(dp.lse)]
    L.attn_bwd_varlen(dp.q[0], dp.k[0], dp.v[0], dp.o[0], dp.lse[0], dout[0], *(t[0] for t in outs),
                      scale=p.scale, workspace=dp.blockmap, mask=dp.mask)
    doc = torch.from_numpy(W.doc_ids_from_lengths(lengths)[None].copy()).cuda()
    m = L.make_mask(kw["flags"] | DOC, kw.get("window", 0), kw.get("softcap", 0.0), doc)
    mp = torch.empty(L.attn_blockmap_bytes(1, p.N, m), dtype=torch.uint8, device="cuda")
    L.attn_blockmap_build(1, p.N, m, mp)
    outs2 = [torch.full_like(t, float("nan")) for t in (dp.q, dp.k, dp.v)] + [torch.empty_like(dp.lse)]
    L.attn_bwd_gqa(dp.q, dp.k, dp.v, dp.o, dp.lse, dout, *outs2, scale=p.scale, mask=m, blockmap=mp)
    torch.cuda.synchronize()
    f = lambda t: t.float().cpu().numpy().astype(np.float64)
    got = [f(t) for t in outs]
    for a_, b_ in zip(outs, outs2):
        assert torch.equal(a_.view(torch.int16) if a_.dtype == torch.bfloat16 else a_.view(torch.int32),
                           b_.view(torch.int16) if b_.dtype == torch.bfloat16 else b_.view(torch.int32))
    ids = oracle.varlen_doc_ids_ref(p.cu_seqlens, p.N)
    Q, K, V = (oracle.decode_bf16(x) for x in (p.q, p.k, p.v))
    ref = oracle.attention_bwd_ref(Q, K, V, oracle.decode_bf16(dO), scale=p.scale, flags=p.flags | DOC,
                                   window=p.window, softcap=p.softcap, doc_id=ids[None], alibi_slopes=p.alibi_slopes)
    _check(got, ref, f"bwd varlen {mix} {variant}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [1, 7, 300, 1500])
@pytest.mark.parametrize("variant", ["causal", "window", "bidir_window", "alibi_causal", "cfg3like"])
def test_without_map_bit_identical(variant, N, d):
    """Causal and window masks without a block map: the kernels take the intervals from
    the flags, and every gradient is bit for bit the one the map gives."""
    p = W.make_problem(2, 4, N, d, seed=(33, N, sorted(VARIANTS).index(variant)), H_kv=2, **VARIANTS[variant])
    dO = W.make_dout(p, seed=33)
    _announce("bwd without map", variant, N)
    dp = WD.to_device(p)
    WD.step(dp)
    dout = torch.from_numpy(dO.view(np.int16)).cuda().view(torch.bfloat16)
    res = []
    for mp in (dp.blockmap, None):
        outs = [torch.full_like(t, float("nan")) for t in (dp.q, dp.k, dp.v)] + [torch.empty_like(dp.lse)]
        L.attn_bwd_gqa(dp.q, dp.k, dp.v, dp.o, dp.lse, dout, *outs, scale=p.scale, mask=dp.mask, blockmap=mp)
        res.append(outs)
    torch.cuda.synchronize()
    for a_, b_ in zip(*res):
        assert not torch.isnan(a_.float()).any()
        va = a_.view(torch.int16) if a_.dtype == torch.bfloat16 else a_.view(torch.int32)
        vb = b_.view(torch.int16) if b_.dtype == torch.bfloat16 else b_.view(torch.int32)
        assert torch.equal(va, vb)
