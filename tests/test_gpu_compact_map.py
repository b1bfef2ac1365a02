"""GPU parity for the compact block map (the general map without its class and list
sections): its sections against the oracle's map, and the forward and backward passes
with it bit for bit equal to the same passes with the general map."""

import numpy as np
import pytest
import torch

import oracle
import workload as W
from workload import device as WD
from exact_attention_119_amd import lib as L
from _parity import check_work_order

pytestmark = pytest.mark.gpu

C, WI, DOC, AL, SC = W.ATTN_CAUSAL, W.ATTN_WINDOW, W.ATTN_DOCUMENT, W.ATTN_ALIBI, W.ATTN_SOFTCAP

CASES = {
    "doc_causal": dict(flags=C | DOC),
    "doc_window_softcap": dict(flags=C | WI | DOC | SC, window=90, softcap=4.0),
    "doc_bidir_alibi": dict(flags=DOC | AL),
    "causal_window": dict(flags=C | WI, window=200),
}


def _same_bits(a, b):
    v = (lambda t: t.view(torch.int16)) if a.dtype == torch.bfloat16 else (lambda t: t.view(torch.int32))
    return torch.equal(v(a), v(b))


@pytest.mark.parametrize("N", [1, 300, 1000])
@pytest.mark.parametrize("case", list(CASES))
def test_compact_map_sections_and_passes(case, N):
    kw = CASES[case]
    p = W.make_problem(2, 4, N, 128, seed=(40, N, sorted(CASES).index(case)), H_kv=2,
                       doc_len_range=(1, max(1, N // 3)), **kw)
    print("CASE compact map", case, N, flush=True)
    dp = WD.to_device(p)
    WD.build_map(dp)
    full = dp.blockmap
    comp = torch.empty(L.attn_blockmap_compact_bytes(p.B, p.N, dp.mask), dtype=torch.uint8, device="cuda")
    L.attn_blockmap_build_compact(p.B, p.N, dp.mask, comp)
    torch.cuda.synchronize()
    assert comp.numel() < full.numel()
    got = L.read_blockmap(comp, p.B, p.N, compact=True)
    ref = oracle.blockmap_ref(p.B, p.N, p.flags & L.POSITIONAL, p.window, p.doc_id)
    hd = got["header"]
    assert (hd["B"], hd["N"], hd["flags"], hd["compact"]) == (p.B, p.N, p.flags & L.POSITIONAL, 1)
    np.testing.assert_array_equal(got["status"], ref["status"])
    for key in ("counts", "row_lo", "row_hi", "col_lo", "col_hi"):
        np.testing.assert_array_equal(got[key], ref[key], err_msg=key)
    np.testing.assert_array_equal(got["pairs"], ref["qb_pairs"])
    check_work_order(got["order"], got["counts"], hd, bool(p.flags & L.ATTN_DOCUMENT))
    assert L.attn_blockmap_status(comp) == L.ATTN_OK

    def fwd(mp):
        o, lse = torch.full_like(dp.o, float("nan")), torch.full_like(dp.lse, float("nan"))
        L.attn_fwd_gqa(dp.q, dp.k, dp.v, o, lse, scale=p.scale, mask=dp.mask, blockmap=mp)
        return o, lse

    (o1, l1), (o2, l2) = fwd(full), fwd(comp)
    dout = torch.from_numpy(W.make_dout(p, seed=40).view(np.int16)).cuda().view(torch.bfloat16)

    def bwd(mp):
        outs = [torch.full_like(t, float("nan")) for t in (dp.q, dp.k, dp.v)] + [torch.empty_like(dp.lse)]
        L.attn_bwd_gqa(dp.q, dp.k, dp.v, o1, l1, dout, *outs, scale=p.scale, mask=dp.mask, blockmap=mp)
        return outs

    g1, g2 = bwd(full), bwd(comp)
    torch.cuda.synchronize()
    assert not torch.isnan(o1).any() and _same_bits(o1, o2) and _same_bits(l1, l2)
    for a, b in zip(g1, g2):
        assert not torch.isnan(a.float()).any() and _same_bits(a, b)


@pytest.mark.parametrize("case", ["doc_causal", "doc_window_softcap"])
def test_compact_map_fp8_forward(case):
    """The fp8 forward pass (e4m3 inputs with block scales) with the compact map equals
    the pass with the general map bit for bit."""
    kw = CASES[case]
    p = W.make_problem(2, 4, 700, 128, dtype="fp8", n_outliers=4, seed=(41, sorted(CASES).index(case)), H_kv=2,
                       doc_len_range=(1, 300), **kw)
    print("CASE compact map fp8", case, flush=True)
    dp = WD.to_device(p)
    WD.build_map(dp)
    comp = torch.empty(L.attn_blockmap_compact_bytes(p.B, p.N, dp.mask), dtype=torch.uint8, device="cuda")
    L.attn_blockmap_build_compact(p.B, p.N, dp.mask, comp)
    res = []
    for mp in (dp.blockmap, comp):
        o, lse = torch.full_like(dp.o, float("nan")), torch.full_like(dp.lse, float("nan"))
        L.attn_fwd_gqa(dp.q, dp.k, dp.v, o, lse, scale=p.scale, dtype=dp.dtype, mask=dp.mask, blockmap=mp,
                       fp8=dp.fp8)
        res.append((o, lse))
    torch.cuda.synchronize()
    (o1, l1), (o2, l2) = res
    assert not torch.isnan(o1).any() and _same_bits(o1, o2) and _same_bits(l1, l2)
