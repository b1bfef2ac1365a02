"""GPU parity for packed variable-length batches: attn_varlen_prepare (sequence ids and
the compact block map, bit-exact against the oracle's) and attn_fwd_varlen against the
fp64 oracle, which runs every sequence on its own."""

import numpy as np
import pytest
import torch

import oracle
import workload as W
from workload import device as WD
from exact_attention_119_amd import lib as L
from _parity import assert_close, check_work_order, sample_rows

pytestmark = pytest.mark.gpu

C, WI, AL, SC = W.ATTN_CAUSAL, W.ATTN_WINDOW, W.ATTN_ALIBI, W.ATTN_SOFTCAP

VARIANTS = {
    "plain": dict(flags=0),
    "causal": dict(flags=C),
    "window": dict(flags=C | WI, window=37),
    "bidir_window": dict(flags=WI, window=50),
    "alibi_causal": dict(flags=C | AL),
    "softcap": dict(flags=SC, softcap=2.0),
    "cfg3like": dict(flags=C | WI | SC, window=100, softcap=3.0),
}


def _lengths(kind):
    rng = np.random.default_rng([119, 77, len(kind)])
    if kind == "one":
        return [300]
    if kind == "single_token":
        return [1]
    if kind == "ragged":
        return [0, 5, 129, 0, 1, 200, 64, 3]
    if kind == "block_aligned":
        return [128, 256, 128]
    if kind == "short_many":
        return [int(x) for x in rng.integers(1, 21, 40)]
    if kind == "mixed":
        return [int(x) for x in rng.integers(1, 401, 8)]
    raise ValueError(kind)


MIXES = ["one", "single_token", "ragged", "block_aligned", "short_many", "mixed"]


def _announce(*a):
    print("CASE", *a, flush=True)


def _run(p, tau=8.0):
    dp = WD.to_device(p)
    dp.o.fill_(float("nan"))
    dp.lse.fill_(float("nan"))
    WD.step(dp, rescale_tau=tau)
    o, lse = WD.outputs(dp)
    return dp, o, lse


def _classes_from_intervals(row_lo, row_hi, N):
    """Class of every 128x128 block from the intervals of each query block's first and
    last rows alone: non-empty where the key block meets [lo(r0), hi(r1)], FULL where it
    lies inside [lo(r1), hi(r0)] (128 rows, 128 keys)."""
    nb = (N + 127) // 128
    cls = np.zeros((nb, nb), dtype=np.uint8)
    for qb in range(nb):
        r0, r1 = 128 * qb, min(N, 128 * qb + 128) - 1
        lo0, lo1, hi0, hi1 = (int(x) for x in (row_lo[r0], row_lo[r1], row_hi[r0], row_hi[r1]))
        if hi1 >= lo0:
            cls[qb, lo0 // 128:hi1 // 128 + 1] = 1
        if r1 - r0 == 127:
            fa, fz = -(-lo1 // 128), (hi0 + 1) // 128 - 1
            if fz >= fa:
                cls[qb, fa:fz + 1] = 2
    return cls


def _check_prepared(dp):
    """Sequence ids and the compact block map in the workspace equal the oracle's byte for
    byte, and the intervals give the oracle's block classes."""
    p = dp.p
    lay = L.attn_varlen_layout_of(p.N)
    mb = lay["total"]
    assert lay["cls"] == 0 and lay["idx"] == 0
    assert dp.blockmap.numel() == mb + (4 * p.N + 255) // 256 * 256
    raw = dp.blockmap.cpu().numpy()
    ids = raw[mb:mb + 4 * p.N].view(np.int32)
    ids_ref = oracle.varlen_doc_ids_ref(p.cu_seqlens, p.N)
    np.testing.assert_array_equal(ids, ids_ref)
    got = L.read_blockmap(dp.blockmap[:mb], 1, p.N, compact=True)
    flags = (p.flags & L.POSITIONAL) | L.ATTN_DOCUMENT
    ref = oracle.blockmap_ref(1, p.N, flags, p.window, ids_ref[None])
    hd = got["header"]
    assert (hd["B"], hd["N"], hd["flags"], hd["compact"]) == (1, p.N, flags, 1)
    np.testing.assert_array_equal(got["status"], ref["status"])
    for key in ("counts", "row_lo", "row_hi", "col_lo", "col_hi"):
        np.testing.assert_array_equal(got[key], ref[key], err_msg=key)
    np.testing.assert_array_equal(_classes_from_intervals(got["row_lo"][0], got["row_hi"][0], p.N), ref["cls"][0])
    check_work_order(got["order"], got["counts"], got["header"], True)
    np.testing.assert_array_equal(got["pairs"], ref["qb_pairs"])
    assert L.attn_blockmap_status(dp.blockmap[:mb]) == L.ATTN_OK
    assert L.attn_blockmap_status(dp.blockmap) == L.ATTN_OK


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("variant", list(VARIANTS))
@pytest.mark.parametrize("mix", MIXES)
def test_varlen_bf16(mix, variant, d):
    lengths = _lengths(mix)
    Hkv = 2 if MIXES.index(mix) % 2 else 4
    p = W.make_varlen_problem(lengths, 4, d, seed=(MIXES.index(mix), sorted(VARIANTS).index(variant), d),
                              H_kv=Hkv, **VARIANTS[variant])
    _announce("varlen bf16", mix, variant, d, p.N, len(lengths))
    dp, o, lse = _run(p)
    _check_prepared(dp)
    o_ref, lse_ref = oracle.attention_problem(p)
    assert_close(p, o, lse, o_ref, lse_ref, f"varlen bf16 {mix} {variant} d={d}")


@pytest.mark.parametrize("variant", ["plain", "causal", "cfg3like"])
@pytest.mark.parametrize("mix", ["ragged", "mixed"])
def test_varlen_fp8(mix, variant):
    p = W.make_varlen_problem(_lengths(mix), 4, 128, dtype="fp8", n_outliers=4, H_kv=2,
                              seed=(MIXES.index(mix), 8), **VARIANTS[variant])
    _announce("varlen fp8", mix, variant, p.N)
    dp, o, lse = _run(p)
    o_ref, lse_ref = oracle.attention_problem(p)
    assert_close(p, o, lse, o_ref, lse_ref, f"varlen fp8 {mix} {variant}")


@pytest.mark.parametrize("variant", ["causal", "cfg3like", "alibi_causal"])
def test_varlen_bit_identical_to_document_mask(variant):
    """The packed call is the document-mask pass over the same ids: same bits."""
    lengths = _lengths("mixed")
    p = W.make_varlen_problem(lengths, 8, 128, seed=(5, 5), H_kv=2, **VARIANTS[variant])
    _announce("varlen vs document", variant)
    dp, o, lse = _run(p)
    doc = torch.from_numpy(W.doc_ids_from_lengths(lengths)[None].copy()).cuda()
    kw = VARIANTS[variant]
    m = L.make_mask(kw["flags"] | L.ATTN_DOCUMENT, kw.get("window", 0), kw.get("softcap", 0.0), doc)
    mp = torch.empty(L.attn_blockmap_bytes(1, p.N, m), dtype=torch.uint8, device="cuda")
    L.attn_blockmap_build(1, p.N, m, mp)
    o2 = torch.full_like(dp.o, float("nan"))
    lse2 = torch.full_like(dp.lse, float("nan"))
    L.attn_fwd_gqa(dp.q, dp.k, dp.v, o2, lse2, scale=p.scale, mask=m, blockmap=mp)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(o, o2.float().cpu().numpy())
    np.testing.assert_array_equal(lse, lse2.cpu().numpy())


@pytest.mark.parametrize("cu", [[0, 100, 50, 300], [1, 150, 300], [0, 150, 299], [0, 300, 300, 299]])
def test_varlen_bad_offsets_reported_and_output_poisoned(cu):
    """Offsets out of order, or not from 0 to total: attn_blockmap_status reports
    ATTN_ERR_BAD_DOC_ID and the forward pass writes NaN to every O and LSE element."""
    p = W.make_varlen_problem([300], 2, 64, flags=C, seed=9)
    p.cu_seqlens = np.asarray(cu, dtype=np.int32)
    _announce("varlen bad offsets", cu)
    dp, o, lse = _run(p)
    mb = L.attn_varlen_layout_of(p.N)["total"]
    assert L.attn_blockmap_status(dp.blockmap[:mb]) == L.ATTN_ERR_BAD_DOC_ID
    assert L.attn_blockmap_status(dp.blockmap) == L.ATTN_ERR_BAD_DOC_ID
    assert np.isnan(o).all() and np.isnan(lse).all()


def test_varlen_full_size_sampled():
    """H16 d128, 16384 packed tokens in sequences of 512 .. 4096 tokens, causal."""
    rng = np.random.default_rng([119, 78])
    lengths = W.draw_doc_lengths(rng, 16384, 512, 4096)
    p = W.make_varlen_problem(lengths, 16, 128, flags=C, seed=78, H_kv=4)
    _announce("varlen full size", p.name, len(lengths))
    dp, o, lse = _run(p)
    _check_prepared(dp)
    rows = sample_rows(p.N, 32, seed=78)
    heads = [(0, h) for h in range(p.H)]
    o_ref, lse_ref = oracle.attention_problem(p, rows=rows, heads=heads, workers=8)
    assert_close(p, o[:, :, rows], lse[:, :, rows], o_ref, lse_ref, "varlen full size sampled")


def test_varlen_million_tokens_compact_workspace():
    """1,048,576 packed tokens in causal sequences of 512 .. 8192 (H1 d64): the workspace
    is the compact map plus the ids, under 24 bytes per token (the map with classes and
    lists would take 0.62 GB); its row and column intervals on sampled positions and its
    FULL/PARTIAL counts on sampled query blocks equal the oracle's, and so do O and LSE on
    sampled rows."""
    rng = np.random.default_rng([119, 79])
    lengths = W.draw_doc_lengths(rng, 1 << 20, 512, 8192)
    p = W.make_varlen_problem(lengths, 1, 64, flags=C, seed=79)
    _announce("varlen 1M tokens", p.name, len(lengths))
    dp, o, lse = _run(p)
    N = p.N
    lay = L.attn_varlen_layout_of(N)
    assert dp.blockmap.numel() == L.attn_varlen_workspace_bytes(N, dp.mask) < 24 * N
    assert L.attn_blockmap_status(dp.blockmap) == L.ATTN_OK
    got = L.read_blockmap(dp.blockmap[:lay["total"]], 1, N, compact=True)
    ids = oracle.varlen_doc_ids_ref(p.cu_seqlens, N)
    flags = C | L.ATTN_DOCUMENT
    kpos = np.arange(N)
    rows = sample_rows(N, 64, seed=79)
    vis = oracle.visible(rows, kpos, flags, 0, ids)
    np.testing.assert_array_equal(got["row_lo"][0][rows], vis.argmax(axis=1))
    np.testing.assert_array_equal(got["row_hi"][0][rows], N - 1 - vis[:, ::-1].argmax(axis=1))
    visk = oracle.visible(kpos, rows, flags, 0, ids)  # [every query][sampled keys]
    np.testing.assert_array_equal(got["col_lo"][0][rows], visk.argmax(axis=0))
    np.testing.assert_array_equal(got["col_hi"][0][rows], N - 1 - visk[::-1].argmax(axis=0))
    nb = N // 128
    for qb in sorted({0, 1, nb - 1, *np.random.default_rng(79).choice(nb, 3, replace=False).tolist()}):
        blk = oracle.visible(np.arange(128 * qb, 128 * qb + 128), kpos, flags, 0, ids).reshape(128, nb, 128)
        anyv, allv = blk.any(axis=(0, 2)), blk.all(axis=(0, 2))
        full, part = int(allv.sum()), int((anyv & ~allv).sum())
        assert tuple(got["counts"][0, qb]) == (full, part), qb
    o_ref, lse_ref = oracle.attention_problem(p, rows=rows)
    assert_close(p, o[:, :, rows], lse[:, :, rows], o_ref, lse_ref, "varlen 1M tokens sampled")
