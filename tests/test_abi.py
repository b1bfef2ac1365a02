"""The C ABI on the CPU: the library loads, exports every declared entry point,
and validates arguments before any HIP call (no GPU needed)."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn119.h")


@pytest.fixture(scope="module")
def L():
    from exact_attention_119_amd import lib
    if not os.path.exists(lib.LIB_PATH):
        pytest.fail("libattn119.so is not built (python -m exact_attention_119_amd.build)")
    lib.load()
    return lib


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol(L):
    names = _declared()
    assert set(names) == set(L.EXPORTS)
    cdll = ctypes.CDLL(L.LIB_PATH)
    for n in names:
        assert hasattr(cdll, n), n


def test_status_strings(L):
    for s in (0, -1, -2, -3, -4, -5):
        assert L.status_str(s) and L.status_str(s) != "unknown status"
    assert L.status_str(7) == "unknown status"


def test_blockmap_layout(L):
    lay = L.attn_blockmap_layout_of(2, 300)
    nb = 3
    assert lay["cls"] == 256
    order = ["cls", "counts", "idx", "row_lo", "row_hi", "col_lo", "col_hi", "pairs", "status", "order", "total"]
    for a, b in zip(order, order[1:]):
        assert lay[a] < lay[b] and lay[b] % 256 == 0
    assert lay["counts"] - lay["cls"] >= 2 * nb * nb
    assert lay["row_hi"] - lay["row_lo"] >= 2 * 300 * 4
    assert L.attn_blockmap_bytes(2, 300, L.make_mask(L.ATTN_CAUSAL)) == lay["total"]
    with pytest.raises(L.AttnError):
        L.attn_blockmap_bytes(0, 300)
    with pytest.raises(L.AttnError):
        L.attn_blockmap_bytes(1, 300, L.make_mask(L.ATTN_WINDOW, window=0))


def test_compact_blockmap_layout_and_either_form_accepted(L):
    """The compact form: the general layout without cls and idx, O(B N) bytes; every call
    that takes a map accepts either form (told apart by the byte count) and nothing else."""
    full, comp = L.attn_blockmap_layout_of(2, 300), L.attn_blockmap_compact_layout_of(2, 300)
    assert comp["cls"] == 0 and comp["idx"] == 0 and comp["counts"] == 256
    names = ["counts", "row_lo", "row_hi", "col_lo", "col_hi", "pairs", "status", "order", "total"]
    for a, b in zip(names, names[1:]):
        assert comp[a] < comp[b] and comp[b] % 256 == 0
        if a != "counts":
            assert comp[b] - comp[a] == full[b] - full[a]
    m = L.make_mask(L.ATTN_CAUSAL | L.ATTN_DOCUMENT, doc_id=P)
    assert L.attn_blockmap_compact_bytes(2, 300, m) == comp["total"] < L.attn_blockmap_bytes(2, 300, m)
    for B, N in ((1, 1), (3, 129), (1, 1 << 20)):
        assert L.attn_blockmap_compact_bytes(B, N) < L.attn_blockmap_bytes(B, N)
    lib = L.load()
    chk = lambda nbytes: lib.attn_check_args(P, P, P, P, P, 2, 4, 300, 128, 0.1, 0, ctypes.byref(m), P, nbytes,
                                             None, 8.0)
    assert chk(full["total"]) == L.ATTN_OK and chk(comp["total"]) == L.ATTN_OK
    for bad in (comp["total"] - 256, comp["total"] + 256, full["total"] - 256, 0):
        assert chk(bad) == L.ATTN_ERR_BAD_BLOCKMAP
    build = lambda nbytes: lib.attn_blockmap_build_compact(2, 300, ctypes.byref(m), P, nbytes, None)
    assert build(full["total"]) == L.ATTN_ERR_BAD_BLOCKMAP


P = 0x10000  # fake, 16-byte aligned "device" addresses: never dereferenced by validation


def _args(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, B=2, H=4, N=300, d=128, scale=0.1, dtype=0, mask=None, blockmap=None,
             blockmap_bytes=0, fp8=None, rescale_tau=8.0)
    a.update(kw)
    return a


def test_check_args_ok_and_errors(L):
    ck = lambda **kw: L.attn_check_args(**_args(**kw))
    assert ck() == L.ATTN_OK
    assert ck(d=64) == L.ATTN_OK
    assert ck(q=None) == L.ATTN_ERR_INVALID_ARG
    assert ck(lse=P + 4) == L.ATTN_ERR_INVALID_ARG
    assert ck(d=96) == L.ATTN_ERR_UNSUPPORTED
    assert ck(B=0) == L.ATTN_ERR_INVALID_ARG
    assert ck(H=0) == L.ATTN_ERR_INVALID_ARG
    assert ck(N=0) == L.ATTN_ERR_INVALID_ARG
    assert ck(scale=0.0) == L.ATTN_ERR_INVALID_ARG
    assert ck(scale=float("inf")) == L.ATTN_ERR_INVALID_ARG
    assert ck(scale=float("nan")) == L.ATTN_ERR_INVALID_ARG
    assert ck(rescale_tau=-1.0) == L.ATTN_ERR_INVALID_ARG
    assert ck(rescale_tau=9.0) == L.ATTN_ERR_INVALID_ARG
    assert ck(dtype=2) == L.ATTN_ERR_UNSUPPORTED
    assert ck(mask=L.make_mask(64)) == L.ATTN_ERR_UNSUPPORTED
    assert ck(mask=L.make_mask(L.ATTN_ALIBI | L.ATTN_SOFTCAP, softcap=30.0)) == L.ATTN_OK
    assert ck(mask=L.make_mask(L.ATTN_SOFTCAP, softcap=0.0)) == L.ATTN_ERR_INVALID_ARG
    assert ck(mask=L.make_mask(L.ATTN_SOFTCAP, softcap=float("inf"))) == L.ATTN_ERR_INVALID_ARG
    # a block map, when given, must have exactly the right size; causal and window masks
    # may come without one, document masks (and e4m3 Q.K^T) may not
    m = L.make_mask(L.ATTN_CAUSAL)
    nbytes = L.attn_blockmap_bytes(2, 300, m)
    assert ck(mask=m) == L.ATTN_OK
    assert ck(mask=L.make_mask(L.ATTN_CAUSAL | L.ATTN_WINDOW, window=5)) == L.ATTN_OK
    assert ck(mask=L.make_mask(L.ATTN_DOCUMENT | L.ATTN_CAUSAL, doc_id=P)) == L.ATTN_ERR_BAD_BLOCKMAP
    f8 = L.make_fp8(P, P, P, qk_mode=L.ATTN_QK_E4M3)
    assert ck(mask=m, dtype=1, fp8=f8) == L.ATTN_OK
    assert ck(mask=m, dtype=1, fp8=f8, blockmap=P, blockmap_bytes=nbytes) == L.ATTN_OK
    assert ck(mask=m, dtype=1, fp8=L.make_fp8(P, P, P)) == L.ATTN_OK
    assert ck(mask=m, blockmap=P, blockmap_bytes=nbytes - 1) == L.ATTN_ERR_BAD_BLOCKMAP
    assert ck(mask=m, blockmap=P, blockmap_bytes=nbytes) == L.ATTN_OK
    assert ck(mask=L.make_mask(L.ATTN_WINDOW | L.ATTN_CAUSAL, window=0), blockmap=P,
              blockmap_bytes=nbytes) == L.ATTN_ERR_INVALID_ARG
    assert ck(mask=L.make_mask(L.ATTN_DOCUMENT), blockmap=P, blockmap_bytes=nbytes) == L.ATTN_ERR_INVALID_ARG
    assert ck(mask=L.make_mask(L.ATTN_DOCUMENT, doc_id=P), blockmap=P, blockmap_bytes=nbytes) == L.ATTN_OK
    # fp8 needs its scales; the e4m3 PV mode is not built
    assert ck(dtype=1) == L.ATTN_ERR_INVALID_ARG
    assert ck(dtype=1, fp8=L.make_fp8(P, P, None)) == L.ATTN_ERR_INVALID_ARG
    assert ck(dtype=1, fp8=L.make_fp8(P, P, P)) == L.ATTN_OK
    assert ck(dtype=1, fp8=L.make_fp8(P, P, P, pv_mode=5)) == L.ATTN_ERR_UNSUPPORTED
    # the fp8/fp4 P.V: with the e4m3 Q.K^T, d = 128, no mask or modifier
    for pv in (L.ATTN_PV_E4M3, L.ATTN_PV_FP4):
        f = L.make_fp8(P, P, P, pv_mode=pv, qk_mode=L.ATTN_QK_E4M3)
        assert ck(dtype=1, fp8=f) == L.ATTN_OK
        assert ck(dtype=1, fp8=L.make_fp8(P, P, P, pv_mode=pv)) == L.ATTN_ERR_UNSUPPORTED
        assert ck(dtype=1, fp8=f, d=64) == L.ATTN_ERR_UNSUPPORTED
        assert ck(dtype=1, fp8=f, mask=L.make_mask(L.ATTN_CAUSAL)) == L.ATTN_ERR_UNSUPPORTED
        assert ck(dtype=1, fp8=f, mask=L.make_mask(L.ATTN_SOFTCAP, softcap=5.0)) == L.ATTN_ERR_UNSUPPORTED


def test_check_args_grouped_heads(L):
    """H_kv key/value heads: must be at least 1 and divide H; H_kv = H is the plain call."""
    ck = lambda H_kv, **kw: L.attn_check_args_gqa(H_kv=H_kv, **_args(**kw))
    assert ck(4) == L.ATTN_OK
    assert ck(2) == L.ATTN_OK
    assert ck(1) == L.ATTN_OK
    assert ck(1, dtype=1, fp8=L.make_fp8(P, P, P)) == L.ATTN_OK
    assert ck(0) == L.ATTN_ERR_INVALID_ARG
    assert ck(-2) == L.ATTN_ERR_INVALID_ARG
    assert ck(3) == L.ATTN_ERR_INVALID_ARG
    assert ck(8) == L.ATTN_ERR_INVALID_ARG
    assert ck(3, H=6) == L.ATTN_OK
    assert ck(2, d=96) == L.ATTN_ERR_UNSUPPORTED
    lib = L.load()
    st = lib.attn_fwd_gqa(P, P, P, P, P, 1, 4, 3, 16, 64, 0.1, 0, None, None, 0, None, 8.0, None)
    assert st == L.ATTN_ERR_INVALID_ARG


def test_varlen_validation(L):
    """Packed variable-length batches: workspace = the compact block map of (1, total)
    (no class and list sections: O(total) bytes), then int32 ids."""
    m = L.make_mask(L.ATTN_CAUSAL)
    for total in (1, 300, 4096, 1 << 20):
        lay = L.attn_varlen_layout_of(total)
        nb = (total + 127) // 128
        full = L.attn_blockmap_layout_of(1, total)
        assert lay["cls"] == 0 and lay["idx"] == 0 and lay["counts"] == 256
        names = ["counts", "row_lo", "row_hi", "col_lo", "col_hi", "pairs", "status", "order", "total"]
        for a, b in zip(names, names[1:]):
            assert lay[a] < lay[b] and lay[b] % 256 == 0
            if a != "counts":  # the same sections as the full map's, without cls and idx
                assert lay[b] - lay[a] == full[b] - full[a]
        assert lay["row_lo"] - lay["counts"] >= 8 * nb
        assert lay["total"] <= 256 * 9 + 16 * total + 24 * nb  # O(total)
        assert L.attn_varlen_workspace_bytes(total, m) == lay["total"] + ((4 * total + 255) // 256) * 256
        assert L.attn_varlen_workspace_bytes(total, None) == L.attn_varlen_workspace_bytes(total, m)
    with pytest.raises(L.AttnError):
        L.attn_varlen_workspace_bytes(300, L.make_mask(L.ATTN_DOCUMENT, doc_id=P))
    with pytest.raises(L.AttnError):
        L.attn_varlen_workspace_bytes(0, m)
    lib = L.load()
    ws = L.attn_varlen_workspace_bytes(300, m)
    prep = lambda cu, nseq, total, bytes_, wsp=P: lib.attn_varlen_prepare(cu, nseq, total, ctypes.byref(m), wsp,
                                                                         bytes_, None)
    assert prep(None, 2, 300, ws) == L.ATTN_ERR_INVALID_ARG
    assert prep(P + 2, 2, 300, ws) == L.ATTN_ERR_INVALID_ARG
    assert prep(P, 0, 300, ws) == L.ATTN_ERR_INVALID_ARG
    assert prep(P, 2, 0, ws) == L.ATTN_ERR_INVALID_ARG
    assert prep(P, 2, 300, ws - 1) == L.ATTN_ERR_BAD_BLOCKMAP
    assert prep(P, 2, 300, ws, P + 8) == L.ATTN_ERR_INVALID_ARG
    fwd = lambda H, H_kv, bytes_, mask=m: lib.attn_fwd_varlen(P, P, P, P, P, H, H_kv, 300, 128, 0.1, 0,
                                                             ctypes.byref(mask) if mask else None, P, bytes_,
                                                             None, 8.0, None)
    assert fwd(4, 2, ws + 256) == L.ATTN_ERR_BAD_BLOCKMAP
    assert fwd(4, 3, ws) == L.ATTN_ERR_INVALID_ARG
    assert fwd(4, 2, ws, L.make_mask(L.ATTN_DOCUMENT, doc_id=P)) == L.ATTN_ERR_INVALID_ARG


def test_fp8_quantize_validation(L):
    lib = L.load()
    q = lambda x=P, c=P, s=P, B=1, H=2, N=300, d=128: lib.attn_fp8_quantize(x, c, s, B, H, N, d, None, None)
    assert q(x=None) == L.ATTN_ERR_INVALID_ARG
    assert q(c=P + 8) == L.ATTN_ERR_INVALID_ARG
    assert q(s=P + 2) == L.ATTN_ERR_INVALID_ARG
    assert q(d=96) == L.ATTN_ERR_UNSUPPORTED
    assert q(B=0) == L.ATTN_ERR_INVALID_ARG
    assert q(N=0) == L.ATTN_ERR_INVALID_ARG


def test_fwd_rejects_before_launch(L):
    """attn_fwd with bad arguments returns the validation error without touching the GPU."""
    lib = L.load()
    st = lib.attn_fwd(P, P, P, P, P, 1, 1, 16, 80, 0.1, 0, None, None, 0, None, 8.0, None)
    assert st == L.ATTN_ERR_UNSUPPORTED
    st = lib.attn_fwd(None, P, P, P, P, 1, 1, 16, 64, 0.1, 0, None, None, 0, None, 8.0, None)
    assert st == L.ATTN_ERR_INVALID_ARG


def test_kernel_variant_selection(L):
    """A masked kernel variant (the one that reads the block map) is selected exactly
    when the mask has a positional flag; the score-modifier mode follows the flags."""
    C, WI, DOC, AL, SC = L.ATTN_CAUSAL, L.ATTN_WINDOW, L.ATTN_DOCUMENT, L.ATTN_ALIBI, L.ATTN_SOFTCAP
    name = lambda d, flags, **kw: L.attn_fwd_kernel_name(d, 0, L.make_mask(flags, **kw) if flags else None)
    for d in (64, 128):
        assert name(d, 0) == f"bf16 d{d} unmasked linear"
        assert name(d, SC, softcap=5.0) == f"bf16 d{d} unmasked softcap"
        assert name(d, AL) == f"bf16 d{d} unmasked generic-alibi"
        assert name(d, AL | SC, softcap=5.0) == f"bf16 d{d} unmasked generic-alibi-softcap"
        assert name(d, C) == f"bf16 d{d} masked linear"
        assert name(d, C | WI | SC, window=9, softcap=50.0) == f"bf16 d{d} masked softcap"
        assert name(d, C | DOC | AL, doc_id=P) == f"bf16 d{d} masked alibi-causal"
        assert name(d, WI | AL, window=9) == f"bf16 d{d} masked generic-alibi"
        assert name(d, DOC | AL | SC, doc_id=P, softcap=1.0) == f"bf16 d{d} masked generic-alibi-softcap"
    for flags in range(32):
        kw = dict(window=3 if flags & WI else 0, softcap=2.0 if flags & SC else 0.0,
                  doc_id=P if flags & DOC else None)
        n = name(128, flags, **kw)
        assert n is not None and ("unmasked" not in n) == bool(flags & (C | WI | DOC)), (flags, n)
    fp8 = L.make_fp8(P, P, P)
    assert L.attn_fwd_kernel_name(128, 1, None, fp8) == "fp8 d128 unmasked linear"
    assert L.attn_fwd_kernel_name(64, 1, L.make_mask(C | AL), fp8) == "fp8 d64 masked alibi-causal"
    assert L.attn_fwd_kernel_name(128, 1, L.make_mask(C | WI | SC, window=9, softcap=50.0), fp8) == \
        "fp8 d128 masked softcap"
    fp8q = L.make_fp8(P, P, P, qk_mode=L.ATTN_QK_E4M3)
    assert L.attn_fwd_kernel_name(128, 1, None, fp8q) == "fp8-qk8 d128 unmasked linear"
    assert L.attn_fwd_kernel_name(64, 1, L.make_mask(C | AL), fp8q) == "fp8-qk8 d64 masked alibi-causal"
    assert L.attn_fwd_kernel_name(128, 1, None, L.make_fp8(P, P, P, pv_mode=L.ATTN_PV_FP4, qk_mode=L.ATTN_QK_E4M3)) \
        == "fp8-qk8-pv4 d128 unmasked linear"
    assert L.attn_fwd_kernel_name(96, 0, None, None) is None
    assert L.attn_fwd_kernel_name(128, 1, None, None) is None


def test_noalloc_backward_rejects_more_rows_than_its_scratch(L):
    """attn_bwd_gqa_noalloc keeps the row sums in a 4,194,304-row scratch array: a call with
    more rows (B * H * N) is refused before anything is launched."""
    lib = L.load()
    st = lib.attn_bwd_gqa_noalloc(P, P, P, P, P, P, P, P, P, 1, 64, 64, 65537, 128, 0.1, None, None, 0, None)
    assert st == L.ATTN_ERR_INVALID_ARG
    st = lib.attn_bwd_gqa_noalloc(P, P, P, P, P, None, P, P, P, 1, 4, 4, 300, 128, 0.1, None, None, 0, None)
    assert st == L.ATTN_ERR_INVALID_ARG


def test_header_is_plain_c():
    """include/attn119.h declares a C ABI: it compiles as C (and as C++) on its own."""
    import shutil
    import subprocess
    hdr = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "attn119.h")
    for cc, lang in (("gcc", "c"), ("g++", "c++")):
        if shutil.which(cc) is None:
            pytest.skip(f"{cc} not installed")
        r = subprocess.run([cc, "-fsyntax-only", "-Wall", "-Wextra", "-Werror", "-x", lang, hdr],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr
