"""Pins for the brute-force block map and visible-pair counts (CPU only)."""

import numpy as np
import pytest

import oracle as O
from oracle.attention import CAUSAL, WINDOW, DOCUMENT
from oracle.blockmap import EMPTY, PARTIAL, FULL


def _loop_blockmap(N, flags, W, doc, block):
    """Scalar re-derivation with explicit per-position loops (tiny sizes only)."""
    def vis(q, k):
        ok = True
        if flags & CAUSAL:
            ok &= k <= q
        if flags & WINDOW:
            ok &= abs(q - k) < W
        if flags & DOCUMENT:
            ok &= doc[q] == doc[k]
        return ok
    nb = -(-N // block)
    cls = np.zeros((nb, nb), np.uint8)
    for qb in range(nb):
        for kb in range(nb):
            seen = [vis(q, k) for q in range(qb * block, min(N, qb * block + block))
                    for k in range(kb * block, min(N, kb * block + block))]
            inside = len(seen) == block * block
            cls[qb, kb] = EMPTY if not any(seen) else (FULL if all(seen) and inside else PARTIAL)
    return cls


@pytest.mark.parametrize("N,flags,W", [(10, CAUSAL, 0), (9, 0, 0), (13, CAUSAL | WINDOW, 3), (12, WINDOW, 2),
                                       (11, DOCUMENT, 0), (16, CAUSAL | DOCUMENT, 0),
                                       (17, CAUSAL | WINDOW | DOCUMENT, 4)])
def test_blockmap_matches_scalar_loops(N, flags, W):
    doc = np.repeat(np.arange(4), [3, 5, 1, 100])[:N].astype(np.int32)
    m = O.blockmap_ref(1, N, flags, W, doc[None], block=4)
    cls = _loop_blockmap(N, flags, W, doc, 4)
    np.testing.assert_array_equal(m["cls"][0], cls)
    for qb in range(cls.shape[0]):
        full = [kb for kb in range(cls.shape[1]) if cls[qb, kb] == FULL]
        part = [kb for kb in range(cls.shape[1]) if cls[qb, kb] == PARTIAL]
        assert list(m["counts"][0, qb]) == [len(full), len(part)]
        row = m["idx"][0, qb]
        assert list(row[0]) == full + [-1] * (cls.shape[1] - len(full))
        assert list(row[1]) == part + [-1] * (cls.shape[1] - len(part))


@pytest.mark.parametrize("nqb", [1, 2, 5, 16])
def test_causal_closed_form_counts(nqb):
    N = 128 * nqb
    m = O.blockmap_ref(2, N, CAUSAL)
    for b in range(2):
        assert (m["cls"][b] == PARTIAL).sum() == nqb
        assert (m["cls"][b] == FULL).sum() == nqb * (nqb - 1) // 2
        assert np.array_equal(np.diag(m["cls"][b]), np.full(nqb, PARTIAL))
    assert m["visible_pairs"] == 2 * N * (N + 1) // 2


def test_causal_window_closed_form_counts():
    """Causal + window 1024 over 8192 tokens: per batch row 420 FULL and 120
    PARTIAL blocks; visible pairs W(W+1)/2 + (N-W)W."""
    N, W = 8192, 1024
    m = O.blockmap_ref(1, N, CAUSAL | WINDOW, W)
    assert (m["cls"] == FULL).sum() == 420
    assert (m["cls"] == PARTIAL).sum() == 120
    assert m["visible_pairs"] == W * (W + 1) // 2 + (N - W) * W


def test_noncausal_all_full_and_tail_partial():
    m = O.blockmap_ref(1, 1024, 0)
    assert (m["cls"] == FULL).all()
    m = O.blockmap_ref(1, 300, 0)
    assert m["cls"][0, 0, 0] == FULL and m["cls"][0, 0, 2] == PARTIAL and m["cls"][0, 2, 0] == PARTIAL
    assert m["visible_pairs"] == 300 * 300


def test_pair_count_consistent_with_classes():
    """#visible = 128*128*#FULL + visible pairs inside PARTIAL blocks."""
    rng = np.random.default_rng(0)
    N = 1000
    lengths = [137, 300, 1, 262, 300]
    doc = np.repeat(np.arange(5), lengths).astype(np.int32)[None]
    for flags, W in ((CAUSAL, 0), (CAUSAL | WINDOW, 200), (CAUSAL | DOCUMENT, 0), (DOCUMENT, 0), (WINDOW, 77)):
        m = O.blockmap_ref(1, N, flags, W, doc)
        vis = O.visible(np.arange(N), np.arange(N), flags, W, doc[0])
        part = 0
        for qb, kb in zip(*np.nonzero(m["cls"][0] == PARTIAL)):
            part += vis[qb * 128:(qb + 1) * 128, kb * 128:(kb + 1) * 128].sum()
        assert m["visible_pairs"] == 128 * 128 * (m["cls"] == FULL).sum() + part
        assert m["visible_pairs"] == O.visible_pairs_ref(1, N, flags, W, doc)


def test_row_intervals_closed_forms():
    N, W = 500, 64
    m = O.blockmap_ref(1, N, CAUSAL)
    assert np.array_equal(m["row_lo"][0], np.zeros(N)) and np.array_equal(m["row_hi"][0], np.arange(N))
    m = O.blockmap_ref(1, N, CAUSAL | WINDOW, W)
    assert np.array_equal(m["row_lo"][0], np.maximum(0, np.arange(N) - W + 1))
    m = O.blockmap_ref(1, N, WINDOW, W)
    assert np.array_equal(m["row_hi"][0], np.minimum(N - 1, np.arange(N) + W - 1))
    lengths = [100, 250, 150]
    starts = np.repeat(np.cumsum([0] + lengths[:-1]), lengths)
    ends = np.repeat(np.cumsum(lengths) - 1, lengths)
    doc = np.repeat(np.arange(3), lengths).astype(np.int32)[None]
    m = O.blockmap_ref(1, N, DOCUMENT, 0, doc)
    assert np.array_equal(m["row_lo"][0], starts) and np.array_equal(m["row_hi"][0], ends)
    m = O.blockmap_ref(1, N, DOCUMENT | CAUSAL, 0, doc)
    assert np.array_equal(m["row_lo"][0], starts) and np.array_equal(m["row_hi"][0], np.arange(N))
    lo, hi, contiguous = O.row_intervals_ref(N, DOCUMENT | CAUSAL | WINDOW, 30, doc[0])
    assert contiguous
    assert np.array_equal(lo, np.maximum(starts, np.arange(N) - 29)) and np.array_equal(hi, np.arange(N))
    # non-contiguous documents are not intervals
    _, _, contiguous = O.row_intervals_ref(6, DOCUMENT, 0, np.array([0, 1, 0, 1, 0, 1]))
    assert not contiguous


def test_column_intervals_closed_forms_and_brute_force():
    """col_lo/col_hi: the first and last query that sees each key, in closed form for the
    flag masks and documents, and against a scalar scan of the predicate on small cases
    (with block sizes that cut the sequence and documents across blocks)."""
    N, W = 500, 64
    k = np.arange(N)
    m = O.blockmap_ref(1, N, CAUSAL)
    assert np.array_equal(m["col_lo"][0], k) and np.array_equal(m["col_hi"][0], np.full(N, N - 1))
    m = O.blockmap_ref(1, N, CAUSAL | WINDOW, W)
    assert np.array_equal(m["col_lo"][0], k) and np.array_equal(m["col_hi"][0], np.minimum(N - 1, k + W - 1))
    m = O.blockmap_ref(1, N, WINDOW, W)
    assert np.array_equal(m["col_lo"][0], np.maximum(0, k - W + 1))
    assert np.array_equal(m["col_hi"][0], np.minimum(N - 1, k + W - 1))
    lengths = [100, 250, 150]
    starts = np.repeat(np.cumsum([0] + lengths[:-1]), lengths)
    ends = np.repeat(np.cumsum(lengths) - 1, lengths)
    doc = np.repeat(np.arange(3), lengths).astype(np.int32)[None]
    m = O.blockmap_ref(1, N, DOCUMENT | CAUSAL, 0, doc)
    assert np.array_equal(m["col_lo"][0], k) and np.array_equal(m["col_hi"][0], ends)
    m = O.blockmap_ref(1, N, DOCUMENT, 0, doc)
    assert np.array_equal(m["col_lo"][0], starts) and np.array_equal(m["col_hi"][0], ends)
    rng = np.random.default_rng([119, 58])
    for _ in range(8):
        n = int(rng.integers(1, 40))
        flags = int(rng.choice([CAUSAL, WINDOW, DOCUMENT, CAUSAL | WINDOW, CAUSAL | WINDOW | DOCUMENT]))
        w = int(rng.integers(1, 9))
        dd = np.repeat(np.arange(n), rng.integers(1, 8, n))[:n].astype(np.int32)
        m = O.blockmap_ref(1, n, flags, w, dd[None], block=4)
        for key in range(n):
            rows = [q for q in range(n)
                    if (not flags & CAUSAL or key <= q) and (not flags & WINDOW or abs(q - key) < w)
                    and (not flags & DOCUMENT or dd[q] == dd[key])]
            assert (m["col_lo"][0, key], m["col_hi"][0, key]) == (min(rows), max(rows)), (flags, w, key)


def test_qb_pairs_and_doc_status():
    doc = np.array([[0] * 100 + [1] * 200 + [2] * 20, [0] * 130 + [2] * 10 + [1] * 180]).astype(np.int32)
    m = O.blockmap_ref(2, 320, CAUSAL | DOCUMENT, 0, doc)
    assert m["qb_pairs"].sum() == m["visible_pairs"]
    assert m["qb_pairs"][0].sum() == 100 * 101 // 2 + 200 * 201 // 2 + 20 * 21 // 2
    assert m["status"][0].tolist() == [0, 0, 0]
    assert m["status"][1].tolist() == [0, 1, 0]  # the decrease 2 -> 1 is at row 139
    assert O.blockmap_ref(2, 320, CAUSAL, 0, doc)["status"].sum() == 0


def test_work_order_checker_accepts_the_order_and_rejects_mistakes():
    """The GPU tests check the device's work order (a scheduling choice, not part of the
    method) with tests/_parity.check_work_order.  The checker itself: it accepts an
    order sorted by the stated cost and rejects a swapped pair, a repeated entry and a
    non-identity order without documents."""
    from _parity import check_work_order
    rng = np.random.default_rng(7)
    lengths = rng.integers(40, 700, size=12)
    doc = np.repeat(np.arange(len(lengths)), lengths)[:1500].astype(np.int32)
    doc = np.stack([doc, np.sort(rng.integers(0, 5, size=1500)).astype(np.int32)])
    m = O.blockmap_ref(2, 1500, CAUSAL | DOCUMENT, 0, doc)
    hd = dict(order_full_cost=2, order_partial_cost=5)
    c = m["counts"].reshape(-1, 2).astype(np.int64)
    work = 2 * c[:, 0] + 5 * c[:, 1]
    assert len(set(work.tolist())) > 3  # the workload does spread the work
    order = np.array(sorted(range(len(work)), key=lambda e: (-work[e], e)))
    check_work_order(order, m["counts"], hd, True)
    i = int(np.nonzero(work[order][:-1] > work[order][1:])[0][0])
    bad = order.copy()
    bad[[i, i + 1]] = bad[[i + 1, i]]
    for wrong in (bad, np.concatenate([order[:-1], order[:1]])):
        with pytest.raises(AssertionError):
            check_work_order(wrong, m["counts"], hd, True)
    check_work_order(np.arange(len(work)), m["counts"], hd, False)
    with pytest.raises(AssertionError):
        check_work_order(order, m["counts"], hd, False)


def _classes_from_end_rows(lo, hi, N, block):
    """The rule the kernels use to find a query block's key blocks without listing them:
    non-empty are the key blocks that meet [lo(r0), hi(r1)] of its first and last rows r0,
    r1; FULL are those inside [lo(r1), hi(r0)], for a block of `block` rows and keys."""
    nb = -(-N // block)
    cls = np.zeros((nb, nb), np.uint8)
    for qb in range(nb):
        r0, r1 = qb * block, min(N, qb * block + block) - 1
        if hi[r1] >= lo[r0]:
            cls[qb, lo[r0] // block:hi[r1] // block + 1] = PARTIAL
        if r1 - r0 + 1 == block:
            fa, fz = -(-lo[r1] // block), (hi[r0] + 1) // block - 1
            if fz >= fa:
                cls[qb, fa:fz + 1] = FULL
    return cls


@pytest.mark.parametrize("seed", range(12))
def test_end_row_interval_rule_gives_every_class(seed):
    """Every supported mask (causal, window, contiguous documents and their conjunctions)
    gives each row one interval of keys whose ends never decrease and which holds the row
    itself, so a block's classes follow from its first and last rows' intervals alone:
    checked against the brute-force classes on random masks, lengths and block sizes."""
    rng = np.random.default_rng([119, 57, seed])
    block = int(rng.choice([4, 8, 16]))
    N = int(rng.integers(1, 12 * block))
    flags = int(rng.choice([CAUSAL, WINDOW, DOCUMENT, CAUSAL | WINDOW, CAUSAL | DOCUMENT, WINDOW | DOCUMENT,
                            CAUSAL | WINDOW | DOCUMENT]))
    W = int(rng.integers(1, 3 * block))
    doc = np.repeat(np.arange(N), rng.integers(1, 3 * block, N))[:N].astype(np.int32)
    m = O.blockmap_ref(1, N, flags, W, doc[None], block=block)
    lo, hi, contiguous = O.row_intervals_ref(N, flags, W, doc)
    assert contiguous and np.all(np.diff(lo) >= 0) and np.all(np.diff(hi) >= 0)
    assert np.all((lo <= np.arange(N)) & (np.arange(N) <= hi))
    np.testing.assert_array_equal(_classes_from_end_rows(lo, hi, N, block), m["cls"][0])
