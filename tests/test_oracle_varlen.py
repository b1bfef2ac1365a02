"""Pins of the oracle's packed variable-length batches against routes that do not go
through its per-sequence slicing: brute force with a document mask over global
positions, a batch of equal-length rows, and the closed form of one-token sequences."""

import math

import numpy as np
import pytest

import oracle
import workload as W
from test_oracle_pins import _brute

CAUSAL, WINDOW, DOCUMENT, ALIBI, SOFTCAP = 1, 2, 4, 8, 16


def test_doc_ids_written_out_by_hand():
    # sequence 1 is empty: tokens 3, 4 belong to sequence 2
    np.testing.assert_array_equal(oracle.varlen_doc_ids_ref([0, 3, 3, 5, 8], 8), [0, 0, 0, 2, 2, 3, 3, 3])
    np.testing.assert_array_equal(oracle.varlen_doc_ids_ref([0, 1], 1), [0])
    np.testing.assert_array_equal(oracle.varlen_doc_ids_ref([0, 0, 2], 2), [1, 1])
    np.testing.assert_array_equal(oracle.varlen_doc_ids_ref([0, 2, 2, 2], 2), [0, 0])


@pytest.mark.parametrize("lengths", [[1], [5], [3, 0, 4], [1, 1, 1, 2], [0, 6, 1, 0, 2, 0]])
def test_varlen_matches_brute_force_with_document_mask(lengths):
    """Every flag combination (document excluded), H 4 over H_kv 2: the per-sequence
    oracle equals brute force over the packed positions with a document mask."""
    total, d, H, Hkv = sum(lengths), 3, 4, 2
    rng = np.random.default_rng([len(lengths), total])
    Q = rng.standard_normal((H, total, d))
    K = rng.standard_normal((Hkv, total, d))
    V = rng.standard_normal((Hkv, total, d))
    cu = np.concatenate([[0], np.cumsum(lengths)])
    doc = np.repeat(np.arange(len(lengths)), lengths)[None]
    slopes = [0.5, 0.25, 0.125, 0.0625]
    for flags in range(32):
        if flags & DOCUMENT:
            continue
        W_, cap = 2, 1.5
        o, l = oracle.attention_varlen_ref(Q, K, V, cu, scale=0.75, flags=flags, window=W_, softcap=cap,
                                           alibi_slopes=slopes)
        ob, lb = _brute(Q[None], K[None], V[None], 0.75, flags | DOCUMENT, W_, cap, doc, slopes)
        np.testing.assert_allclose(o, ob[0], rtol=1e-12, atol=1e-12, err_msg=f"flags {flags}")
        np.testing.assert_allclose(l, lb[0], rtol=1e-12, atol=1e-12, err_msg=f"flags {flags}")


@pytest.mark.parametrize("flags", [0, CAUSAL, CAUSAL | WINDOW, CAUSAL | ALIBI, SOFTCAP | WINDOW])
def test_equal_lengths_equal_a_batch(flags):
    """nseq sequences of one length L packed: the same as B = nseq rows of N = L."""
    nseq, L, H, Hkv, d = 3, 40, 4, 1, 8
    rng = np.random.default_rng([flags, 7])
    Q = rng.standard_normal((H, nseq * L, d))
    K = rng.standard_normal((Hkv, nseq * L, d))
    V = rng.standard_normal((Hkv, nseq * L, d))
    kw = dict(scale=0.3, flags=flags, window=9, softcap=2.0)
    o, l = oracle.attention_varlen_ref(Q, K, V, np.arange(nseq + 1) * L, **kw)
    to_b = lambda X: X.reshape(X.shape[0], nseq, L, d).transpose(1, 0, 2, 3)
    ob, lb = oracle.attention_ref(to_b(Q), to_b(K), to_b(V), **kw)
    np.testing.assert_allclose(o, ob.transpose(1, 0, 2, 3).reshape(H, nseq * L, d), rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(l, lb.transpose(1, 0, 2).reshape(H, nseq * L), rtol=1e-13, atol=1e-13)


def test_one_token_sequences_closed_form():
    """A sequence of one token sees only itself: O is its value row and LSE its own
    (soft-capped) score; ALiBi adds nothing at distance 0."""
    total, H, d = 6, 2, 5
    rng = np.random.default_rng(3)
    Q, K, V = (rng.standard_normal((H, total, d)) for _ in range(3))
    cap, scale = 2.0, 0.625  # exact in fp32, as the oracle takes the fp32 scale
    o, l = oracle.attention_varlen_ref(Q, K, V, np.arange(total + 1), scale=scale,
                                       flags=CAUSAL | ALIBI | SOFTCAP, softcap=cap)
    np.testing.assert_allclose(o, V, rtol=0, atol=1e-15)
    s = np.array([[cap * math.tanh(scale * float(Q[h, t] @ K[h, t]) / cap) for t in range(total)]
                  for h in range(H)])
    np.testing.assert_allclose(l, s, rtol=1e-14, atol=1e-15)


def test_rows_and_heads_subset_match_full():
    p = W.make_varlen_problem([0, 50, 7, 130, 1], 4, 16, flags=CAUSAL | WINDOW, window=20, seed=2, H_kv=2)
    o, l = oracle.attention_problem(p)
    rows = np.array([0, 49, 50, 56, 57, 100, 186, 187])
    os_, ls_ = oracle.attention_problem(p, rows=rows, heads=[(0, 1), (0, 3)])
    for h in (1, 3):
        np.testing.assert_array_equal(os_[0, h], o[0, h, rows])
        np.testing.assert_array_equal(ls_[0, h], l[0, h, rows])
    assert np.isnan(os_[0, 0]).all() and np.isnan(ls_[0, 2]).all()


def test_rejects_document_flag_and_bad_offsets():
    Q = np.zeros((1, 4, 2))
    with pytest.raises(ValueError):
        oracle.attention_varlen_ref(Q, Q, Q, [0, 4], scale=1.0, flags=DOCUMENT)
    for cu in ([1, 4], [0, 3], [0, 3, 2, 4]):
        with pytest.raises(ValueError):
            oracle.attention_varlen_ref(Q, Q, Q, cu, scale=1.0)
    with pytest.raises(ValueError):
        W.make_varlen_problem([2, 2], 2, 8, flags=DOCUMENT)
    with pytest.raises(ValueError):
        W.make_varlen_problem([0, 0], 2, 8)
