"""Pins for the fp64 attention oracle (CPU only).

Each check ties the oracle to something other than itself:
  * brute force -- scalar Python loops over explicitly enumerated visible keys,
    math.fsum and math.exp -- on tiny shapes, every flag combination;
  * library special cases -- torch's CPU scaled_dot_product_attention and
    logsumexp in float64, with masks built from torch.tril/triu;
  * closed forms -- zero queries give uniform (or ALiBi-geometric) weights;
  * invariants named for the method -- weights sum to one, constant V, single
    visible key, permutation of keys with values, linearity, degenerate masks.
"""

import itertools
import math

import numpy as np
import pytest
import torch

import oracle as O
from oracle.attention import CAUSAL, WINDOW, DOCUMENT, ALIBI, SOFTCAP, _softmax_rows

ALL_FLAGS = [CAUSAL, WINDOW, DOCUMENT, ALIBI, SOFTCAP]


# ---------------------------------------------------------------------------
# brute force
# ---------------------------------------------------------------------------

def _segments(doc_row):
    segs, start = [], 0
    for i in range(1, len(doc_row) + 1):
        if i == len(doc_row) or doc_row[i] != doc_row[start]:
            segs.append((start, i - 1))
            start = i
    return segs


def _visible_keys(q, N, flags, W, doc_row):
    """Enumerate the keys query q may see, written per mask kind as ranges."""
    lo, hi = 0, N - 1
    if flags & CAUSAL:
        hi = min(hi, q)
    if flags & WINDOW:
        lo = max(lo, q - (W - 1))
        if not flags & CAUSAL:
            hi = min(hi, q + (W - 1))
    if flags & DOCUMENT:
        for a, b in _segments(list(doc_row)):
            if a <= q <= b:
                lo, hi = max(lo, a), min(hi, b)
    return list(range(lo, hi + 1))


def _brute(Q, K, V, scale, flags, W, cap, doc, slopes):
    B, H, N, d = Q.shape
    g = H // K.shape[1]  # query heads per key/value head
    Ob = np.zeros((B, H, N, V.shape[3]))
    Lb = np.zeros((B, H, N))
    for b, h, q in itertools.product(range(B), range(H), range(N)):
        keys = _visible_keys(q, N, flags, W, None if doc is None else doc[b])
        sc = []
        for k in keys:
            s = math.fsum(float(Q[b, h, q, i]) * float(K[b, h // g, k, i]) for i in range(d)) * scale
            if flags & SOFTCAP:
                s = cap * math.tanh(s / cap)
            if flags & ALIBI:
                s += slopes[h] * (k - q) if k <= q else -slopes[h] * (k - q)
            sc.append(s)
        if not keys:
            Lb[b, h, q] = -math.inf
            continue
        m = max(sc)
        w = [math.exp(s - m) for s in sc]
        l = math.fsum(w)
        Lb[b, h, q] = m + math.log(l)
        for j in range(V.shape[3]):
            Ob[b, h, q, j] = math.fsum(wi * float(V[b, h // g, k, j]) for wi, k in zip(w, keys)) / l
    return Ob, Lb


def _doc_rows(B, N, rng):
    rows = []
    for _ in range(B):
        cuts = np.sort(rng.choice(np.arange(1, N), size=min(N - 1, 2), replace=False)) if N > 2 else []
        ids = np.zeros(N, dtype=np.int32)
        for c in cuts:
            ids[c:] += 1
        rows.append(ids)
    return np.stack(rows)


@pytest.mark.parametrize("N,d", [(1, 4), (2, 1), (3, 8), (7, 4), (16, 8), (33, 4)])
def test_oracle_matches_brute_force_all_flag_combinations(N, d):
    rng = np.random.default_rng(N * 100 + d)
    B, H = 1, 2
    Q = rng.standard_normal((B, H, N, d)) * 1.5
    K = rng.standard_normal((B, H, N, d)) * 1.5
    V = rng.standard_normal((B, H, N, d))
    doc = _doc_rows(B, N, rng)
    slopes = [0.5, 0.125]
    for r in range(len(ALL_FLAGS) + 1):
        for combo in itertools.combinations(ALL_FLAGS, r):
            flags = sum(combo)
            W = max(1, N // 3)
            cap = 2.5
            o, l = O.attention_ref(Q, K, V, scale=0.7, flags=flags, window=W, softcap=cap,
                                   doc_id=doc, alibi_slopes=slopes)
            ob, lb = _brute(Q, K, V, float(np.float32(0.7)), flags, W, float(np.float32(cap)), doc, slopes)
            np.testing.assert_allclose(o, ob, rtol=1e-12, atol=1e-12, err_msg=f"flags={flags}")
            np.testing.assert_allclose(l, lb, rtol=1e-12, atol=1e-12, err_msg=f"flags={flags}")


@pytest.mark.parametrize("H_kv", [1, 2])
def test_oracle_matches_brute_force_grouped_heads(H_kv):
    """GQA (H_kv = 2) and MQA (H_kv = 1) with four query heads: query head h reads
    key/value head h // (4 / H_kv), for a spread of flag combinations."""
    rng = np.random.default_rng(70 + H_kv)
    B, H, N, d = 1, 4, 9, 4
    Q = rng.standard_normal((B, H, N, d)) * 1.5
    K = rng.standard_normal((B, H_kv, N, d)) * 1.5
    V = rng.standard_normal((B, H_kv, N, d))
    doc = _doc_rows(B, N, rng)
    slopes = [0.5, 0.25, 0.125, 0.0625]
    for flags in (0, CAUSAL, CAUSAL | WINDOW | SOFTCAP, DOCUMENT | ALIBI, CAUSAL | DOCUMENT | ALIBI | SOFTCAP):
        o, l = O.attention_ref(Q, K, V, scale=0.7, flags=flags, window=3, softcap=2.5, doc_id=doc,
                               alibi_slopes=slopes)
        ob, lb = _brute(Q, K, V, float(np.float32(0.7)), flags, 3, float(np.float32(2.5)), doc, slopes)
        np.testing.assert_allclose(o, ob, rtol=1e-12, atol=1e-12, err_msg=f"flags={flags}")
        np.testing.assert_allclose(l, lb, rtol=1e-12, atol=1e-12, err_msg=f"flags={flags}")


@pytest.mark.parametrize("causal", [False, True])
def test_vs_torch_sdpa_grouped_heads(causal):
    """torch's scaled_dot_product_attention with enable_gqa (float64, CPU)."""
    rng = np.random.default_rng(77)
    Q = rng.standard_normal((2, 6, 90, 16))
    K = rng.standard_normal((2, 2, 90, 16))
    V = rng.standard_normal((2, 2, 90, 16))
    o, l = O.attention_ref(Q, K, V, scale=0.25, flags=CAUSAL if causal else 0)
    q, k, v = (torch.from_numpy(x) for x in (Q, K, V))
    ot = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=causal, scale=0.25, enable_gqa=True)
    np.testing.assert_allclose(o, ot.numpy(), rtol=1e-11, atol=1e-12)
    with pytest.raises(ValueError):
        O.attention_ref(Q, K[:, :1].repeat(4, axis=1), V[:, :1].repeat(4, axis=1), scale=0.25)


def test_empty_row_convention():
    s = np.array([[-np.inf, -np.inf, -np.inf], [0.0, -np.inf, 1.0]])
    V = np.arange(6.0).reshape(3, 2)
    o, l = _softmax_rows(s, V)
    assert np.all(o[0] == 0) and l[0] == -np.inf
    w = np.array([1.0, 0.0, math.e]) / (1 + math.e)
    np.testing.assert_allclose(o[1], w @ V, rtol=1e-14)
    np.testing.assert_allclose(l[1], 1 + math.log(1 + math.exp(-1)), rtol=1e-14)


# ---------------------------------------------------------------------------
# library special cases: torch SDPA in float64 on the CPU
# ---------------------------------------------------------------------------

def _torch_sdpa(Q, K, V, scale, mask=None, causal=False, bias=None, cap=None):
    q, k, v = (torch.from_numpy(x) for x in (Q, K, V))
    if cap is None and bias is None:
        o = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask, is_causal=causal,
                                                             scale=scale)
    else:
        s = (q @ k.transpose(-1, -2)) * scale
        if cap is not None:
            s = cap * torch.tanh(s / cap)
        if bias is not None:
            s = s + bias
        if mask is not None:
            s = s.masked_fill(~mask, float("-inf"))
        o = torch.softmax(s, dim=-1) @ v
    s = (q @ k.transpose(-1, -2)) * scale
    if cap is not None:
        s = cap * torch.tanh(s / cap)
    if bias is not None:
        s = s + bias
    if causal:
        mask = torch.ones(s.shape[-2:], dtype=torch.bool).tril()
    if mask is not None:
        s = s.masked_fill(~mask, float("-inf"))
    return o.numpy(), torch.logsumexp(s, dim=-1).numpy()


@pytest.fixture(scope="module")
def qkv():
    rng = np.random.default_rng(11)
    B, H, N, d = 2, 3, 150, 32
    return tuple(rng.standard_normal((B, H, N, d)) for _ in range(3))


def test_vs_torch_sdpa_noncausal(qkv):
    Q, K, V = qkv
    sc = float(np.float32(1 / math.sqrt(32)))
    o, l = O.attention_ref(Q, K, V, scale=sc)
    ot, lt = _torch_sdpa(Q, K, V, sc)
    np.testing.assert_allclose(o, ot, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(l, lt, rtol=1e-12, atol=1e-12)


def test_vs_torch_sdpa_causal(qkv):
    Q, K, V = qkv
    o, l = O.attention_ref(Q, K, V, scale=0.25, flags=CAUSAL)
    ot, lt = _torch_sdpa(Q, K, V, 0.25, causal=True)
    np.testing.assert_allclose(o, ot, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(l, lt, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("W", [1, 17, 64, 400])
def test_vs_torch_causal_window(qkv, W):
    Q, K, V = qkv
    N = Q.shape[2]
    mask = torch.ones(N, N, dtype=torch.bool).tril().triu(-(W - 1))
    o, l = O.attention_ref(Q, K, V, scale=0.25, flags=CAUSAL | WINDOW, window=W)
    ot, lt = _torch_sdpa(Q, K, V, 0.25, mask=mask)
    np.testing.assert_allclose(o, ot, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(l, lt, rtol=1e-12, atol=1e-12)


def test_vs_torch_bidirectional_window(qkv):
    Q, K, V = qkv
    N, W = Q.shape[2], 20
    mask = torch.ones(N, N, dtype=torch.bool).tril(W - 1).triu(-(W - 1))
    o, l = O.attention_ref(Q, K, V, scale=0.25, flags=WINDOW, window=W)
    ot, lt = _torch_sdpa(Q, K, V, 0.25, mask=mask)
    np.testing.assert_allclose(o, ot, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(l, lt, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_vs_torch_document(qkv, causal):
    Q, K, V = qkv
    N = Q.shape[2]
    lengths = [40, 1, 70, 39]
    doc = np.repeat(np.arange(4), lengths).astype(np.int32)
    doc_id = np.stack([doc, np.repeat(np.arange(2), [75, 75]).astype(np.int32)])
    outs = O.attention_ref(Q, K, V, scale=0.375, flags=DOCUMENT | (CAUSAL if causal else 0), doc_id=doc_id)
    for b in range(2):
        # block-diagonal mask built from the segment table, not from doc ids
        mask = torch.zeros(N, N, dtype=torch.bool)
        segs = [(0, 40), (40, 41), (41, 111), (111, 150)] if b == 0 else [(0, 75), (75, 150)]
        for a, e in segs:
            mask[a:e, a:e] = True
        if causal:
            mask &= torch.ones(N, N, dtype=torch.bool).tril()
        ot, lt = _torch_sdpa(Q[b:b + 1], K[b:b + 1], V[b:b + 1], 0.375, mask=mask)
        np.testing.assert_allclose(outs[0][b:b + 1], ot, rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(outs[1][b:b + 1], lt, rtol=1e-12, atol=1e-12)


def test_vs_torch_alibi_causal(qkv):
    Q, K, V = qkv
    B, H, N, d = Q.shape
    slopes = O.default_alibi_slopes(H)
    pos = torch.arange(N, dtype=torch.float64)
    bias = torch.stack([float(s) * (pos[None, :] - pos[:, None]) for s in slopes])[None]
    o, l = O.attention_ref(Q, K, V, scale=0.1875, flags=CAUSAL | ALIBI)
    ot, lt = _torch_sdpa(Q, K, V, 0.1875, bias=bias, causal=True, mask=torch.ones(N, N, dtype=torch.bool).tril())
    np.testing.assert_allclose(o, ot, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(l, lt, rtol=1e-12, atol=1e-12)


def test_vs_torch_alibi_bidirectional_is_symmetric_distance(qkv):
    Q, K, V = qkv
    B, H, N, d = Q.shape
    slopes = [0.3, 0.01, 1.0]
    pos = torch.arange(N, dtype=torch.float64)
    bias = torch.stack([-s * (pos[None, :] - pos[:, None]).abs() for s in slopes])[None]
    o, l = O.attention_ref(Q, K, V, scale=0.1875, flags=ALIBI, alibi_slopes=slopes)
    ot, lt = _torch_sdpa(Q, K, V, 0.1875, bias=bias)
    np.testing.assert_allclose(o, ot, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(l, lt, rtol=1e-12, atol=1e-12)


def test_vs_torch_softcap(qkv):
    Q, K, V = qkv
    Q = Q * 6.0  # scores large enough for the cap to bite
    o, l = O.attention_ref(Q, K, V, scale=0.5, flags=SOFTCAP | CAUSAL, softcap=5.0)
    ot, lt = _torch_sdpa(Q, K, V, 0.5, cap=5.0, causal=True, mask=torch.ones(150, 150, dtype=torch.bool).tril())
    np.testing.assert_allclose(o, ot, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(l, lt, rtol=1e-12, atol=1e-12)
    s = O.scores_ref(Q[0, 0], K[0, 0], np.arange(150), scale=0.5, flags=SOFTCAP, softcap=5.0)
    assert np.abs(s).max() < 5.0 and np.abs(s).max() > 4.9


def test_default_alibi_slopes():
    s = O.default_alibi_slopes(16)
    assert s[0] == 2.0 ** -0.5 and s[-1] == 2.0 ** -8
    np.testing.assert_allclose(s[1:] / s[:-1], 2.0 ** -0.5)
    assert O.default_alibi_slopes(8)[0] == 0.5


# ---------------------------------------------------------------------------
# closed forms
# ---------------------------------------------------------------------------

def test_zero_queries_uniform_weights():
    rng = np.random.default_rng(2)
    N, d = 40, 8
    Q = np.zeros((1, 1, N, d))
    K = rng.standard_normal((1, 1, N, d))
    V = rng.standard_normal((1, 1, N, d))
    o, l = O.attention_ref(Q, K, V, scale=1.0, flags=CAUSAL | SOFTCAP, softcap=3.0)
    for q in range(N):
        np.testing.assert_allclose(o[0, 0, q], V[0, 0, :q + 1].mean(axis=0), rtol=1e-12, atol=1e-14)
        assert abs(l[0, 0, q] - math.log(q + 1)) < 1e-12
    o, l = O.attention_ref(Q, K, V, scale=1.0, flags=CAUSAL | WINDOW, window=5)
    for q in range(N):
        lo = max(0, q - 4)
        np.testing.assert_allclose(o[0, 0, q], V[0, 0, lo:q + 1].mean(axis=0), rtol=1e-12, atol=1e-14)
        assert abs(l[0, 0, q] - math.log(q + 1 - lo)) < 1e-12


def test_zero_queries_alibi_geometric_series():
    rng = np.random.default_rng(3)
    N, d, H = 30, 4, 4
    Q = np.zeros((1, H, N, d))
    K = rng.standard_normal((1, H, N, d))
    V = rng.standard_normal((1, H, N, d))
    o, l = O.attention_ref(Q, K, V, scale=1.0, flags=CAUSAL | ALIBI)
    for h in range(H):
        m = 2.0 ** (-8.0 * (h + 1) / H)
        for q in range(N):
            n = q + 1
            closed = math.log((1 - math.exp(-m * n)) / (1 - math.exp(-m)))
            assert abs(l[0, h, q] - closed) < 1e-12
            w = np.exp(-m * (q - np.arange(n)))
            np.testing.assert_allclose(o[0, h, q], (w / w.sum()) @ V[0, h, :n], rtol=1e-11, atol=1e-13)


# ---------------------------------------------------------------------------
# invariants
# ---------------------------------------------------------------------------

def _rand(shape, seed, s=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * s


def test_weights_sum_to_one_and_lse_is_logsumexp():
    Q, K = _rand((1, 2, 50, 8), 1), _rand((1, 2, 50, 8), 2)
    for flags in (0, CAUSAL, CAUSAL | WINDOW | ALIBI, SOFTCAP):
        s = O.scores_ref(Q[0, 1], K[0, 1], np.arange(50), scale=0.4, flags=flags, window=7, softcap=2.0,
                         slope=0.25)
        p = np.exp(s - s.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=1e-14)
        V = np.eye(50)[None, None].repeat(2, axis=1)  # O with V = I is the weight matrix itself
        o, l = O.attention_ref(Q, K, V, scale=0.4, flags=flags, window=7, softcap=2.0,
                               alibi_slopes=[0.0, 0.25])
        np.testing.assert_allclose(o[0, 1], p, rtol=1e-12, atol=1e-15)
        np.testing.assert_allclose(o[0, 1].sum(axis=1), 1.0, rtol=1e-13)
        ref_lse = torch.logsumexp(torch.from_numpy(s), dim=1).numpy()
        np.testing.assert_allclose(l[0, 1], ref_lse, rtol=1e-13)


def test_constant_v_gives_constant_o():
    Q, K = _rand((1, 2, 64, 16), 4, 3.0), _rand((1, 2, 64, 16), 5, 3.0)
    V = np.full((1, 2, 64, 16), 0.37)
    o, _ = O.attention_ref(Q, K, V, scale=0.5, flags=CAUSAL | ALIBI | SOFTCAP, softcap=4.0)
    np.testing.assert_allclose(o, 0.37, rtol=1e-13)


def test_single_visible_key_returns_its_value_row():
    Q, K, V = _rand((1, 2, 30, 8), 6), _rand((1, 2, 30, 8), 7), _rand((1, 2, 30, 8), 8)
    # W = 1: each query sees only itself
    o, l = O.attention_ref(Q, K, V, scale=0.5, flags=CAUSAL | WINDOW, window=1)
    np.testing.assert_allclose(o, V, rtol=1e-14)
    s_self = np.einsum("bhnd,bhnd->bhn", Q, K) * 0.5
    np.testing.assert_allclose(l, s_self, rtol=1e-13, atol=1e-14)
    # causal row 0 and the first token of every document
    doc = np.repeat(np.arange(3), [10, 12, 8]).astype(np.int32)[None]
    o, _ = O.attention_ref(Q, K, V, scale=0.5, flags=CAUSAL | DOCUMENT, doc_id=doc)
    for q0 in (0, 10, 22):
        np.testing.assert_allclose(o[0, :, q0], V[0, :, q0], rtol=1e-14)


def test_noncausal_permutation_invariance():
    Q, K, V = _rand((1, 2, 45, 8), 9), _rand((1, 2, 45, 8), 10), _rand((1, 2, 45, 8), 11)
    perm = np.random.default_rng(12).permutation(45)
    for flags in (0, SOFTCAP):
        o1, l1 = O.attention_ref(Q, K, V, scale=0.3, flags=flags, softcap=1.5)
        o2, l2 = O.attention_ref(Q, K[:, :, perm], V[:, :, perm], scale=0.3, flags=flags, softcap=1.5)
        np.testing.assert_allclose(o1, o2, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(l1, l2, rtol=1e-13)


def test_linear_in_v():
    Q, K, V1, V2 = (_rand((1, 2, 33, 8), s) for s in (13, 14, 15, 16))
    kw = dict(scale=0.3, flags=CAUSAL | ALIBI)
    o1, _ = O.attention_ref(Q, K, V1, **kw)
    o2, _ = O.attention_ref(Q, K, V2, **kw)
    o3, _ = O.attention_ref(Q, K, 2.0 * V1 - 0.5 * V2, **kw)
    np.testing.assert_allclose(o3, 2.0 * o1 - 0.5 * o2, rtol=1e-11, atol=1e-13)


def test_degenerate_masks():
    Q, K, V = _rand((2, 2, 40, 8), 17), _rand((2, 2, 40, 8), 18), _rand((2, 2, 40, 8), 19)
    ref = O.attention_ref(Q, K, V, scale=0.3, flags=CAUSAL)
    wide = O.attention_ref(Q, K, V, scale=0.3, flags=CAUSAL | WINDOW, window=40)
    one_doc = O.attention_ref(Q, K, V, scale=0.3, flags=CAUSAL | DOCUMENT, doc_id=np.zeros((2, 40), np.int32))
    nocap = O.attention_ref(Q, K, V, scale=0.3, flags=CAUSAL | SOFTCAP, softcap=1e30)
    for other in (wide, one_doc, nocap):
        np.testing.assert_allclose(other[0], ref[0], rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(other[1], ref[1], rtol=1e-12)
    zero_slope = O.attention_ref(Q, K, V, scale=0.3, flags=CAUSAL | ALIBI, alibi_slopes=[0.0, 0.0])
    np.testing.assert_allclose(zero_slope[0], ref[0], rtol=1e-12, atol=1e-14)


def test_alibi_row_shift():
    """In the causal case the -slope*q part of slope*(k - q) is constant per row:
    the weights equal those of a bias slope*k, and LSE shifts by exactly -slope*q."""
    Q, K, V = _rand((1, 1, 50, 8), 20), _rand((1, 1, 50, 8), 21), _rand((1, 1, 50, 8), 22)
    slope = 0.125
    o, l = O.attention_ref(Q, K, V, scale=0.3, flags=CAUSAL | ALIBI, alibi_slopes=[slope])
    q = torch.from_numpy(Q[0, 0]); k = torch.from_numpy(K[0, 0]); v = torch.from_numpy(V[0, 0])
    s = (q @ k.T) * float(np.float32(0.3)) + slope * torch.arange(50, dtype=torch.float64)[None, :]
    s = s.masked_fill(~torch.ones(50, 50, dtype=torch.bool).tril(), float("-inf"))
    np.testing.assert_allclose(o[0, 0], (torch.softmax(s, 1) @ v).numpy(), rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(l[0, 0], torch.logsumexp(s, 1).numpy() - slope * np.arange(50), rtol=1e-12,
                               atol=1e-12)


def test_rows_subset_matches_full():
    Q, K, V = _rand((1, 2, 300, 16), 23), _rand((1, 2, 300, 16), 24), _rand((1, 2, 300, 16), 25)
    rows = np.array([0, 1, 127, 128, 255, 299])
    full = O.attention_ref(Q, K, V, scale=0.25, flags=CAUSAL | WINDOW, window=100, chunk=64)
    sub = O.attention_ref(Q, K, V, scale=0.25, flags=CAUSAL | WINDOW, window=100, rows=rows)
    np.testing.assert_array_equal(sub[0], full[0][:, :, rows])
    np.testing.assert_array_equal(sub[1], full[1][:, :, rows])


# ---------------------------------------------------------------------------
# decoding
# ---------------------------------------------------------------------------

def test_decode_bf16_matches_torch():
    bits = np.arange(0, 65536, 7, dtype=np.uint32).astype(np.uint16)
    ours = O.decode_bf16(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    np.testing.assert_array_equal(ours[ok], ref[ok])


def test_decode_e4m3_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ours = O.decode_e4m3(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    np.testing.assert_array_equal(ours[ok], ref[ok])
    assert ours[0x7E] == 448.0 and ours[0x01] == 2.0 ** -9 and ours[0x38] == 1.0


def test_dequant_blocks_uses_row_block_scale():
    codes = np.full((1, 1, 260, 2), 0x38, dtype=np.uint8)  # 1.0
    scales = np.array([[[2.0, 3.0, 0.5]]], dtype=np.float32)
    x = O.dequant_blocks(codes, scales)
    assert x[0, 0, 0, 0] == 2.0 and x[0, 0, 127, 1] == 2.0
    assert x[0, 0, 128, 0] == 3.0 and x[0, 0, 255, 0] == 3.0 and x[0, 0, 256, 0] == 0.5


def test_oracle_cfg1_regression_fixture():
    """Oracle output on sampled rows of configuration 1, written by
    tests/golden/make_golden.py (calls only the generator and the oracle)."""
    import json
    import os
    import workload as W
    with open(os.path.join(os.path.dirname(__file__), "golden", "oracle_cfg1.json")) as f:
        g = json.load(f)
    o, l = O.attention_problem(W.config_problem(1), rows=np.array(g["rows"]))
    np.testing.assert_allclose(o, np.array(g["O"]), rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(l, np.array(g["LSE"]), rtol=1e-13)
