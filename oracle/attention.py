"""Exact scaled-dot-product attention in float64 -- the definition, written out.

Test infrastructure (see package doc).  Nothing here is blocked, fused or
reordered: for each (batch, head) the full score rows are built, modified,
masked and normalised, then multiplied by V.

Definition (pages: "FlashAttention 4: ... για LLMs", el.linux-konsole.com,
section "Εισαγωγή": scores are queries times keys, a softmax normalises them,
the result multiplies the values; the score/mask variants are the four named
in the opening section of "PyTorchs FlexAttention mit FlashAttention-4 ist ein
Game-Changer", liora.io):

  s[q, k]   = (Q[q] . K[k]) * scale                       (scale: the fp32 value)
  softcap:    s <- cap * tanh(s / cap)                     (applied to scaled scores)
  ALiBi:      s <- s - slope_h * |q - k|                   (= slope_h*(k - q) when k <= q)
  mask:       s <- -inf where (q, k) is not visible
  visible  =  [k <= q             if CAUSAL]
            & [|q - k| <= W - 1    if WINDOW]   (with CAUSAL: exactly W keys, self included)
            & [doc[q] == doc[k]    if DOCUMENT]
  m = max_k s,  l = sum_k exp(s - m),  LSE = m + ln l,  O = sum_k exp(s - m) V[k] / l
  a row with no visible key: O = 0, LSE = -inf.
  grouped-query attention (GQA; MQA with one key/value head): K and V carry H_kv
  heads, H_kv dividing H, and query head h reads key/value head h // (H / H_kv)
  (same page, section "Συμβατότητα και τρέχουσα κατάσταση": several query heads
  share one key/value projection).
  variable-length batches (same section: sequences of different lengths batched
  without padding): sequences packed back to back along one token axis, given by
  cumulative offsets cu[0] = 0 <= cu[1] <= ... <= cu[nseq] = total; each sequence
  is the definition above applied to its own tokens, positions counted from its
  first token.

Readings where the pages are silent: scale first, then softcap, then ALiBi,
then the mask; default ALiBi slopes 2^(-8(h+1)/H) for heads h = 0..H-1;
natural-log LSE; under GQA consecutive query heads share a key/value head;
a packed batch keeps the head-major [H][total][d] layout of one batch row.
"""

from __future__ import annotations

import math
import os
from typing import Optional, Sequence

import numpy as np

from .decode import decode_problem

CAUSAL, WINDOW, DOCUMENT, ALIBI, SOFTCAP = 1, 2, 4, 8, 16


def default_alibi_slopes(H: int) -> np.ndarray:
    """Geometric ALiBi slopes 2^(-8/H), 2^(-16/H), ..., 2^(-8) (float64)."""
    return np.array([2.0 ** (-8.0 * (h + 1) / H) for h in range(H)], dtype=np.float64)


def visible(qpos: np.ndarray, kpos: np.ndarray, flags: int, window: int,
            doc_row: Optional[np.ndarray]) -> np.ndarray:
    """Boolean [len(qpos), len(kpos)]: may query qpos[i] attend to key kpos[j]?"""
    qpos = np.asarray(qpos, dtype=np.int64)[:, None]
    kpos = np.asarray(kpos, dtype=np.int64)[None, :]
    vis = np.ones((qpos.shape[0], kpos.shape[1]), dtype=bool)
    if flags & CAUSAL:
        vis &= kpos <= qpos
    if flags & WINDOW:
        vis &= np.abs(qpos - kpos) <= window - 1
    if flags & DOCUMENT:
        doc_row = np.asarray(doc_row)
        vis &= doc_row[qpos] == doc_row[kpos]
    return vis


def scores_ref(Qh: np.ndarray, Kh: np.ndarray, rows: np.ndarray, *, scale: float, flags: int,
               window: int = 0, softcap: float = 0.0, doc_row=None, slope: float = 0.0) -> np.ndarray:
    """Masked, modified scores s[rows, :] for one (batch, head); -inf where hidden."""
    N = Kh.shape[0]
    kpos = np.arange(N)
    s = (Qh[rows] @ Kh.T) * float(np.float32(scale))
    if flags & SOFTCAP:
        cap = float(np.float32(softcap))
        s = cap * np.tanh(s / cap)
    if flags & ALIBI:
        s = s - slope * np.abs(rows[:, None].astype(np.float64) - kpos[None, :].astype(np.float64))
    vis = visible(rows, kpos, flags, window, doc_row)
    return np.where(vis, s, -np.inf)


def _softmax_rows(s: np.ndarray, Vh: np.ndarray):
    m = s.max(axis=1)
    empty = ~np.isfinite(m)
    m_safe = np.where(empty, 0.0, m)
    p = np.exp(s - m_safe[:, None])  # exp(-inf) = 0 for hidden keys
    l = p.sum(axis=1)
    with np.errstate(divide="ignore", invalid="ignore"):
        o = (p @ Vh) / l[:, None]
        lse = m_safe + np.log(l)
    o[empty] = 0.0
    lse[empty] = -np.inf
    return o, lse


def attention_ref(Q: np.ndarray, K: np.ndarray, V: np.ndarray, *, scale: float, flags: int = 0,
                  window: int = 0, softcap: float = 0.0, doc_id: Optional[np.ndarray] = None,
                  alibi_slopes: Optional[Sequence[float]] = None, rows: Optional[np.ndarray] = None,
                  heads: Optional[Sequence[tuple]] = None, chunk: int = 1024):
    """O [B][H][R][d] and LSE [B][H][R] (float64) for query rows `rows` (default: all).

    Q: float64 [B][H][N][d]; K, V: float64 [B][H_kv][N][d] with H_kv dividing H
    (H_kv = H: one key/value head per query head).  `heads`, if given, restricts the
    work to a list of (b, h) pairs; the other outputs are left as NaN.
    """
    B, H, N, d = Q.shape
    H_kv = K.shape[1]
    if H_kv < 1 or H % H_kv or V.shape[1] != H_kv:
        raise ValueError(f"{H} query heads cannot share {H_kv} key/value heads")
    group = H // H_kv
    rows = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64)
    R = rows.shape[0]
    slopes = default_alibi_slopes(H) if alibi_slopes is None else np.asarray(alibi_slopes, np.float64)
    O = np.full((B, H, R, Q.shape[3] if V is None else V.shape[3]), np.nan)
    L = np.full((B, H, R), np.nan)
    pairs = [(b, h) for b in range(B) for h in range(H)] if heads is None else list(heads)
    for (b, h) in pairs:
        doc_row = None if doc_id is None else doc_id[b]
        for c0 in range(0, R, chunk):
            rr = rows[c0:c0 + chunk]
            s = scores_ref(Q[b, h], K[b, h // group], rr, scale=scale, flags=flags, window=window,
                           softcap=softcap, doc_row=doc_row, slope=float(slopes[h]))
            O[b, h, c0:c0 + chunk], L[b, h, c0:c0 + chunk] = _softmax_rows(s, V[b, h // group])
    return O, L


def varlen_doc_ids_ref(cu_seqlens: np.ndarray, total: int) -> np.ndarray:
    """int32 [total]: the index of the sequence each packed token belongs to (the last
    sequence starting at or before it, so empty sequences own no token)."""
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    ids = np.zeros(total, dtype=np.int32)
    for i in range(len(cu) - 1):
        ids[cu[i]:cu[i + 1]] = i
    return ids


def attention_varlen_ref(Q: np.ndarray, K: np.ndarray, V: np.ndarray, cu_seqlens, *, scale: float,
                         flags: int = 0, window: int = 0, softcap: float = 0.0,
                         alibi_slopes: Optional[Sequence[float]] = None, rows: Optional[np.ndarray] = None,
                         heads: Optional[Sequence[int]] = None):
    """O [H][R][d] and LSE [H][R] of a packed variable-length batch: every sequence on
    its own (attention_ref on its slice, positions local to it), results placed back
    at the packed rows.  Q: [H][total][d]; K, V: [H_kv][total][d]; cu_seqlens:
    [nseq + 1].  `rows` selects packed query rows, `heads` query heads (others NaN)."""
    if flags & DOCUMENT:
        raise ValueError("the sequences of a packed batch are its documents")
    H, total, _ = Q.shape
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    if cu[0] != 0 or cu[-1] != total or np.any(np.diff(cu) < 0):
        raise ValueError("cu_seqlens must run from 0 to total without decreasing")
    rows = np.arange(total) if rows is None else np.asarray(rows, dtype=np.int64)
    O = np.full((H, len(rows), V.shape[2]), np.nan)
    L = np.full((H, len(rows)), np.nan)
    hs = range(H) if heads is None else list(heads)
    for i in range(len(cu) - 1):
        a, e = int(cu[i]), int(cu[i + 1])
        sel = np.nonzero((rows >= a) & (rows < e))[0]
        if len(sel) == 0:
            continue
        o, l = attention_ref(Q[None, :, a:e], K[None, :, a:e], V[None, :, a:e], scale=scale, flags=flags,
                             window=window, softcap=softcap, alibi_slopes=alibi_slopes, rows=rows[sel] - a,
                             heads=[(0, h) for h in hs])
        O[:, sel], L[:, sel] = o[0], l[0]
    return O, L


# ---------------------------------------------------------------------------
# Whole-problem driver (optionally over a process pool: one task per (b, h))
# ---------------------------------------------------------------------------

_POOL_STATE = {}


def _pool_task(bh):
    st = _POOL_STATE
    Q, K, V = st["qkv"]
    o, l = attention_ref(Q, K, V, heads=[bh], **st["kw"])
    b, h = bh
    return bh, o[b, h], l[b, h]


def attention_problem(p, rows: Optional[np.ndarray] = None, heads: Optional[Sequence[tuple]] = None,
                      workers: int = 1):
    """Oracle outputs for a workload.Problem (decoded exactly to float64 first).

    Returns (O, LSE) with the same shapes as attention_ref.  With workers > 1
    the (b, h) pairs are spread over a fork()ed process pool, one BLAS thread
    per worker.
    """
    Q, K, V = decode_problem(p)
    if getattr(p, "cu_seqlens", None) is not None:
        hs = None if heads is None else sorted({h for (_, h) in heads})
        o, l = attention_varlen_ref(Q[0], K[0], V[0], p.cu_seqlens, scale=p.scale, flags=p.flags,
                                    window=p.window, softcap=p.softcap, alibi_slopes=p.alibi_slopes, rows=rows,
                                    heads=hs)
        return o[None], l[None]
    kw = dict(scale=p.scale, flags=p.flags, window=p.window, softcap=p.softcap, doc_id=p.doc_id,
              alibi_slopes=p.alibi_slopes, rows=rows)
    if workers <= 1:
        return attention_ref(Q, K, V, heads=heads, **kw)
    import multiprocessing as mp
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # pragma: no cover
        threadpool_limits = None
    B, H, N, d = Q.shape
    R = N if rows is None else len(rows)
    pairs = [(b, h) for b in range(B) for h in range(H)] if heads is None else list(heads)
    O = np.full((B, H, R, d), np.nan)
    L = np.full((B, H, R), np.nan)
    _POOL_STATE["qkv"] = (Q, K, V)
    _POOL_STATE["kw"] = kw
    ctx = mp.get_context("fork")
    init = (lambda: threadpool_limits(1)) if threadpool_limits else None
    try:
        with ctx.Pool(processes=min(workers, len(pairs)), initializer=init) as pool:
            for (b, h), o, l in pool.imap_unordered(_pool_task, pairs):
                O[b, h], L[b, h] = o, l
    finally:
        _POOL_STATE.clear()
    return O, L


def available_cores() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1
