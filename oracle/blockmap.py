"""Block map by brute force -- test infrastructure (see package doc).

Block sparsity (skipping fully masked blocks) is named in "PyTorchs
FlexAttention mit FlashAttention-4 ist ein Game-Changer" (liora.io), section
"Aktuelle Einschränkungen".  The map is defined here directly from the
visibility predicate, evaluated for every (query, key) position:

  class[b][qb][kb] (blocks of 128 queries x 128 keys):
      EMPTY   = 0  no in-range position of the block is visible
      FULL    = 2  all 128 x 128 positions are in range and visible
      PARTIAL = 1  otherwise (so blocks cut by the sequence end are never FULL)
  counts[b][qb] = (#FULL, #PARTIAL)
  idx[b][qb][0][:] = FULL kb in ascending order, then -1 padding
  idx[b][qb][1][:] = PARTIAL kb in ascending order, then -1 padding
  row_lo[b][q], row_hi[b][q] = smallest and largest visible key of query q
      (0 and -1 for a row with no visible key)
  col_lo[b][k], col_hi[b][k] = smallest and largest query that sees key k
      (0 and -1 for a key no query sees)
  qb_pairs[b][qb] = visible (q, k) pairs of the query rows of block qb
  status[b][qb] = 1 if doc_id[b][q + 1] < doc_id[b][q] for some row q of block qb
      (documents must be contiguous runs; only evaluated with the DOCUMENT flag)

(The device map also holds a work order of the query blocks; that is the library's
scheduling choice, not part of the method, so it has no definition here: the tests
check it as a property of the device's own stated cost.)

The visible-pair count is the number of (b, q, k) with visible(q, k); the
metric's "unmasked FLOPs" are 4 * H * d times it.
"""

from __future__ import annotations

from typing import Optional

import numpy as np

from .attention import DOCUMENT, visible

EMPTY, PARTIAL, FULL = 0, 1, 2
BLOCK = 128


def blockmap_ref(B: int, N: int, flags: int, window: int = 0, doc_id: Optional[np.ndarray] = None,
                 block: int = BLOCK) -> dict:
    nqb = (N + block - 1) // block
    cls = np.zeros((B, nqb, nqb), dtype=np.uint8)
    counts = np.zeros((B, nqb, 2), dtype=np.int32)
    idx = np.full((B, nqb, 2, nqb), -1, dtype=np.int32)
    row_lo = np.zeros((B, N), dtype=np.int32)
    row_hi = np.full((B, N), -1, dtype=np.int32)
    col_lo = np.zeros((B, N), dtype=np.int32)
    col_hi = np.full((B, N), -1, dtype=np.int32)
    pairs = np.zeros(B, dtype=np.int64)
    qb_pairs = np.zeros((B, nqb), dtype=np.int64)
    status = np.zeros((B, nqb), dtype=np.int32)
    kpos = np.arange(N)
    for b in range(B):
        doc_row = None if doc_id is None else np.asarray(doc_id[b])
        for qb in range(nqb):
            q0, q1 = qb * block, min(N, (qb + 1) * block)
            vis = visible(np.arange(q0, q1), kpos, flags, window, doc_row)  # [rows][N]
            qb_pairs[b, qb] = int(vis.sum())
            pairs[b] += qb_pairs[b, qb]
            if flags & DOCUMENT:
                rows = np.arange(q0, min(q1, N - 1))
                status[b, qb] = int(np.any(doc_row[rows + 1] < doc_row[rows]))
            anyv = vis.any(axis=1)
            r = np.nonzero(anyv)[0]
            row_lo[b, q0 + r] = vis[r].argmax(axis=1)
            row_hi[b, q0 + r] = N - 1 - vis[r, ::-1].argmax(axis=1)
            # blocks go by increasing query: a key's first seeing block gives col_lo, its
            # last one col_hi
            seen = vis.any(axis=0)
            first = seen & (col_hi[b] < 0)
            col_lo[b, first] = q0 + vis[:, first].argmax(axis=0)
            col_hi[b, seen] = q1 - 1 - vis[::-1, seen].argmax(axis=0)
            for kb in range(nqb):
                k0, k1 = kb * block, min(N, (kb + 1) * block)
                sub = vis[:, k0:k1]
                if not sub.any():
                    c = EMPTY
                elif sub.all() and (q1 - q0) == block and (k1 - k0) == block:
                    c = FULL
                else:
                    c = PARTIAL
                cls[b, qb, kb] = c
            full = np.nonzero(cls[b, qb] == FULL)[0]
            part = np.nonzero(cls[b, qb] == PARTIAL)[0]
            counts[b, qb] = (len(full), len(part))
            idx[b, qb, 0, :len(full)] = full
            idx[b, qb, 1, :len(part)] = part
    return dict(cls=cls, counts=counts, idx=idx, row_lo=row_lo, row_hi=row_hi, col_lo=col_lo, col_hi=col_hi,
                pairs=pairs,
                qb_pairs=qb_pairs, status=status, visible_pairs=int(pairs.sum()))


def row_intervals_ref(N: int, flags: int, window: int = 0, doc_row=None):
    """(lo, hi, contiguous) per query for one batch row, by brute force.

    `contiguous` tells whether every row's visible keys form the single
    interval [lo, hi] (true for causal/window masks and for documents that are
    contiguous runs of tokens)."""
    vis = visible(np.arange(N), np.arange(N), flags, window, doc_row)
    anyv = vis.any(axis=1)
    lo = np.where(anyv, vis.argmax(axis=1), 0)
    hi = np.where(anyv, N - 1 - vis[:, ::-1].argmax(axis=1), -1)
    kpos = np.arange(N)[None, :]
    interval = (kpos >= lo[:, None]) & (kpos <= hi[:, None])
    return lo.astype(np.int32), hi.astype(np.int32), bool((interval == vis).all())


def visible_pairs_ref(B: int, N: int, flags: int, window: int = 0, doc_id=None) -> int:
    total = 0
    kpos = np.arange(N)
    for b in range(B):
        doc_row = None if doc_id is None else np.asarray(doc_id[b])
        for q0 in range(0, N, 1024):
            total += int(visible(np.arange(q0, min(N, q0 + 1024)), kpos, flags, window, doc_row).sum())
    return total
