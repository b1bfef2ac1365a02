"""Gradients of the attention definition in float64 -- test infrastructure (see package doc).

The backward pass is the one piece the page "FlashAttention 4: ... για LLMs"
(el.linux-konsole.com) says FA4 still lacks (sections "Κύρια Συμπεράσματα" and
"Συμβατότητα και τρέχουσα κατάσταση": forward-only, no backward pass for training).
Here it is the chain rule through the forward definition of oracle.attention, for
L = sum(O * dO), per (batch, query head h, key/value head h // (H / H_kv)):

  r  = Q K^T                                   (raw dot products)
  s  = r * scale, or cap * tanh(r * scale / cap) with softcap; s -= slope_h |q - k|
       with ALiBi; s = -inf where (q, k) is hidden
  P  = exp(s - LSE)                            (LSE from the same s)
  O  = P V
  dV = P^T dO                                  (summed over the query heads sharing it)
  dP = dO V^T,  D = rowsum(P * dP) = rowsum(dO * O)
  dS = P * (dP - D)
  dR = dS * ds/dr,  ds/dr = scale, or scale * (1 - tanh^2) with softcap
  dQ = dR K,  dK = dR^T Q                      (dK summed over the sharing heads)

Nothing is blocked or fused: every (b, h) builds its full score matrix.
"""

from __future__ import annotations

from typing import Optional, Sequence

import numpy as np

from .attention import ALIBI, SOFTCAP, default_alibi_slopes, visible
from .decode import decode_bf16


def attention_bwd_ref(Q: np.ndarray, K: np.ndarray, V: np.ndarray, dO: np.ndarray, *, scale: float,
                      flags: int = 0, window: int = 0, softcap: float = 0.0,
                      doc_id: Optional[np.ndarray] = None, alibi_slopes: Optional[Sequence[float]] = None,
                      heads: Optional[Sequence[tuple]] = None):
    """(dQ [B][H][N][d], dK [B][H_kv][N][d], dV [B][H_kv][N][d], D [B][H][N]) in float64.
    `heads`, if given, restricts the work to those (b, h) query heads; the gradients of a
    key/value head are then complete only if every query head sharing it is listed."""
    B, H, N, d = Q.shape
    H_kv = K.shape[1]
    if H_kv < 1 or H % H_kv:
        raise ValueError(f"{H} query heads cannot share {H_kv} key/value heads")
    g = H // H_kv
    sc = float(np.float32(scale))
    cap = float(np.float32(softcap))
    slopes = default_alibi_slopes(H) if alibi_slopes is None else np.asarray(alibi_slopes, np.float64)
    pos = np.arange(N)
    dQ = np.zeros(Q.shape)
    dK = np.zeros(K.shape)
    dV = np.zeros(V.shape)
    Dr = np.zeros((B, H, N))
    todo = {(b, h) for b in range(B) for h in range(H)} if heads is None else set(heads)
    for b in range(B):
        vis = visible(pos, pos, flags, window, None if doc_id is None else doc_id[b])
        for h in range(H):
            if (b, h) not in todo:
                continue
            kv = h // g
            r = Q[b, h] @ K[b, kv].T
            if flags & SOFTCAP:
                t = np.tanh(r * sc / cap)
                s = cap * t
                dsdr = sc * (1.0 - t * t)
            else:
                s = r * sc
                dsdr = np.full_like(r, sc)
            if flags & ALIBI:
                s = s - slopes[h] * np.abs(pos[:, None] - pos[None, :]).astype(np.float64)
            s = np.where(vis, s, -np.inf)
            m = s.max(axis=1, keepdims=True)
            e = np.exp(s - m)
            lse = m + np.log(e.sum(axis=1, keepdims=True))
            P = np.exp(s - lse)
            O = P @ V[b, kv]
            dP = dO[b, h] @ V[b, kv].T
            D = (dO[b, h] * O).sum(axis=1)
            dS = P * (dP - D[:, None])
            dR = dS * dsdr
            dQ[b, h] = dR @ K[b, kv]
            dK[b, kv] += dR.T @ Q[b, h]
            dV[b, kv] += P.T @ dO[b, h]
            Dr[b, h] = D
    return dQ, dK, dV, Dr


def attention_bwd_problem(p, dO_bits: np.ndarray, heads: Optional[Sequence[tuple]] = None):
    """Gradients for a bf16 workload.Problem and bf16 output gradients dO [B][H][N][d]."""
    if p.dtype != "bf16":
        raise ValueError("the backward pass takes bf16 inputs")
    Q, K, V = decode_bf16(p.q), decode_bf16(p.k), decode_bf16(p.v)
    return attention_bwd_ref(Q, K, V, decode_bf16(dO_bits), scale=p.scale, flags=p.flags, window=p.window,
                             softcap=p.softcap, doc_id=p.doc_id, alibi_slopes=p.alibi_slopes, heads=heads)
