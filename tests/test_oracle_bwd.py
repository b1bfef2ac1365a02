"""Pins of the oracle's backward pass (oracle/attention_bwd.py) against routes that do
not share its hand-derived chain rule: torch autograd in float64 through a forward
written with torch ops, central finite differences of the forward oracle, and an
invariance of softmax attention."""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle.attention_bwd import attention_bwd_ref

CAUSAL, WINDOW, DOCUMENT, ALIBI, SOFTCAP = 1, 2, 4, 8, 16


def _torch_grads(Q, K, V, dO, scale, flags, W, cap, doc, slopes):
    """Autograd of L = sum(O * dO) through the definition written in torch ops (GQA by
    repeating the key/value heads, so the gradients of the shared heads are summed)."""
    q = torch.tensor(Q, requires_grad=True)
    k = torch.tensor(K, requires_grad=True)
    v = torch.tensor(V, requires_grad=True)
    B, H, N, d = Q.shape
    g = H // K.shape[1]
    kk = torch.repeat_interleave(k, g, dim=1)
    vv = torch.repeat_interleave(v, g, dim=1)
    r = q @ kk.transpose(-1, -2)
    s = cap * torch.tanh(r * scale / cap) if flags & SOFTCAP else r * scale
    i = torch.arange(N)
    dist = (i[:, None] - i[None, :]).abs().double()
    if flags & ALIBI:
        s = s - torch.tensor(slopes, dtype=torch.float64)[None, :, None, None] * dist
    vis = torch.ones(B, 1, N, N, dtype=torch.bool)
    if flags & CAUSAL:
        vis &= (i[None, :] <= i[:, None])
    if flags & WINDOW:
        vis &= dist <= W - 1
    if flags & DOCUMENT:
        dd = torch.tensor(doc)
        vis &= (dd[:, None, :, None] == dd[:, None, None, :])
    s = s.masked_fill(~vis, float("-inf"))
    o = torch.softmax(s, dim=-1) @ vv
    (o * torch.tensor(dO)).sum().backward()
    return q.grad.numpy(), k.grad.numpy(), v.grad.numpy()


@pytest.mark.parametrize("H,H_kv", [(2, 2), (4, 2), (3, 1)])
@pytest.mark.parametrize("N,d", [(1, 4), (7, 3), (20, 8)])
def test_matches_torch_autograd_all_flag_combinations(N, d, H, H_kv):
    rng = np.random.default_rng([N, d, H, H_kv])
    B = 2
    Q = rng.standard_normal((B, H, N, d))
    K = rng.standard_normal((B, H_kv, N, d))
    V = rng.standard_normal((B, H_kv, N, d))
    dO = rng.standard_normal((B, H, N, d))
    doc = np.stack([np.sort(rng.integers(0, 3, N)) for _ in range(B)]).astype(np.int32)
    slopes = [0.5 / (h + 1) for h in range(H)]
    scale, W, cap = 0.375, 4, 1.25  # exact in fp32
    for flags in range(32):
        dQ, dK, dV, _ = attention_bwd_ref(Q, K, V, dO, scale=scale, flags=flags, window=W, softcap=cap,
                                          doc_id=doc, alibi_slopes=slopes)
        tq, tk, tv = _torch_grads(Q, K, V, dO, scale, flags, W, cap, doc, slopes)
        for a, b_, name in ((dQ, tq, "dQ"), (dK, tk, "dK"), (dV, tv, "dV")):
            np.testing.assert_allclose(a, b_, rtol=1e-9, atol=1e-11, err_msg=f"{name} flags {flags}")


@pytest.mark.parametrize("flags", [0, CAUSAL | SOFTCAP, WINDOW | ALIBI, CAUSAL | DOCUMENT | ALIBI | SOFTCAP])
def test_matches_finite_differences_of_the_forward_oracle(flags):
    """Central differences of L = sum(attention_ref(...) * dO) in each of Q, K and V."""
    rng = np.random.default_rng([flags, 11])
    B, H, H_kv, N, d = 1, 2, 1, 6, 3
    Q = rng.standard_normal((B, H, N, d))
    K = rng.standard_normal((B, H_kv, N, d))
    V = rng.standard_normal((B, H_kv, N, d))
    dO = rng.standard_normal((B, H, N, d))
    kw = dict(scale=0.5, flags=flags, window=3, softcap=2.0, doc_id=np.array([[0, 0, 0, 1, 1, 1]], np.int32),
              alibi_slopes=[0.25, 0.125])
    dQ, dK, dV, _ = attention_bwd_ref(Q, K, V, dO, **kw)

    def loss(Q_, K_, V_):
        o, _ = oracle.attention_ref(Q_, K_, V_, **kw)
        return float((o * dO).sum())

    eps = 1e-6
    for X, G, which in ((Q, dQ, 0), (K, dK, 1), (V, dV, 2)):
        for idx in [(0, 0, 0, 0), (0, X.shape[1] - 1, N - 1, d - 1), (0, 0, 3, 1)]:
            Xp, Xm = X.copy(), X.copy()
            Xp[idx] += eps
            Xm[idx] -= eps
            args_p = [Q, K, V]
            args_m = [Q, K, V]
            args_p[which], args_m[which] = Xp, Xm
            fd = (loss(*args_p) - loss(*args_m)) / (2 * eps)
            assert math.isclose(fd, G[idx], rel_tol=1e-6, abs_tol=1e-8), (which, idx, fd, G[idx])


@pytest.mark.parametrize("flags", [0, CAUSAL, CAUSAL | WINDOW | ALIBI])
def test_key_shift_changes_nothing_without_softcap(flags):
    """Adding one vector c to every key adds q.c to a whole score row: softmax, O, dV and
    dQ stay (the rows of dS sum to zero), and dK gains nothing either."""
    rng = np.random.default_rng([flags, 12])
    Q, K, V, dO = (rng.standard_normal((1, 2, 9, 4)) for _ in range(4))
    c = rng.standard_normal(4)
    kw = dict(scale=0.5, flags=flags, window=4, alibi_slopes=[0.3, 0.1])
    a = attention_bwd_ref(Q, K, V, dO, **kw)
    b = attention_bwd_ref(Q, K + c, V, dO, **kw)
    for x, y in zip(a, b):
        np.testing.assert_allclose(x, y, rtol=1e-9, atol=1e-10)


def test_delta_is_the_row_sum_of_dO_times_O():
    rng = np.random.default_rng(13)
    Q, K, V, dO = (rng.standard_normal((1, 1, 10, 4)) for _ in range(4))
    _, _, _, D = attention_bwd_ref(Q, K, V, dO, scale=0.5, flags=CAUSAL)
    o, _ = oracle.attention_ref(Q, K, V, scale=0.5, flags=CAUSAL)
    np.testing.assert_allclose(D, (o * dO).sum(-1), rtol=1e-12)
