"""GPU parity at the largest inputs: a causal forward pass whose Q, K, V and O hold 2^31
elements each (4 GiB apiece in bf16), so that the heads past the 2^31-byte and 2^32-byte
marks are reached only through 64-bit offsets.  The 64 heads are built on the device from
two generated heads, each scaled by its own combination of powers of two (exact in bf16),
so that no two heads hold the same inputs and a head read at the wrong offset would give
other outputs; the fp64 oracle runs on sampled rows of eight heads spread over the range."""

import numpy as np
import pytest
import torch

import oracle
import workload as W
from exact_attention_119_amd import lib as L
from _parity import assert_close, sample_rows

pytestmark = pytest.mark.gpu


def _scales(h):
    """Q, K and V multipliers of head h: powers of two, a different triple (with the
    base head h % 2) for each of the 64 heads; V's are at most 1, so that |O| stays
    within the unit-scale range the absolute bf16 tolerance is set for."""
    return 2.0 ** ((h >> 1) % 4 - 2), 2.0 ** ((h >> 3) % 2 - 1), 2.0 ** -((h >> 4) % 4)


def test_two_to_the_31_elements_per_tensor_causal_sampled():
    H, N, d = 64, 1 << 18, 128
    assert H * N * d == 1 << 31
    base = W.make_problem(1, 2, N, d, flags=W.ATTN_CAUSAL, seed=(31, 1))
    print("CASE large: B1 H64 N262144 d128 causal, two base heads", flush=True)
    dev = [torch.from_numpy(np.ascontiguousarray(x.view(np.int16))).cuda().view(torch.bfloat16)
           for x in (base.q, base.k, base.v)]
    q, k, v = (torch.empty((1, H, N, d), dtype=torch.bfloat16, device="cuda") for _ in range(3))
    for h in range(H):
        for t, src, s in zip((q, k, v), dev, _scales(h)):
            t[0, h] = src[0, h % 2] * s  # a power of two: exact
    del dev
    o = torch.full_like(q, float("nan"))
    lse = torch.full((1, H, N), float("nan"), dtype=torch.float32, device="cuda")
    L.attn_fwd(q, k, v, o, lse, scale=base.scale, mask=L.make_mask(L.ATTN_CAUSAL))
    torch.cuda.synchronize()
    assert not torch.isnan(o).any().item() and not torch.isnan(lse).any().item()
    rows = sample_rows(N, 24, seed=31)
    rows_t = torch.from_numpy(rows).cuda()
    Qb, Kb, Vb = (oracle.decode_bf16(x)[0] for x in (base.q, base.k, base.v))  # [2][N][d] float64
    for h in (0, 1, 15, 16, 31, 32, 47, 63):
        sq, sk, sv = _scales(h)
        b = h % 2
        o_ref, lse_ref = oracle.attention_ref((Qb[b] * sq)[None, None], (Kb[b] * sk)[None, None],
                                              (Vb[b] * sv)[None, None], scale=base.scale, flags=L.ATTN_CAUSAL,
                                              rows=rows)
        og = o[0, h].index_select(0, rows_t).float().cpu().numpy()[None, None]
        lg = lse[0, h].index_select(0, rows_t).cpu().numpy()[None, None]
        assert_close(base, og, lg, o_ref, lse_ref, f"2^31 elements, head {h}")
