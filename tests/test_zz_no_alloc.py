"""The backward pass without a workspace (attn_bwd_gqa_noalloc), for callers that cannot
allocate: its row sums live in the library's per-GPU scratch array.  Through the C ABI it
must give the same bits as attn_bwd_gqa with a caller-owned delta buffer, on two calls in
a row, the second smaller than the first (the scratch array keeps the first call's
contents; nothing of it may leak into the second)."""

import numpy as np
import pytest
import torch

import workload as W
from workload import device as WD
from exact_attention_119_amd import lib as L

pytestmark = pytest.mark.gpu

C, WI, DOC, AL, SC = W.ATTN_CAUSAL, W.ATTN_WINDOW, W.ATTN_DOCUMENT, W.ATTN_ALIBI, W.ATTN_SOFTCAP


def _prepare(p, seed):
    dp = WD.to_device(p)
    WD.step(dp)
    dout = torch.from_numpy(W.make_dout(p, seed=seed).view(np.int16)).cuda().view(torch.bfloat16)
    return dp, dout


def _grads(dp, dout, noalloc):
    p = dp.p
    dq = torch.full_like(dp.q, float("nan"))
    dk = torch.full_like(dp.k, float("nan"))
    dv = torch.full_like(dp.v, float("nan"))
    if noalloc:
        L.attn_bwd_gqa_noalloc(dp.q, dp.k, dp.v, dp.o, dp.lse, dout, dq, dk, dv, scale=p.scale, mask=dp.mask,
                               blockmap=dp.blockmap)
    else:
        delta = torch.empty_like(dp.lse)
        L.attn_bwd_gqa(dp.q, dp.k, dp.v, dp.o, dp.lse, dout, dq, dk, dv, delta, scale=p.scale, mask=dp.mask,
                       blockmap=dp.blockmap)
    return dq, dk, dv


def test_noalloc_backward_equals_the_workspace_call_twice_in_a_row():
    big = W.make_problem(2, 8, 1000, 128, flags=C | WI | SC, window=300, softcap=20.0, seed=(91, 1), H_kv=4)
    small = W.make_problem(1, 4, 300, 64, flags=C | DOC | AL, seed=(91, 2), doc_len_range=(40, 150), H_kv=2)
    print("CASE no-alloc backward", big.name, small.name, flush=True)
    prepared = [_prepare(big, 1), _prepare(small, 2)]
    refs = [_grads(dp, dout, noalloc=False) for dp, dout in prepared]
    torch.cuda.synchronize()
    got = [_grads(dp, dout, noalloc=True) for dp, dout in prepared]  # two calls in a row, the second smaller
    torch.cuda.synchronize()
    for (dp, _), r, g in zip(prepared, refs, got):
        for name, a, b in zip(("dQ", "dK", "dV"), r, g):
            assert not torch.isnan(b.float()).any(), f"{dp.p.name} {name}: not fully written"
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"{dp.p.name} {name}: bits differ"
        print(f"{dp.p.name}: dQ, dK, dV bit-identical to the workspace call", flush=True)
