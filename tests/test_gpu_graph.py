"""GPU: the forward pass captured in a HIP graph (as bench.py times short kernels) gives
the eager result on every replay, with eager work and synchronisation between replays.
Every case prints what it is before it touches the GPU."""

import pytest
import torch

import workload as W
from workload import device as WD

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("case", ["cfg1", "causal_derived", "document_with_map"])
def test_graph_replays_match_eager(case):
    if case == "cfg1":
        p, use_map = W.config_problem(1), False
    elif case == "causal_derived":
        p, use_map = W.make_problem(2, 4, 700, 128, flags=W.ATTN_CAUSAL, seed=60), False
    else:
        p, use_map = W.make_problem(1, 4, 900, 64, flags=W.ATTN_CAUSAL | W.ATTN_DOCUMENT | W.ATTN_ALIBI,
                                    seed=61, doc_len_range=(50, 300)), True
    print("CASE graph", case, flush=True)
    dp = WD.to_device(p)
    WD.step(dp, use_map=use_map)
    torch.cuda.synchronize()
    o_ref, l_ref = dp.o.clone(), dp.lse.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        WD.step(dp, use_map=use_map)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        WD.step(dp, use_map=use_map)
    for _ in range(3):
        dp.o.zero_()
        dp.lse.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(dp.o.view(torch.int16), o_ref.view(torch.int16))
        assert torch.equal(dp.lse.view(torch.int32), l_ref.view(torch.int32))
