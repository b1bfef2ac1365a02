"""Rescale events of the online softmax (attn_fwd_rescale_counts): the count per query row
of steps in which the offset in use was replaced, for the threshold tau (the page "FlashAttention
4: ... για LLMs", section "Έξυπνος επανακανονισμός Softmax ...").  Pinned by a closed form
on inputs whose per-step maximum rises by a fixed amount, and by properties on the
configuration workloads: every row counts at least its first visible step, never more than its
steps, and tau = 8 never counts more than tau = 0 (an event at tau = 8 means the maximum passed
the offset by more than 8, so it also passed the running maximum, the tau = 0 offset)."""

import math

import numpy as np
import pytest
import torch

import oracle
import workload as W
from workload import device as WD
from exact_attention_119_amd import lib as L
from _parity import assert_close

pytestmark = pytest.mark.gpu


def _announce(*a):
    print("CASE", *a, flush=True)


def _counts(dp, tau, use_map=False):
    p = dp.p
    counts = torch.full((p.B, p.H, p.N), -1, dtype=torch.int32, device="cuda")
    dp.o.fill_(float("nan"))
    dp.lse.fill_(float("nan"))
    if use_map or WD.needs_map(dp):
        WD.build_map(dp)
    L.attn_fwd_rescale_counts(dp.q, dp.k, dp.v, dp.o, dp.lse, counts, scale=p.scale, dtype=dp.dtype, mask=dp.mask,
                              blockmap=dp.blockmap if (use_map or WD.needs_map(dp)) else None, rescale_tau=tau)
    torch.cuda.synchronize()
    return counts.cpu().numpy(), WD.outputs(dp)


@pytest.mark.parametrize("d", [64, 128])
def test_closed_form_on_a_rising_maximum(d):
    """No mask, N = 1024 (16 steps of 64 keys, taken in ascending order): every key of step
    s scores 3s in log2 units for every query, so the maximum rises by 3 per step.  tau = 0
    replaces the offset in every step (16 events); tau = 8 only once it has risen by more
    than 8, i.e. every third step: steps 0, 3, ..., 15 (6 events)."""
    N, H = 1024, 2
    p = W.make_problem(1, H, N, d, seed=(71, d))
    c = p.scale * math.log2(math.e)
    q = np.zeros((1, H, N, d), np.float32)
    q[..., 0] = 1.0
    k = np.zeros((1, H, N, d), np.float32)
    k[..., 0] = (3.0 * (np.arange(N) // 64) / c)[None, None, :]
    p.q, p.k = W.bf16_bits_from_f32(q), W.bf16_bits_from_f32(k)
    _announce("rescale closed form", d)
    dp = WD.to_device(p)
    o_ref, lse_ref = oracle.attention_problem(p)
    for tau, expect in ((0.0, 16), (8.0, 6)):
        counts, (o, lse) = _counts(dp, tau)
        np.testing.assert_array_equal(counts, expect, err_msg=f"tau={tau}")
        assert_close(p, o, lse, o_ref, lse_ref, f"rescale counting pass tau={tau}")


@pytest.mark.parametrize("cfg", [2, 3])
def test_config_counts_properties_and_rate(cfg):
    """Configurations 2 and 3: mean rescale events per row at tau = 0 and tau = 8, with the
    properties above; the forward outputs of the counting pass match the plain pass."""
    p = W.config_problem(cfg)
    _announce("rescale counts cfg", cfg)
    dp = WD.to_device(p)
    c0, (o0, l0) = _counts(dp, 0.0)
    c8, (o8, l8) = _counts(dp, 8.0)
    WD.step(dp, 8.0, use_map=False)
    o, lse = WD.outputs(dp)
    np.testing.assert_array_equal(o8, o)
    np.testing.assert_array_equal(l8, lse)
    # steps with a visible key per row: the row's visible keys span its 64-key steps
    q = np.arange(p.N)
    lo = np.maximum(0, q - p.window + 1) if p.flags & W.ATTN_WINDOW else np.zeros_like(q)
    steps_max = q // 64 - lo // 64 + 1  # (an upper bound: the steps touching [lo, q])
    assert (c0 >= 1).all() and (c8 >= 1).all()
    assert (c8 <= c0).all()
    assert (c0 <= steps_max[None, None, :]).all()
    r0, r8 = float((c0 - 1).mean()), float((c8 - 1).mean())
    print(f"cfg{cfg}: rescales per row after the first step: tau=0 {r0:.3f}, tau=8 {r8:.4f} "
          f"(events incl. the first: {c0.mean():.3f} / {c8.mean():.3f})", flush=True)
