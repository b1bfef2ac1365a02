"""P.V on the f8f6f4 MFMA with P in e4m3 (ATTN_PV_E4M3, FlashAttention-3's all-FP8 product)
or in E2M1 with one E8M0 scale per 32 keys (ATTN_PV_FP4, the "Direct-P" of "Hardware-Aware
FP4 FlashAttention-4"): measured variants for non-causal inference.

Their operand layouts are pinned exactly: on inputs whose probabilities are all powers of
two that both formats hold (every key scores 0, -1, -2 or -3 in log2 units, V block scales
equal), rounding P changes nothing, so the variants must match the fp64 oracle like any
exact path; a V^T byte taken from the wrong key, a P value in the wrong nibble or a wrong
block scale would show there.  On configuration 5 their error against the oracle is
measured and printed (it is the rounding of P, not gated)."""

import math

import numpy as np
import pytest
import torch

import oracle
import workload as W
from workload import device as WD
from exact_attention_119_amd import lib as L
from oracle import fp4 as F4
from _parity import assert_close, errors, sample_rows

pytestmark = pytest.mark.gpu

MODES = {"e4m3": L.ATTN_PV_E4M3, "fp4": L.ATTN_PV_FP4}


def _announce(*a):
    print("CASE", *a, flush=True)


def _run(p, pv_mode, tau=8.0):
    dp = WD.to_device(p, pv_mode=pv_mode, qk_mode=L.ATTN_QK_E4M3)
    dp.o.fill_(float("nan"))
    dp.lse.fill_(float("nan"))
    WD.step(dp, tau)
    return WD.outputs(dp)


def _exact_p_problem(N, seed):
    """B1 H2 d128 fp8: Q = e_0, key j = -k_j e_0 with k_j in {0, 1, 2, 3} drawn per key, all
    scales 1 (V's shared by every block), scale = ln 2 so that a score in log2 units is
    exactly -k_j: P = 2^-k_j, held exactly by e4m3 and by E2M1 with the block scale 2^-2."""
    p = W.make_problem(1, 2, N, 128, dtype="fp8", seed=(88, N, seed))
    rng = np.random.default_rng([119, 88, N, seed])
    k = rng.integers(0, 4, size=(1, 2, N))
    q = np.zeros_like(p.q)
    q[..., 0] = 0x38
    kc = np.zeros_like(p.k)
    kc[..., 0] = oracle.e4m3_encode(-k.astype(np.float64))
    p.q, p.k = q, kc
    p.q_scale = np.ones_like(p.q_scale)
    p.k_scale = np.ones_like(p.k_scale)
    p.v_scale = np.full_like(p.v_scale, 1.0 / 64)
    p.scale = float(np.float32(math.log(2.0)))
    return p


@pytest.mark.parametrize("N", [256, 300, 1000])
@pytest.mark.parametrize("mode", list(MODES))
def test_exactly_representable_p_matches_the_oracle(mode, N):
    p = _exact_p_problem(N, 1)
    _announce("low-precision P.V, exact P", mode, N)
    o, lse = _run(p, MODES[mode])
    o_ref, lse_ref = oracle.attention_problem(p)
    # the inputs are e4m3 codes, but nothing is rounded on the way: the bf16 gate applies
    e_o, e_ob, e_l = errors(o, lse, o_ref, lse_ref)
    print(f"exact-P {mode} N={N}: max|dO|={e_o:.3e} max|dLSE|={e_l:.3e}", flush=True)
    assert e_o <= 2e-2 and e_l <= 1e-3


@pytest.mark.parametrize("mode", list(MODES))
def test_cfg5_rotated_error_is_measured(mode):
    """Configuration 5 (incoherent processing): the error of the rounded P against the oracle,
    reported; the outputs must be finite and every row written."""
    p = W.config_problem(5, rotate=True)
    _announce("low-precision P.V cfg5 rotated", mode)
    o, lse = _run(p, MODES[mode])
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    rows = sample_rows(p.N, 32, seed=55)
    heads = [(0, h) for h in range(p.H)]
    o_ref, lse_ref = oracle.attention_problem(p, rows=rows, heads=heads, workers=8)
    e_o, e_ob, e_l = errors(o[:, :, rows], lse[:, :, rows], o_ref, lse_ref)
    print(f"cfg5 rotated, Q.K^T e4m3, P {mode}: max|dO|={e_o:.3e} beyond-half-ulp={e_ob:.3e} "
          f"max|dLSE|={e_l:.3e} (max|O_ref|={np.abs(o_ref).max():.1f})", flush=True)


def test_unsupported_combinations_are_refused():
    p = W.make_problem(1, 2, 300, 128, dtype="fp8", flags=W.ATTN_CAUSAL, seed=3)
    dp = WD.to_device(p, pv_mode=L.ATTN_PV_E4M3, qk_mode=L.ATTN_QK_E4M3)
    with pytest.raises(L.AttnError):
        WD.forward(dp)
    dp = WD.to_device(W.make_problem(1, 2, 300, 128, dtype="fp8", seed=3), pv_mode=L.ATTN_PV_FP4)
    with pytest.raises(L.AttnError):
        WD.forward(dp)
