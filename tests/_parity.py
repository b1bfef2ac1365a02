"""Helpers shared by the GPU parity tests: tolerances and error metrics.

Tolerances (attention forward, against the fp64 oracle on the same inputs):
  bf16 inputs, fp32 accumulation: max |O - O_ref| <= 2e-2, max |LSE - LSE_ref| <= 1e-3.
  fp8 e4m3 inputs with block scales (oracle on the dequantised inputs):
      max(|O - O_ref| - ulp_bf16(O_ref)/2) <= 6e-2   (error beyond the bf16 output's
      own rounding: with outlier channels |O| reaches ~64, where rounding to bf16
      alone costs up to 0.125), and max |LSE - LSE_ref| <= 1e-3.
"""

import numpy as np

TOL_O_BF16 = 2e-2
TOL_LSE = 1e-3
TOL_O_FP8 = 6e-2


def half_ulp_bf16(x: np.ndarray) -> np.ndarray:
    ax = np.abs(x)
    e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    e = np.maximum(e, -126)
    return np.where(ax > 0, 2.0 ** (e - 7) / 2, 0.0)


def errors(o, lse, o_ref, lse_ref):
    """Max errors, with -inf LSE values required to match exactly."""
    assert np.array_equal(np.isneginf(lse), np.isneginf(lse_ref)), "empty-row pattern differs"
    fin = np.isfinite(lse_ref)
    assert np.all(np.isfinite(o)), "non-finite O"
    e_o = float(np.max(np.abs(o - o_ref))) if o.size else 0.0
    e_o_beyond = float(np.max(np.abs(o - o_ref) - half_ulp_bf16(o_ref))) if o.size else 0.0
    e_l = float(np.max(np.abs(lse[fin] - lse_ref[fin]))) if fin.any() else 0.0
    return e_o, e_o_beyond, e_l


def assert_close(p, o, lse, o_ref, lse_ref, what=""):
    e_o, e_ob, e_l = errors(o, lse, o_ref, lse_ref)
    msg = f"{what}: max|dO|={e_o:.3e} beyond-half-ulp={e_ob:.3e} max|dLSE|={e_l:.3e}"
    print(msg, flush=True)
    if p.dtype == "bf16":
        assert e_o <= TOL_O_BF16, msg
    else:
        assert e_ob <= TOL_O_FP8, msg
    assert e_l <= TOL_LSE, msg
    return e_o, e_ob, e_l


def sample_rows(N: int, n: int, seed: int) -> np.ndarray:
    """Rows to compare at full size: edges of every 128-row block and of the
    sequence, plus a seeded random sample."""
    fixed = {0, 1, N - 1, N - 2}
    for q0 in range(0, N, 128 * max(1, N // (128 * 8))):
        fixed.update({q0, min(N - 1, q0 + 127), min(N - 1, q0 + 31), min(N - 1, q0 + 32)})
    rng = np.random.default_rng(seed)
    extra = rng.choice(N, size=min(N, n), replace=False)
    return np.array(sorted(fixed.union(extra.tolist()).intersection(range(N))), dtype=np.int64)


def check_work_order(order, counts, header, document: bool, what: str = "order"):
    """The block map's work order (the library's scheduling choice, not part of the
    method) as a property of the device's own stated cost: a permutation of the (batch
    row, query block) entries; under a document mask the work order_full_cost * #FULL +
    order_partial_cost * #PARTIAL (weights read from the map header, counts from the
    map) never increases along it and equal work keeps index order; otherwise the
    identity."""
    order = np.asarray(order, dtype=np.int64)
    M = order.size
    assert np.array_equal(np.sort(order), np.arange(M)), f"{what}: not a permutation"
    if not document:
        assert np.array_equal(order, np.arange(M)), f"{what}: not the identity"
        return
    wf, wp = int(header["order_full_cost"]), int(header["order_partial_cost"])
    assert wf > 0 and wp > 0, f"{what}: no stated cost"
    c = np.asarray(counts, dtype=np.int64).reshape(-1, 2)
    w = (wf * c[:, 0] + wp * c[:, 1])[order]
    ok = (w[:-1] > w[1:]) | ((w[:-1] == w[1:]) & (order[:-1] < order[1:]))
    assert np.all(ok), f"{what}: work increases along the order at {np.nonzero(~ok)[0][:5]}"
