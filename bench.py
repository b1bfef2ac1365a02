"""Benchmark of the fused attention forward pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 3] [--no-cpu]

A step is one pass of the whole path over one batch of synthetic input already
resident in HBM: the block-map build (document masks and packed batches; causal and
window masks have their block lists derived inside the forward kernel) followed by
the forward pass, both on the current stream.  `value` is attention TFLOP/s over the
unmasked FLOPs, 4*d*H*(visible (q, k) pairs) per step, divided by the step time: the
host clock around K steps launched back to back, synchronised on both sides.

Warm-up: at least W steps and at least --warmup-s seconds (default 3), so that the
engine clock has settled at the board's power limit before the timed steps.  The K
timed steps are split into up to 5 windows by HIP events recorded on the stream
between them (one event per window, none inside a step): the median and minimum of
the per-window step times are reported beside the host-clock mean.  When a step is
the forward kernel alone, the kernel's time is that window's (so it can never exceed
the step time); otherwise the forward kernel is timed the same way in a second run
of K launches right after.  The engine clock is sampled (amdsmi) through the last
second of warm-up and the timed steps.

Default workload: B=2 H=32 N=8192 d=128 bf16, causal + sliding window of 1024 keys
+ tanh soft-cap 50 (configuration 3).  Other --config values are the other synthetic
workloads (1: B1 H2 N256 d64 plain; 2: B4 H16 N2048 d128 causal; 4: B1 H16 N16384
d128 document-causal+ALiBi; 5: B1 H16 N16384 d128 fp8 plain), --plain-causal the
configuration-3 shape with a plain causal mask, and --shape B,H,N,d [--mask causal]
any other bf16 shape (--kv-heads H_kv for grouped-query attention), --varlen a packed
batch of causal sequences of different lengths.

Printed on stdout: ONE JSON line.  Extra diagnostics go to stderr.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0}  # MI355X dense MFMA, published
HBM_PEAK_GBS = 8000.0
KERNEL_SOURCES = ["exact_attention_119_amd/csrc/fwd_bf16.hpp",
                  "exact_attention_119_amd/csrc/fwd_args.hpp", "exact_attention_119_amd/csrc/common.hpp",
                  "exact_attention_119_amd/build.py"]
QUANT_SOURCES = ["exact_attention_119_amd/csrc/quant.hip", "exact_attention_119_amd/csrc/common.hpp",
                 "exact_attention_119_amd/build.py"]
QUANT_WORKLOAD = "quantise B1 H16 N16384 d128 bf16, rotated"
METRIC = "attention fwd TFLOP/s (unmasked FLOPs) and % of MI355X bf16/fp8 MFMA peak"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash(files=None) -> str:
    h = hashlib.sha256()
    for f in (KERNEL_SOURCES if files is None else files):
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def median(v):
    v = sorted(v)
    n = len(v)
    return v[n // 2] if n % 2 else 0.5 * (v[n // 2 - 1] + v[n // 2])


def arithmetic_dtype(dp) -> str:
    """The types the MFMAs compute in: bf16; for e4m3 inputs the codes are widened for
    Q.K^T (bf16) and P.V (fp16), or Q.K^T runs on the e4m3 MFMA (qk8)."""
    if dp.fp8 is None:
        return "bf16"
    from exact_attention_119_amd import lib as L
    qk = "e4m3" if dp.fp8.qk_mode == L.ATTN_QK_E4M3 else "bf16"
    pv = {L.ATTN_PV_E4M3: "e4m3", L.ATTN_PV_FP4: "e2m1 (E8M0 block scales)"}.get(dp.fp8.pv_mode, "f16")
    return f"{qk} QK^T + {pv} PV (e4m3 inputs)"


def workload_name(p) -> str:
    mods = []
    if p.cu_seqlens is not None:
        mods.append(f"varlen{len(p.cu_seqlens) - 1}")
    if p.flags & 4:
        mods.append("document")
    if p.flags & 1:
        mods.append("causal")
    if p.flags & 2:
        mods.append(f"window{p.window}")
    if p.flags & 16:
        mods.append(f"softcap{p.softcap:g}")
    if p.flags & 8:
        mods.append("alibi")
    kv = "" if p.Hkv == p.H else f" Hkv{p.Hkv}"
    rot = " rotated" if p.rotate_signs is not None else ""
    return f"B{p.B} H{p.H}{kv} N{p.N} d{p.d} {'+'.join(mods) or 'no-mask'} {p.dtype}{rot}"


def visible_pairs(p) -> int:
    """Exact visible (q, k) pairs for one head, from the positional mask's row intervals."""
    import numpy as np
    N, total = p.N, 0
    for b in range(p.B):
        q = np.arange(N)
        lo, hi = np.zeros(N, np.int64), np.full(N, N - 1, np.int64)
        if p.flags & 1:
            hi = np.minimum(hi, q)
        if p.flags & 2:
            lo = np.maximum(lo, q - (p.window - 1))
            if not p.flags & 1:
                hi = np.minimum(hi, q + (p.window - 1))
        d = None
        if p.flags & 4:
            d = p.doc_id[b]
        elif p.cu_seqlens is not None:
            d = np.repeat(np.arange(len(p.cu_seqlens) - 1), np.diff(p.cu_seqlens))
        if d is not None:
            first = np.searchsorted(d, d, side="left")
            last = np.searchsorted(d, d, side="right") - 1
            lo, hi = np.maximum(lo, first), np.minimum(hi, last)
        total += int(np.maximum(0, hi - lo + 1).sum())
    return total


def cpu_baseline(p, budget_s: float):
    """The fp64 oracle timed on the host cores over a bounded sample of the same
    workload: whole (b, h) heads, as many as fit the time budget."""
    import numpy as np
    import oracle
    from oracle.attention import available_cores
    cores = min(available_cores(), 16)  # the host CPUs one GPU's share of the box holds
    heads_all = [(b, h) for b in range(p.B) for h in range(p.H)]
    t0 = time.perf_counter()
    oracle.attention_problem(p, heads=heads_all[:1], workers=1)
    t1 = time.perf_counter() - t0
    n = int(max(1, min(len(heads_all), budget_s / max(t1, 1e-3) * cores)))
    n = max(1, min(len(heads_all), (n // cores) * cores or n))
    heads = heads_all[:n]
    t0 = time.perf_counter()
    oracle.attention_problem(p, heads=heads, workers=cores)
    dt = time.perf_counter() - t0
    pairs_per_head = visible_pairs(p) / p.B
    flops = 4.0 * p.d * pairs_per_head * n
    dense = 4.0 * p.d * p.N * p.N * n  # the oracle forms every score of a row, masked or not
    cpu = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            cpu = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), cpu)
    except OSError:
        pass
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"{n} of {len(heads_all)} (b,h) heads, all {p.N} query rows, fp64 numpy, "
                      f"{dt:.1f} s wall",
            "cpu_model": cpu, "wall_s": round(dt, 3),
            "dense_tflops": round(dense / dt / 1e12, 6)}


def timed_windows(torch, stream, steps: int, launch, nwin: int = 5):
    """Times `steps` calls of `launch` back to back: the host clock around all of them
    (synchronised on both sides) and HIP events on `stream` at the boundaries of up to
    `nwin` windows.  Returns (host ms per call, [event ms per call of each window],
    event ms per call over all windows)."""
    nwin = max(1, min(nwin, steps))
    bounds = [round(i * steps / nwin) for i in range(nwin + 1)]
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(nwin + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev[0].record(stream)
    for w in range(nwin):
        for _ in range(bounds[w + 1] - bounds[w]):
            launch()
        ev[w + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = [ev[w].elapsed_time(ev[w + 1]) / (bounds[w + 1] - bounds[w]) for w in range(nwin)]
    return wall * 1e3 / steps, per, ev[0].elapsed_time(ev[nwin]) / steps


def warm_up(torch, launch, min_steps: int, min_seconds: float):
    """At least min_steps calls and at least min_seconds of them (the queue is drained
    every 32 calls so the host does not run far ahead of the GPU)."""
    n, t0 = 0, time.perf_counter()
    while n < min_steps or time.perf_counter() - t0 < min_seconds:
        launch()
        n += 1
        if n % 32 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    return n, time.perf_counter() - t0


class ClockSampler:
    """Samples the GPU's engine (gfx) clock through amdsmi in a background thread,
    every `period` seconds, between start() and stop().  Reports nothing where amdsmi or
    the metric is unavailable."""

    def __init__(self, period: float = 0.05):
        import threading
        self.period, self.samples, self.source = period, [], None
        self._stop = threading.Event()
        self._thread = None
        self._read = None
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            handles = amdsmi.amdsmi_get_processor_handles()
            if not handles:
                return
            h = handles[0]

            def read_clock_info():
                return float(amdsmi.amdsmi_get_clock_info(h, amdsmi.AmdSmiClkType.GFX)["clk"])

            def read_metrics():
                m = amdsmi.amdsmi_get_gpu_metrics_info(h)
                v = m.get("current_gfxclks") or m.get("current_gfxclk")
                if isinstance(v, (list, tuple)):
                    v = [x for x in v if isinstance(x, (int, float)) and 0 < x < 10000]
                    return float(sum(v) / len(v)) if v else None
                return float(v) if isinstance(v, (int, float)) and 0 < v < 10000 else None

            for name, fn in (("amdsmi gpu_metrics current_gfxclk", read_metrics),
                             ("amdsmi clock_info gfx", read_clock_info)):
                try:
                    if fn() is not None:
                        self._read, self.source = fn, name
                        break
                except Exception:  # noqa: BLE001 - any failure means: not available
                    continue
        except Exception:  # noqa: BLE001
            self._read = None

    def _run(self):
        while not self._stop.is_set():
            try:
                v = self._read()
                if v is not None:
                    self.samples.append((time.perf_counter(), v))
            except Exception:  # noqa: BLE001
                pass
            self._stop.wait(self.period)

    def start(self):
        import threading
        if self._read is not None:
            self._thread = threading.Thread(target=self._run, daemon=True)
            self._thread.start()

    def stop(self):
        self._stop.set()
        if self._thread is not None:
            self._thread.join()

    def summary(self, since: float):
        v = sorted(x for t, x in self.samples if t >= since)
        if not v:
            return None
        return {"median_mhz": v[len(v) // 2], "min_mhz": v[0], "max_mhz": v[-1], "samples": len(v),
                "source": self.source, "peak_mhz": 2400}


def rescale_events(torch, dp) -> dict:
    """Mean rescale events per query row of the online softmax at tau = 0 and tau = 8
    (attn_fwd_rescale_counts; one untimed pass each), the first visible step excluded."""
    from exact_attention_119_amd import lib as L
    from workload import device as WD
    p = dp.p
    out = {}
    counts = torch.empty((p.B, p.H, p.N), dtype=torch.int32, device="cuda")
    for tau in (0.0, 8.0):
        if WD.needs_map(dp):
            WD.build_map(dp)
        L.attn_fwd_rescale_counts(dp.q, dp.k, dp.v, dp.o, dp.lse, counts, scale=p.scale, dtype=dp.dtype,
                                  mask=dp.mask, blockmap=dp.blockmap if WD.needs_map(dp) else None, rescale_tau=tau)
        torch.cuda.synchronize()
        out[f"tau{tau:g}_per_row_after_first"] = round(float((counts.double() - 1).mean().item()), 5)
    r0, r8 = out["tau0_per_row_after_first"], out["tau8_per_row_after_first"]
    out["ratio_tau0_over_tau8"] = round(r0 / r8, 2) if r8 > 0 else None
    return out


def loop_ms(torch, stream, n: int, launch) -> float:
    """Average duration of `launch` over n back-to-back calls on `stream` (HIP events)."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(n):
        launch()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n


def graph_loop_ms(torch, stream, n: int, launch) -> float:
    """The same over one HIP graph of n launches, replayed once: the kernels run back to back
    with no host launch gaps (for kernels shorter than the host's launch interval)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        launch()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(n):
            launch()
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n


def traffic_record(name: str, files=None):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were taken on
    the current kernel sources."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f).get(name)
    if not rec or rec.get("kernel_source_hash") != kernel_source_hash(files):
        return None
    return rec.get("bytes_per_launch")


def bench_bwd(args):
    """One step = the two backward launches for the configuration's workload."""
    import numpy as np
    import torch
    import workload as W
    from workload import device as WD
    from exact_attention_119_amd import lib as L
    p = W.config_problem(args.config)
    if p.dtype != "bf16":
        raise SystemExit("the backward pass takes bf16 inputs")
    dp = WD.to_device(p)
    WD.step(dp)
    dout = torch.from_numpy(W.make_dout(p, seed=2).view(np.int16)).cuda().view(torch.bfloat16)
    dq, dk, dv = torch.empty_like(dp.q), torch.empty_like(dp.k), torch.empty_like(dp.v)
    delta = torch.empty_like(dp.lse)
    stream = torch.cuda.current_stream()

    def step():
        L.attn_bwd_gqa(dp.q, dp.k, dp.v, dp.o, dp.lse, dout, dq, dk, dv, delta, scale=p.scale, mask=dp.mask,
                       blockmap=dp.blockmap)

    warm_up(torch, step, args.warmup, args.warmup_s)  # (the clock settles, as for the forward pass)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    avg = loop_ms(torch, stream, args.steps, step)
    pairs = visible_pairs(p)
    flop = 10.0 * p.d * p.H * pairs  # five products of 2*d flop per visible pair
    step_ms = wall * 1e3 / args.steps
    name = workload_name(p)
    log(f"bench: backward step {step_ms:.4f} ms (wall), two launches avg {avg:.4f} ms (back-to-back, events)")
    out = {"metric": "attention bwd TFLOP/s (five products of 2d flop per visible pair)",
           "value": round(flop / (step_ms * 1e-3) / 1e12, 3), "unit": "TFLOP/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(step_ms, 5), "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded N(0,1))",
           "config": {"workload": name + " backward", "visible_pairs": pairs, "flop_per_step": flop,
                      "step": "row sums + dQ + dK/dV, given O and LSE", "parallelism": "single GPU"},
           "roofline": {"bound": "mfma", "achieved": round(flop / (avg * 1e-3) / 1e12, 3), "peak": PEAK_TFLOPS["bf16"],
                        "unit": "TFLOP/s", "frac": round(flop / (avg * 1e-3) / 1e12 / PEAK_TFLOPS["bf16"], 4),
                        "traffic": None, "kernel": "dq (with the row sums D) + dkdv (two launches)",
                        "kernel_avg_ms": round(avg, 5)}}
    if not args.no_cpu:
        import oracle
        t0 = time.perf_counter()
        n = 0
        while time.perf_counter() - t0 < min(args.cpu_budget, 10.0) and n < p.B * p.H:
            oracle.attention_bwd_problem(p, W.make_dout(p, seed=2), heads=[divmod(n, p.H)])
            n += 1
        dt = time.perf_counter() - t0
        out["cpu_baseline"] = {"value": round(flop * n / (p.B * p.H) / dt / 1e12, 6), "unit": "TFLOP/s",
                               "cores": 1, "kind": "oracle",
                               "sample": f"{n} of {p.B * p.H} (b,h) heads, fp64 numpy, {dt:.1f} s"}
    print(json.dumps(out), flush=True)
    return 0


QUANT_SIGNS = [0x9E3779B9, 0x7F4A7C15, 0x2545F491, 0x4F6CDD1D]


def bench_quant(args):
    """One step = block-quantise Q and K (rotated, one sign vector) and V (plain) from bf16."""
    import numpy as np
    import torch
    import workload as W
    from exact_attention_119_amd import lib as L
    p = W.make_problem(1, 16, 16384, 128, n_outliers=4, outlier_gain=20.0, seed=55)
    nblk = (p.N + 127) // 128
    xs = [torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16) for x in (p.q, p.k, p.v)]
    codes = [torch.empty(x.shape, dtype=torch.uint8, device="cuda") for x in xs]
    scales = [torch.empty((p.B, p.H, nblk), dtype=torch.float32, device="cuda") for _ in xs]
    signs = [QUANT_SIGNS, QUANT_SIGNS, None]
    stream = torch.cuda.current_stream()

    def step():
        for i in range(3):
            L.attn_fp8_quantize(xs[i], codes[i], scales[i], signs[i])

    warm_up(torch, step, args.warmup, args.warmup_s)  # (the clock settles, as for the forward pass)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    rot_avg = loop_ms(torch, stream, 2 * args.steps, lambda: L.attn_fp8_quantize(xs[0], codes[0], scales[0], signs[0]))
    elems = p.B * p.H * p.N * p.d
    bytes_launch = elems * 3 + 4 * p.B * p.H * nblk
    step_ms = wall * 1e3 / args.steps
    achieved = bytes_launch / (rot_avg * 1e-3) / 1e9
    log(f"bench: quantise step {step_ms:.4f} ms (3 launches), rotated launch avg {rot_avg:.4f} ms")
    out = {"metric": "fp8 block quantisation with incoherent processing, GB/s of algorithmic HBM traffic",
           "value": round(3 * bytes_launch / (step_ms * 1e-3) / 1e9, 2), "unit": "GB/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(step_ms, 5),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16->fp8",
           "data": "synthetic (seeded N(0,1), four channels x20)",
           "config": {"workload": "quantise Q, K (rotated) and V: B1 H16 N16384 d128 bf16", "elements_per_launch": elems,
                      "bytes_per_launch": bytes_launch, "parallelism": "single GPU"},
           "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": round(achieved / HBM_PEAK_GBS, 4),
                        "traffic": traffic_record(QUANT_WORKLOAD, QUANT_SOURCES),
                        "kernel": "quant_kernel<128> (rotated)", "kernel_avg_ms": round(rot_avg, 5)}}
    if not args.no_cpu:
        from oracle import quant as Qz
        t0 = time.perf_counter()
        n = 0
        while time.perf_counter() - t0 < min(args.cpu_budget, 10.0) and n < p.H:
            Qz.quantize_blocks_ref(p.q[:, n:n + 1], np.array(QUANT_SIGNS, np.uint32))
            n += 1
        dt = time.perf_counter() - t0
        out["cpu_baseline"] = {"value": round(n * p.N * p.d * 3 / dt / 1e9, 4), "unit": "GB/s", "cores": 1,
                               "kind": "oracle", "sample": f"{n} of {p.H} heads of Q, rotated, float32 numpy, "
                                                           f"{dt:.1f} s"}
    print(json.dumps(out), flush=True)
    return 0


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--config", type=int, default=3, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--warmup-s", type=float, default=3.0,
                    help="minimum seconds of warm-up steps (the engine clock settles at the power limit)")
    ap.add_argument("--plain-causal", action="store_true", help="configuration-3 shape, plain causal mask")
    ap.add_argument("--shape", type=str, default=None,
                    help="supplementary bf16 workload B,H,N,d (with --mask, --kv-heads), instead of a "
                         "configuration")
    ap.add_argument("--mask", choices=["none", "causal"], default="none", help="mask of a --shape workload")
    ap.add_argument("--varlen", action="store_true",
                    help="packed variable-length batch: 16384 tokens in causal sequences of 512..4096, "
                         "H16 d128 (with --kv-heads)")
    ap.add_argument("--kv-heads", type=int, default=None,
                    help="key/value heads of a --shape workload (grouped-query attention)")
    ap.add_argument("--tau", type=float, default=8.0)
    ap.add_argument("--qk8", action="store_true",
                    help="fp8 workloads: Q.K^T on the e4m3 MFMA (a measured mode: its truncating accumulation "
                         "misses the fp8 LSE tolerance on configuration 5)")
    ap.add_argument("--pv", choices=["f16", "e4m3", "fp4"], default="f16",
                    help="fp8 workloads with --qk8: P.V precision (e4m3 or fp4 P are measured modes)")
    ap.add_argument("--rotate", action="store_true",
                    help="configuration 5 with incoherent processing: Q and K quantised after the rotation")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle work to time")
    ap.add_argument("--bwd", action="store_true",
                    help="instead: the backward pass (row sums, dQ, dK/dV) on the configuration's workload "
                         "(bf16), given the forward pass's O and LSE")
    ap.add_argument("--quant", action="store_true",
                    help="instead: the device fp8 quantiser (Q and K rotated, V plain) on the fp8 workload's "
                         "shape B1 H16 N16384 d128 from bf16")
    ap.add_argument("--copy-calib", type=int, default=0,
                    help="instead: run a plain device copy of this many MiB (counter calibration)")
    args = ap.parse_args(argv)

    if args.gpus != 1:
        print(f"bench.py: the benchmark runs on one GPU only (asked for --gpus {args.gpus}); the attention pass "
              f"would shard over (b, h) heads with no communication.",
              file=sys.stderr)
        return 2

    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)

    if args.copy_calib:
        n = args.copy_calib << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calib_bytes_read": n, "bytes_written": n, "launches": 5}))
        return 0

    import workload as W
    from workload import device as WD

    if args.quant:
        return bench_quant(args)
    if args.bwd:
        return bench_bwd(args)

    if args.varlen:
        import numpy as np
        lengths = W.draw_doc_lengths(np.random.default_rng([119, 78]), 16384, 512, 4096)
        p = W.make_varlen_problem(lengths, 16, 128, flags=W.ATTN_CAUSAL, seed=78, H_kv=args.kv_heads)
    elif args.shape:
        B, H, N, d = (int(x) for x in args.shape.split(","))
        p = W.make_problem(B, H, N, d, flags=W.ATTN_CAUSAL if args.mask == "causal" else 0, seed=4,
                           H_kv=args.kv_heads)
    elif args.plain_causal:
        p = W.make_problem(2, 32, 8192, 128, flags=W.ATTN_CAUSAL, seed=3)
    else:
        p = W.config_problem(args.config, rotate=args.rotate)
    name = workload_name(p)
    log(f"bench: {name}; generating done, staging to HBM")
    from exact_attention_119_amd import lib as L
    pv_mode = {"f16": L.ATTN_PV_F16, "e4m3": L.ATTN_PV_E4M3, "fp4": L.ATTN_PV_FP4}[args.pv]
    # (the forward pass reads only the map's interval, status and order sections: the compact
    # form, without the class and list sections the backward tests compare, is what it needs)
    dp = WD.to_device(p, qk_mode=L.ATTN_QK_E4M3 if args.qk8 else L.ATTN_QK_BF16, pv_mode=pv_mode,
                      compact_map=True)
    pairs = visible_pairs(p)
    flop_per_step = 4.0 * p.d * p.H * pairs
    stream = torch.cuda.current_stream()

    # A step builds the block map where the forward pass needs one (document masks, packed
    # batches); causal and window masks go without, their block lists derived in the kernel.
    map_in_step = WD.needs_map(dp)

    def one_step():
        WD.step(dp, args.tau, use_map=False)

    def one_forward():
        WD.forward(dp, args.tau, use_map=False)

    clock = ClockSampler()
    clock.start()
    nwarm, twarm = warm_up(torch, one_step, args.warmup, args.warmup_s)
    t_settled = time.perf_counter() - min(1.0, twarm)

    # The timed region: K whole steps back to back with nothing else on the stream (one
    # event between windows, none inside a step).
    step_ms, step_win, step_ev = timed_windows(torch, stream, args.steps, one_step)
    if map_in_step:
        # the forward kernel alone, K launches right after, timed the same way
        _, fwd_win, fwd_mean = timed_windows(torch, stream, args.steps, one_forward)
    else:
        fwd_win, fwd_mean = step_win, step_ev  # the step is the forward kernel: its own window
    clock.stop()
    fwd_med, fwd_min = fwd_mean, min(fwd_win)
    graph_note = None
    if fwd_med < 0.05:  # short kernel: the windows above measure the host's launch rate
        graph_note = fwd_med
        fwd_med = fwd_min = graph_loop_ms(torch, stream, args.steps, one_forward)
        log(f"bench: forward kernel {graph_note:.4f} ms launched from the host, {fwd_med:.4f} ms from a graph")
    map_avg = loop_ms(torch, stream, args.steps, lambda: WD.build_map(dp)) if dp.blockmap is not None else 0.0
    consistent = fwd_med <= step_ms
    log(f"bench: warm-up {nwarm} steps in {twarm:.2f} s; step {step_ms:.4f} ms (host clock, mean of {args.steps}), "
        f"windows median {median(step_win):.4f} min {min(step_win):.4f} ms; forward kernel mean {fwd_med:.4f} "
        f"(window median {median(fwd_win):.4f}) min {fwd_min:.4f} ms; block map build avg {map_avg:.4f} ms")
    if not consistent:
        log("bench: WARNING the forward kernel's mean exceeds the step time (it was timed in its own run; "
            "the clock differed)")

    dtype = p.dtype
    achieved = flop_per_step / (fwd_med * 1e-3) / 1e12
    peak = PEAK_TFLOPS[dtype]
    traffic = traffic_record(name)
    from exact_attention_119_amd import lib as L
    kernel_name = L.attn_fwd_kernel_name(p.d, dp.dtype, dp.mask, dp.fp8)
    eb = 1 if dtype == "fp8" else 2
    alg_bytes = p.B * p.N * (p.H * (p.d * (eb + 2) + 4) + p.Hkv * 2 * p.d * eb)
    log(f"bench: algorithmic HBM bytes per launch {alg_bytes}; at the forward kernel's time that is "
        f"{alg_bytes / (fwd_med * 1e-3) / 1e9:.1f} GB/s of {HBM_PEAK_GBS:.0f}")

    out = {
        "metric": METRIC,
        "value": round(flop_per_step / (step_ms * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": arithmetic_dtype(dp),
        "data": "synthetic (seeded N(0,1) inputs of the workload's shape)",
        "config": {"workload": name, "B": p.B, "H": p.H, "N": p.N, "d": p.d, "visible_pairs": pairs,
                   "unmasked_flop_per_step": flop_per_step, "rescale_tau": args.tau, "input_dtype": dtype,
                   "step": "block-map build (compact form) + forward pass" if map_in_step else
                           ("forward pass (block lists derived from the mask in the kernel)" if dp.blockmap is not None
                            else "forward pass"), "parallelism": "single GPU",
                   "warmup_run": {"steps": nwarm, "seconds": round(twarm, 3)},
                   "step_ms_windows": {"median": round(median(step_win), 5), "min": round(min(step_win), 5),
                                       "windows": len(step_win)},
                   "engine_clock": clock.summary(t_settled)},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 3), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(achieved / peak, 4), "traffic": traffic,
                     "kernel": kernel_name, "kernel_avg_ms": round(fwd_med, 5),
                     "kernel_window_median_ms": round(median(fwd_win), 5), "kernel_min_ms": round(fwd_min, 5),
                     "kernel_timing": ("HIP events around the timed steps, each step being this kernel alone: "
                                       "mean per launch, and the median and minimum of the windows"
                                       if not map_in_step else
                                       "HIP events around K forward launches right after the timed steps: mean per "
                                       "launch, and the median and minimum of the windows"),
                     "kernel_le_step": consistent, "map_build_avg_ms": round(map_avg, 5)},
    }
    if dtype == "fp8":
        out["roofline"]["note"] = ("fp8 peak; Q.K^T on the bf16 MFMA and P.V on the fp16 MFMA (both half the fp8 "
                                   "rate) unless the kernel name says fp8-qk8")
    # Below the ridge (peak flop/s over 8 TB/s) the kernel's roofline is HBM bandwidth.
    if flop_per_step / alg_bytes < peak * 1e12 / (HBM_PEAK_GBS * 1e9):
        gbs = alg_bytes / (fwd_med * 1e-3) / 1e9
        out["roofline"].update({"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                "frac": round(gbs / HBM_PEAK_GBS, 5), "achieved_tflops": round(achieved, 3),
                                "algorithmic_bytes": alg_bytes})
    if p.dtype == "bf16" and p.cu_seqlens is None:
        out["config"]["rescale_events"] = rescale_events(torch, dp)
    if not args.no_cpu:
        log("bench: timing the CPU oracle on a bounded sample ...")
        out["cpu_baseline"] = cpu_baseline(p, args.cpu_budget)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
