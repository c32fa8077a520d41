"""Ring attention forward benchmark on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--gpus 1]

A step is one pass of the whole hot path over the workload's synthetic input:
the striped (or contiguous) shard layout of K and V (ra_stripe_permute), then
ra_ring_forward: every ring step's blockwise attention, the log-sum-exp merges
and the final normalisation.  Inputs are generated on the host from a seeded
counter-based generator and are resident in HBM before timing starts.

Printed: one JSON line.  `value` is attention TFLOP/s counting only unmasked
(query, key) pairs (4 * head_dim FLOPs per pair per query head), over the timed
steps.  `roofline` describes the block-attention kernel (achieved FLOP rate from
HIP events on its own stream vs the bf16 dense MFMA peak), with the gfx clock
sampled while it ran and the fraction of the MFMA rate at that clock; `merge`
the log-sum-exp merge kernel's algorithmic HBM rate; `cpu_baseline` times the
CPU fp64 oracle on a bounded sample of the same workload.  With the default
workload (the Llama-3-8B-shaped 1M-token share) `companion` holds the same
figures for the causal 256K-token striped share, measured in the same run.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6  # MI355X dense bf16 MFMA: 256 CU x 4096 FLOP/clk x 2.4 GHz
PEAK_HBM_GBPS = 8000.0

WORKLOADS = {
    # Llama-3-8B-shaped causal GQA, 1M tokens striped over 32 positions:
    # one position's share (32768 queries against 32 KV blocks of 32768).
    "llama3-8b-gqa-1m-striped-share": dict(B=1, Hq=32, Hkv=8, S=1 << 20, D=128, N=32, layout="striped",
                                           causal=True, share=31),
    # causal striped, 8 heads, 256K tokens over 8 positions: one position's share
    "causal-256k-striped-share": dict(B=1, Hq=8, Hkv=8, S=262144, D=128, N=8, layout="striped", causal=True,
                                      share=7),
    # causal contiguous, 32 heads, 32K tokens over 4 positions: the whole ring
    "causal-32k-contiguous-ring": dict(B=1, Hq=32, Hkv=32, S=32768, D=128, N=4, layout="contiguous",
                                       causal=True, share=None),
    # non-causal, 4 heads, 4K tokens, d 64 over 2 positions: the whole ring
    "noncausal-4k-ring": dict(B=1, Hq=4, Hkv=4, S=4096, D=64, N=2, layout="contiguous", causal=False,
                              share=None),
}
DEFAULT = "llama3-8b-gqa-1m-striped-share"


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def traffic_from_profile(kernel_src, workload, record="block_attn_traffic.json"):
    """HBM bytes per block-kernel launch (or block pair, for the backward) from
    committed rocprofv3 counters, if they were taken on the current kernel
    source and on this workload (else None).  The record holds one entry per
    workload (``workloads``: name -> {kernel_sha256, bytes_per_launch, ...})."""
    path = os.path.join(ROOT, "profiles", record)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    with open(kernel_src, "rb") as f:
        digest = hashlib.sha256(f.read()).hexdigest()
    entry = rec.get("workloads", {}).get(workload)
    if not entry or entry.get("kernel_sha256") != digest:
        return None
    return entry.get("bytes_per_launch")


def _openmp():
    """The OpenMP runtime the oracle library runs on (to pin its thread count)."""
    import ctypes

    try:
        return ctypes.CDLL("libgomp.so.1")
    except OSError:
        return None


def cpu_baseline(cfg, k_np, v_np, q_rows_fn, budget_s, max_rows=20000, seed=2, threads=None, g_rows_fn=None):
    """Time the oracle on seeded query rows of the workload, in chunks of 32 rows,
    until about budget_s seconds of CPU work have been done.  threads=None uses
    every host core the process may run on.  With g_rows_fn (the rows' output
    gradients) the oracle computes the rows' dQ instead of their output: it
    forms the scores, lse, D = dO . O and dQ, 8 d FLOPs a visible pair."""
    import oracle

    gomp = _openmp()
    avail = len(os.sched_getaffinity(0))
    if threads is None:
        threads = min(int(os.environ.get("OMP_NUM_THREADS", "0")) or avail, avail)
    if gomp is not None:
        gomp.omp_set_num_threads(threads)

    rng = np.random.Generator(np.random.PCG64(seed))
    S, N, Hq, Hkv = cfg["S"], cfg["N"], cfg["Hq"], cfg["Hkv"]
    g = Hq // Hkv
    pairs, rows, dt = 0, 0, 0.0
    while dt < budget_s and rows < max_rows:
        h = int(rng.integers(0, Hq))
        if cfg["share"] is not None:
            sb = S // N
            r = rng.integers(0, sb, 32)
            t = cfg["share"] + N * r if cfg["layout"] == "striped" else cfg["share"] * sb + r
        else:
            t = rng.integers(0, S, 32)
        t = np.sort(t).astype(np.int64)
        qr = q_rows_fn(h, t)
        gr = g_rows_fn(h, t) if g_rows_fn is not None else None
        t0 = time.perf_counter()
        if gr is None:
            oracle.rows(qr, k_np[0, h // g], v_np[0, h // g], q_pos=t, causal=cfg["causal"])
        else:
            oracle.grads(qr, k_np[0, h // g], v_np[0, h // g], gr, q_pos=t, causal=cfg["causal"], key_grads=False)
        dt += time.perf_counter() - t0
        pairs += int(np.sum(t + 1)) if cfg["causal"] else len(t) * S
        rows += len(t)
    per_pair = 4.0 if g_rows_fn is None else 8.0
    flops = per_pair * cfg["D"] * pairs
    what = "output" if g_rows_fn is None else "dQ (scores, lse, D = dO . O and dQ: 8 d FLOPs a pair)"
    return {"value": round(flops / dt / 1e12, 5), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{rows} seeded query rows of this workload (one head per 32-row chunk), their {what} over "
                      f"the full causal key range, fp64: {flops / 1e9:.1f} GFLOP in {dt:.1f} s"}


def run_backward(args, cfg, ra, torch, fwd_step, q_sh, k_sh, v_sh, o_sh, lse, first, n_run, dev, k_np, v_np,
                 q_rows):
    """Time ra_ring_backward over the workload: one forward provides o and lse,
    then each timed step is the whole backward (delta, every block pair's
    dQ / dK / dV share).  FLOPs: 10 head_dim per unmasked pair (five products)."""
    import ra_inputs

    B, Hq, S, D, N, lay = (cfg[k] for k in ("B", "Hq", "S", "D", "N", "layout"))
    sb = S // N
    fwd_step(False)
    if cfg["share"] is not None:
        t0, ts = (first, N) if lay == "striped" else (first * sb, 1)
        g_np = ra_inputs.normal((B, Hq, S, D), 3, seed=args.seed, dtype="bf16", t0=t0, t_stride=ts, n_rows=sb)[None]
    else:
        g_full = ra_inputs.normal((B, Hq, S, D), 3, seed=args.seed, dtype="bf16")
        g_np = None
    if g_np is not None:
        dout = torch.from_numpy(g_np.view(np.int16)).view(torch.bfloat16).to(dev)
    else:
        gf = torch.from_numpy(g_full.view(np.int16)).view(torch.bfloat16).to(dev)
        dout = torch.empty_like(q_sh)
        ra.ra_stripe_permute(gf, dout, layout=lay, inverse=False, n_pos=N)
        del gf
    dq = torch.empty(q_sh.shape, dtype=torch.float32, device=dev)
    dk = torch.empty(k_sh.shape, dtype=torch.float32, device=dev)
    dv = torch.empty_like(dk)
    kw = dict(n_pos=N, first_pos=first, layout=lay, causal=cfg["causal"])
    log(f"backward warmup {args.warmup}")
    timed_kw = dict(kw, n_streams=args.n_streams)
    for _ in range(args.warmup):
        ra.ra_ring_backward(q_sh, k_sh, v_sh, o_sh, dout, lse, dq, dk, dv, **timed_kw)
    torch.cuda.synchronize()
    log(f"backward timing {args.steps} steps")
    marks = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for e0, e1 in marks:
        e0.record()
        ra.ra_ring_backward(q_sh, k_sh, v_sh, o_sh, dout, lse, dq, dk, dv, **timed_kw)
        e1.record()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    step_ms = [e0.elapsed_time(e1) for e0, e1 in marks]
    ms_per_step = elapsed / args.steps * 1e3
    # launch timing (HIP events around every block pair) in 3 more steps, on
    # one stream for a whole ring (where the positions' launches overlap)
    tot = {"block_ms": 0.0, "block_launches": 0, "flops": 0.0}
    for _ in range(3):
        st = ra.ra_ring_backward(q_sh, k_sh, v_sh, o_sh, dout, lse, dq, dk, dv, stats=True,
                                 n_streams=1 if n_run > 1 else 0, **kw)
        for key in tot:
            tot[key] += st[key]
    clock = sustained_clock(lambda _s: ra.ra_ring_backward(q_sh, k_sh, v_sh, o_sh, dout, lse, dq, dk, dv,
                                                           **timed_kw), torch)
    flops_per_step = tot["flops"] / 3
    value = flops_per_step / (ms_per_step * 1e-3) / 1e12
    per_launch_ms = tot["block_ms"] / max(1, tot["block_launches"])
    achieved = tot["flops"] / max(1, tot["block_launches"]) / (per_launch_ms * 1e-3) / 1e12
    line = {
        "metric": "ring-attention bwd TFLOP/s (causal-adjusted, five products) + % of MI355X bf16 MFMA peak",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4), "ms_per_step_median": round(float(np.median(step_ms)), 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "pct_of_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "config": {"workload": args.workload, "pass": "backward", "n_streams": args.n_streams, "batch": B,
                   "q_heads": Hq,
                   "kv_heads": cfg["Hkv"], "seq_len": S, "head_dim": D, "ring_positions": N, "layout": lay,
                   "causal": cfg["causal"], "positions_run": n_run, "first_position": first,
                   "unmasked_flops_per_step": flops_per_step},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic_from_profile(os.path.join(ROOT, "ring_attention_step_amd", "csrc",
                                                                  "block_attn_bwd_mfma.hip"),
                                                     args.workload, "block_attn_bwd_traffic.json"),
                     "kernel": "dq_kernel + dkdv_kernel (one block pair)", "launches": tot["block_launches"],
                     "mean_launch_ms": round(per_launch_ms, 4),
                     "timing": "HIP events around each block pair's pair of launches, 3 steps after the "
                               "timed ones",
                     "clock": clock,
                     "frac_at_clock": None if clock is None else round(achieved / mfma_peak_at(clock), 4)},
        "cpu_baseline": None,
    }
    if args.cpu_seconds > 0:
        if g_np is not None:
            def g_rows(h, t):
                r = (t - first) // N if lay == "striped" else t - first * sb
                return g_np[0][0][h, r]
        else:
            def g_rows(h, t):
                return g_full[0][h, t]
        log(f"cpu baseline: oracle dQ rows for about {args.cpu_seconds:.0f} s on all cores")
        cpu = cpu_baseline(cfg, k_np, v_np, q_rows, args.cpu_seconds, g_rows_fn=g_rows)
        # the oracle over one whole backward step at the measured rate (extrapolated; 10 d a pair)
        cpu["extrapolated_step_s"] = round(flops_per_step / (cpu["value"] * 1e12), 1)
        line["cpu_baseline"] = cpu
    print(json.dumps(line), flush=True)


def ring_balance(ra, torch, q_sh, k_sh, v_sh, N, sb, causal, layout_name):
    """Modeled ring time from measured block-pair times: on a real ring the N
    positions step in lockstep, so step s lasts as long as the slowest
    position's block (i - s) mod N; t(i, j) is one ra_block_attn_fwd launch
    of position i's queries against block j (0 when fully masked).  Returns
    the modeled time, the perfectly balanced time (sum / N) and their ratio,
    for the workload's layout and for the other layout of the same tokens."""
    out = {}
    lay = layout_name
    B, Hq, D = q_sh.shape[1], q_sh.shape[2], q_sh.shape[4]
    o = torch.empty((B, Hq, sb, D), dtype=torch.float32, device=q_sh.device)
    m = torch.empty((B, Hq, sb), dtype=torch.float32, device=q_sh.device)
    l = torch.empty_like(m)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for name in (lay, "striped" if lay == "contiguous" else "contiguous"):
        t = np.zeros((N, N))
        for i in range(N):
            for j in range(N):
                off = ra.ra_ring_pair_offset(name, N, sb, i, j)
                if causal and ra.ra_unmasked_pairs(sb, sb, True, off) == 0:
                    continue
                # the mask offset alone decides the work of a pair; the data of the
                # workload's own shards stands in for the other layout's
                kw = dict(causal=causal, q_pos0=off, k_pos0=0)
                ra.ra_block_attn_fwd(q_sh[i], k_sh[j], v_sh[j], o, m, l, **kw)  # warm
                e0.record()
                for _ in range(3):
                    ra.ra_block_attn_fwd(q_sh[i], k_sh[j], v_sh[j], o, m, l, **kw)
                e1.record()
                torch.cuda.synchronize()
                t[i, j] = e0.elapsed_time(e1) / 3
        steps = [max(t[i, (i - s) % N] for i in range(N)) for s in range(N)]
        modeled, balanced = float(sum(steps)), float(t.sum() / N)
        out[name] = {"modeled_ring_ms": round(modeled, 4), "balanced_ms": round(balanced, 4),
                     "imbalance": round(modeled / balanced, 4) if balanced else None}
    return out


class ClockSampler:
    """Samples the GPU's gfx clock (mean over its XCDs) in a background thread
    while a timed region runs, so that each rate is reported beside the clock
    it ran at (the chip holds well under its 2.4 GHz peak clock under a full
    MFMA load, and its XCDs differ).  Reads the GPU metrics through the amdsmi
    library in this process (no helper program is started); without amdsmi
    the summary is None."""

    def __init__(self, gpu=0, period_s=0.05):
        import threading
        self.period_s = period_s
        self.samples = []
        self.per_xcd = []
        self._stop = threading.Event()
        self._thread = None
        self._threading = threading
        self._handle = None
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            self._amdsmi = amdsmi
            self._handle = amdsmi.amdsmi_get_processor_handles()[gpu]
        except Exception:  # no library, no permission: no clock figures
            self._handle = None

    def _read(self):
        m = self._amdsmi.amdsmi_get_gpu_metrics_info(self._handle)
        clks = m.get("current_gfxclks")
        if isinstance(clks, (list, tuple)):
            vals = [float(x) for x in clks if isinstance(x, (int, float)) and 0 < x < 10000]
            if vals:
                return vals
        c = m.get("current_gfxclk")
        return [float(c)] if isinstance(c, (int, float)) and 0 < c < 10000 else []

    def _loop(self):
        while not self._stop.is_set():
            try:
                mhz = self._read()
                if mhz and min(mhz) > 500:  # skip samples taken while the GPU idled
                    self.samples.append(sum(mhz) / len(mhz))
                    self.per_xcd.append(mhz)
            except Exception:  # a failed read is just a missing sample
                pass
            self._stop.wait(self.period_s)

    def __enter__(self):
        if self._handle is not None:
            self._thread = self._threading.Thread(target=self._loop, daemon=True)
            self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        if self._thread:
            self._thread.join(timeout=15)

    def summary(self, skip_frac=0.0):
        """Mean clock over the samples, the first skip_frac of them dropped (the
        clock settles during the first part of a sustained load)."""
        n0 = int(len(self.samples) * skip_frac)
        s, x = self.samples[n0:], self.per_xcd[n0:]
        if not s:
            return None
        widths = {len(r) for r in x}
        xcd = np.mean(np.array(x), axis=0).tolist() if len(widths) == 1 else None
        return {"mean_mhz": round(float(np.mean(s)), 1), "min_mhz": round(float(np.min(s)), 1),
                "max_mhz": round(float(np.max(s)), 1), "samples": len(s),
                "per_xcd_mean_mhz": None if xcd is None else [round(float(v), 1) for v in xcd],
                "source": "amdsmi gpu metrics (current gfx clock of each XCD)"}


def sustained_clock(run_step, torch, seconds=2.5):
    """The gfx clock under this workload's sustained load: the step repeated
    back to back for about `seconds` while the clock is sampled (first third
    of the samples dropped)."""
    with ClockSampler() as clk:
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < seconds:
            run_step(False)
            torch.cuda.synchronize()
    return clk.summary(skip_frac=1 / 3)


def mfma_peak_at(clock):
    """Dense bf16 MFMA rate of the whole chip at a clock (256 CUs x 4096 FLOP/clk)."""
    return None if clock is None else 256 * 4096 * clock["mean_mhz"] * 1e6 / 1e12


def run_forward(args, name, ra, torch, dev, cpu_seconds, quiet=False):
    """Forward measurement of one workload: the timed steps, the block kernel's
    roofline, the merge rate, ring balance and the CPU baseline.  Returns the
    JSON record (without printing it)."""
    import ra_inputs

    cfg = WORKLOADS[name]
    B, Hq, Hkv, S, D, N, lay = (cfg[k] for k in ("B", "Hq", "Hkv", "S", "D", "N", "layout"))
    sb = S // N
    log(f"workload {name}: generating inputs")
    t0 = time.perf_counter()
    k_np = ra_inputs.normal((B, Hkv, S, D), ra_inputs.STREAM_K, seed=args.seed, dtype="bf16")
    v_np = ra_inputs.normal((B, Hkv, S, D), ra_inputs.STREAM_V, seed=args.seed, dtype="bf16")
    if cfg["share"] is not None:
        i = cfg["share"]
        t0q, tstride = (i, N) if lay == "striped" else (i * sb, 1)
        q_np = ra_inputs.normal((B, Hq, S, D), ra_inputs.STREAM_Q, seed=args.seed, dtype="bf16", t0=t0q,
                                t_stride=tstride, n_rows=sb)

        def q_rows(h, t):
            r = (t - i) // N if lay == "striped" else t - i * sb
            return q_np[0][h, r]
    else:
        q_np = ra_inputs.normal((B, Hq, S, D), ra_inputs.STREAM_Q, seed=args.seed, dtype="bf16")

        def q_rows(h, t):
            return q_np[0][h, t]
    log(f"inputs generated in {time.perf_counter() - t0:.1f} s; uploading")

    def to_dev(x):
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev)

    k_g, v_g = to_dev(k_np), to_dev(v_np)
    k_sh = torch.empty((N, B, Hkv, sb, D), dtype=torch.bfloat16, device=dev)
    v_sh = torch.empty_like(k_sh)
    if cfg["share"] is not None:
        q_sh = to_dev(q_np)[None]
        first, n_run = cfg["share"], 1
        q_g = None
    else:
        q_g = to_dev(q_np)
        q_sh = torch.empty((N, B, Hq, sb, D), dtype=torch.bfloat16, device=dev)
        first, n_run = 0, N
    o_sh = torch.empty_like(q_sh)
    lse = torch.empty(q_sh.shape[:4], dtype=torch.float32, device=dev)
    o_full = torch.empty((B, Hq, S, D), dtype=torch.bfloat16, device=dev) if q_g is not None else None
    desc = ra.ring_desc(q_sh, k_sh, n_pos=N, first_pos=first, layout=lay, causal=cfg["causal"],
                        separate_merge=args.separate_merge, kv_splits=args.kv_splits)
    workspace = torch.empty(ra.ra_ring_workspace_size(desc), dtype=torch.uint8, device=dev)
    kv_splits = args.kv_splits

    def step(stats, n_streams=args.n_streams):
        ra.ra_stripe_permute(k_g, k_sh, layout=lay, inverse=False, n_pos=N)
        ra.ra_stripe_permute(v_g, v_sh, layout=lay, inverse=False, n_pos=N)
        if q_g is not None:
            ra.ra_stripe_permute(q_g, q_sh, layout=lay, inverse=False, n_pos=N)
        st = ra.ra_ring_forward(q_sh, k_sh, v_sh, o_sh, lse, n_pos=N, first_pos=first, layout=lay,
                                causal=cfg["causal"], workspace=workspace, stats=stats,
                                separate_merge=args.separate_merge, n_streams=n_streams, kv_splits=kv_splits)
        if o_full is not None:
            ra.ra_stripe_permute(o_sh, o_full, layout=lay, inverse=True, n_pos=N)
        return st

    if args.backward:
        run_backward(args, cfg, ra, torch, step, q_sh, k_sh, v_sh, o_sh, lse, first, n_run, dev, k_np, v_np, q_rows)
        return None

    log(f"warmup {args.warmup}")
    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    # the step's work accounting (FLOPs, key ranges) from one untimed step
    st = step(True)
    torch.cuda.synchronize()
    flops_per_step = st["flops"]
    splits = int(st["kv_splits"])  # key ranges per block launch
    run_step = step
    if args.graph:  # the library's streams and events exist after the eager steps above
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step(False)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(graph):
            step(False)
        torch.cuda.synchronize()

        def run_step(_stats):
            graph.replay()
    log(f"timing {args.steps} steps")
    # steps are enqueued back to back; events on the caller's stream (which
    # every step's work joins) give per-step times without a host round trip
    marks = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for e0, e1 in marks:
        e0.record()
        run_step(False)
        e1.record()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    step_ms = [e0.elapsed_time(e1) for e0, e1 in marks]
    ms_per_step = elapsed / args.steps * 1e3
    value = flops_per_step / (ms_per_step * 1e-3) / 1e12
    log(f"{ms_per_step:.3f} ms/step, {value:.1f} TFLOP/s")
    log("clock under sustained load")
    clock = sustained_clock(run_step, torch)

    # block-attention kernel roofline: algorithmic FLOPs per launch / mean launch
    # time, from HIP events around every launch in 3 steps after the timed
    # region.  The timed schedule may run launches on several streams (the
    # positions of a whole ring, the two accumulation chains of a share), where
    # launches overlap and event spans overstate each one; the launches are
    # therefore timed on one stream, with the key ranges of the timed steps.
    n_stat = 3
    rt = {"block_ms": 0.0, "block_launches": 0, "merge_ms": 0.0, "merge_launches": 0, "flops": 0.0}
    stat_streams = 1
    if n_run > 1:
        kv_splits = splits  # whatever one stream alone would choose
        if splits > 1:
            workspace = torch.empty(ra.ra_ring_workspace_size(ra.ring_desc(
                q_sh, k_sh, n_pos=N, first_pos=first, layout=lay, causal=cfg["causal"], n_streams=1,
                kv_splits=splits)), dtype=torch.uint8, device=dev)
    for _ in range(n_stat):
        st = step(True, n_streams=stat_streams)
        for key in rt:
            rt[key] += st[key]
    torch.cuda.synchronize()
    per_launch_flops = rt["flops"] / max(1, rt["block_launches"])
    per_launch_ms = rt["block_ms"] / max(1, rt["block_launches"])
    achieved = per_launch_flops / (per_launch_ms * 1e-3) / 1e12
    traffic = traffic_from_profile(os.path.join(ROOT, "ring_attention_step_amd", "csrc", "block_attn_mfma.hip"),
                                   name)
    at_clock = mfma_peak_at(clock)
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                "kernel": "block_mfma_kernel<128>" if D == 128 else "block_mfma_kernel<64>",
                "launches": rt["block_launches"], "mean_launch_ms": round(per_launch_ms, 4),
                "timing": "HIP events around each launch on its stream, 3 steps after the timed ones" +
                          (" (on one stream)" if n_run > 1 else ""),
                "clock": clock,  # gfx clock while the step repeats back to back (amdsmi)
                "peak_at_clock": None if at_clock is None else round(at_clock, 1),
                "frac_at_clock": None if at_clock is None else round(achieved / at_clock, 4)}

    # merge kernel: algorithmic bytes per step.  A state (fp32 O, m, l) is
    # 4 D + 8 bytes a row, a finalised row (bf16 output, log-sum-exp) 2 D + 4.
    # Fused schedule: the block kernel folds each partial into the running
    # state, and the merge kernel only finalises (read a state, write a row).
    # Separate schedule: per position with c computed blocks, c - 2 plain folds
    # (read two states, write one) and one fold that finalises.  Key splits
    # (n ranges): every computed block's fold reads n partials and the running
    # state (none at the first), and writes the state (or, at the last, a row).
    rows_pos = B * Hq * sb
    st_b, row_b = 4 * D + 8, 2 * D + 4
    merge_bytes = 0
    for p in range(n_run):
        c = sum(1 for j in range(N)
                if not (cfg["causal"] and ra.ra_unmasked_pairs(
                    sb, sb, True, ra.ra_ring_pair_offset(lay, N, sb, first + p, j)) == 0))
        if splits > 1:
            for s_i in range(c):
                merge_bytes += rows_pos * (splits * st_b + (st_b if s_i else 0) + (row_b if s_i == c - 1 else st_b))
        elif c == 1 or not args.separate_merge:
            merge_bytes += rows_pos * (st_b + row_b)
        else:
            merge_bytes += (c - 2) * rows_pos * 3 * st_b + rows_pos * (2 * st_b + row_b)
    n_merge = rt["merge_launches"]
    merge = None
    if n_merge:
        gbps = merge_bytes * n_stat / (rt["merge_ms"] * 1e-3) / 1e9
        merge = {"bound": "hbm", "achieved": round(gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                 "frac": round(gbps / PEAK_HBM_GBPS, 4), "launches": n_merge,
                 "mean_launch_ms": round(rt["merge_ms"] / n_merge, 4),
                 "bytes_per_step": merge_bytes}

    balance = None
    if n_run > 1 and cfg["causal"]:
        log("ring balance: timing every (position, block) pair")
        balance = ring_balance(ra, torch, q_sh, k_sh, v_sh, N, sb, cfg["causal"], lay)

    cpu = None
    if cpu_seconds > 0:
        log(f"cpu baseline: oracle for about {cpu_seconds:.0f} s on all cores, then a third of that on one")
        cpu = cpu_baseline(cfg, k_np, v_np, q_rows, cpu_seconds)
        one = cpu_baseline(cfg, k_np, v_np, q_rows, cpu_seconds / 3, threads=1)
        cpu["one_core"] = {"value": one["value"], "unit": one["unit"], "cores": 1, "sample": one["sample"]}
        # the oracle over one whole step of this workload, at the measured rate (extrapolated)
        cpu["extrapolated_step_s"] = round(flops_per_step / (cpu["value"] * 1e12), 1)

    return {
        "metric": "ring-attention fwd TFLOP/s (causal-adjusted) + % of MI355X bf16 MFMA peak",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "ms_per_step_median": round(float(np.median(step_ms)), 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "pct_of_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "config": {"workload": name, "batch": B, "q_heads": Hq, "kv_heads": Hkv, "seq_len": S,
                   "head_dim": D, "ring_positions": N, "layout": lay, "causal": cfg["causal"],
                   "positions_run": n_run, "first_position": first,
                   "merge_schedule": "separate" if args.separate_merge else "fused", "kv_splits": splits,
                   "launch": "hip graph replay" if args.graph else "eager",
                   "unmasked_flops_per_step": flops_per_step},
        "roofline": roofline, "merge": merge, "cpu_baseline": cpu,
        "ring_balance": balance,
    }


# the second causal striped workload measured beside the default one
COMPANION = "causal-256k-striped-share"


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=DEFAULT, choices=sorted(WORKLOADS))
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="CPU time budget of the oracle baseline (0 = skip)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--backward", action="store_true",
                    help="time the ring backward (dQ, dK, dV) instead of the forward")
    ap.add_argument("--separate-merge", action="store_true",
                    help="fold each block's partial with a separate merge launch instead of in the block kernel")
    ap.add_argument("--graph", action="store_true",
                    help="capture one step in a HIP graph and time its replays (launch overhead removed)")
    ap.add_argument("--kv-splits", type=int, default=0,
                    help="key ranges per block launch (0: the library's automatic choice, 1: none)")
    ap.add_argument("--n-streams", type=int, default=0,
                    help="library streams a whole ring's positions run on (0: the library's choice)")
    ap.add_argument("--no-companion", action="store_true",
                    help=f"with the default workload, skip the {COMPANION} measurement reported beside it")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the ring positions are virtual positions on a single "
              "MI355X; run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    import ring_attention_step_amd as ra

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    ra.load_library()

    line = run_forward(args, args.workload, ra, torch, dev, args.cpu_seconds)
    if line is None:  # the backward printed its own line
        return
    if args.workload == DEFAULT and not args.no_companion and not args.backward:
        # the other causal striped workload, whose block kernel carries the same
        # 50%-of-peak target: measured in the same run, on the same GPU
        torch.cuda.empty_cache()
        comp = run_forward(args, COMPANION, ra, torch, dev, 0)
        line["companion"] = {k: comp[k] for k in ("config", "value", "ms_per_step", "ms_per_step_median",
                                                  "pct_of_bf16_peak", "roofline", "merge")}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
