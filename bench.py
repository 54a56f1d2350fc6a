"""Throughput of the Taylor linear attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config cfg2] [--no-extra] [--no-cpu]

A step is one ``based_prefill`` call over one batch of the headline
workload (default cfg2: the BASED-360M-shaped prefill layer, B=8, H=16,
L=2048, d'=16, d_v=64, bf16, chunk 64), inputs already resident in HBM.
Steps cycle over four distinct input/output buffer sets so that consecutive
steps do not re-read the previous step's data from the 256 MB Infinity
Cache.  Before anything is timed the GPU runs the step untimed for a fixed
wall-clock time (the settle phase: the first ~20 ms of work run at the idle
clock), then W warm-up steps; the K timed steps are captured once in a HIP
graph and replayed, so that host-side launch gaps do not enter the step
time.  Rank 0 prints one JSON line with:

* value: tokens/s (tokens = B*L per step, each token covering all H heads);
* roofline: the prefill kernel's algorithmic bytes per launch / its mean
  launch duration (HIP events on the launch stream around the timed replay,
  over the number of launches), against 8 TB/s HBM (the kernel's
  arithmetic intensity is below the bf16 MFMA ridge), plus its algorithmic
  flop rate against the 2.5 PFLOP/s dense bf16 MFMA peak and the median,
  p10 and p90 of single launches; `traffic` comes from the committed
  rocprofv3 FETCH_SIZE/WRITE_SIZE summary when that summary was taken on
  the current kernel source;
* cpu_baseline: the fp64 oracle (recurrent form) timed on the host cores on
  a sample of whole heads of the same workload, with the thread count, the
  CPU model and a one-core rate;
* extra: every other configuration, each leg with its own roofline (bytes
  or flops per launch, mean and median/p10/p90 launch time, fraction of
  peak, counter traffic where a summary exists) and, where the oracle has
  the routine, its CPU rate on a sample: the 1.3B decode (its 1024-token
  setup prefill at d_v = 128, then 1024 next-token steps), the 8K window
  layer (linear branch, window branch with fused add, the fused hybrid
  layer), the 64K prefill, the tiny fp32 layer, the window's next-token
  step, the gradients of the prefill and of the window, and the other
  feature dims and window sizes.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synthetic_inputs as si  # noqa: E402

HBM_PEAK = 8.0e12          # B/s, MI355X HBM3E
MFMA_BF16_PEAK = 2.5e15    # flop/s, dense bf16
MFMA_F32_PEAK = 157.3e12   # flop/s, dense fp32 matrix cores
METRIC = "tokens/sec for Taylor lin-attn prefill & decode; % of HBM / MFMA peak"
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "linear_attention_sequence_taylor_amd", "csrc")
BUILD_SCRIPT = os.path.join(ROOT, "linear_attention_sequence_taylor_amd", "build.py")
# the sources of the bf16 prefill and fused hybrid kernels (their counter
# summaries are valid while these are unchanged)
PREFILL_SOURCES = ("prefill_mfma.hip", "prefill_mfma_kernels.hpp", "prefill_mfma_ilp.hip", "common.hpp")
N_SETS = 4
F = 273


# ---------------------------------------------------------------- algorithmic work
def prefill_bytes(wl) -> int:
    """q,k,v read once, y written once (fp32), final state written once."""
    es = 2 if wl.dtype == "bf16" else 4
    tok_heads = wl.B * wl.H * wl.L
    per_tok = 2 * wl.d * es + wl.dv * es + wl.dv * 4
    state = (F * wl.dv + F) * 4
    return tok_heads * per_tok + wl.B * wl.H * state


def prefill_flops(wl) -> int:
    """Per token-head: 4*F*d_v (state update + readout, 2 flop per MAC) plus
    the causal on-diagonal term (C+1)*(d'+d_v)."""
    return wl.B * wl.H * wl.L * (4 * F * wl.dv + (wl.chunk + 1) * (wl.d + wl.dv))


def decode_bytes(wl) -> int:
    es = 2
    per_head = 2 * (F * wl.dv + F) * 4 + 2 * wl.d * es + wl.dv * es + wl.dv * 4
    return wl.B * wl.H * per_head


def swa_bytes(wl) -> int:
    es = 2
    per_tok = 2 * wl.d_qk * es + wl.dv * es + 2 * wl.dv * 4
    return wl.B * wl.H * wl.L * per_tok


def hybrid_bytes(wl) -> int:
    """The whole hybrid layer in one pass: both branches' q, k and the shared
    v read once, y written once (fp32), the final linear-attention state
    written once."""
    es = 2
    per_tok = 2 * wl.d * es + 2 * wl.d_qk * es + wl.dv * es + wl.dv * 4
    return wl.B * wl.H * wl.L * per_tok + wl.B * wl.H * (F * wl.dv + F) * 4


def window_decode_bytes(wl) -> int:
    """Per tok-head: the window-1 cached key/value rows read, the new row
    written to its slot, q,k,v read, the fused-add input read and y written."""
    es = 2
    row = (wl.d_qk + wl.dv) * es
    per_head = (wl.window - 1) * row + row + (2 * wl.d_qk + wl.dv) * es + 2 * wl.dv * 4
    return wl.B * wl.H * per_head


# ---------------------------------------------------------------- helpers
def source_digest(*names) -> str:
    """Digest of the named csrc/ files and of the build script (whose
    per-source compiler flags change the kernels as much as the sources do)."""
    h = hashlib.sha256()
    for path in [os.path.join(CSRC, n) for n in names] + [BUILD_SCRIPT]:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(summary: str, digest: str, launches_per_kernel: int = 1):
    """HBM bytes per launch from a committed rocprofv3 --pmc summary, or None
    if absent or taken on a different kernel source."""
    path = os.path.join(PROFILES, summary)
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            key, val = line.split(":", 1)
            vals[key.strip()] = val.strip()
    if vals.get("kernel_source_sha256_16") != digest:
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


class RegionTimer:
    """HIP events on the launch stream around a whole timed region: the mean
    launch duration is the region's GPU time over the launches in it, with
    no event between launches (events between back-to-back launches add
    their own gaps)."""

    def __init__(self):
        self.e0 = torch.cuda.Event(enable_timing=True)
        self.e1 = torch.cuda.Event(enable_timing=True)

    def start(self):
        self.e0.record(torch.cuda.current_stream())

    def stop(self):
        self.e1.record(torch.cuda.current_stream())

    def seconds(self) -> float:
        self.e1.synchronize()
        return self.e0.elapsed_time(self.e1) / 1e3


def launch_distribution(launch, n: int) -> dict:
    """Median, p10 and p90 of single launches, each between its own pair of
    events (created beforehand), in a pass after the timed region."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    st = torch.cuda.current_stream()
    for i, (a, b) in enumerate(evs):
        a.record(st)
        launch(i)
        b.record(st)
    torch.cuda.synchronize()
    ts = sorted(a.elapsed_time(b) * 1e3 for a, b in evs)

    def pct(p):
        return ts[min(len(ts) - 1, int(round(p * (len(ts) - 1))))]

    return {"median_us": pct(0.5), "p10_us": pct(0.1), "p90_us": pct(0.9), "launches": n}


def settle(fn, seconds: float) -> int:
    """Runs fn(i) untimed for a wall-clock time (the GPU leaves its idle
    clock state only after ~20 ms of continuous work); returns the count."""
    t_end = time.perf_counter() + seconds
    i = 0
    while time.perf_counter() < t_end:
        fn(i)
        i += 1
        if i % 64 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    return i


def time_leg(fn, n: int, settle_s: float = 0.1, dist_n: int = 30):
    """Mean launch seconds of fn over n launches (events around the region on
    the launch stream), after a settle phase, and the per-launch
    distribution of a separate pass."""
    settle(fn, settle_s)
    timer = RegionTimer()
    torch.cuda.synchronize()
    timer.start()
    for i in range(n):
        fn(i)
    timer.stop()
    mean = timer.seconds() / n
    return mean, launch_distribution(fn, dist_n)


def roofline(nbytes: float, sec: float, traffic=None, flops: float | None = None, flop_peak: float = None,
             flop_unit: str = "bf16 MFMA") -> dict:
    """HBM roofline of one launch (algorithmic bytes / mean launch time), with
    the flop rate against a matrix-core peak where the kernel has one."""
    out = {"bound": "hbm", "achieved": nbytes / sec / 1e9, "peak": HBM_PEAK / 1e9, "unit": "GB/s",
           "frac": nbytes / sec / HBM_PEAK, "traffic": traffic, "algorithmic_bytes": nbytes}
    if flops is not None:
        out.update({"algorithmic_flops": flops, "tflops": flops / sec / 1e12,
                    "mfma_frac": flops / sec / (flop_peak or MFMA_BF16_PEAK), "mfma_peak": flop_unit})
    return out


def counter_mfma_busy(name: str, sec: float):
    """Matrix-core busy fraction from the committed SQ counter summary of the
    workload's prefill kernel (SQ_VALU_MFMA_BUSY_CYCLES: SIMD-cycles with an
    MFMA in flight, summed over the chip), over 1024 SIMDs x the mean launch
    time at the 2.4 GHz peak engine clock; None if the summary is absent or
    taken on other kernel sources.  It counts the hi/lo pairs' extra
    products, which the algorithmic fraction does not."""
    path = os.path.join(PROFILES, f"sq_counters_{name}.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if not line.startswith("#"):
            parts = line.replace(":", " ").split()
            if len(parts) >= 2:
                vals[parts[0]] = parts[1]
    if vals.get("kernel_source_sha256_16") != source_digest(*PREFILL_SOURCES):
        return None
    try:
        return float(vals["SQ_VALU_MFMA_BUSY_CYCLES"]) / (1024 * sec * 2.4e9)
    except (KeyError, ValueError):
        return None


def cpu_info() -> dict:
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        avail = os.cpu_count()
    return {"cpu_model": model, "nproc": avail, "os_cpu_count": os.cpu_count()}


def make_sets(tensors, n):
    out = [tuple(t.to("cuda") for t in tensors)]
    for _ in range(n - 1):
        out.append(tuple(t.clone() for t in out[0]))
    return out


# ---------------------------------------------------------------- legs
def prefill_sets(based, wl, n_sets=N_SETS):
    q, k, v = si.linear_inputs(wl)
    ins = make_sets((q, k, v), n_sets)
    outs = [(torch.empty(wl.B, wl.H, wl.L, wl.dv, device="cuda"), torch.empty(wl.B, wl.H, F, wl.dv, device="cuda"),
             torch.empty(wl.B, wl.H, F, device="cuda")) for _ in range(n_sets)]
    nbytes = based.based_prefill_workspace_bytes(wl.B, wl.H, wl.L, wl.dv)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device="cuda")

    def step(i):
        (qq, kk, vv), (y, S, z) = ins[i % n_sets], outs[i % n_sets]
        based.based_prefill(qq, kk, vv, chunk=wl.chunk, eps=wl.eps, y=y, S=S, z=z, workspace=ws)

    return step


def bench_headline(step, steps, warmup, settle_s=0.3):
    """The headline leg.  Settle phase, W warm-up steps, then K steps
    captured in a HIP graph and replayed once: returns (wall seconds per
    step, mean launch seconds from events around the replay, per-launch
    distribution)."""
    settle(step, settle_s)
    for i in range(warmup):
        step(i)
    # capture on a side stream after an eager run there (as torch requires)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(0)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(steps):
            step(i)
    g.replay()  # untimed: first replay of a new graph
    settle(step, 0.05)
    timer = RegionTimer()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    timer.start()
    g.replay()
    timer.stop()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    dist = launch_distribution(step, min(max(steps, 20), 50))
    return wall / steps, timer.seconds() / steps, dist


def headline_spec(based, cfg: str) -> dict:
    """The step of the headline configuration: the library call(s) of one
    step over synthetic inputs of the configuration's shape, tokens per step,
    algorithmic bytes (and flops where the matrix cores carry the leg), the
    counter summary behind `traffic` and the JSON `config`."""
    wl = si.WORKLOADS[CONFIGS[cfg]]
    conf = {"workload": wl.name, "B": wl.B, "H": wl.H, "L": wl.L, "d_feat": wl.d, "d_v": wl.dv, "chunk": wl.chunk,
            "scale": wl.scale, "parallelism": "single GPU"}
    if cfg in ("cfg2", "cfg5"):
        return {"wl": wl, "step": prefill_sets(based, wl), "tokens": wl.B * wl.L, "bytes": prefill_bytes(wl),
                "flops": prefill_flops(wl), "kernel": "based_prefill (bf16 MFMA)",
                "traffic": (f"prefill_mfma_{wl.name}_pmc.txt", PREFILL_SOURCES), "config": conf}
    if cfg == "cfg3":
        # the state of a 1024-token prefix, then steps cycling over 4 input sets
        q, k, v = (t.cuda() for t in si.linear_inputs(wl))
        S = torch.empty(wl.B, wl.H, F, wl.dv, device="cuda")
        z = torch.empty(wl.B, wl.H, F, device="cuda")
        based.based_prefill(q, k, v, chunk=wl.chunk, eps=wl.eps, S=S, z=z)
        del q, k, v
        ins = [tuple(t.cuda() for t in si.decode_inputs(wl, t)) for t in range(N_SETS)]
        y = torch.empty(wl.B, wl.H, wl.dv, device="cuda")

        def step(i):
            based.based_decode_step(*ins[i % N_SETS], S, z, eps=wl.eps, y=y)
        conf.update({"L": 1, "prefix": wl.L})
        return {"wl": wl, "step": step, "tokens": wl.B, "bytes": decode_bytes(wl), "flops": None,
                "kernel": "based_decode_step", "traffic": ("decode_step_decode_1p3b_pmc.txt", ("decode.hip", "common.hpp")),
                "config": conf}
    if cfg == "cfg4":
        q, k, v = si.linear_inputs(wl)
        qw, kw = si.window_inputs(wl)
        sets = make_sets((q, k, qw, kw, v), 2)
        ws = torch.empty(max(based.based_hybrid_prefill_workspace_bytes(wl.B, wl.H, wl.L, wl.dv), 1),
                         dtype=torch.uint8, device="cuda")
        ys = [torch.empty(wl.B, wl.H, wl.L, wl.dv, device="cuda") for _ in range(2)]

        def step(i):
            based.based_hybrid_prefill(*sets[i % 2], chunk=wl.chunk, eps=wl.eps, window=wl.window,
                                       scale=wl.swa_scale, y=ys[i % 2], workspace=ws)
        conf.update({"window": wl.window, "d_qk": wl.d_qk})
        return {"wl": wl, "step": step, "tokens": wl.B * wl.L, "bytes": hybrid_bytes(wl), "flops": None,
                "kernel": "based_hybrid_prefill", "config": conf,
                "traffic": ("prefill_mfma_hybrid_window_8k_pmc.txt", PREFILL_SOURCES)}
    # cfg1: the tiny fp32 layer, linear attention then the window adding into y
    q, k, v = (t.cuda() for t in si.linear_inputs(wl))
    y = torch.empty(1, 1, wl.L, wl.dv, device="cuda")
    S, z = torch.empty(1, 1, F, wl.dv, device="cuda"), torch.empty(1, 1, F, device="cuda")

    def step(i):
        based.based_prefill(q, k, v, chunk=wl.chunk, eps=wl.eps, y=y, S=S, z=z)
        based.swa_forward(q, k, v, window=wl.window, scale=wl.swa_scale, add=y, y=y)
    conf.update({"window": wl.window})
    return {"wl": wl, "step": step, "tokens": wl.L, "bytes": prefill_bytes(wl) + swa_bytes(wl), "flops": None,
            "kernel": "based_prefill + swa_forward (fp32)", "traffic": None, "config": conf}


def bench_prefill_leg(based, wl, n=50):
    """A prefill workload as an extra leg: mean launch time and distribution."""
    return time_leg(prefill_sets(based, wl), n, settle_s=0.15, dist_n=30)


def bench_decode(based, wl, n_steps):
    """1024-token prefill (the d_v = 128 setup, timed as its own leg), then
    n_steps next-token steps timed as one region, and a per-step
    distribution on a copy of the state.  Returns (setup mean seconds,
    setup distribution, wall seconds per step, event seconds per step, step
    distribution)."""
    q, k, v = si.linear_inputs(wl)
    qd, kd, vd = (t.cuda() for t in (q, k, v))
    del q, k, v
    S = torch.empty(wl.B, wl.H, F, wl.dv, device="cuda")
    z = torch.empty(wl.B, wl.H, F, device="cuda")
    yp = torch.empty(wl.B, wl.H, wl.L, wl.dv, device="cuda")
    ws = torch.empty(max(1, based.based_prefill_workspace_bytes(wl.B, wl.H, wl.L, wl.dv)), dtype=torch.uint8,
                     device="cuda")

    def setup(i):
        based.based_prefill(qd, kd, vd, chunk=wl.chunk, eps=wl.eps, y=yp, S=S, z=z, workspace=ws)

    setup_s, setup_dist = time_leg(setup, 10, settle_s=0.1, dist_n=10)
    setup(0)
    del qd, kd, vd, yp
    step_in = [tuple(t.cuda() for t in si.decode_inputs(wl, t)) for t in range(n_steps)]
    y = torch.empty(wl.B, wl.H, wl.dv, device="cuda")
    # untimed settle on a copy of the state
    S2, z2 = S.clone(), z.clone()
    settle(lambda t: based.based_decode_step(*step_in[t % n_steps], S2, z2, eps=wl.eps, y=y), 0.1)
    dist = launch_distribution(lambda t: based.based_decode_step(*step_in[t % n_steps], S2, z2, eps=wl.eps, y=y), 50)
    del S2, z2
    timer = RegionTimer()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    timer.start()
    for t in range(n_steps):
        based.based_decode_step(*step_in[t], S, z, eps=wl.eps, y=y)
    timer.stop()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return setup_s, setup_dist, wall / n_steps, timer.seconds() / n_steps, dist


def bench_swa(based, wl, reps, window=None):
    """Window kernel with fused add, alternating two input/output sets;
    returns (mean launch seconds over the timed region, distribution)."""
    window = wl.window if window is None else window
    q, k, v = si.linear_inputs(wl)
    qw, kw = si.window_inputs(wl)
    sets = make_sets((qw, kw, v), 2)
    del q, k
    adds = [torch.randn(wl.B, wl.H, wl.L, wl.dv, device="cuda") for _ in range(2)]
    ys = [torch.empty_like(adds[0]) for _ in range(2)]

    def launch(i):
        based.swa_forward(*sets[i % 2], window=window, scale=wl.swa_scale, add=adds[i % 2], y=ys[i % 2])

    return time_leg(launch, reps, settle_s=0.1, dist_n=30)


def bench_hybrid(based, wl, reps):
    """The whole hybrid layer (linear attention + window, summed) through
    based_hybrid_prefill with each path: "auto" (the library's choice),
    "fused" (one kernel) and "two_pass" (prefill, then the window adding into
    y).  Two input/output sets alternate (1.4 GB, past the Infinity Cache).
    Returns {path: event seconds per layer}."""
    q, k, v = si.linear_inputs(wl)
    qw, kw = si.window_inputs(wl)
    sets = make_sets((q, k, qw, kw, v), 2)
    del q, k, v, qw, kw
    outs = [(torch.empty(wl.B, wl.H, wl.L, wl.dv, device="cuda"), torch.empty(wl.B, wl.H, F, wl.dv, device="cuda"),
             torch.empty(wl.B, wl.H, F, device="cuda")) for _ in range(2)]
    ws = torch.empty(max(based.based_hybrid_prefill_workspace_bytes(wl.B, wl.H, wl.L, wl.dv), 1), dtype=torch.uint8,
                     device="cuda")

    def layer(i, path):
        qq, kk, qqw, kkw, vv = sets[i % 2]
        y, S, z = outs[i % 2]
        based.based_hybrid_prefill(qq, kk, qqw, kkw, vv, chunk=wl.chunk, eps=wl.eps, window=wl.window,
                                   scale=wl.swa_scale, path=path, y=y, S=S, z=z, workspace=ws)

    res = {}
    for path in ("auto", "fused", "two_pass"):
        sec, dist = time_leg(lambda i: layer(i, path), reps, settle_s=0.1, dist_n=20)
        res[path] = sec
        res[path + "_dist"] = dist
    return res


def bench_window_decode(based, wl, n_steps, graph_steps=64, n_sets=16):
    """Window next-token steps (fused add of a fixed fp32 tensor standing in
    for the linear-attention output), captured as a HIP graph of 64 steps and
    replayed; the steps cycle over 16 filled cache sets (805 MB) so that every
    step reads its ring from HBM, not from the 256 MB Infinity Cache.
    Returns event seconds per step over the timed replays."""
    _, k = si.window_inputs(wl)
    v = si.linear_inputs(wl)[2]
    kd, vd = k.cuda(), v.cuda()
    caches = [based.swa_cache_fill(kd, vd, window=wl.window) for _ in range(n_sets)]
    del kd, vd, k, v
    steps = [tuple(t.cuda() for t in si.window_decode_inputs(wl, t)) for t in range(graph_steps)]
    pos = [torch.full((wl.B,), wl.L + t, dtype=torch.int64, device="cuda") for t in range(graph_steps)]
    add = torch.randn(wl.B, wl.H, wl.dv, device="cuda")
    y = torch.empty_like(add)

    def run_all():
        for t in range(graph_steps):
            kc, vc = caches[t % n_sets]
            based.swa_decode_step(*steps[t], kc, vc, pos[t], scale=wl.swa_scale, add=add, y=y)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run_all()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run_all()
    for _ in range(100):  # untimed warm-up, ~50 ms
        g.replay()
    reps = max(1, n_steps // graph_steps)
    timer = RegionTimer()
    torch.cuda.synchronize()
    timer.start()
    for _ in range(reps):
        g.replay()
    timer.stop()
    return timer.seconds() / (reps * graph_steps)


def bench_layer_decode(based, wd, ww, n_steps, graph_steps=64):
    """One BASED-1.3B layer's next-token step: the linear-attention step
    (state from a 1024-token prefill) and then the window step on the same
    token (shared v; its ring filled from the same prefix), adding into the
    linear output.  HIP graph of 64 layer steps, replayed; returns event
    seconds per layer step."""
    q, k, v = si.linear_inputs(wd)
    qd, kd, vd = (t.cuda() for t in (q, k, v))
    del q, k, v
    S = torch.empty(wd.B, wd.H, F, wd.dv, device="cuda")
    z = torch.empty(wd.B, wd.H, F, device="cuda")
    yp = torch.empty(wd.B, wd.H, wd.L, wd.dv, device="cuda")
    ws = torch.empty(max(1, based.based_prefill_workspace_bytes(wd.B, wd.H, wd.L, wd.dv)), dtype=torch.uint8,
                     device="cuda")
    based.based_prefill(qd, kd, vd, chunk=wd.chunk, eps=wd.eps, y=yp, S=S, z=z, workspace=ws)
    del yp, ws
    kw = si.randn((wd.B, wd.H, wd.L, ww.d_qk), 1000 * ww.index + 11, 1.0, torch.bfloat16).cuda()
    kc, vc = based.swa_cache_fill(kw, vd, window=ww.window)
    del qd, kd, vd, kw
    steps = []
    for t in range(graph_steps):
        ql, kl, vl = (x.cuda() for x in si.decode_inputs(wd, t))
        qw, kww = (x.cuda() for x in si.window_decode_inputs(ww, t)[:2])
        steps.append((ql, kl, vl, qw, kww))
    pos = [torch.full((wd.B,), wd.L + t, dtype=torch.int64, device="cuda") for t in range(graph_steps)]
    y = torch.empty(wd.B, wd.H, wd.dv, device="cuda")

    def run_all():
        for t in range(graph_steps):
            ql, kl, vl, qw, kww = steps[t]
            based.based_decode_step(ql, kl, vl, S, z, eps=wd.eps, y=y)
            based.swa_decode_step(qw, kww, vl, kc, vc, pos[t], scale=ww.swa_scale, add=y, y=y)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run_all()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run_all()
    for _ in range(3):  # untimed warm-up
        g.replay()
    reps = max(1, n_steps // graph_steps)
    timer = RegionTimer()
    torch.cuda.synchronize()
    timer.start()
    for _ in range(reps):
        g.replay()
    timer.stop()
    return timer.seconds() / (reps * graph_steps)


def bench_other_sizes(based):
    """The pages' other design points (feature dim 32, window 128), on the
    paths that carry them: seeded inputs, event-timed regions.  Returns a
    dict of legs (report only)."""
    out = {}
    # window 128 over the 8K window workload inputs (matrix cores, two-tile
    # halo), timed exactly as the w = 64 leg
    ww = si.WORKLOADS["window_8k"]
    sec, _ = bench_swa(based, ww, 100, window=128)
    sb = swa_bytes(ww)
    out["window_8k_w128"] = {"kernel_us": sec * 1e6, "hbm_GBps": sb / sec / 1e9, "hbm_frac": sb / sec / HBM_PEAK,
                             "algorithmic_bytes": sb, "note": "w=128, fused add, matrix cores with a two-tile halo"}
    # next-token step with feature dim 32 (F = 1057), the 1.3B decode batch
    # (B=128, H=16, d_v=128; 1.1 GB of fp32 state), from a zero state
    B, H, d, dv, F32 = 128, 16, 32, 128, 1 + 32 + 32 * 32
    steps = [tuple(x.cuda() for x in si.custom((B, H, d), (B, H, dv), seed=2000 + i)) for i in range(16)]
    S = torch.zeros(B, H, F32, dv, device="cuda")
    z = torch.zeros(B, H, F32, device="cuda")
    yd = torch.empty(B, H, dv, device="cuda")
    for i in range(300):
        based.based_decode_step(*steps[i % 16], S, z, y=yd)
    t = RegionTimer()
    torch.cuda.synchronize()
    t.start()
    for i in range(256):
        based.based_decode_step(*steps[i % 16], S, z, y=yd)
    t.stop()
    sec = t.seconds() / 256
    db = B * H * (2 * (F32 * dv + F32) * 4 + 2 * d * 2 + dv * 2 + dv * 4)
    out["decode_d32"] = {"kernel_us": sec * 1e6, "hbm_GBps": db / sec / 1e9, "hbm_frac": db / sec / HBM_PEAK,
                         "algorithmic_bytes": db, "note": "feature dim 32, B=128, H=16, d_v=128, bf16 inputs"}
    del S, z, steps
    # prefill with feature dim 32 (bf16 inputs widened, fp32 matrix cores), B=2, H=16, L=2048, d_v=64
    B, H, L, dv = 2, 16, 2048, 64
    q, k, v = (x.cuda() for x in si.custom((B, H, L, d), (B, H, L, dv), seed=2100, scale=0.5))
    outs = dict(y=torch.empty(B, H, L, dv, device="cuda"), S=torch.empty(B, H, F32, dv, device="cuda"),
                z=torch.empty(B, H, F32, device="cuda"),
                workspace=torch.empty(max(1, based.based_prefill_workspace_bytes(B, H, L, dv, d)), dtype=torch.uint8,
                                      device="cuda"))
    for _ in range(100):  # untimed warm-up, ~50 ms
        based.based_prefill(q, k, v, **outs)
    t = RegionTimer()
    torch.cuda.synchronize()
    t.start()
    for _ in range(20):
        based.based_prefill(q, k, v, **outs)
    t.stop()
    sec = t.seconds() / 20
    pb = B * H * L * (2 * d * 2 + dv * 2 + dv * 4) + B * H * (F32 * dv + F32) * 4
    # per tok-head: 4 F d_v (state update and readout) + the causal intra-chunk term
    pf = B * H * L * (4 * F32 * dv + 65 * (d + dv))
    out["prefill_d32"] = {"kernel_us": sec * 1e6, "tokens_per_s": B * L / sec, "hbm_frac": pb / sec / HBM_PEAK,
                          "algorithmic_bytes": pb, "algorithmic_flops": pf, "tflops": pf / sec / 1e12,
                          "mfma_f32_frac": pf / sec / MFMA_F32_PEAK,
                          "note": "feature dim 32, B=2, H=16, L=2048, fp32 arithmetic on the fp32 matrix cores; "
                                  "each head in 2 sequence segments (a state-only pass over the first, the prefix, "
                                  "then 256 workgroups: one per head, segment and 16 value columns)"}
    return out


SYM_FEATURES = 1 + 16 + 16 * 17 // 2  # 153 distinct Taylor features for d' = 16


def backward_flops(wl, form: str) -> float:
    """Algorithmic flops of the gradients over a workload.  Direct form: per
    causal (i, j) pair 8d + 6d_v + 12 (scores twice, weights, g.v, dq, dk,
    dv and N).  Chunked form (64-token chunks): per token six products
    with the 153 distinct features of d' = 16 (readout y, g S^T, S update,
    R update, R v, phi(k) R: 2 x 153 x d_v flops each) plus the direct
    form's pairs inside the token's chunk (65/2 per token on average)."""
    per_pair = 8 * wl.d + 6 * wl.dv + 12
    if form == "direct":
        return wl.B * wl.H * wl.L * (wl.L + 1) // 2 * per_pair
    return wl.B * wl.H * wl.L * (6 * 2 * SYM_FEATURES * wl.dv + (wl.chunk + 1) / 2 * per_pair)


def backward_bytes(wl) -> float:
    """Algorithmic HBM bytes of the gradients: q, k, v (bf16) and dy (fp32)
    read once, dq, dk, dv (fp32) written once."""
    return wl.B * wl.H * wl.L * (2 * (2 * wl.d + wl.dv) + 4 * wl.dv + 4 * (2 * wl.d + wl.dv))


def backward_sets(based, wl, form: str):
    """One gradient call over the workload (bf16 inputs with feature dim 16,
    a seeded dy), as fn(i) for time_leg."""
    q, k, v = (x.cuda() for x in si.linear_inputs(wl))
    dy = torch.randn(wl.B, wl.H, wl.L, wl.dv, generator=torch.Generator().manual_seed(2300)).cuda()
    outs = (torch.empty(wl.B, wl.H, wl.L, wl.d, device="cuda"), torch.empty(wl.B, wl.H, wl.L, wl.d, device="cuda"),
            torch.empty(wl.B, wl.H, wl.L, wl.dv, device="cuda"))
    ws = torch.empty(based.based_prefill_backward_workspace_bytes(wl.B, wl.H, wl.L, wl.dv, wl.d), dtype=torch.uint8,
                     device="cuda")

    def run(i):
        based.based_prefill_backward(q, k, v, dy, eps=wl.eps, form=form, dq=outs[0], dk=outs[1], dv=outs[2],
                                     workspace=ws)
    return run


def bench_backward(based, wl, form: str, n: int):
    """Mean seconds per gradient call and the per-call distribution."""
    return time_leg(backward_sets(based, wl, form), n, settle_s=0.1, dist_n=10)


def swa_backward_bytes(wl) -> int:
    """Algorithmic HBM bytes of the window's gradients: q, k, v (bf16) and dy
    (fp32) read once, dq, dk, dv (fp32) written once."""
    return wl.B * wl.H * wl.L * (2 * (2 * wl.d_qk + wl.dv) + 4 * wl.dv + 4 * (2 * wl.d_qk + wl.dv))


def swa_backward_flops(wl) -> int:
    """Algorithmic flops of the window's gradients: per (query, key) pair
    inside the window, the score, dy . v, and the dq, dk, dv updates
    (2 flop per multiply-add each: 6 d_qk + 4 d_v)."""
    pairs = sum(min(wl.window, i + 1) for i in range(wl.L))
    return wl.B * wl.H * pairs * (6 * wl.d_qk + 4 * wl.dv)


def swa_backward_sets(based, wl):
    """One window-gradient call over the workload (bf16 q, k, v, a seeded
    fp32 dy), as fn(i) for time_leg."""
    _, _, v = si.linear_inputs(wl)
    q, k = si.window_inputs(wl)
    q, k, v = q.cuda(), k.cuda(), v.cuda()
    dy = torch.randn(wl.B, wl.H, wl.L, wl.dv, generator=torch.Generator().manual_seed(2301)).cuda()
    outs = (torch.empty(wl.B, wl.H, wl.L, wl.d_qk, device="cuda"), torch.empty(wl.B, wl.H, wl.L, wl.d_qk, device="cuda"),
            torch.empty(wl.B, wl.H, wl.L, wl.dv, device="cuda"))
    ws = torch.empty(based.swa_backward_workspace_bytes(wl.B, wl.H, wl.L), dtype=torch.uint8, device="cuda")

    def fn(i):
        based.swa_backward(q, k, v, dy, window=wl.window, scale=wl.swa_scale, dq=outs[0], dk=outs[1], dv=outs[2],
                           workspace=ws)

    return fn


def bench_swa_backward(based, wl, n: int):
    """Mean seconds per window-gradient call and the per-call distribution."""
    return time_leg(swa_backward_sets(based, wl), n, settle_s=0.1, dist_n=10)


def _oracle():
    import oracle

    oracle.build()
    return oracle


def cpu_baseline(wl, budget_s=8.0):
    """Oracle recurrent form on whole heads of the workload, sized to about
    budget_s of host time (at most the full workload), OpenMP over heads on
    every host core; plus one head alone (one core)."""
    oracle = _oracle()
    q, k, v = (t.reshape(-1, wl.L, t.shape[-1]) for t in si.linear_inputs(wl))
    threads = oracle.num_threads()
    t0 = time.perf_counter()
    oracle.la_recurrent(q[:1], k[:1], v[:1], eps=wl.eps)  # one head: one thread
    one = time.perf_counter() - t0
    rounds = max(1, int(budget_s / max(one, 1e-9)))
    n_heads = min(q.shape[0], threads * rounds)
    t0 = time.perf_counter()
    oracle.la_recurrent(q[:n_heads], k[:n_heads], v[:n_heads], eps=wl.eps)
    dt = time.perf_counter() - t0
    tokens = n_heads * wl.L / wl.H  # a token covers all H heads
    return {"value": tokens / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{n_heads} of {q.shape[0]} heads x {wl.L} tokens of {wl.name} "
                      f"(fp64 recurrent form, OpenMP over heads), {dt:.1f} s; tokens = head-tokens / H",
            "single_core_tokens_per_s": wl.L / wl.H / one, **cpu_info()}


def cpu_baseline_for(cfg: str, wl) -> dict:
    """The oracle timed on the headline configuration's own work: the
    prefill configurations through cpu_baseline; the 1.3B next-token steps,
    the 8K hybrid layer and the tiny layer on a bounded sample of them."""
    if cfg in ("cfg2", "cfg5"):
        return cpu_baseline(wl)
    oracle = _oracle()
    th = oracle.num_threads()
    if cfg == "cfg3":
        # one sequence (all H heads) from the oracle's state of its 1024-token prefix, 64 steps
        q, k, v = (t[0] for t in si.linear_inputs(wl, B=1))
        _, S, z = oracle.la_recurrent(q, k, v, eps=wl.eps, want_y=False)
        steps = [tuple(t[0] for t in si.decode_inputs(wl, i, B=1)) for i in range(wl.decode_steps)]

        def dec(n):
            Sx, zx = S[:n], z[:n]
            for qt, kt, vt in steps:
                _, Sx, zx = oracle.decode_step(qt[:n], kt[:n], vt[:n], Sx, zx, eps=wl.eps)
        dt, one = cpu_heads(dec, wl.H, th)
        return {"value": len(steps) / dt, "unit": "tokens/s", "cores": th, "kind": "oracle",
                "sample": f"1 of {wl.B} sequences ({wl.H} heads), {len(steps)} decode_step calls from the state of "
                          f"its {wl.L}-token prefix, {dt:.2f} s",
                "single_core_tokens_per_s": len(steps) / wl.H / one, **cpu_info()}
    if cfg == "cfg4":
        q, k, v = (t[0] for t in si.linear_inputs(wl, B=1))
        qw, kw = (t[0] for t in si.window_inputs(wl, B=1))

        def layer(n):
            oracle.la_recurrent(q[:n], k[:n], v[:n], eps=wl.eps)
            oracle.swa(qw[:n], kw[:n], v[:n], wl.window, wl.swa_scale)
        dt, one = cpu_heads(layer, wl.H, th)
        return {"value": wl.L / dt, "unit": "tokens/s", "cores": th, "kind": "oracle",
                "sample": f"1 of {wl.B} sequences ({wl.H} heads x {wl.L} tokens): la_recurrent then swa, {dt:.2f} s",
                "single_core_tokens_per_s": wl.L / wl.H / one, **cpu_info()}
    q, k, v = si.linear_inputs(wl)
    t0 = time.perf_counter()
    oracle.la_quadratic(q, k, v, eps=wl.eps)
    oracle.swa(q, k, v, wl.window, wl.swa_scale)
    dt = time.perf_counter() - t0
    return {"value": wl.L / dt, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"the whole layer (la_quadratic + swa; one head, one thread), {dt*1e3:.1f} ms", **cpu_info()}


def cpu_heads(fn, n_heads, threads):
    """Seconds of fn over a sample (called once; OpenMP over its heads) and of
    fn over one head (one core)."""
    t0 = time.perf_counter()
    fn(1)
    one = time.perf_counter() - t0
    t0 = time.perf_counter()
    fn(n_heads)
    return time.perf_counter() - t0, one


def cpu_legs() -> dict:
    """The oracle on a sample of every other configuration (a batch of one:
    the config's H heads; values drawn for that shape), timed on the host
    cores: tokens/s on all cores and on one."""
    oracle = _oracle()
    th = oracle.num_threads()
    out = {"threads": th, **cpu_info()}
    # 1.3B decode: the 1024-token prefill and 1024 next-token steps of every head of one sequence
    wl = si.WORKLOADS["decode_1p3b"]
    q, k, v = (t[0] for t in si.linear_inputs(wl, B=1))
    steps = [tuple(t[0] for t in si.decode_inputs(wl, t, B=1)) for t in range(wl.decode_steps)]
    dt, one = cpu_heads(lambda n: oracle.la_recurrent(q[:n], k[:n], v[:n], eps=wl.eps), wl.H, th)
    _, S, z = oracle.la_recurrent(q, k, v, eps=wl.eps, want_y=False)

    def dec(n):
        Sx, zx = S[:n], z[:n]
        for qt, kt, vt in steps:
            _, Sx, zx = oracle.decode_step(qt[:n], kt[:n], vt[:n], Sx, zx, eps=wl.eps)

    ddt, done = cpu_heads(dec, wl.H, th)
    out["decode_1p3b"] = {
        "prefill_tokens_per_s": wl.L / dt, "prefill_single_core_tokens_per_s": wl.L / wl.H / one,
        "decode_tokens_per_s": wl.decode_steps / ddt, "decode_single_core_tokens_per_s": wl.decode_steps / wl.H / done,
        "sample": f"1 of {wl.B} sequences ({wl.H} heads): la_recurrent over {wl.L} tokens ({dt:.2f} s), then "
                  f"{wl.decode_steps} decode_step calls ({ddt:.2f} s); tokens = head-tokens / H"}
    # 8K window layer: both branches over every head of one sequence
    wl = si.WORKLOADS["window_8k"]
    q, k, v = (t[0] for t in si.linear_inputs(wl, B=1))
    qw, kw = (t[0] for t in si.window_inputs(wl, B=1))
    dt, one = cpu_heads(lambda n: oracle.la_recurrent(q[:n], k[:n], v[:n], eps=wl.eps, want_y=True), wl.H, th)
    sdt, sone = cpu_heads(lambda n: oracle.swa(qw[:n], kw[:n], v[:n], wl.window, wl.swa_scale), wl.H, th)
    out["window_8k"] = {"linear_tokens_per_s": wl.L / dt, "linear_single_core_tokens_per_s": wl.L / wl.H / one,
                        "window_tokens_per_s": wl.L / sdt, "window_single_core_tokens_per_s": wl.L / wl.H / sone,
                        "sample": f"1 of {wl.B} sequences ({wl.H} heads x {wl.L} tokens): la_recurrent {dt:.2f} s, "
                                  f"swa (brute force) {sdt:.2f} s"}
    # 64K sequence: every head
    wl = si.WORKLOADS["long_64k"]
    q, k, v = (t[0] for t in si.linear_inputs(wl))
    dt, one = cpu_heads(lambda n: oracle.la_recurrent(q[:n], k[:n], v[:n], eps=wl.eps), wl.H, th)
    out["long_64k"] = {"tokens_per_s": wl.L / dt, "single_core_tokens_per_s": wl.L / wl.H / one,
                       "sample": f"the whole workload ({wl.H} heads x {wl.L} tokens), la_recurrent {dt:.2f} s"}
    # tiny fp32 layer: the closed (quadratic) form and the window
    wl = si.WORKLOADS["tiny_f32"]
    q, k, v = si.linear_inputs(wl)
    t0 = time.perf_counter()
    oracle.la_quadratic(q, k, v, eps=wl.eps)
    oracle.swa(q, k, v, wl.window, wl.swa_scale)
    dt = time.perf_counter() - t0
    out["tiny_f32"] = {"tokens_per_s": wl.L / dt, "sample": f"the whole layer (la_quadratic + swa), {dt*1e3:.1f} ms"}
    return out


# gradient legs with a counter summary: leg name -> (workload, form)
BACKWARD_PROFILE_LEGS = {"backward_360m": ("prefill_360m", "chunked"), "backward_360m_direct": ("prefill_360m", "direct"),
                         "backward_64k": ("long_64k", "chunked"), "backward_1p3b": ("decode_1p3b", "chunked"),
                         "backward_1p3b_direct": ("decode_1p3b", "direct")}
BACKWARD_SOURCES = ("prefill_backward_mfma.hip", "common.hpp")


def backward_summary(wname: str, form: str) -> str:
    """Name of the counter summary of one gradient leg."""
    leg = next(k for k, v in BACKWARD_PROFILE_LEGS.items() if v == (wname, form))
    return f"prefill_backward_mfma_{leg}_pmc.txt"


def profile_leg(name: str, launches: int = 8) -> None:
    """Launches of one leg's library call, untimed, for counter passes: each
    dispatch of the call's kernels is one launch of that call."""
    import linear_attention_sequence_taylor_amd as based

    if name in ("prefill_360m", "long_64k", "setup_1p3b", "linear_8k"):
        wl = si.WORKLOADS[{"setup_1p3b": "decode_1p3b", "linear_8k": "window_8k"}.get(name, name)]
        step = prefill_sets(based, wl)
    elif name == "hybrid_8k":
        wl = si.WORKLOADS["window_8k"]
        q, k, v = si.linear_inputs(wl)
        qw, kw = si.window_inputs(wl)
        sets = make_sets((q, k, qw, kw, v), 2)
        ws = torch.empty(max(based.based_hybrid_prefill_workspace_bytes(wl.B, wl.H, wl.L, wl.dv), 1),
                         dtype=torch.uint8, device="cuda")

        def step(i):
            based.based_hybrid_prefill(*sets[i % 2], chunk=wl.chunk, eps=wl.eps, window=wl.window, scale=wl.swa_scale,
                                       workspace=ws)
    elif name == "decode_1p3b":
        wl = si.WORKLOADS["decode_1p3b"]
        S = torch.zeros(wl.B, wl.H, F, wl.dv, device="cuda")
        z = torch.zeros(wl.B, wl.H, F, device="cuda")
        steps = [tuple(t.cuda() for t in si.decode_inputs(wl, t)) for t in range(4)]

        def step(i):
            based.based_decode_step(*steps[i % 4], S, z, eps=wl.eps)
    elif name in BACKWARD_PROFILE_LEGS:
        wname, form = BACKWARD_PROFILE_LEGS[name]
        step = backward_sets(based, si.WORKLOADS[wname], form)
    elif name == "window_backward_8k":
        step = swa_backward_sets(based, si.WORKLOADS["window_8k"])
    elif name == "window_8k":
        wl = si.WORKLOADS["window_8k"]
        qw, kw = si.window_inputs(wl)
        v = si.linear_inputs(wl)[2]
        sets = make_sets((qw, kw, v), 2)
        adds = [torch.randn(wl.B, wl.H, wl.L, wl.dv, device="cuda") for _ in range(2)]

        def step(i):
            based.swa_forward(*sets[i % 2], window=wl.window, scale=wl.swa_scale, add=adds[i % 2])
    else:
        wl = si.WORKLOADS["window_decode_1p3b"]
        _, k = si.window_inputs(wl)
        v = si.linear_inputs(wl)[2]
        caches = [based.swa_cache_fill(k.cuda(), v.cuda(), window=wl.window) for _ in range(8)]
        steps = [tuple(t.cuda() for t in si.window_decode_inputs(wl, t)) for t in range(8)]
        pos = torch.full((wl.B,), wl.L, dtype=torch.int64, device="cuda")
        add = torch.randn(wl.B, wl.H, wl.dv, device="cuda")

        def step(i):
            based.swa_decode_step(*steps[i % 8], *caches[i % 8], pos, scale=wl.swa_scale, add=add)
    for i in range(launches):
        step(i)
    torch.cuda.synchronize()
    print(json.dumps({"profile_leg": name, "launches": launches}), flush=True)


CONFIGS = {"cfg1": "tiny_f32", "cfg2": "prefill_360m", "cfg3": "decode_1p3b", "cfg4": "window_8k", "cfg5": "long_64k"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # A settle phase of fixed wall time runs before the warm-up steps, so the
    # timed steps never see the idle clock whatever --warmup is.
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--config", default="cfg2", choices=sorted(CONFIGS),
                    help="headline configuration: cfg2 (360M-shaped prefill layer, the default), cfg5 (64K "
                         "sequence), cfg3 (1.3B next-token steps), cfg4 (8K hybrid layer through "
                         "based_hybrid_prefill) or cfg1 (the tiny fp32 layer); the others are extra legs")
    ap.add_argument("--workload", default=None, choices=sorted(CONFIGS.values()), help="same, by name")
    ap.add_argument("--no-extra", action="store_true", help="skip every leg but the headline")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baselines")
    ap.add_argument("--decode-steps", type=int, default=1024)
    ap.add_argument("--window-decode-steps", type=int, default=4096)
    ap.add_argument("--profile-leg", default=None,
                    choices=["prefill_360m", "long_64k", "hybrid_8k", "decode_1p3b", "window_8k", "window_decode_1p3b",
                             "setup_1p3b", "linear_8k", "window_backward_8k", *BACKWARD_PROFILE_LEGS],
                    help="only launch one leg's kernels a few times (untimed), for rocprofv3 counter passes")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (5 times), to calibrate "
                         "rocprofv3 FETCH_SIZE/WRITE_SIZE against known bytes")
    args = ap.parse_args()
    if args.copy_calibration:
        n = args.copy_calibration * (1 << 20) // 4
        src = torch.ones(n, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n * 4, "copy_bytes_written": n * 4, "launches": 5}))
        return

    if args.profile_leg:
        profile_leg(args.profile_leg)
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(every (batch, head) is independent, so a larger job splits over batch and heads "
              "with no communication between GPUs). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import linear_attention_sequence_taylor_amd as based

    cfg = args.config
    if args.workload:
        cfg = {name: c for c, name in CONFIGS.items()}[args.workload]
    spec = headline_spec(based, cfg)
    wl = spec["wl"]
    print(f"[bench] workload {wl.name}: {wl.description}", file=sys.stderr, flush=True)
    step_s, kern_s, dist = bench_headline(spec["step"], args.steps, args.warmup)
    tokens = spec["tokens"]
    abytes, aflops = spec["bytes"], spec["flops"]
    digest = source_digest(*PREFILL_SOURCES)
    traffic = None
    if spec["traffic"]:
        traffic = read_traffic(spec["traffic"][0], source_digest(*spec["traffic"][1]))
    achieved = abytes / kern_s
    line = {
        "metric": METRIC,
        "value": tokens / step_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": step_s * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"bf16": "bf16", "f32": "f32"}.get(wl.dtype, wl.dtype),
        "data": "synthetic (seeded N(0,1)*scale" + (", bf16-rounded)" if wl.dtype == "bf16" else ")"),
        "config": spec["config"],
        "roofline": {
            "bound": "hbm",
            "achieved": achieved / 1e9,
            "peak": HBM_PEAK / 1e9,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK,
            "traffic": traffic,
            "kernel": spec["kernel"],
            "kernel_ms": kern_s * 1e3,
            "kernel_timing": "HIP events on the launch stream around one replay of the K steps captured in a HIP "
                             "graph, / K; before it a 0.3 s settle phase and W warm-up steps",
            "single_launch_us": dist,
            "algorithmic_bytes": abytes,
        },
    }
    if aflops is not None:
        line["roofline"].update({"algorithmic_flops": aflops, "mfma_tflops": aflops / kern_s / 1e12,
                                 "mfma_frac": aflops / kern_s / MFMA_BF16_PEAK})
    busy = counter_mfma_busy(wl.name, kern_s)
    if busy is not None:
        line["roofline"]["counter_mfma_busy_frac"] = busy
    if spec["traffic"]:
        line["roofline"]["kernel_source_sha256_16"] = source_digest(*spec["traffic"][1])
    print(f"[bench] headline {wl.name}: {kern_s*1e6:.1f} us/step, {achieved/1e9:.0f} GB/s", file=sys.stderr,
          flush=True)

    if not args.no_extra:
        extra = {}
        # cfg3: the 1.3B decode, its d_v = 128 setup prefill and 1024 steps
        wd = si.WORKLOADS["decode_1p3b"]
        ssec, sdist, dstep, dkern, ddist = bench_decode(based, wd, args.decode_steps)
        db = decode_bytes(wd)
        extra["decode_1p3b"] = {
            "tokens_per_s": wd.B / dstep, "ms_per_step": dstep * 1e3, "kernel_us": dkern * 1e6,
            "step_us": ddist, "steps": args.decode_steps,
            "roofline": roofline(db, dkern, read_traffic("decode_step_decode_1p3b_pmc.txt",
                                                         source_digest("decode.hip", "common.hpp"))),
            "setup_prefill": {"kernel_us": ssec * 1e6, "launch_us": sdist, "tokens_per_s": wd.B * wd.L / ssec,
                              "roofline": roofline(prefill_bytes(wd), ssec, read_traffic(
                                  "prefill_mfma_decode_1p3b_setup_pmc.txt", digest), prefill_flops(wd)),
                              "note": "B=128, H=16, L=1024, d_v=128 prefill that builds the decode state"},
            "note": "1024-token prefill then next-token steps; fp32 state; events around the step loop"}
        print(f"[bench] decode: setup prefill {ssec*1e6:.1f} us, {dkern*1e6:.1f} us/step", file=sys.stderr,
              flush=True)
        # cfg4: the 8K layer -- linear branch, window branch (fused add), whole layer
        ww = si.WORKLOADS["window_8k"]
        lsec, ldist = bench_prefill_leg(based, ww, 40)
        skern, sdist2 = bench_swa(based, ww, 100)
        sb = swa_bytes(ww)
        ht = bench_hybrid(based, ww, 100)
        hb = hybrid_bytes(ww)
        extra["window_8k"] = {
            "linear_branch": {"kernel_us": lsec * 1e6, "launch_us": ldist, "tokens_per_s": ww.B * ww.L / lsec,
                              "roofline": roofline(prefill_bytes(ww), lsec, read_traffic(
                                  "prefill_mfma_window_8k_linear_pmc.txt", digest), prefill_flops(ww))},
            "window_branch": {"kernel_us": skern * 1e6, "launch_us": sdist2, "tokens_per_s": ww.B * ww.L / skern,
                              "roofline": roofline(sb, skern, read_traffic("swa_mfma_window_8k_pmc.txt",
                                                                           source_digest("swa_mfma.hip",
                                                                                         "common.hpp")))},
            "hybrid_layer": {"kernel_us": ht["auto"] * 1e6, "launch_us": ht["auto_dist"],
                             "tokens_per_s": ww.B * ww.L / ht["auto"],
                             "roofline": roofline(hb, ht["auto"], read_traffic(
                                 "prefill_mfma_hybrid_window_8k_pmc.txt",
                                 source_digest(*PREFILL_SOURCES))),
                             "fused_us": ht["fused"] * 1e6, "two_pass_us": ht["two_pass"] * 1e6,
                             "note": "linear attention + w=64 window through based_hybrid_prefill; kernel_us is the "
                                     "library's own choice (auto), fused_us the one-kernel path, two_pass_us "
                                     "based_prefill then the window adding into y; algorithmic bytes are those of "
                                     "one pass"}}
        print(f"[bench] 8K layer: linear {lsec*1e6:.1f} us, window {skern*1e6:.1f} us, hybrid auto "
              f"{ht['auto']*1e6:.1f} / fused {ht['fused']*1e6:.1f} / two passes {ht['two_pass']*1e6:.1f} us",
              file=sys.stderr, flush=True)
        # cfg5: the 64K sequence (or cfg2 when the headline is cfg5)
        for oname in ("prefill_360m", "long_64k"):
            if oname == wl.name:
                continue
            other = si.WORKLOADS[oname]
            osec, odist = bench_prefill_leg(based, other, 40 if other.name == "long_64k" else 200)
            extra[other.name] = {"kernel_us": osec * 1e6, "launch_us": odist,
                                 "tokens_per_s": other.B * other.L / osec,
                                 "roofline": roofline(prefill_bytes(other), osec, read_traffic(
                                     f"prefill_mfma_{other.name}_pmc.txt", digest), prefill_flops(other))}
            print(f"[bench] {other.name}: {osec*1e6:.1f} us", file=sys.stderr, flush=True)
        # cfg1: the tiny fp32 layer (linear attention + window, summed)
        wt = si.WORKLOADS["tiny_f32"]
        tq, tk, tv = (t.cuda() for t in si.linear_inputs(wt))
        ty = torch.empty(1, 1, wt.L, wt.dv, device="cuda")
        tS, tz = torch.empty(1, 1, F, wt.dv, device="cuda"), torch.empty(1, 1, F, device="cuda")

        def tiny(i):
            based.based_prefill(tq, tk, tv, chunk=wt.chunk, eps=wt.eps, y=ty, S=tS, z=tz)
            based.swa_forward(tq, tk, tv, window=wt.window, scale=wt.swa_scale, add=ty, y=ty)

        tsec, tdist = time_leg(tiny, 200, settle_s=0.05, dist_n=30)
        extra["tiny_f32"] = {"layer_us": tsec * 1e6, "launch_us": tdist, "tokens_per_s": wt.L / tsec,
                             "note": "fp32 inputs: prefill (fp32 matrix cores) then the window adding into y; "
                                     "launch-latency bound (256 tokens)"}
        # window next-token step, gradients, other sizes
        wwd = si.WORKLOADS["window_decode_1p3b"]
        wkern = bench_window_decode(based, wwd, args.window_decode_steps)
        wb = window_decode_bytes(wwd)
        extra["window_decode_1p3b"] = {
            "tokens_per_s": wwd.B / wkern, "kernel_us": wkern * 1e6, "steps": args.window_decode_steps,
            "roofline": roofline(wb, wkern, read_traffic("swa_decode_window_decode_1p3b_pmc.txt",
                                                         source_digest("swa_decode.hip", "common.hpp"))),
            "note": "w=64 ring, B=128, H=16, d_qk=64, d_v=128, fused add; HIP graph of 64 steps "
                    "replayed, 16 cache sets"}
        print(f"[bench] window decode: {wkern*1e6:.1f} us/step", file=sys.stderr, flush=True)
        wd3 = si.WORKLOADS["decode_1p3b"]
        lsec = bench_layer_decode(based, wd3, wwd, 256)
        lb = decode_bytes(wd3) + window_decode_bytes(wwd)
        # the layer step's launches are the two legs' launches, so its counter
        # traffic is the sum of their summaries' (None if either is stale)
        lparts = (read_traffic("decode_step_decode_1p3b_pmc.txt", source_digest("decode.hip", "common.hpp")),
                  read_traffic("swa_decode_window_decode_1p3b_pmc.txt", source_digest("swa_decode.hip", "common.hpp")))
        ltraffic = None if None in lparts else sum(lparts)
        extra["layer_decode_1p3b"] = {
            "tokens_per_s": wd3.B / lsec, "layer_step_us": lsec * 1e6, "steps": 256,
            "roofline": roofline(lb, lsec, ltraffic),
            "note": "one BASED-1.3B layer's next-token step: the linear-attention step (fp32 state 273x128 per "
                    "head, read and written once) then the w=64 window step on the same token adding into its "
                    "output; B=128, H=16; HIP graph of 64 layer steps replayed 4 times; bytes are the two "
                    "launches' algorithmic bytes"}
        print(f"[bench] layer decode: {lsec*1e6:.1f} us/step", file=sys.stderr, flush=True)
        for bname, forms in (("prefill_360m", ("chunked", "direct")), ("long_64k", ("chunked",)),
                             ("decode_1p3b", ("chunked", "direct"))):
            bw = si.WORKLOADS[bname]
            leg = {}
            for form in forms:
                bsec, bdist = bench_backward(based, bw, form, 100 if bname == "prefill_360m" else 30)
                traffic = read_traffic(backward_summary(bname, form), source_digest(*BACKWARD_SOURCES))
                leg[form] = {"kernel_us": bsec * 1e6, "tokens_per_s": bw.B * bw.L / bsec, "dist_us": bdist,
                             "roofline": roofline(backward_bytes(bw), bsec, traffic, backward_flops(bw, form))}
                print(f"[bench] backward {bname} {form}: {bsec*1e6:.1f} us", file=sys.stderr, flush=True)
            leg["auto_form"] = "chunked"
            leg["note"] = ("dq, dk, dv for a seeded dy, bf16 inputs, fp32 accumulation on the bf16 matrix cores "
                           "(non-input operands as bf16 hi/lo pairs).  chunked: linear in L through the carried "
                           "state (segment sums, scans, query sweep, key sweep); direct: pair by pair, O(L^2) "
                           "per head.  Flops are each form's own algorithmic count (backward_flops).")
            if bname == "decode_1p3b":
                leg["note"] += ("  The 1.3B-shaped layer (B=128, H=16, L=1024, d_v=128) of the decode workload's "
                                "prefill; the chunked form runs once per 64-column half of v.")
                extra["layer_1p3b_backward"] = leg
            else:
                extra[f"{bname}_backward"] = leg
        ww8 = si.WORKLOADS["window_8k"]
        wsec, wdist = bench_swa_backward(based, ww8, 100)
        extra["window_8k_backward"] = {
            "kernel_us": wsec * 1e6, "tokens_per_s": ww8.B * ww8.L / wsec, "dist_us": wdist,
            "roofline": roofline(swa_backward_bytes(ww8), wsec,
                                 read_traffic("swa_backward_window_8k_pmc.txt", source_digest("swa_backward.hip", "common.hpp")),
                                 swa_backward_flops(ww8)),
            "note": "dq, dk, dv of the w=64 window of the 8K layer (B=4, H=16, L=8192, d_qk=d_v=64) for a seeded "
                    "dy: query side then key side on the bf16 matrix cores, P, dS and dy as bf16 hi/lo pairs; "
                    "flops are the window-exact pairs' (swa_backward_flops)"}
        print(f"[bench] window backward window_8k: {wsec*1e6:.1f} us", file=sys.stderr, flush=True)
        oth = bench_other_sizes(based)
        extra.update(oth)
        print("[bench] other sizes: " + ", ".join(f"{k} {v['kernel_us']:.1f} us" for k, v in oth.items()),
              file=sys.stderr, flush=True)
        line["extra"] = extra

    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline_for(cfg, wl)
        if not args.no_extra:
            line["extra"]["cpu_baselines"] = cpu_legs()
            print("[bench] cpu baselines done", file=sys.stderr, flush=True)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
