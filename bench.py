"""Throughput of the Taylor linear attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-extra]

A step is one ``based_prefill`` call over one batch of the workload
(default: the BASED-360M-shaped prefill layer, B=8, H=16, L=2048, d'=16,
d_v=64, bf16, chunk 64), inputs already resident in HBM.  Steps cycle over
four distinct input/output buffer sets so that consecutive steps do not
re-read the previous step's data from the 256 MB Infinity Cache.  Rank 0
prints one JSON line with:

* value: tokens/s (tokens = B*L per step, each token covering all H heads);
* roofline: the prefill kernel's algorithmic bytes per launch / its mean
  launch duration (HIP events on the launch stream around the timed loop,
  over the number of launches), against 8 TB/s HBM (the kernel's
  arithmetic intensity is below the bf16 MFMA ridge), plus its algorithmic
  flop rate against the 2.5 PFLOP/s dense bf16 MFMA peak; `traffic` comes
  from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE summary when that
  summary was taken on the current kernel source;
* cpu_baseline: the fp64 oracle (recurrent form) timed on the host cores on
  a sample of whole heads of the same workload;
* extra: the next-token step (1.3B-shaped decode, 1024 steps), the w=64
  window kernel with fused add, the window's next-token step on its ring
  cache, and the 64K-token prefill, each with its own HBM roofline fraction;
  the whole 8K hybrid layer fused (and as two passes);
  the gradients of the prefill over the same layer (matrix-core fraction);
  and the other feature dims and window sizes.
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
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(CSRC, n), "rb") as f:
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


def make_sets(tensors, n):
    out = [tuple(t.to("cuda") for t in tensors)]
    for _ in range(n - 1):
        out.append(tuple(t.clone() for t in out[0]))
    return out


# ---------------------------------------------------------------- legs
def bench_prefill(based, wl, steps, warmup):
    """Returns (wall seconds per step, mean launch seconds from the events
    around the timed region, per-launch distribution)."""
    q, k, v = si.linear_inputs(wl)
    ins = make_sets((q, k, v), N_SETS)
    outs = []
    for _ in range(N_SETS):
        outs.append((torch.empty(wl.B, wl.H, wl.L, wl.dv, device="cuda"),
                     torch.empty(wl.B, wl.H, F, wl.dv, device="cuda"),
                     torch.empty(wl.B, wl.H, F, device="cuda")))
    nbytes = based.based_prefill_workspace_bytes(wl.B, wl.H, wl.L, wl.dv)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device="cuda")

    def step(i):
        (qq, kk, vv), (y, S, z) = ins[i % N_SETS], outs[i % N_SETS]
        based.based_prefill(qq, kk, vv, chunk=wl.chunk, eps=wl.eps, y=y, S=S, z=z, workspace=ws)

    for i in range(warmup):
        step(i)
    timer = RegionTimer()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    timer.start()
    for i in range(steps):
        step(i)
    timer.stop()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    dist = launch_distribution(step, min(max(steps, 20), 50))
    return wall / steps, timer.seconds() / steps, dist


def bench_decode(based, wl, n_steps):
    """1024-token prefill, then n_steps next-token steps timed as one region.
    Returns (wall seconds per step, event seconds per step)."""
    q, k, v = si.linear_inputs(wl)
    _, S, z = based.based_prefill(*(t.cuda() for t in (q, k, v)), chunk=wl.chunk, eps=wl.eps)
    del q, k, v
    step_in = [tuple(t.cuda() for t in si.decode_inputs(wl, t)) for t in range(n_steps)]
    y = torch.empty(wl.B, wl.H, wl.dv, device="cuda")
    # untimed warm-up (~50 ms, out of the idle clock state) on a copy of the state
    S2, z2 = S.clone(), z.clone()
    for t in range(500):
        based.based_decode_step(*step_in[t % n_steps], S2, z2, eps=wl.eps, y=y)
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
    return wall / n_steps, timer.seconds() / n_steps


def bench_swa(based, wl, reps, window=None):
    """Window kernel with fused add, alternating two input/output sets;
    returns event seconds per launch over the timed region."""
    window = wl.window if window is None else window
    q, k, v = si.linear_inputs(wl)
    qw, kw = si.window_inputs(wl)
    sets = make_sets((qw, kw, v), 2)
    del q, k
    adds = [torch.randn(wl.B, wl.H, wl.L, wl.dv, device="cuda") for _ in range(2)]
    ys = [torch.empty_like(adds[0]) for _ in range(2)]

    def launch(i):
        based.swa_forward(*sets[i % 2], window=window, scale=wl.swa_scale, add=adds[i % 2], y=ys[i % 2])

    for i in range(500):  # untimed warm-up, ~45 ms
        launch(i)
    timer = RegionTimer()
    torch.cuda.synchronize()
    timer.start()
    for i in range(reps):
        launch(i)
    timer.stop()
    return timer.seconds() / reps


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
        for i in range(200):  # untimed warm-up
            layer(i, path)
        timer = RegionTimer()
        torch.cuda.synchronize()
        timer.start()
        for i in range(reps):
            layer(i, path)
        timer.stop()
        res[path] = timer.seconds() / reps
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


def bench_other_sizes(based):
    """The pages' other design points (feature dim 32, window 128), on the
    paths that carry them: seeded inputs, event-timed regions.  Returns a
    dict of legs (report only)."""
    out = {}
    # window 128 over the 8K window workload inputs (matrix cores, two-tile
    # halo), timed exactly as the w = 64 leg
    ww = si.WORKLOADS["window_8k"]
    sec = bench_swa(based, ww, 100, window=128)
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
    for _ in range(100):  # untimed warm-up, ~50 ms
        based.based_prefill(q, k, v)
    t = RegionTimer()
    torch.cuda.synchronize()
    t.start()
    for _ in range(20):
        based.based_prefill(q, k, v)
    t.stop()
    sec = t.seconds() / 20
    pb = B * H * L * (2 * d * 2 + dv * 2 + dv * 4) + B * H * (F32 * dv + F32) * 4
    # per tok-head: 4 F d_v (state update and readout) + the causal intra-chunk term
    pf = B * H * L * (4 * F32 * dv + 65 * (d + dv))
    out["prefill_d32"] = {"kernel_us": sec * 1e6, "tokens_per_s": B * L / sec, "hbm_frac": pb / sec / HBM_PEAK,
                          "algorithmic_bytes": pb, "algorithmic_flops": pf, "tflops": pf / sec / 1e12,
                          "mfma_f32_frac": pf / sec / MFMA_F32_PEAK,
                          "note": "feature dim 32, B=2, H=16, L=2048, fp32 arithmetic on the fp32 matrix cores "
                                  "(128 workgroups: one per head and 16 value columns)"}
    return out


def bench_backward(based, wl, reps=40):
    """Gradients of the prefill output over the workload (bf16 inputs with
    feature dim 16: the matrix-core kernels, direct form).  Returns (event
    seconds per call, algorithmic flops): per causal (i, j) pair
    8d + 6d_v + 12 flops (scores twice, weights, g.v, dq, dk, dv and N)."""
    q, k, v = (x.cuda() for x in si.linear_inputs(wl))
    dy = torch.randn(wl.B, wl.H, wl.L, wl.dv, device="cuda")
    outs = (torch.empty(wl.B, wl.H, wl.L, wl.d, device="cuda"), torch.empty(wl.B, wl.H, wl.L, wl.d, device="cuda"),
            torch.empty(wl.B, wl.H, wl.L, wl.dv, device="cuda"))
    ws = torch.empty(based.based_prefill_backward_workspace_bytes(wl.B, wl.H, wl.L, wl.dv, wl.d), dtype=torch.uint8,
                     device="cuda")
    run = lambda: based.based_prefill_backward(q, k, v, dy, eps=wl.eps, dq=outs[0], dk=outs[1], dv=outs[2],
                                               workspace=ws)
    for _ in range(100):  # untimed warm-up, ~50 ms
        run()
    t = RegionTimer()
    torch.cuda.synchronize()
    t.start()
    for _ in range(reps):
        run()
    t.stop()
    pairs = wl.B * wl.H * wl.L * (wl.L + 1) // 2
    return t.seconds() / reps, pairs * (8 * wl.d + 6 * wl.dv + 12)


def cpu_baseline(wl, budget_s=12.0):
    """Oracle recurrent form on whole heads of the workload, sized to about
    budget_s of host time (at most the full workload)."""
    import oracle

    oracle.build()
    q, k, v = (t.reshape(-1, wl.L, t.shape[-1]) for t in si.linear_inputs(wl))
    threads = oracle.num_threads()
    t0 = time.perf_counter()
    oracle.la_recurrent(q[:2], k[:2], v[:2], eps=wl.eps)  # two heads run on two threads
    per_head = time.perf_counter() - t0
    rounds = max(1, int(budget_s / max(per_head, 1e-9)))
    n_heads = min(q.shape[0], threads * rounds)
    t0 = time.perf_counter()
    oracle.la_recurrent(q[:n_heads], k[:n_heads], v[:n_heads], eps=wl.eps)
    dt = time.perf_counter() - t0
    tokens = n_heads * wl.L / wl.H  # a token covers all H heads
    return {"value": tokens / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{n_heads} of {q.shape[0]} heads x {wl.L} tokens of {wl.name} "
                      f"(fp64 recurrent form, OpenMP over heads), {dt:.1f} s; tokens = head-tokens / H"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # The GPU leaves its idle clock state only after ~20 ms of continuous
    # work (the first 50 prefill launches run ~75% slower), so the default
    # untimed warm-up is 1000 steps (~45 ms) before 400 timed ones.
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=1000)
    ap.add_argument("--workload", default="prefill_360m", choices=["prefill_360m", "long_64k"])
    ap.add_argument("--no-extra", action="store_true", help="skip decode/window/64K legs")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--decode-steps", type=int, default=1024)
    ap.add_argument("--window-decode-steps", type=int, default=4096)
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

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(every (batch, head) is independent, so a larger job splits over batch and heads "
              "with no communication between GPUs). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import linear_attention_sequence_taylor_amd as based

    wl = si.WORKLOADS[args.workload]
    print(f"[bench] workload {wl.name}: {wl.description}", file=sys.stderr, flush=True)
    step_s, kern_s, dist = bench_prefill(based, wl, args.steps, args.warmup)
    tokens = wl.B * wl.L
    abytes, aflops = prefill_bytes(wl), prefill_flops(wl)
    digest = source_digest("prefill_mfma.hip", "common.hpp")
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
        "dtype": wl.dtype,
        "data": "synthetic (seeded N(0,1)*scale, bf16-rounded)",
        "config": {"workload": wl.name, "B": wl.B, "H": wl.H, "L": wl.L, "d_feat": wl.d,
                   "d_v": wl.dv, "chunk": wl.chunk, "scale": wl.scale, "parallelism": "single GPU"},
        "roofline": {
            "bound": "hbm",
            "achieved": achieved / 1e9,
            "peak": HBM_PEAK / 1e9,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK,
            "traffic": read_traffic(f"prefill_mfma_{wl.name}_pmc.txt", digest),
            "kernel": "based_prefill (bf16 MFMA)",
            "kernel_ms": kern_s * 1e3,
            "kernel_timing": "HIP events around the timed region on the launch stream / steps",
            "single_launch_us": dist,
            "algorithmic_bytes": abytes,
            "algorithmic_flops": aflops,
            "mfma_tflops": aflops / kern_s / 1e12,
            "mfma_frac": aflops / kern_s / MFMA_BF16_PEAK,
            "kernel_source_sha256_16": digest,
        },
    }
    print(f"[bench] prefill {wl.name}: {kern_s*1e6:.1f} us/launch, {achieved/1e9:.0f} GB/s", file=sys.stderr,
          flush=True)

    if not args.no_extra:
        extra = {}
        wd = si.WORKLOADS["decode_1p3b"]
        dstep, dkern = bench_decode(based, wd, args.decode_steps)
        db = decode_bytes(wd)
        extra["decode_1p3b"] = {
            "tokens_per_s": wd.B / dstep, "ms_per_step": dstep * 1e3, "kernel_us": dkern * 1e6,
            "hbm_GBps": db / dkern / 1e9, "hbm_frac": db / dkern / HBM_PEAK, "algorithmic_bytes": db,
            "steps": args.decode_steps, "note": "1024-token prefill then next-token steps; fp32 state"}
        print(f"[bench] decode: {dkern*1e6:.1f} us/step, {db/dkern/1e9:.0f} GB/s", file=sys.stderr, flush=True)
        ww = si.WORKLOADS["window_8k"]
        skern = bench_swa(based, ww, 100)
        sb = swa_bytes(ww)
        extra["window_8k_swa"] = {"tokens_per_s": ww.B * ww.L / skern, "kernel_us": skern * 1e6,
                                  "hbm_GBps": sb / skern / 1e9, "hbm_frac": sb / skern / HBM_PEAK,
                                  "algorithmic_bytes": sb}
        print(f"[bench] swa: {skern*1e6:.1f} us, {sb/skern/1e9:.0f} GB/s", file=sys.stderr, flush=True)
        ht = bench_hybrid(based, ww, 100)
        hb = hybrid_bytes(ww)
        extra["window_8k_hybrid_layer"] = {
            "tokens_per_s": ww.B * ww.L / ht["auto"], "kernel_us": ht["auto"] * 1e6,
            "hbm_GBps": hb / ht["auto"] / 1e9, "hbm_frac": hb / ht["auto"] / HBM_PEAK, "algorithmic_bytes": hb,
            "fused_us": ht["fused"] * 1e6, "two_pass_us": ht["two_pass"] * 1e6,
            "note": "linear attention + w=64 window over B=4, H=16, L=8192 through based_hybrid_prefill; kernel_us "
                    "is the library's own choice (auto), fused_us the one-kernel path (32-column groups with a "
                    "segment split), two_pass_us based_prefill then the window adding into y; algorithmic bytes "
                    "are those of one pass"}
        print(f"[bench] hybrid layer: auto {ht['auto']*1e6:.1f} us, fused {ht['fused']*1e6:.1f} us, two passes "
              f"{ht['two_pass']*1e6:.1f} us", file=sys.stderr, flush=True)
        wwd = si.WORKLOADS["window_decode_1p3b"]
        wkern = bench_window_decode(based, wwd, args.window_decode_steps)
        wb = window_decode_bytes(wwd)
        extra["window_decode_1p3b"] = {
            "tokens_per_s": wwd.B / wkern, "kernel_us": wkern * 1e6, "hbm_GBps": wb / wkern / 1e9,
            "hbm_frac": wb / wkern / HBM_PEAK, "algorithmic_bytes": wb, "steps": args.window_decode_steps,
            "note": "w=64 ring, B=128, H=16, d_qk=64, d_v=128, fused add; HIP graph of 64 steps "
                    "replayed, 16 cache sets"}
        print(f"[bench] window decode: {wkern*1e6:.1f} us/step, {wb/wkern/1e9:.0f} GB/s", file=sys.stderr,
              flush=True)
        if wl.name != "long_64k":
            wlong = si.WORKLOADS["long_64k"]
            lstep, lkern, _ = bench_prefill(based, wlong, 50, 100)
            lb = prefill_bytes(wlong)
            extra["long_64k_prefill"] = {"tokens_per_s": wlong.B * wlong.L / lstep, "kernel_ms": lkern * 1e3,
                                         "hbm_GBps": lb / lkern / 1e9, "hbm_frac": lb / lkern / HBM_PEAK,
                                         "mfma_frac": prefill_flops(wlong) / lkern / MFMA_BF16_PEAK}
            print(f"[bench] long prefill: {lkern*1e3:.3f} ms", file=sys.stderr, flush=True)
        bsec, bflops = bench_backward(based, wl)
        extra["prefill_360m_backward"] = {
            "kernel_ms": bsec * 1e3, "tokens_per_s": wl.B * wl.L / bsec, "direct_form_flops": bflops,
            "tflops": bflops / bsec / 1e12, "mfma_frac": bflops / bsec / MFMA_BF16_PEAK,
            "note": "dq, dk, dv for a seeded dy; bf16 matrix cores (weights as bf16 hi/lo pairs, fp32 "
                    "accumulation), direct form (O(L^2) per head)"}
        print(f"[bench] backward: {bsec*1e3:.2f} ms, {bflops/bsec/1e12:.1f} TFLOP/s", file=sys.stderr, flush=True)
        other = bench_other_sizes(based)
        extra.update(other)
        print("[bench] other sizes: " + ", ".join(f"{k} {v['kernel_us']:.1f} us" for k, v in other.items()),
              file=sys.stderr, flush=True)
        line["extra"] = extra

    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(wl)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
