"""Benchmark of the expert-ID matmul path on one MI355X.

One step = one pass of the whole path over one batch of seeded synthetic
input: router (sigmoid + selection bias, top-k) -> expert-ID matmul ->
gate-weighted combine, all in the library's HIP kernels.

Headline (`value`): decode, m=1, k=4096, n=1536, top-8 of 256 bf16 experts,
as effective GB/s of touched expert weights (8 x 1536 x 4096 x 2 B per step)
over the whole step.  Decode is timed cold: step i routes with the experts
relabelled so that its picks are experts 8(i mod 32)..8(i mod 32)+7, so 32
consecutive steps sweep all 3.2 GB of weights and none is served from the
256 MB Infinity Cache.  The prefill configurations (m=2048 down projection
with per-slot input; m=512 balanced and maximally skewed) are reported next
to it in TFLOP/s.

A decode step is one launch of the fused kernel (route, Direct matmul and
combine).  Exactly --steps steps are captured into one HIP graph and replayed
once between two HIP events on the replaying stream, right behind a replay
of the warm-up graph (so the GPU is busy and at its working clocks when the
start event is taken), so the per-step time is that kernel's average launch
duration plus the graph's gaps and its one-time start and end.  The GPU clocks take a few hundred
milliseconds of load to ramp up, so every measurement is preceded by at
least --warmup steps and at least half a second of the same work; the line
reports both what was asked and what ran.  Prefill matmul calls (id map +
Grouped kernel) are timed the same way, after their own warm-up: a graph of
back-to-back calls between HIP events.
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import subprocess
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from expert_id_matmul_amd import binding as B  # noqa: E402
from expert_id_matmul_amd import workloads as W  # noqa: E402

HBM_PEAK = 8.0e12            # B/s, MI355X HBM3E
F32_PEAK = 157.3e12          # flop/s, MI355X dense f32 matrix
MX16_PEAK = 2.5e15           # flop/s, MI355X dense bf16 / f16 matrix
ROT = 32                     # decode steps per full sweep of the experts
PREFILL_STEPS = 16           # matmul calls per timed prefill graph


def _dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _percentiles(v):
    v = sorted(v)
    n = len(v)
    return {"p25": v[(n - 1) // 4], "median": v[n // 2], "p75": v[3 * (n - 1) // 4]}


def _relabel(n_experts: int, picks: np.ndarray, target: np.ndarray) -> np.ndarray:
    """A permutation p of experts with p[picks[j]] = target[j]; every other
    expert keeps its order among the remaining labels."""
    p = np.full(n_experts, -1, dtype=np.int64)
    p[picks] = target
    rest_src = [e for e in range(n_experts) if p[e] < 0]
    used = set(int(t) for t in target)
    rest_dst = [e for e in range(n_experts) if e not in used]
    p[rest_src] = rest_dst
    return p


WARMUP_FLOOR_S = 0.5  # seconds of the same work before any timed region
SPIN_CYCLES = 200_000  # ~80 us of GPU spin: the host enqueues the timed work meanwhile


def _capture(step_fn, n: int, start: int = 0) -> torch.cuda.CUDAGraph:
    """A HIP graph of step_fn(start) .. step_fn(start + n - 1), captured on a
    side stream after one eager pass of the same steps."""
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for i in range(start, start + n):
            step_fn(i)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        for i in range(start, start + n):
            step_fn(i)
    torch.cuda.synchronize()
    return g


class Timed:
    """Warm up on a graph of `warm_n` steps for at least `warmup` steps and
    WARMUP_FLOOR_S seconds, replay the timed graph once untimed, then time
    one replay of that graph of exactly `steps` steps, queued right behind
    one more replay of the warm-up graph (all untimed steps are counted in
    warmup_steps_run)."""

    def __init__(self, step_fn, warm_n: int):
        self.step_fn = step_fn
        self.warm = _capture(step_fn, warm_n)
        self.warm_n = warm_n

    def warm_up(self, warmup: int, floor_s: float = WARMUP_FLOOR_S):
        done, t0 = 0, time.perf_counter()
        while done < warmup or time.perf_counter() - t0 < floor_s:
            self.warm.replay()
            done += self.warm_n
            if done % (self.warm_n * 16) == 0:
                torch.cuda.synchronize()
        torch.cuda.synchronize()
        return done, time.perf_counter() - t0

    def run(self, steps: int, warmup: int, repeats: int = 1):
        timed = _capture(self.step_fn, steps)
        wsteps, wsecs = self.warm_up(warmup)
        # one untimed replay of the timed graph itself: a graph's first launch
        # also uploads it to the device, which is not part of a step
        timed.replay()
        torch.cuda.synchronize()
        wsteps += steps
        times = []
        for _ in range(repeats):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            # the warm-up graph runs right ahead of the start event: the GPU
            # stays busy (and at its working clocks) while the host submits
            # the timed graph, so the interval holds the steps only
            self.warm.replay()
            wsteps += self.warm_n
            start.record()
            timed.replay()
            end.record()
            torch.cuda.synchronize()
            times.append((start.elapsed_time(end), time.perf_counter() - t0))
        gpu_ms, wall_s = times[0]
        return {"steps": steps, "gpu_ms_per_step": gpu_ms / steps, "wall_ms_per_step": wall_s * 1e3 / steps,
                "warmup_steps_run": wsteps, "warmup_s": round(wsecs, 3),
                "repeats_gpu_ms_per_step": [t[0] / steps for t in times]}




def kernel_times(call, steps: int, before=None, after=None):
    """HIP events around `call(i)` for i < steps, on the stream the kernels run
    on.  A short GPU spin is queued ahead of each start event so the GPU is
    still busy while the host enqueues event, launch and event: the interval
    then holds the kernel alone, not the host's launch latency."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    for i in range(steps):
        if before is not None:
            before(i)
        torch.cuda._sleep(SPIN_CYCLES)
        evs[i][0].record()
        call(i)
        evs[i][1].record()
        if after is not None:
            after(i)
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in evs]


# ---------------------------------------------------------------------- decode
def decode_bytes(wl) -> dict:
    """Algorithmic HBM bytes of one decode step: the touched experts' weights
    (top_k distinct experts, n*k each) plus every other input and output once."""
    touched = wl.top_k * wl.n * wl.k * W.DTYPE_SIZE[wl.dtype]
    other = (wl.m * wl.k * 4                  # x
             + wl.m * wl.n_experts * 4 + wl.n_experts * 4   # logits, bias
             + wl.routed_rows * wl.n * 4      # y
             + wl.m * wl.n * 4                # out
             + wl.routed_rows * 8)            # ids, gates
    return {"touched_weights": touched, "algorithmic": touched + other}


def bench_decode(lib, steps: int, warmup: int):
    wl = W.WORKLOADS["decode"]
    shape = B.shape_of(wl)
    weights = torch.empty(wl.weight_bytes, dtype=torch.uint8, device="cuda")
    W.fill_weights(wl, weights)
    x = _dev(W.activations(wl))
    logits0 = W.router_logits(wl)[0]
    bias0 = W.router_bias(wl)
    # the picks of the unrelabelled router, from the library's own router
    ids0 = torch.empty((1, wl.top_k), dtype=torch.int32, device="cuda")
    lib.route_topk(_dev(logits0[None]), _dev(bias0), wl.top_k, ids0, None)
    picks = ids0.cpu().numpy().view(np.uint32)[0].astype(np.int64)
    logits = np.empty((ROT, wl.n_experts), np.float32)
    bias = np.empty((ROT, wl.n_experts), np.float32)
    for i in range(ROT):
        p = _relabel(wl.n_experts, picks, np.arange(wl.top_k) + wl.top_k * i)
        logits[i, p] = logits0
        bias[i, p] = bias0
    logits_d, bias_d = _dev(logits), _dev(bias)
    ids = torch.empty((wl.m, wl.top_k), dtype=torch.int32, device="cuda")
    gates = torch.empty((wl.m, wl.top_k), dtype=torch.float32, device="cuda")
    y = torch.empty((wl.routed_rows, wl.n), dtype=torch.float32, device="cuda")
    out = torch.empty((wl.m, wl.n), dtype=torch.float32, device="cuda")

    def step(i):
        # route -> Direct matmul -> combine: one fused kernel
        lib.moe_forward(shape, B.DIRECT, weights, x, logits_d[i % ROT][None], bias_d[i % ROT], ids, gates,
                        y, out, None, weight_bytes=wl.weight_bytes)

    def step_unfused(i):
        lib.route_topk(logits_d[i % ROT][None], bias_d[i % ROT], wl.top_k, ids, gates)
        lib.matmul_id(shape, B.DIRECT, weights, x, ids, y, weight_bytes=wl.weight_bytes)
        lib.combine(y, gates, out)

    timed = Timed(step, ROT)
    res = timed.run(steps, warmup)
    # the graph's last step against the same step run eagerly, and against
    # the three separate calls
    last = steps - 1
    graph_out, graph_ids = out.clone(), ids.clone()
    step(last)
    torch.cuda.synchronize()
    assert torch.equal(graph_out, out) and torch.equal(graph_ids, ids), "graph replay differs from eager"
    assert sorted(graph_ids.cpu().numpy()[0].tolist()) == list(range(8 * (last % ROT), 8 * (last % ROT) + 8))
    step_unfused(last)
    torch.cuda.synchronize()
    assert torch.equal(graph_out.view(torch.int32), out.view(torch.int32)), "fused and unfused steps differ"
    unfused = Timed(step_unfused, ROT).run(ROT * 4, ROT, repeats=1)
    nbytes = decode_bytes(wl)
    t = res["gpu_ms_per_step"] * 1e-3
    res.update({
        "kernel": "moe_direct_kernel (route + Direct matmul + combine, one launch per step)",
        "touched_bytes": nbytes["touched_weights"],
        "algorithmic_bytes": nbytes["algorithmic"],
        "value_gbs": nbytes["touched_weights"] / t / 1e9,
        "algorithmic_gbs": nbytes["algorithmic"] / t / 1e9,
        "unfused_ms_per_step": unfused["gpu_ms_per_step"],
    })
    del weights
    torch.cuda.empty_cache()
    return res


# ---------------------------------------------------------------------- prefill
def bench_prefill(lib, name: str, steps: int, warmup: int):
    wl = W.WORKLOADS[name]
    shape = B.shape_of(wl)
    weights = torch.empty(wl.weight_bytes, dtype=torch.uint8, device="cuda")
    W.fill_weights(wl, weights)
    x = _dev(W.activations(wl))
    ids = torch.empty((wl.m, wl.top_k), dtype=torch.int32, device="cuda")
    gates = torch.empty((wl.m, wl.top_k), dtype=torch.float32, device="cuda")
    routed = wl.ids_kind == "logits"
    if routed:
        logits = _dev(W.router_logits(wl))
        bias = _dev(W.router_bias(wl))
    else:
        ids.copy_(_dev(W.ids(wl).view(np.int32)))
        gates.copy_(_dev(W.gates(wl)))
    y = torch.empty((wl.routed_rows, wl.n), dtype=torch.float32, device="cuda")
    out = torch.empty((wl.m, wl.n), dtype=torch.float32, device="cuda")
    scratch = torch.empty(lib.query(shape, B.GROUPED).scratch_bytes, dtype=torch.uint8, device="cuda")

    def matmul(i, route=B.GROUPED):
        lib.matmul_id(shape, route, weights, x, ids, y, scratch, weight_bytes=wl.weight_bytes)

    def step(i):
        if routed:
            lib.route_topk(logits, bias, wl.top_k, ids, gates)
        matmul(i)
        lib.combine(y, gates, out)

    # whole steps (route, matmul, combine), then the matmul call alone
    res = Timed(step, 4).run(PREFILL_STEPS, 8)
    mm = Timed(matmul, 4).run(PREFILL_STEPS, 8, repeats=3)
    flops = 2.0 * wl.routed_rows * wl.n * wl.k
    per_call = float(np.median(mm["repeats_gpu_ms_per_step"]))
    res.update({
        "flops": flops,
        "tflops": flops / (res["gpu_ms_per_step"] * 1e-3) / 1e12,
        "matmul_ms": {"per_call": per_call, "repeats": mm["repeats_gpu_ms_per_step"],
                      "calls_per_repeat": PREFILL_STEPS, "warmup_s": mm["warmup_s"]},
        "grouped_tflops": flops / (per_call * 1e-3) / 1e12,
    })
    # Direct on the same inputs, for the route comparison (not the headline)
    dm = kernel_times(lambda i: matmul(i, B.DIRECT), 3)
    res["direct_tflops"] = flops / (float(np.median(dm)) * 1e-3) / 1e12
    # the same matmul in the split-16 arithmetic (activation split + map +
    # Grouped per call); its roofline is the 16-bit matrix peak, on the
    # algorithmic flops (the three parts per activation are not counted)
    s16_shape = B.shape_of(wl.with_(arith=B.ARITH_SPLIT16))
    s16_scratch = torch.empty(lib.query(s16_shape, B.GROUPED).scratch_bytes, dtype=torch.uint8, device="cuda")

    def matmul16(i):
        lib.matmul_id(s16_shape, B.GROUPED, weights, x, ids, y, s16_scratch, weight_bytes=wl.weight_bytes)

    m16 = Timed(matmul16, 4).run(PREFILL_STEPS, 8, repeats=3)
    per16 = float(np.median(m16["repeats_gpu_ms_per_step"]))
    res["split16"] = {"per_call_ms": per16, "repeats": m16["repeats_gpu_ms_per_step"],
                      "tflops": flops / (per16 * 1e-3) / 1e12}
    del s16_scratch
    del weights
    torch.cuda.empty_cache()
    return res


# ---------------------------------------------------------------------- expert FFN
def bench_ffn(lib, steps: int, warmup: int):
    """The expert FFN (route, gate/up, silu * up, down, combine) on the
    prefill FFN workload, whole calls in a graph."""
    fw = W.FFN_WORKLOADS["ffn_prefill"]
    shape = B.ffn_shape_of(fw)
    wdev = {}
    for w in ("gate", "up", "down"):
        p = fw.part(w)
        wdev[w] = torch.empty(p.weight_bytes, dtype=torch.uint8, device="cuda")
        W.fill_weights(p, wdev[w])
    xh, lh, bh = W.ffn_inputs(fw)
    x, logits, bias = _dev(xh), _dev(lh), _dev(bh)
    ids = torch.empty((fw.m, fw.top_k), dtype=torch.int32, device="cuda")
    gates = torch.empty((fw.m, fw.top_k), dtype=torch.float32, device="cuda")
    out = torch.empty((fw.m, fw.hidden), dtype=torch.float32, device="cuda")
    scratch = torch.empty(lib.moe_ffn_scratch_bytes(shape), dtype=torch.uint8, device="cuda")

    def step(i):
        lib.moe_ffn(shape, B.AUTO, wdev["gate"], wdev["up"], wdev["down"], x, logits, bias, ids, gates, out,
                    scratch)

    res = Timed(step, 4).run(PREFILL_STEPS, 8)
    flops = 3 * 2.0 * fw.m * fw.top_k * fw.hidden * fw.inter
    res["flops"] = flops
    res["tflops"] = flops / (res["gpu_ms_per_step"] * 1e-3) / 1e12
    del wdev
    torch.cuda.empty_cache()
    return res


# ---------------------------------------------------------------------- counters
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "moe_direct_kernel_decode_hbm_counters.txt")
DECODE_SOURCES = ("moe_direct.hip", "direct_wave.hpp", "route_wave.hpp", "eidm_device.hpp",
                  "eidm_internal.hpp")


def decode_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for name in DECODE_SOURCES:
        with open(os.path.join(ROOT, "expert_id_matmul_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def decode_traffic():
    """HBM bytes per launch of the fused decode kernel, from the committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE summary, scaled by the same counters on
    a copy of known size; None when that summary is missing or was taken on
    other kernel sources than the ones built now."""
    try:
        fields = {}
        with open(TRAFFIC_FILE) as f:
            for ln in f:
                if ":" in ln:
                    k, v = ln.split(":", 1)
                    fields[k.strip()] = v.strip()
        if fields.get("sources_sha256") != decode_source_hash():
            return None
        return int(fields["hbm_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


# ---------------------------------------------------------------------- CPU oracle
def _host_cpus() -> dict:
    """Host core count (affinity and online) and the CPU model name."""
    model = platform.processor() or platform.machine()
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for ln in out.splitlines():
            if ln.lower().startswith("model name"):
                model = ln.split(":", 1)[1].strip()
                break
    except (OSError, subprocess.SubprocessError):
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count() or 1
    return {"usable": usable, "online": os.cpu_count() or usable, "model": model}


def _median_time(fn, runs: int = 3) -> float:
    ts = []
    for _ in range(runs):
        t0 = time.perf_counter()
        fn()
        ts.append(time.perf_counter() - t0)
    return float(np.median(ts))


def cpu_baseline():
    """The CPU oracle, as it stands (double-precision sums, one routine per
    output), on bounded samples of two workloads, each the median of 3 runs,
    on one host thread and on every usable host thread (the outputs split into
    contiguous ranges):
      decode: whole steps (route + the 8 routed rows x 1536 x 4096 bf16 matmul
              + combine), 4 steps per run, in GB/s of touched weights;
      prefill balanced: the 256 routed rows of experts 0-7 (m=512, k=2048,
              n=768, top-8 of 128 bf16), in GFLOP/s.
    `value` is the all-threads decode figure."""
    import oracle

    host = _host_cpus()
    threads = host["usable"]
    legs = {}
    # decode
    wl = W.WORKLOADS["decode"]
    logits, bias, x = W.router_logits(wl), W.router_bias(wl), W.activations(wl)
    ids0, _, _, _ = oracle.route(logits, bias, wl.top_k)
    # the touched experts packed at indices 0..7 (placement does not change y)
    packed = np.concatenate([W.expert_weights(wl, int(e)).contiguous().view(torch.uint8).numpy().reshape(-1)
                             for e in ids0[0]])
    local_ids = np.arange(wl.top_k, dtype=np.uint32)[None]
    touched = wl.top_k * wl.n * wl.k * W.DTYPE_SIZE[wl.dtype]
    steps = 4
    for th in (1, threads):
        def run(th=th):
            for _ in range(steps):
                _, g, _, _ = oracle.route(logits, bias, wl.top_k)
                y = oracle.matmul_id_threads(wl.dtype, wl.m, wl.n, wl.k, wl.top_k, wl.top_k, wl.stride, wl.layout,
                                             packed, x, local_ids, th)
                oracle.combine(y, g, wl.top_k)
        t = _median_time(run) / steps
        legs[f"decode_{th}t"] = {"value": touched / t / 1e9, "unit": "GB/s", "threads": th,
                                 "ms_per_step": t * 1e3}
    # prefill balanced sample: routed rows of experts 0..7, as a slotted problem
    wl = W.WORKLOADS["prefill_balanced"]
    n_e = 8
    packed = np.concatenate([W.expert_weights(wl, e).contiguous().view(torch.uint8).numpy().reshape(-1)
                             for e in range(n_e)])
    ids = W.ids(wl).reshape(-1)
    rows = np.nonzero(ids < n_e)[0]
    xs = W.activations(wl)[rows // wl.top_k]
    sids = ids[rows].astype(np.uint32)[:, None]
    flops = 2.0 * rows.size * wl.n * wl.k
    for th in (1, threads):
        t = _median_time(lambda th=th: oracle.matmul_id_threads(wl.dtype, rows.size, wl.n, wl.k, 1, n_e, wl.stride,
                                                                 W.LAYOUT_SLOTTED, packed, xs, sids, th))
        legs[f"prefill_balanced_{th}t"] = {"value": flops / t / 1e9, "unit": "GFLOP/s", "threads": th,
                                           "s_per_run": t}
    best = legs[f"decode_{threads}t"]
    return {"value": best["value"], "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"decode: {steps} whole steps per run (route + 8x1536x4096 bf16 matmul + combine); "
                      f"prefill balanced: the {rows.size} routed rows of experts 0-{n_e - 1} "
                      f"({flops / 1e9:.2f} GFLOP); median of 3 runs each, on 1 and {threads} threads",
            "host_cpus": host, "legs": legs}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=640, help="decode steps timed (exactly this many)")
    ap.add_argument("--warmup", type=int, default=64,
                    help="decode warm-up steps (at least; the warm-up also lasts at least half a second)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-ffn", action="store_true", help="skip the expert-FFN line")
    ap.add_argument("--no-decode", action="store_true",
                    help="prefill configurations only (the line then has no headline value)")
    ap.add_argument("--prefill", default="down_proj,prefill_balanced,prefill_skewed",
                    help="comma-separated prefill configurations to run")
    ap.add_argument("--copy-calibration", type=int, metavar="MIB", default=0,
                    help="only run a plain device copy of MIB MiB five times (the known-size "
                         "kernel that scales HBM byte counters) and exit")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the expert-ID matmul path here has no multi-GPU "
              "form (expert or column sharding is a design, not built); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    if args.steps < 1 or args.warmup < 0:
        print("--steps must be at least 1 and --warmup at least 0", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    if args.copy_calibration:
        n = args.copy_calibration * (1 << 20) // 4
        src = torch.empty(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": n * 4, "bytes_written": n * 4, "launches": 5}))
        return
    lib = B.load()
    dec = None
    if not args.no_decode:
        print(f"[bench] decode: {args.steps} steps, warmup {args.warmup} (and >= {WARMUP_FLOOR_S} s)",
              file=sys.stderr, flush=True)
        dec = bench_decode(lib, args.steps, args.warmup)
        print(f"[bench] decode warm-up ran {dec['warmup_steps_run']} steps in {dec['warmup_s']} s",
              file=sys.stderr, flush=True)
    prefill = {}
    if not args.no_prefill:
        for name in [p for p in args.prefill.split(",") if p]:
            print(f"[bench] {name}", file=sys.stderr, flush=True)
            prefill[name] = bench_prefill(lib, name, args.steps, args.warmup)
    ffn = None
    if not args.no_prefill and not args.no_ffn:
        print("[bench] ffn_prefill", file=sys.stderr, flush=True)
        ffn = bench_ffn(lib, args.steps, args.warmup)
    cpu = None
    if not args.no_cpu and not args.no_decode:
        print("[bench] cpu oracle baseline", file=sys.stderr, flush=True)
        cpu = cpu_baseline()
    prefill_out = {k: {"tflops_step": round(v["tflops"], 2),
                       "tflops_matmul": round(v["grouped_tflops"], 2),
                       "frac_f32_peak_matmul": round(v["grouped_tflops"] * 1e12 / F32_PEAK, 4),
                       "ms_per_step": round(v["gpu_ms_per_step"], 4),
                       "matmul_ms": v["matmul_ms"], "direct_tflops": round(v["direct_tflops"], 2),
                       "split16": {"tflops_matmul": round(v["split16"]["tflops"], 2),
                                   "ms": round(v["split16"]["per_call_ms"], 4),
                                   "frac_16bit_peak": round(v["split16"]["tflops"] * 1e12 / MX16_PEAK, 4),
                                   "vs_f32_order": round(v["split16"]["tflops"] / v["grouped_tflops"], 3)}}
                   for k, v in prefill.items()}
    if dec is None:
        print(json.dumps({"prefill": prefill_out}), flush=True)
        return
    line = {
        "metric": "expert-ID matmul: decode weight GB/s (m=1) + prefill TFLOP/s (m=2048) at 1 GPU",
        "value": round(dec["value_gbs"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": dec["steps"],
        "warmup": args.warmup,
        "warmup_steps_run": dec["warmup_steps_run"],
        "warmup_s": dec["warmup_s"],
        "ms_per_step": round(dec["gpu_ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "decode: m=1 k=4096 n=1536 n_experts=256 top_k=8, bf16 weights, "
                               "f32 activations, sigmoid+bias routing, cold experts",
                   "weights": "bf16", "m": 1, "n": 1536, "k": 4096, "n_experts": 256, "top_k": 8},
        "roofline": {"kernel": "moe_direct_kernel<bf16> (fused decode step)", "bound": "hbm",
                     "achieved": round(dec["algorithmic_gbs"], 1), "peak": HBM_PEAK / 1e9,
                     "unit": "GB/s", "frac": round(dec["algorithmic_gbs"] * 1e9 / HBM_PEAK, 4),
                     "traffic": decode_traffic()},
        "decode_detail": dec,
        "prefill": prefill_out,
        "ffn_prefill": None if ffn is None else {
            "workload": "m=512 hidden=2048 inter=768 top-8 of 128 bf16 experts: route, gate/up, "
                        "silu*up, down, combine", "ms_per_step": round(ffn["gpu_ms_per_step"], 4),
            "tflops": round(ffn["tflops"], 2)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
