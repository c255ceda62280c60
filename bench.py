#!/usr/bin/env python3
"""Bench of the MI355X decode GEMV: achieved HBM TB/s and fraction of peak at Llama-8B shapes.

Headline ("step" = one full GEMV pass): the down_proj GEMV, W 4096 x 14336 bf16, x bf16, fp32
outputs, batch 1. Inputs are seeded synthetic tensors already resident in HBM. Each step uses
the next of >= 1 GB of distinct weight copies, so no step is served from the 256 MB Infinity
Cache or the 32 MB of L2 (the decode-GEMV page warns about matrices small enough to sit in
cache, "Common mistakes"). Every launch in the timed region is bracketed by HIP events on the
stream it runs on; throughput is whole-region bytes / whole-region time, and the roofline's
`achieved` is algorithmic bytes / mean launch duration.

Also reported on the same JSON line: the graph-replayed decode step (32 layers x [QKV,
o_proj, gate_up, down] + lm_head), per-GEMV numbers for the other workload shapes, the
oracle timed on the host cores, and the pages' H100 context.

    python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import statistics
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
PEAK_HBM = 8.0e12                 # MI355X HBM3E, published peak, B/s
METRIC = "achieved HBM TB/s and % of peak, bf16 GEMV batch 1 at Llama-8B shapes"
ROTATION_BYTES = 1.0e9            # >= 1 GB of distinct weights per rotation arena
COUNTERS_FILE = os.path.join(HERE, "profiles", "counters_down_4096x14336.json")
# The headline (batch-1, whole-burst rows) kernel's sources; the committed counter summary
# is valid only for the sources it was taken on.
KERNEL_SOURCES = [os.path.join(HERE, "bandwidth_bound_decode_amd", "csrc", f)
                  for f in ("whole.hip", "device.h")]

# The pages' H100 SXM context (decode-GEMV page and GPU performance chains page).
H100 = {"hbm_TBps": 3.35, "sms": 132, "k_proj_transfer_us_at_peak": 2.5,
        "goal_fraction_of_peak": 0.80}


# ---------------------------------------------------------------------------- arithmetic
def alg_bytes(n: int, k: int, m: int = 1) -> int:
    """Bytes a perfect GEMV moves: W and X read once in bf16, Y written once in fp32."""
    return 2 * n * k + 2 * m * k + 4 * m * n


def seconds_at(nbytes: float, bytes_per_s: float) -> float:
    return nbytes / bytes_per_s


def mbu(nbytes: float, seconds: float, bytes_per_s: float) -> float:
    """Memory-bandwidth utilisation: bytes moved per second over the peak."""
    return nbytes / seconds / bytes_per_s


def waves(programs: int, units: int) -> int:
    return math.ceil(programs / units)


def wave_efficiency(programs: int, units: int) -> float:
    return programs / (waves(programs, units) * units)


def ridge(flops_per_s: float, bytes_per_s: float) -> float:
    return flops_per_s / bytes_per_s


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for path in KERNEL_SOURCES:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def counter_traffic(plan_info: dict):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or None when there
    is none, or the kernel source or the launch configuration changed since it was taken."""
    try:
        with open(COUNTERS_FILE) as f:
            c = json.load(f)
    except (OSError, ValueError):
        return None, "no counter summary"
    if c.get("kernel_source_sha256") != kernel_source_hash():
        return None, "kernel source changed since the counters were taken"
    if any(plan_info.get(k) != v for k, v in c.get("plan", {}).items()):
        return None, "launch configuration changed since the counters were taken"
    fetch = c["fetch_kib_per_launch"] * 1024 * c["fetch_scale"]
    write = c["write_kib_per_launch"] * 1024 * c["write_scale"]
    return round(fetch + write), ("rocprofv3 FETCH_SIZE + WRITE_SIZE per launch, scaled by a "
                                  "plain copy of known size (profiles/counters_down_4096x14336.json)")


def log(msg: str):
    print(msg, file=sys.stderr, flush=True)


def pct(xs, q):
    xs = sorted(xs)
    i = min(len(xs) - 1, max(0, int(round(q * (len(xs) - 1)))))
    return xs[i]


# ---------------------------------------------------------------------------- GPU timing
def time_launches(torch, launch, count: int, warmup: int, stream):
    """Run `launch(i)` warmup + count times; every timed launch is bracketed by events on
    `stream`. Returns (total seconds over the timed region, list of per-launch seconds)."""
    for i in range(warmup):
        launch(i)
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(count)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(count)]
    for i in range(count):
        starts[i].record(stream)
        launch(warmup + i)
        ends[i].record(stream)
    torch.cuda.synchronize()
    total = starts[0].elapsed_time(ends[-1]) / 1e3
    per = [s.elapsed_time(e) / 1e3 for s, e in zip(starts, ends)]
    return total, per


def time_graph(torch, launch, count: int, stream):
    """Capture `count` launches (launch(i), i = 0..count-1) into one graph on `stream`,
    replay it once untimed, then time one replay with events. Returns seconds for all
    `count` launches back to back, with no host in between."""
    import bandwidth_bound_decode_amd as bbd
    g = bbd.Graph(stream)
    with torch.cuda.stream(stream):
        with g:
            for i in range(count):
                launch(i)
    g.launch(stream)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    g.launch(stream)
    end.record(stream)
    torch.cuda.synchronize()
    g.destroy()
    return start.elapsed_time(end) / 1e3


def time_windows(torch, launch, per_graph: int, windows: int, min_launches: int, stream):
    """Per-launch time of `launch` run back to back, independent of the graph size.

    The launches are captured into one graph on `stream`: `per_graph` of them, repeated to a
    whole multiple of `per_graph` that reaches `min_launches`. Each of `windows` windows is
    an untimed leading replay, then two replays back to back (more if `min_launches` asks
    for it) bracketed by HIP events on `stream`: while the GPU runs the leading replay the
    host has already queued the timed ones, so the window holds the launches and none of the
    host's submission latency (which an idle GPU would wait for, see replay_cost). The
    per-launch time of a window is its span over the launches in it. Returns a dict of
    medians and the per-window figures."""
    import bandwidth_bound_decode_amd as bbd
    # One graph holds a whole multiple of the K launches, at least min_launches of them, so
    # that the replay's own cost is spread over as many launches whatever K is.
    per_graph = per_graph * max(1, math.ceil(min_launches / per_graph))
    g = bbd.Graph(stream)
    with torch.cuda.stream(stream):
        with g:
            for i in range(per_graph):
                launch(i)
    reps = max(2, math.ceil(min_launches / per_graph))
    for _ in range(2):                       # untimed replays
        g.launch(stream)
    torch.cuda.synchronize()
    per = []
    for _ in range(windows):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        g.launch(stream)                     # leading replay, untimed
        a.record(stream)
        for _ in range(reps):
            g.launch(stream)
        b.record(stream)
        torch.cuda.synchronize()
        per.append(a.elapsed_time(b) / 1e3 / (reps * per_graph))
    g.destroy()
    launch_s = statistics.median(per)
    return {"launch_s": launch_s, "per_window_s": per, "windows": windows, "reps": reps,
            "per_graph": per_graph, "timed_launches": windows * reps * per_graph,
            "spread": (max(per) - min(per)) / launch_s}


def replay_cost(torch, bbd, stream, replays: int = 11) -> float:
    """Seconds one replay of a graph holding a single tiny GEMV launch (1 x 512) takes
    between two events on an idle stream, median of `replays`: the host's submission of the
    replay, the events and one near-empty kernel. What a timing window would pay once if it
    started on an idle GPU; time_windows starts its windows behind a leading replay instead."""
    w = torch.zeros((1, 512), dtype=torch.bfloat16, device="cuda")
    x = torch.zeros((1, 512), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((1, 1), dtype=torch.float32, device="cuda")
    plan = bbd.Plan(1, 512, 1)
    ws = plan.alloc_workspace()
    g = bbd.Graph(stream)
    with torch.cuda.stream(stream):
        with g:
            bbd.run(plan, w, x, y, ws, stream)
    for _ in range(2):
        g.launch(stream)
    torch.cuda.synchronize()
    ts = []
    for _ in range(replays):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        g.launch(stream)
        b.record(stream)
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b) / 1e3)
    g.destroy()
    return statistics.median(ts)


def rotation_arena(torch, w, min_bytes=ROTATION_BYTES):
    nbytes = w.numel() * w.element_size()
    copies = max(2, math.ceil(min_bytes / nbytes) + 1)
    arena = torch.empty((copies,) + tuple(w.shape), dtype=w.dtype, device="cuda")
    for i in range(copies):
        arena[i].copy_(w)
    return arena


def bench_gemv(torch, bbd, g, w, x, steps, warmup, segments=(), windows=5, min_launches=200,
               **plan_opts):
    """Rotated timing of one GEMV shape (fused when `segments` is given): the launches back
    to back from one graph over several windows (the figure reported), and isolated
    launches each bracketed by its own events (these include the events' overhead)."""
    W = w.to("cuda")
    X = x.to("cuda")
    arena = rotation_arena(torch, W)
    plan = bbd.Plan(g.n, g.k, g.m, **plan_opts)
    ws = plan.alloc_workspace()
    Y = torch.empty((g.m, g.n), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    copies = arena.shape[0]
    if segments:
        bounds = [0]
        for s in segments:
            bounds.append(bounds[-1] + s)
        ys = [Y[:, a:b] for a, b in zip(bounds[:-1], bounds[1:])]

        def launch(i, stream=None):
            wi = arena[i % copies]
            bbd.fused_run(plan, [(wi[a:b], y) for (a, b), y in
                                 zip(zip(bounds[:-1], bounds[1:]), ys)], X, ws, stream)
    else:
        def launch(i, stream=None):
            bbd.run(plan, arena[i % copies], X, Y, ws, stream)
    # isolated launches: every launch bracketed by its own events (host-paced; the figure
    # includes the events' own ~2 us, so it is context, not the bandwidth figure)
    _, per = time_launches(torch, launch, steps, warmup, stream)
    # back to back: the same rotated launches replayed from one graph on a side stream
    side = torch.cuda.Stream()
    tw = time_windows(torch, lambda i: launch(i, side), steps, windows, min_launches, side)
    nb = alg_bytes(g.n, g.k, g.m)
    t = tw["launch_s"]
    res = {"shape": f"{g.n}x{g.k}", "m": g.m, "plan": plan.info, "alg_bytes": nb,
           "rotation_copies": copies,
           "us_per_launch": t * 1e6, "TBps": nb / t / 1e12, "pct_peak": 100 * nb / t / PEAK_HBM,
           "windows": tw["windows"], "launches_per_window": tw["reps"] * tw["per_graph"],
           "window_spread": tw["spread"],
           "isolated_launch_us_median": statistics.median(per) * 1e6,
           "isolated_launch_us_p10": pct(per, 0.1) * 1e6,
           "isolated_launch_us_p90": pct(per, 0.9) * 1e6}
    del arena
    return res, tw, per, plan


def bench_int4(torch, bbd, workloads, name, n, k, steps, warmup):
    """Rotated timing of one INT4-weight GEMV (batch 1): per-launch event pairs and the same
    launches back to back from one graph. Algorithmic bytes: packed weights, scales, x, y."""
    gen = workloads.generator(2000 + n % 997, "cuda")
    packed, scales, _ = workloads.draw_int4(n, k, gen, "cuda")
    x = workloads.bf16_normal((1, k), workloads.SIGMA_X, gen, "cuda")
    unit = packed.numel() + scales.numel() * 2
    copies = max(2, math.ceil(ROTATION_BYTES / unit) + 1)
    wa = torch.empty((copies,) + tuple(packed.shape), dtype=packed.dtype, device="cuda")
    sa = torch.empty((copies,) + tuple(scales.shape), dtype=scales.dtype, device="cuda")
    for i in range(copies):
        wa[i].copy_(packed)
        sa[i].copy_(scales)
    plan = bbd.Plan(n, k, 1, weights="int4")
    Y = torch.empty((1, n), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def launch(i, stream=None):
        bbd.run_int4(plan, wa[i % copies], sa[i % copies], x, Y, stream)
    _, per = time_launches(torch, launch, steps, warmup, stream)
    side = torch.cuda.Stream()
    tw = time_windows(torch, lambda i: launch(i, side), steps, 5, 200, side)
    t = tw["launch_s"]
    nb = unit + 2 * k + 4 * n
    info = plan.info
    res = {"name": name, "weights": "int4", "shape": f"{n}x{k}", "m": 1, "alg_bytes": nb,
           "plan": {key: info[key] for key in ("rows_per_wave", "unroll", "waves_per_block",
                                               "grid_x", "lds_bytes")},
           "rotation_copies": copies, "us_per_launch": t * 1e6, "TBps": nb / t / 1e12,
           "pct_peak": 100 * nb / t / PEAK_HBM, "window_spread": tw["spread"],
           "isolated_launch_us_median": statistics.median(per) * 1e6}
    del wa, sa
    return res


def bench_rmsnorm(torch, bbd, workloads, name, segments, k, steps):
    """A projection with its RMSNorm prologue fused (gemv_rmsnorm_run) against the same
    projection without it (gemv_fused_run on an already normalised x), both rotated and back
    to back in one graph, and against the norm as a separate launch (torch's rms_norm),
    timed back to back eagerly."""
    n = sum(segments)
    gen = workloads.generator(4000 + n % 997, "cuda")
    w = workloads.bf16_normal((n, k), workloads.SIGMA_W, gen, "cuda")
    h = workloads.bf16_normal((k,), workloads.SIGMA_X, gen, "cuda")
    gain = (1.0 + 0.1 * torch.randn((k,), generator=gen, device="cuda")).to(torch.bfloat16)
    arena = rotation_arena(torch, w)
    copies = arena.shape[0]
    bounds = [0]
    for seg in segments:
        bounds.append(bounds[-1] + seg)
    y = torch.empty((1, n), dtype=torch.float32, device="cuda")
    ys = [y[0, a:b] for a, b in zip(bounds[:-1], bounds[1:])]
    ys2 = [y[:, a:b] for a, b in zip(bounds[:-1], bounds[1:])]
    norm_plan = bbd.Plan(n, k, 1, prologue="rmsnorm")
    plain_plan = bbd.Plan(n, k, 1)
    x = h[None, :].clone()

    def fused(i, stream=None):
        wi = arena[i % copies]
        bbd.rmsnorm_run(norm_plan, [(wi[a:b], yy) for (a, b), yy in
                                    zip(zip(bounds[:-1], bounds[1:]), ys)], h, gain, 1e-5,
                        stream)

    def plain(i, stream=None):
        wi = arena[i % copies]
        if len(segments) == 1:
            bbd.run(plain_plan, wi, x, y, None, stream)
        else:
            bbd.fused_run(plain_plan, [(wi[a:b], yy) for (a, b), yy in
                                       zip(zip(bounds[:-1], bounds[1:]), ys2)], x, None, stream)
    side = torch.cuda.Stream()
    t_fused = time_windows(torch, lambda i: fused(i, side), steps, 5, 200, side)["launch_s"]
    t_plain = time_windows(torch, lambda i: plain(i, side), steps, 5, 200, side)["launch_s"]
    # the norm as its own launch, eagerly back to back (torch's kernel; not on the GEMV path)
    for _ in range(10):
        torch.nn.functional.rms_norm(h.float(), (k,), gain.float(), 1e-5)
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        torch.nn.functional.rms_norm(h.float(), (k,), gain.float(), 1e-5)
    b.record()
    torch.cuda.synchronize()
    t_norm = a.elapsed_time(b) / 1e3 / steps
    del arena
    return {"name": name, "shape": f"{n}x{k}", "segments": list(segments),
            "fused_norm_gemv_us": t_fused * 1e6, "gemv_without_norm_us": t_plain * 1e6,
            "prologue_cost_us": (t_fused - t_plain) * 1e6,
            "separate_torch_rms_norm_eager_us": t_norm * 1e6,
            "plan": {key: norm_plan.info[key] for key in ("unroll", "waves_per_block",
                                                          "grid_x", "lds_bytes")}}


def bench_decode_step_int4(torch, bbd, workloads, replays):
    """The same 129-GEMV decode step with INT4 weights: every projection (QKV and gate_up as
    one row-concatenated matrix each) through gemv_int4_run, captured in one graph, in stream
    order. Weights are drawn freshly (about 3.8 GB packed), so the first replay finds none of
    them in cache and later replays find at most the last ~256 MB."""
    gen = workloads.generator(3000, "cuda")
    plans, steps, nb = {}, [], 0
    for g in workloads.decode_step_gemvs():
        packed, scales, _ = workloads.draw_int4(g.n, g.k, gen, "cuda")
        x = workloads.bf16_normal((1, g.k), workloads.SIGMA_X, gen, "cuda")
        y = torch.empty((1, g.n), dtype=torch.float32, device="cuda")
        if (g.n, g.k) not in plans:
            plans[(g.n, g.k)] = bbd.Plan(g.n, g.k, 1, weights="int4")
        steps.append((plans[(g.n, g.k)], packed, scales, x, y))
        nb += packed.numel() + scales.numel() * 2 + 2 * g.k + 4 * g.n
    stream = torch.cuda.Stream()
    graph = bbd.Graph(stream)
    with torch.cuda.stream(stream):
        with graph:
            for plan, packed, scales, x, y in steps:
                bbd.run_int4(plan, packed, scales, x, y, stream)
    for _ in range(3):
        graph.launch(stream)
    torch.cuda.synchronize()
    times = []
    for _ in range(replays):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        graph.launch(stream)
        b.record(stream)
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b) / 1e3)
    graph.destroy()
    t = statistics.median(times)
    return {"gemvs": len(steps), "alg_bytes": nb, "replays": replays,
            "graph_ms_median": t * 1e3, "graph_TBps": nb / t / 1e12,
            "graph_mbu": nb / t / PEAK_HBM,
            "note": "INT4 weights (signed nibbles, bf16 scale per 128), batch 1, one graph of "
                    "129 gemv_int4_run launches; QKV and gate_up as one row-concatenated matrix"}


def bench_decode_step(torch, bbd, workloads, replays, warmup):
    """The 129-GEMV decode step three ways: eager launches, one graph of the 129 launches,
    and one graph holding the single persistent chain launch."""
    from bandwidth_bound_decode_amd.decode_step import Call, Sequence
    drawn = workloads.draw_decode_step("cuda")
    calls = [Call(parts, x, [torch.empty((x.shape[0], w.shape[0]), device="cuda")
                             for w in parts]) for _, parts, x in drawn]
    seq = Sequence(calls)
    nb = seq.alg_bytes
    stream = torch.cuda.Stream()
    chain = seq.chain()
    with torch.cuda.stream(stream):
        _, eager_per = time_launches(torch, lambda i: seq.run(stream), replays, warmup, stream)
        seq.capture(stream)
        _, graph_per = time_launches(torch, lambda i: seq.replay(stream), replays, warmup,
                                     stream)
        cg = bbd.Graph(stream)
        with cg:
            chain.run(stream)
        _, chain_per = time_launches(torch, lambda i: cg.launch(stream), replays, warmup,
                                     stream)
    chain.check()
    # The same step with the RMSNorm prologue fused into every call that consumes a
    # normalised vector in a Llama layer (QKV, gate_up) and into lm_head (the final norm):
    # each such call reads its x as the residual stream h plus a gain, eps 1e-5.
    gen = workloads.generator(5000, "cuda")
    norm_plans, norm_gain, nb_norm = {}, [], nb
    for c in calls:
        name_ok = len(c.weights) > 1 or c.weights[0].shape[0] == workloads.VOCAB
        if name_ok:
            key = (c.n, c.x.shape[-1])
            if key not in norm_plans:
                norm_plans[key] = bbd.Plan(c.n, c.x.shape[-1], 1, prologue="rmsnorm")
            norm_gain.append((1.0 + 0.1 * torch.randn((c.x.shape[-1],), generator=gen,
                                                       device="cuda")).to(torch.bfloat16))
            nb_norm += 2 * c.x.shape[-1]
        else:
            norm_gain.append(None)

    def run_with_norms(stream):
        for c, g in zip(calls, norm_gain):
            if g is None:
                if len(c.weights) == 1:
                    bbd.run(c.plan, c.weights[0], c.x, c.ys[0], seq.workspace, stream)
                else:
                    bbd.fused_run(c.plan, list(zip(c.weights, c.ys)), c.x, seq.workspace,
                                  stream)
            else:
                bbd.rmsnorm_run(norm_plans[(c.n, c.x.shape[-1])],
                                [(w, y[0]) for w, y in zip(c.weights, c.ys)], c.x[0], g,
                                1e-5, stream)
    with torch.cuda.stream(stream):
        ng = bbd.Graph(stream)
        with ng:
            run_with_norms(stream)
        _, norm_per = time_launches(torch, lambda i: ng.launch(stream), replays, warmup,
                                    stream)
    ng.destroy()
    out = {"gemvs": len(calls), "alg_bytes": nb, "weight_bytes": seq.weight_bytes,
           "replays": replays}
    t = statistics.median(norm_per)
    out["graph_with_rmsnorm_prologues_ms_median"] = t * 1e3
    out["graph_with_rmsnorm_prologues_mbu"] = mbu(nb_norm, t, PEAK_HBM)
    out["rmsnorm_prologue_calls"] = sum(g is not None for g in norm_gain)
    for name, per in (("eager", eager_per), ("graph", graph_per), ("chain_graph", chain_per)):
        t = statistics.median(per)
        out[f"{name}_ms_median"] = t * 1e3
        out[f"{name}_ms_p10"] = pct(per, 0.1) * 1e3
        out[f"{name}_ms_p90"] = pct(per, 0.9) * 1e3
        out[f"{name}_TBps"] = nb / t / 1e12
        out[f"{name}_mbu"] = mbu(nb, t, PEAK_HBM)
    out["gate_fraction"] = 0.80
    out["meets_gate"] = out["chain_graph_mbu"] >= 0.80 or out["graph_mbu"] >= 0.80
    out["note"] = ("graph: one hipGraph of the 129 GEMV launches (fused QKV and gate_up); "
                   "chain_graph: one hipGraph holding a single persistent launch that runs "
                   "the 129 GEMVs in order, each waiting for the previous one to complete "
                   "while its weights already stream")
    cg.destroy()
    chain.destroy()
    seq.graph.destroy()
    del seq, calls, drawn
    torch.cuda.empty_cache()
    return out


def bench_shards(torch, bbd, workloads, steps, replays):
    """One GPU's share of a decode step spread over G GPUs (G = 2, 4, 8): each projection's
    shard (rows of QKV, gate_up and lm_head, K of o_proj and down_proj) timed back to back on
    rotated weights like the shapes above, and the per-GPU 129-GEMV sequence as one graph.
    The collectives a multi-GPU step adds (the K-sharded partials summed over the GPUs, any
    gather of y) are not built, so the step is the GEMV part of one GPU's time."""
    from bandwidth_bound_decode_amd.decode_step import Call, Sequence
    out = []
    for gpus in workloads.SHARD_GPUS:
        rec = {"gpus": gpus, "shapes": []}
        for i, g in enumerate(workloads.shard_gemvs(gpus)):
            w, x = workloads.draw_gemv(g, workloads.generator(6000 + 10 * gpus + i, "cuda"),
                                       "cuda")
            r, _, _, _ = bench_gemv(torch, bbd, g, w, x, steps, 10, g.segments, windows=5)
            info = r["plan"]
            rec["shapes"].append({
                "name": g.name, "shape": f"{g.n}x{g.k}", "alg_bytes": g.alg_bytes,
                "us_per_launch": round(r["us_per_launch"], 3), "TBps": round(r["TBps"], 4),
                "pct_peak": round(r["pct_peak"], 2),
                "plan": {k: info[k] for k in ("splits", "unroll", "grid_x", "waves_per_cu")}})
            del w, x
        drawn = workloads.draw_decode_step("cuda", seed=6100 + gpus,
                                           gemvs=workloads.shard_decode_step_gemvs(gpus))
        calls = [Call(parts, x, [torch.empty((x.shape[0], w.shape[0]), device="cuda")
                                 for w in parts]) for _, parts, x in drawn]
        seq = Sequence(calls)
        nb = seq.alg_bytes
        stream = torch.cuda.Stream()
        with torch.cuda.stream(stream):
            seq.capture(stream)
            _, per = time_launches(torch, lambda i: seq.replay(stream), replays, 3, stream)
        t = statistics.median(per)
        rec["decode_step"] = {"gemvs": len(calls), "alg_bytes": nb,
                              "graph_ms_median": round(t * 1e3, 4),
                              "graph_TBps": round(nb / t / 1e12, 4),
                              "graph_mbu": round(mbu(nb, t, PEAK_HBM), 4),
                              "at_peak_ms": round(nb / PEAK_HBM * 1e3, 4)}
        seq.graph.destroy()
        del seq, calls, drawn
        torch.cuda.empty_cache()
        out.append(rec)
    return out


def cpu_baseline(w, x, min_seconds=10.0, max_runs=20000):
    """The oracle as it stands, on all host threads, over the same full GEMV, run back to back
    for about `min_seconds` of CPU work (a bounded sample); the median run, and the count."""
    import oracle
    import numpy as np
    wb = w.contiguous().view(__import__("torch").int16).numpy().view(np.uint16)
    xb = x.contiguous().view(__import__("torch").int16).numpy().view(np.uint16)
    threads = oracle.threads(0)
    oracle.gemv(wb, xb, nthreads=threads)                 # untimed warm-up
    times = []
    start = time.perf_counter()
    while len(times) < 3 or (time.perf_counter() - start < min_seconds and len(times) < max_runs):
        t0 = time.perf_counter()
        oracle.gemv(wb, xb, nthreads=threads)
        times.append(time.perf_counter() - t0)
    return statistics.median(times), threads, len(times), time.perf_counter() - start


def read_calibration(torch, bbd, cus, steps, window_launches):
    """The achievable read ceiling and the loaded latency, from the library's pure-read
    streaming kernel (the GEMV's weight stream alone).

    Sweep: 2 GiB read in 64 KiB rows (far beyond the 256 MB Infinity Cache), for U loads in
    flight per lane and a cap of W resident single-wave workgroups per CU; bytes in flight
    on the chip = W * U * 1 KiB * CUs. The ceiling is the best rate; on the points well
    below it (linear part) Little's law gives latency = bytes in flight / rate. Also the
    same read at the headline's shape (4096 rows of 28 KiB, U = 4, W = 8, rotated over
    >= 1 GB of copies), timed like the headline: the floor the GEMV's schedule allows."""
    rows, row_bytes = 32768, 65536
    buf = torch.empty(rows * row_bytes, dtype=torch.uint8, device="cuda")
    buf.fill_(0x5A)
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    side = torch.cuda.Stream()
    sweep = []
    for u in (1, 2, 4, 8):
        for cap in (1, 2, 3, 4, 6, 8, 12, 16, 24, 32):
            tw = time_windows(torch, lambda i: bbd.read_stream(buf, rows, row_bytes, u, cap,
                                                               sink, side), 5, 5, 5, side)
            rate = rows * row_bytes / tw["launch_s"]
            inflight = cap * u * 1024 * cus
            sweep.append({"unroll": u, "waves_per_cu": cap, "inflight_kib_per_cu": cap * u,
                          "TBps": round(rate / 1e12, 4),
                          "latency_us": round(inflight / rate * 1e6, 4)})
    del buf
    torch.cuda.empty_cache()
    ceiling = max(p["TBps"] for p in sweep)
    best = max(sweep, key=lambda p: p["TBps"])
    linear = [p for p in sweep if p["TBps"] < 0.75 * ceiling]
    lat_fit = statistics.median(p["latency_us"] for p in linear)
    # the least bytes in flight per CU that reach 95 % of the ceiling, and the latency there
    knee = min((p for p in sweep if p["TBps"] >= 0.95 * ceiling),
               key=lambda p: p["inflight_kib_per_cu"])
    # the headline's rows read alone
    nrows, rb = 4096, 14336 * 2
    copies = max(2, math.ceil(ROTATION_BYTES / (nrows * rb)) + 1)
    arena = torch.empty(copies * nrows * rb, dtype=torch.uint8, device="cuda")
    arena.fill_(0x3C)
    views = [arena[i * nrows * rb:(i + 1) * nrows * rb] for i in range(copies)]
    tw = time_windows(torch, lambda i: bbd.read_stream(views[i % copies], nrows, rb, 4, 8, sink,
                                                       side), steps, 5, window_launches, side)
    del arena, views
    torch.cuda.empty_cache()
    return {"TBps": ceiling, "frac_of_peak": round(ceiling * 1e12 / PEAK_HBM, 4),
            "best": {"unroll": best["unroll"], "waves_per_cu": best["waves_per_cu"]},
            "latency_us_linear_median": round(lat_fit, 4),
            "latency_us_light": min(p["latency_us"] for p in sweep),
            "knee": knee,
            "headline_shape_read_us": round(tw["launch_s"] * 1e6, 3),
            "headline_shape_read_TBps": round(nrows * rb / tw["launch_s"] / 1e12, 4),
            "sweep": sweep,
            "method": "2 GiB in 64 KiB rows, gemv_read_stream (one single-wave workgroup per "
                      "row, U nontemporal 16-byte loads per lane per burst, at most W "
                      "workgroups per CU); latency = bytes in flight / rate below 75 % of "
                      "the ceiling"}


def oracle_per_config(workloads, runs=3):
    """The oracle on every workload, on 1 thread and on all host threads: 1 untimed run then
    the median of `runs`. The decode step is sampled as one layer (QKV, o_proj, gate_up, down)
    plus lm_head and scaled to 32 layers + lm_head; its inputs are drawn on the host with the
    step's shapes and distributions."""
    import numpy as np
    import oracle
    import torch

    def bits(t):
        return t.contiguous().view(torch.int16).numpy().view(np.uint16)

    def timed(wb, xb, threads):
        oracle.gemv(wb, xb, nthreads=threads)
        ts = []
        for _ in range(runs):
            t0 = time.perf_counter()
            oracle.gemv(wb, xb, nthreads=threads)
            ts.append(time.perf_counter() - t0)
        return statistics.median(ts)

    all_threads = oracle.threads(0)
    rows = []

    def add(name, gemvs, scale=None, sample=None):
        entry = {"config": name, "gemvs": [f"{g.name} {g.n}x{g.k} m={g.m}" for g, _, _ in gemvs]}
        nbytes = sum(alg_bytes(g.n, g.k, g.m) for g, _, _ in gemvs)
        for label, th in (("1_thread", 1), ("all_threads", all_threads)):
            per = [timed(wb, xb, th) for _, wb, xb in gemvs]
            t = sum(per) if scale is None else scale(per)
            entry[f"seconds_{label}"] = round(t, 5)
            entry[f"GBps_{label}"] = round((nbytes if scale is None else scale_bytes) / t / 1e9, 4)
        entry["threads_all"] = all_threads
        if sample:
            entry["sample"] = sample
        rows.append(entry)
        log(f"oracle {name}: {entry['seconds_1_thread'] * 1e3:.1f} ms on 1 thread, "
            f"{entry['seconds_all_threads'] * 1e3:.1f} ms on {all_threads}")

    def drawn(cfg):
        return [(g, bits(w), bits(x)) for g, (w, x) in zip(cfg.gemvs, workloads.draw_config(cfg))]

    scale_bytes = None
    add("k_proj_and_tails", drawn(workloads.K_PROJ_AND_TAILS))
    add("down_proj", drawn(workloads.DOWN_PROJ))
    add("fused_projections", drawn(workloads.FUSED_PROJECTIONS))
    add("skinny_batch", drawn(workloads.SKINNY_BATCH))
    layer = [g for g in workloads.decode_step_gemvs()[:4]] + [workloads.decode_step_gemvs()[-1]]
    gen = workloads.generator(6000)
    sample = []
    for g in layer:
        w = workloads.bf16_normal((g.n, g.k), workloads.SIGMA_W, gen)
        x = workloads.bf16_normal((g.m, g.k), workloads.SIGMA_X, gen)
        sample.append((g, bits(w), bits(x)))
    layers = workloads.LAYERS
    scale_bytes = sum(alg_bytes(g.n, g.k, g.m) for g in workloads.decode_step_gemvs())
    add("decode_step", sample, scale=lambda per: layers * sum(per[:4]) + per[4],
        sample=f"one layer (QKV, o_proj, gate_up, down) and lm_head timed, scaled to "
               f"{layers} layers + lm_head")
    return rows


# ---------------------------------------------------------------------------- main
def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--decode-replays", type=int, default=20)
    ap.add_argument("--shape-steps", type=int, default=100)
    ap.add_argument("--windows", type=int, default=7,
                    help="timing windows for the headline (median reported, at least 5)")
    ap.add_argument("--window-launches", type=int, default=200,
                    help="launches per graph (at least); each timing window replays the "
                         "graph twice back to back behind an untimed leading replay")
    ap.add_argument("--skip-decode", action="store_true")
    ap.add_argument("--skip-shapes", action="store_true")
    ap.add_argument("--skip-cpu", action="store_true")
    ap.add_argument("--sections", default="all",
                    help="comma list of what to run besides the headline: calib, shapes, "
                         "rmsnorm, int4, decode, decode_int4, shards, cpu (default: all)")
    args = ap.parse_args(argv)
    args.windows = max(5, args.windows)
    every = {"calib", "shapes", "rmsnorm", "int4", "decode", "decode_int4", "shards", "cpu"}
    wanted = every if args.sections == "all" else set(args.sections.split(","))
    if wanted - every:
        ap.error(f"unknown sections {sorted(wanted - every)}")
    if args.skip_shapes:
        wanted -= {"shapes", "rmsnorm", "int4"}
    if args.skip_decode:
        wanted -= {"decode", "decode_int4", "shards"}
    if args.skip_cpu:
        wanted -= {"cpu"}
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this GEMV build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        return 2

    import torch

    sys.path.insert(0, HERE)
    import bandwidth_bound_decode_amd as bbd
    import workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    props = torch.cuda.get_device_properties(0)
    arch = getattr(props, "gcnArchName", "?")
    log(f"device: {props.name} {arch} CUs={props.multi_processor_count}")

    # headline: down_proj 4096 x 14336, batch 1
    cfg = workloads.DOWN_PROJ
    g = cfg.gemvs[0]
    (w, x), = workloads.draw_config(cfg)
    res, tw, per, plan = bench_gemv(torch, bbd, g, w, x, args.steps, args.warmup,
                                    windows=args.windows, min_launches=args.window_launches)
    nb = res["alg_bytes"]
    launch_s = tw["launch_s"]                 # median over the windows, back to back
    value_TBps = nb / launch_s / 1e12
    achieved_GBps = nb / launch_s / 1e9
    replay_s = replay_cost(torch, bbd, torch.cuda.Stream())
    log(f"down 4096x14336: {launch_s * 1e6:.3f} us per launch back to back (median of "
        f"{tw['windows']} windows of {tw['reps'] * tw['per_graph']} launches, spread "
        f"{100 * tw['spread']:.2f} %), {value_TBps:.3f} TB/s; a one-launch graph replay "
        f"{replay_s * 1e6:.1f} us; isolated launches "
        f"{res['isolated_launch_us_median']:.2f} us; plan {plan.info}")
    traffic, traffic_note = counter_traffic(plan.info)

    out = {
        "metric": METRIC,
        "value": round(value_TBps, 4),
        "unit": "TB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(launch_s * 1e3, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "down_proj GEMV y = W.x, W 4096x14336 bf16 row-major, x bf16, "
                               "fp32 accumulate and output, batch 1",
                   "n": g.n, "k": g.k, "m": g.m, "sigma_w": workloads.SIGMA_W,
                   "sigma_x": workloads.SIGMA_X, "seed": cfg.seed,
                   "rotation_copies": res["rotation_copies"], "plan": plan.info},
        "timing": {"method": "the K steps (one rotated launch each), repeated to a whole "
                             f"multiple of K of at least {args.window_launches} launches, "
                             "captured in one graph; each window is an untimed leading replay "
                             f"and then {tw['reps']} back-to-back replays between two HIP "
                             "events on the replay stream, its span over the launches in it; "
                             "value and ms_per_step use the median window",
                   "launches_per_graph": tw["per_graph"],
                   "windows": tw["windows"], "launches_per_window": tw["reps"] * tw["per_graph"],
                   "timed_launches": tw["timed_launches"],
                   "per_window_us": [round(t * 1e6, 4) for t in tw["per_window_s"]],
                   "window_spread": round(tw["spread"], 5),
                   "one_launch_graph_replay_us": round(replay_s * 1e6, 3),
                   "one_launch_graph_replay_note": "a replay of a graph holding one tiny GEMV "
                                                   "launch, between events on an idle stream "
                                                   "(mostly the host's submission latency); "
                                                   "each timed window starts behind an untimed "
                                                   "leading replay, so none of it is inside "
                                                   "the windows"},
        "pct_of_peak": round(100 * value_TBps * 1e12 / PEAK_HBM, 2),
        "roofline": {"bound": "hbm", "achieved": round(achieved_GBps, 1), "peak": PEAK_HBM / 1e9,
                     "unit": "GB/s", "frac": round(achieved_GBps * 1e9 / PEAK_HBM, 4),
                     "traffic": traffic, "traffic_note": traffic_note,
                     "alg_bytes_per_launch": nb,
                     "launch_us_mean": round(launch_s * 1e6, 3),
                     "timing": "mean launch duration back to back: median over the windows "
                               "of (window span / launches in it), HIP events on the replay "
                               "stream",
                     "isolated_launch_us_median": round(res["isolated_launch_us_median"], 3),
                     "isolated_launch_us_p10": round(res["isolated_launch_us_p10"], 3),
                     "isolated_launch_us_p90": round(res["isolated_launch_us_p90"], 3),
                     "isolated_note": "each launch bracketed by its own events, host-paced; "
                                      "includes the events' cost"},
        "device": {"name": props.name, "arch": arch, "cus": props.multi_processor_count,
                   "peak_hbm_TBps_assumed": PEAK_HBM / 1e12},
        "h100_context": H100,
    }

    if "calib" in wanted:
        cal = read_calibration(torch, bbd, props.multi_processor_count, args.steps,
                               args.window_launches)
        out["read_ceiling"] = cal
        out["pct_of_read_ceiling"] = round(100 * value_TBps / cal["TBps"], 2)
        out["roofline"]["frac_of_read_ceiling"] = round(value_TBps / cal["TBps"], 4)
        log(f"read ceiling {cal['TBps']:.3f} TB/s at U={cal['best']['unroll']} "
            f"W={cal['best']['waves_per_cu']}; loaded latency {cal['latency_us_linear_median']:.3f} us "
            f"(linear part), knee {cal['knee']['inflight_kib_per_cu']} KiB/CU; headline rows read "
            f"alone {cal['headline_shape_read_us']:.2f} us; GEMV at "
            f"{out['pct_of_read_ceiling']:.1f} % of the ceiling")

    if "cpu" in wanted:
        t_cpu, threads, runs, spent = cpu_baseline(w, x)
        out["cpu_baseline"] = {"value": round(nb / t_cpu / 1e12, 6), "unit": "TB/s",
                               "cores": threads, "kind": "oracle",
                               "sample": f"the full 4096x14336 batch-1 GEMV, fp64 C oracle "
                                         f"(OpenMP over rows), run {runs} times back to back "
                                         f"({spent:.1f} s) after 1 warm-up; the median run",
                               "seconds_per_gemv": round(t_cpu, 5), "runs": runs,
                               "host_cpus": len(os.sched_getaffinity(0))}
        log(f"cpu oracle: {t_cpu * 1e3:.2f} ms per GEMV on {threads} threads "
            f"({runs} runs, {spent:.1f} s)")
        out["cpu_baseline"]["per_config"] = oracle_per_config(workloads)

    if "shapes" in wanted:
        shapes = []
        kproj = workloads.K_PROJ_AND_TAILS.gemvs[0]
        wkp, xkp = workloads.draw_config(workloads.K_PROJ_AND_TAILS)[0]
        shapes.append(("k_proj", kproj, wkp, xkp, ()))
        for gg, (ww, xx) in zip(workloads.FUSED_PROJECTIONS.gemvs, workloads.draw_config(workloads.FUSED_PROJECTIONS)):
            shapes.append((gg.name + "_fused", gg, ww, xx, gg.segments))
        o = workloads.Gemv("o_proj", 4096, 4096)
        shapes.append(("o_proj", o, *workloads.draw_gemv(o, workloads.generator(7)), ()))
        lm = workloads.Gemv("lm_head", workloads.VOCAB, workloads.HIDDEN)
        shapes.append(("lm_head", lm, *workloads.draw_gemv(lm, workloads.generator(8, "cuda"), "cuda"),
                       ()))
        for gg, (ww, xx) in zip(workloads.SKINNY_BATCH.gemvs, workloads.draw_config(workloads.SKINNY_BATCH)):
            shapes.append((gg.name, gg, ww, xx, ()))
        # batches of 9-16 on the 16-row matrix-core form with 16 X vectors (where 32-row blocks
        # would have to split K): down_proj at M = 12 and o_proj at M = 16
        for name, n, k, m in (("batch_m12", workloads.HIDDEN, workloads.INTERMEDIATE, 12),
                              ("o_proj_m16", 4096, 4096, 16)):
            gb = workloads.Gemv(name, n, k, m)
            shapes.append((name, gb, *workloads.draw_gemv(gb, workloads.generator(70 + m)), ()))
        # the unaligned 4097 x 14337 tail at the batches where x no longer fits in LDS whole
        for m in (8, 16):
            gt = workloads.Gemv(f"skinny_tail_m{m}", workloads.HIDDEN + 1,
                                workloads.INTERMEDIATE + 1, m)
            shapes.append((gt.name, gt, *workloads.draw_gemv(gt, workloads.generator(90 + m)),
                           ()))
        for name, gg, ww, xx, segs in shapes:
            r, _, _, _ = bench_gemv(torch, bbd, gg, ww, xx, args.shape_steps, 10, segs,
                                    windows=5, min_launches=args.window_launches)
            r["name"] = name
            info = r["plan"]
            r["plan"] = {k: info[k] for k in ("splits", "rows_per_wave", "unroll",
                                              "grid_x", "grid_y")}
            if gg.k % 8 and not segs and info["mfma_unaligned_depth"]:
                # contiguous rows of odd length sit at 2-byte offsets; from M = 10 such calls
                # run on the matrix cores in 16-row tiles of each row class
                r["plan"] = {"kernel": "gemv_mfma_unaligned", "splits": 1,
                             "classes": 8, "rows_per_block": 16}
            elif gg.k % 8 and not segs and info["splits"] == 1:
                # below that the class-staged unaligned kernel, whose wave shape is its own
                # (not the plan's)
                r["plan"] = {"kernel": "gemv_unaligned_lds", "splits": 1}
            elif info["mfma"]:    # aligned calls of this plan run the matrix-core kernel
                r["plan"] = {"kernel": "gemv_mfma", "splits": info["mfma_splits"],
                             "rows_per_block": info["mfma_rows"], "grid_x": info["mfma_grid_x"],
                             "grid_y": info["mfma_splits"]}
            for k in list(r):
                if isinstance(r[k], float):
                    r[k] = round(r[k], 3)
            log(f"{name}: {r['us_per_launch']:.2f} us back to back, {r['TBps']:.3f} TB/s "
                f"({r['pct_peak']:.1f} %)")
            out.setdefault("shapes", []).append(r)
    if "rmsnorm" in wanted:
        # the RMSNorm prologue fused into the projections that consume the normalised x
        for name, segs in (("rmsnorm_qkv", (4096, 1024, 1024)), ("rmsnorm_gate_up", (14336, 14336))):
            r = bench_rmsnorm(torch, bbd, workloads, name, segs, 4096, args.shape_steps)
            for key in list(r):
                if isinstance(r[key], float):
                    r[key] = round(r[key], 3)
            log(f"{name}: fused {r['fused_norm_gemv_us']:.2f} us, without the norm "
                f"{r['gemv_without_norm_us']:.2f} us, a separate norm launch "
                f"{r['separate_torch_rms_norm_eager_us']:.2f} us")
            out.setdefault("rmsnorm_prologue", []).append(r)
    if "int4" in wanted:
        # INT4 weights at the same projection shapes (batch 1)
        for name, n, k in (("int4_down", 4096, 14336), ("int4_k_proj", 1024, 4096),
                           ("int4_o_proj", 4096, 4096), ("int4_qkv", 6144, 4096),
                           ("int4_gate_up", 28672, 4096), ("int4_lm_head", workloads.VOCAB, 4096)):
            r = bench_int4(torch, bbd, workloads, name, n, k, args.shape_steps, 10)
            for key in list(r):
                if isinstance(r[key], float):
                    r[key] = round(r[key], 3)
            log(f"{name}: {r['us_per_launch']:.2f} us back to back, {r['TBps']:.3f} TB/s "
                f"({r['pct_peak']:.1f} %)")
            out.setdefault("int4_shapes", []).append(r)

    if "decode" in wanted:
        d = bench_decode_step(torch, bbd, workloads, args.decode_replays, 3)
        for k in list(d):
            if isinstance(d[k], float):
                d[k] = round(d[k], 4)
        out["decode_step"] = d
        log(f"decode step: chain in a graph {d['chain_graph_ms_median']:.3f} ms "
            f"(MBU {d['chain_graph_mbu']:.3f}); graph of 129 launches "
            f"{d['graph_ms_median']:.3f} ms (MBU {d['graph_mbu']:.3f}); eager "
            f"{d['eager_ms_median']:.3f} ms; graph with {d['rmsnorm_prologue_calls']} fused "
            f"RMSNorm prologues {d['graph_with_rmsnorm_prologues_ms_median']:.3f} ms")
        torch.cuda.empty_cache()
    if "shards" in wanted:
        out["shards"] = bench_shards(torch, bbd, workloads, args.shape_steps,
                                     args.decode_replays)
        for rec in out["shards"]:
            d = rec["decode_step"]
            log(f"one GPU of {rec['gpus']}: " + ", ".join(
                f"{s['name']} {s['us_per_launch']:.2f} us ({s['pct_peak']:.0f} %)"
                for s in rec["shapes"]) + f"; per-GPU step {d['graph_ms_median']:.3f} ms "
                f"(MBU {d['graph_mbu']:.3f}, {d['at_peak_ms']:.3f} ms at peak)")
    if "decode_int4" in wanted:
        d4 = bench_decode_step_int4(torch, bbd, workloads, args.decode_replays)
        for k in list(d4):
            if isinstance(d4[k], float):
                d4[k] = round(d4[k], 4)
        out["decode_step_int4"] = d4
        log(f"decode step, INT4 weights: graph of 129 launches {d4['graph_ms_median']:.3f} ms "
            f"({d4['graph_TBps']:.3f} TB/s, MBU {d4['graph_mbu']:.3f})")

    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
