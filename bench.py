#!/usr/bin/env python3
"""Boundary-engine benchmark on one MI355X.

Workload: the 32-layer boundary sweep on the 8B GQA shape -- 64 requests with contexts
log-uniform in [512, 16384] tokens, 32 query / 8 KV heads, head_dim 128, bf16 K/V, page
size 16, 30% of the requests planted as broadening demand, page ids shuffled over a
24,576-page pool, every request at its capacity boundary.  A step is one boundary batch
through the C ABI: gp_boundary_scan (logits of both summaries against every retained key,
softmax statistics, Top-p working sets) -> gp_decide (delta, grow pops) ->
gp_compact_prepare (keep-sets, copy-on-write) -> gp_compact_move (in-place K/V moves,
free stack).  Inputs are resident in HBM before timing; between steps the mutated state is
restored from a device copy outside the timed region, so every step sees the same batch.

Prints one JSON line.  `value` is request-level boundary scans per second (each scan
covers all 32 layers); layer-tokens scanned per second and algorithmic HBM GB/s are
reported beside it.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
METRIC = "KV-boundary scans/sec (tokens scanned/s) + achieved HBM GB/s vs peak, 1 GPU"
HBM_PEAK_GBPS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_boundary_sweep.json")
# Sources of the dominant kernel (gather_kernel): a traffic record taken from counters is
# used only while these are unchanged.
KERNEL_SOURCES = ["compact.hip", "device_util.h", "gp_internal.h"]


def source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "demand_paged_kv_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--seed", type=int, default=3000)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=5.0e6,
                    help="layer-tokens of oracle work in the CPU baseline sample")
    ap.add_argument("--copy-probe", action="store_true",
                    help="run only a plain 4 GiB device copy (HBM counter calibration)")
    ap.add_argument("--workload", choices=("boundary_sweep", "decode_loop", "prefix_share", "policies", "overlap",
                                           "one_layer", "single_request"),
                    default="boundary_sweep",
                    help="boundary_sweep (default, the headline line); decode_loop (the 36-layer decode "
                         "loop: 128 requests x 4096 steps) or prefix_share (256 requests x 36 layers, page "
                         "32, shared 2048-token prefixes, pool at 80%% of demand; one shot) or policies (the "
                         "decode loop under each decision policy: grow ratios, and the signal's rank "
                         "correlation with the later working set) or overlap (decode attention with the "
                         "boundary engine serial vs on a second stream) or one_layer (16 requests, one layer, "
                         "summaries from 256 decode queries: a batch small enough to be bound by launch "
                         "latency) or single_request (the boundary of one request, 36 layers, at the "
                         "pages' operating point and at page 16, 4K and 16K tokens: the latency of the "
                         "boundaries that come one at a time), each reported on its own line")
    ap.add_argument("--decode-steps", type=int, default=4096)
    ap.add_argument("--graphs", action="store_true",
                    help="decode_loop: replay each step from HIP graphs (one launch per step) "
                         "instead of launching its kernels eagerly")
    ap.add_argument("--ordinary-pools", action="store_true",
                    help="allocate the K/V pools in ordinary device memory instead of asking for "
                         "physically contiguous memory (the compaction's row moves vary with the "
                         "physical pages behind ordinary allocations)")
    ap.add_argument("--schedules", default="serial,overlap",
                    help="overlap workload: schedules to run (serial, overlap)")
    ap.add_argument("--placements", type=int, default=0,
                    help="boundary sweep on this many fresh K/V pool placements (spacer allocations "
                         "of 1-20 GiB between them): per-placement step and gather times on their "
                         "own line, to show how the physical pages set the gather's speed")
    ap.add_argument("--paper", action="store_true",
                    help="the boundary sweep (or, with --workload decode_loop, the decode loop) at the pages' "
                         "operating point (KV block 256, p 0.99, quota 64), reported on its own line")
    return ap.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def copy_probe():
    import torch
    n = 4 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"copy probe: 3 copies of {n} bytes")


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the boundary engine has no multi-GPU path (each GPU "
              "would own its pool and run the same calls on its own requests). Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)
    if args.copy_probe:
        copy_probe()
        return
    if args.placements > 0:
        placements(args)
        return
    if args.workload == "decode_loop":
        decode_loop(args)
        return
    if args.workload == "prefix_share":
        prefix_share(args)
        return
    if args.workload == "policies":
        policies(args)
        return
    if args.workload == "overlap":
        overlap(args)
        return
    if args.workload == "one_layer":
        one_layer(args)
        return
    if args.workload == "single_request":
        single_request(args)
        return
    import numpy as np
    import torch

    from demand_paged_kv_amd import binding as Bd
    from demand_paged_kv_amd.engine import BoundaryEngine
    from synth import gpu_workloads as GW

    Bd.load()  # the HIP library must be there; no fallback
    t0 = time.time()
    if args.paper:
        from synth import workloads as SW
        gw = GW.boundary_sweep(seed=args.seed + 100, P=256, num_pages=1536, params=dict(SW.PARAMS_PAPER),
                               name="boundary_sweep_paper", contiguous=not args.ordinary_pools)
    else:
        gw = GW.boundary_sweep(seed=args.seed, contiguous=not args.ordinary_pools)
    st = gw.st
    torch.cuda.synchronize()
    log(f"workload generated in {time.time() - t0:.1f}s: {gw.B} requests, {gw.total_tokens()} tokens, "
        f"{st.L} layers, pool {st.num_pages} pages")
    prm = Bd.params_from(gw.params)
    eng = BoundaryEngine(st, gw.B, gw.total_tokens(), prm)
    req = torch.arange(gw.B, dtype=torch.int32, device="cuda")
    backup = GW.StateBackup(st)
    torch.cuda.synchronize()

    names = ("scan", "decide", "compact_prepare", "compact_move")
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
    times = {k: [] for k in names}
    totals = []
    first = None
    for i in range(args.warmup + args.steps):
        backup.restore()
        torch.cuda.synchronize()
        ev[0].record()
        eng.scan(req)
        ev[1].record()
        eng.decide(req)
        ev[2].record()
        eng.compact_prepare(req)
        ev[3].record()
        eng.compact_move(req)
        ev[4].record()
        torch.cuda.synchronize()
        snap = (eng.out.decision[: gw.B].cpu().numpy().copy(), eng.out.counters.cpu().numpy().copy())
        if first is None:
            first = snap
        else:
            assert np.array_equal(first[0], snap[0]) and np.array_equal(first[1], snap[1]), "non-deterministic step"
        if i >= args.warmup:
            for k, name in enumerate(names):
                times[name].append(ev[k].elapsed_time(ev[k + 1]))
            totals.append(ev[0].elapsed_time(ev[4]))
        log(f"step {i} ({'warmup' if i < args.warmup else 'timed'}): {ev[0].elapsed_time(ev[4]):.3f} ms")

    c = dict(zip(Bd.COUNTER_NAMES, [int(x) for x in first[1]]))
    dec = first[0]
    L, Hkv, Hq, d, P = st.L, st.Hkv, st.Hq, st.d, st.P
    esz = 2
    sum_n = gw.total_tokens()
    ms = float(np.mean(totals))
    step_s = ms / 1e3
    scan_bytes = L * Hkv * sum_n * d * esz + 2 * gw.B * L * Hq * d * 4
    move_bytes = c["moved_rows"] * 4 * d * esz
    cow_bytes = c["copied_rows"] * 4 * d * esz
    alg_bytes = scan_bytes + move_bytes + cow_bytes
    mean_ms = {k: float(np.mean(v)) for k, v in times.items()}
    per_kernel = {
        "scan": dict(bytes=scan_bytes, ms=mean_ms["scan"]),
        "compact_move": dict(bytes=move_bytes, ms=mean_ms["compact_move"]),
    }
    dom = max(per_kernel, key=lambda k: per_kernel[k]["ms"])
    kname = {"scan": "gp_boundary_scan (plan_kernel + fused_scan_kernel)",
             "compact_move": "gather_kernel (gp_compact_move)"}[dom]
    achieved = per_kernel[dom]["bytes"] / (per_kernel[dom]["ms"] / 1e3) / 1e9
    traffic = None
    try:
        with open(TRAFFIC_FILE) as fh:
            tf = json.load(fh)
        if tf.get("source_hash") == source_hash() and tf.get("kernel_key") == dom and not args.paper:
            traffic = tf.get("bytes_per_launch")
    except (OSError, ValueError):
        pass
    roofline = {"bound": "hbm", "kernel": kname, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic}

    result = {
        "metric": METRIC,
        "value": round(gw.B / step_s, 2),
        "unit": "scans/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": ("boundary_sweep: 64 requests x 32 layers, 32q/8kv heads, d128, bf16 K/V, "
                                "page 16, contexts log-uniform 512-16384, 30% planted broadening, "
                                "24576-page pool") if not args.paper else
                               ("boundary_sweep_paper: 64 requests x 32 layers, 32q/8kv heads, d128, bf16 K/V, "
                                "page 256, p 0.99, quota 64, contexts log-uniform 512-16384, 30% planted "
                                "broadening, 1536-page pool"),
                   "requests": gw.B, "layers": L, "q_heads": Hq, "kv_heads": Hkv, "head_dim": d,
                   "page_size": P, "tokens": sum_n, "pool_pages": st.num_pages, "top_p": gw.params["top_p"],
                   "n_local": gw.params["n_local"], "seed": gw.seed, "storage_dtype": "bf16",
                   "pool_memory": gw.pool_memory},
        "tokens_scanned_per_s": round(L * sum_n / step_s, 1),
        "algorithmic_GBps": round(alg_bytes / step_s / 1e9, 1),
        "hbm_frac": round(alg_bytes / step_s / 1e9 / HBM_PEAK_GBPS, 4),
        "algorithmic_bytes": {"scan": scan_bytes, "compact_move": move_bytes, "copy_on_write": cow_bytes},
        "breakdown_ms": {k: round(v, 4) for k, v in mean_ms.items()},
        "decisions": {"grow": int((dec == 1).sum()), "compact": int((dec == 0).sum())},
        "counters": c,
        "roofline": roofline,
    }

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(gw, backup, args.cpu_budget)
    print(json.dumps(result), flush=True)


def one_layer(args):
    """One layer, 16 requests (32/8 heads, d 128, bf16, page 16, contexts log-uniform in
    512-8192 tokens, page ids from a shuffled 65,536-page pool): the summaries are built
    on the GPU by gp_update_summaries from 256 bf16 decode queries, then the boundary
    batch is timed like the sweep's (state restored between steps).  About 45K tokens, so
    the step is bound by launch latency rather than HBM; reported, not a target."""
    import numpy as np
    import torch

    from demand_paged_kv_amd import binding as Bd
    from demand_paged_kv_amd.engine import BoundaryEngine
    from synth import device as SD
    from synth import gpu_workloads as GW
    from synth import workloads as SW

    Bd.load()
    wl = SW.config2(seed=2001)
    st = SD.upload(wl, "cuda")
    eng = BoundaryEngine(st, wl.B, wl.total_tokens(), Bd.params_from(wl.params))
    req = torch.arange(wl.B, dtype=torch.int32, device="cuda")
    q = torch.from_numpy(np.ascontiguousarray(wl.queries).view(np.int16)).view(torch.bfloat16).to("cuda")
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record()
    for t in range(q.shape[0]):
        eng.update_summaries(q[t], req)
    ev[1].record()
    torch.cuda.synchronize()
    ema_ms = ev[0].elapsed_time(ev[1]) / q.shape[0]
    backup = GW.StateBackup(st)
    steps = max(1, args.steps) * 10
    times = []
    for i in range(args.warmup + steps):
        backup.restore()
        torch.cuda.synchronize()
        ev[0].record()
        eng.scan(req)
        eng.decide(req)
        eng.compact_prepare(req)
        eng.compact_move(req)
        ev[1].record()
        torch.cuda.synchronize()
        if i >= args.warmup:
            times.append(ev[0].elapsed_time(ev[1]))
    ms = float(np.mean(times))
    c = dict(zip(Bd.COUNTER_NAMES, [int(x) for x in eng.out.counters.cpu().numpy()]))
    tok = wl.total_tokens() * wl.L
    print(json.dumps({"metric": METRIC, "value": round(wl.B / (ms / 1e3), 2), "unit": "scans/s", "n_gpus": 1,
                      "steps": steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
                      "higher_is_better": True, "vs_baseline": None, "dtype": "f32", "data": "synthetic",
                      "config": {"workload": "one_layer: 16 requests x 1 layer, 32q/8kv heads, d128, bf16 K/V, "
                                             "page 16, contexts log-uniform 512-8192, summaries from 256 decode "
                                             "queries", "tokens": wl.total_tokens(), "seed": 2001},
                      "tokens_scanned_per_s": round(tok / (ms / 1e3), 1),
                      "summary_update_ms_per_query": round(ema_ms, 4),
                      "decisions": {"grow": int(c["grows"]), "compact": int(c["compacts"])},
                      "counters": c}), flush=True)


def single_request(args):
    """The boundary batch of one request (36 layers, 32/8 heads, d 128, bf16, a concentrating
    request, so it compacts), timed per call like the sweep (state restored between steps):
    at the pages' operating point (KV block 256, p 0.99, quota 64) with about 4K and 16K
    tokens, and at page 16.  With the pages' block size a request reaches a boundary once
    every 256 decode steps, so boundaries mostly come one request at a time; 288 units
    leave most of the chip to the latency of each unit's walk."""
    import numpy as np
    import torch

    from demand_paged_kv_amd import binding as Bd
    from demand_paged_kv_amd.engine import BoundaryEngine
    from synth import gpu_workloads as GW
    from synth import workloads as SW

    Bd.load()
    L = 36
    names = ("scan", "decide", "compact_prepare", "compact_move")
    cases = []
    for P, ctx in ((256, 16000), (256, 4000), (16, 16000), (16, 4000)):
        prm = dict(SW.PARAMS_PAPER) if P == 256 else dict(SW.PARAMS_DEFAULT)
        gw = GW.boundary_sweep(seed=args.seed + 200, B=1, L=L, P=P, num_pages=ctx // P + 10, ctx=(ctx, ctx),
                               grow_frac=0.0, params=prm, name="single_request",
                               contiguous=not args.ordinary_pools)
        st = gw.st
        eng = BoundaryEngine(st, 1, gw.total_tokens(), Bd.params_from(gw.params))
        req = torch.zeros(1, dtype=torch.int32, device="cuda")
        backup = GW.StateBackup(st)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
        times = []
        for i in range(args.warmup + args.steps):
            backup.restore()
            torch.cuda.synchronize()
            ev[0].record()
            eng.scan(req)
            ev[1].record()
            eng.decide(req)
            ev[2].record()
            eng.compact_prepare(req)
            ev[3].record()
            eng.compact_move(req)
            ev[4].record()
            torch.cuda.synchronize()
            if i >= args.warmup:
                times.append([ev[k].elapsed_time(ev[k + 1]) for k in range(4)])
        med = np.median(np.array(times), axis=0)
        c = dict(zip(Bd.COUNTER_NAMES, [int(x) for x in eng.out.counters.cpu().numpy()]))
        n = gw.total_tokens()
        scan_b = L * st.Hkv * n * st.d * 2
        move_b = c["moved_rows"] * 4 * st.d * 2
        case = {"page_size": P, "tokens": n, "top_p": gw.params["top_p"], "n_local": gw.params["n_local"],
                "ms": {k: round(float(v), 4) for k, v in zip(names, med)}, "total_ms": round(float(med.sum()), 4),
                "scan_GBps": round(float(scan_b / med[0] / 1e6), 1),
                "move_GBps": round(float(move_b / max(med[3], 1e-9) / 1e6), 1),
                "decision": "compact" if c["compacts"] else "grow"}
        log(f"single request P={P} n={n}: {case}")
        cases.append(case)
        del eng, st, gw, backup
        torch.cuda.empty_cache()
    print(json.dumps({"metric": "boundary batch latency of one request (ms, median of the timed steps)",
                      "higher_is_better": False, "steps": args.steps, "warmup": args.warmup,
                      "config": {"workload": "single_request: 1 request x 36 layers, 32q/8kv heads, d128, bf16 K/V, "
                                             "concentrating (it compacts)", "seed": args.seed + 200},
                      "cases": cases, "data": "synthetic"}), flush=True)


def placements(args):
    """The boundary sweep on several fresh pool placements in one process (physically
    contiguous pools unless --ordinary-pools): the same batch (state restored) timed per
    placement.  Between placements a
    spacer allocation of a seeded random size moves where the next pools land."""
    import numpy as np
    import torch

    from demand_paged_kv_amd import binding as Bd
    from demand_paged_kv_amd import pool as PM
    from demand_paged_kv_amd.engine import BoundaryEngine
    from synth import gpu_workloads as GW

    Bd.load()
    contiguous = not args.ordinary_pools
    gw = GW.boundary_sweep(seed=args.seed, contiguous=contiguous)
    st = gw.st
    backup = GW.StateBackup(st)
    shape = tuple(st.k_pool.shape)
    st.k_pool = st.v_pool = None
    torch.cuda.synchronize()
    req = torch.arange(gw.B, dtype=torch.int32, device="cuda")
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    rng = np.random.default_rng(args.seed)
    spacer = None
    out = []
    for i in range(args.placements):
        k, kk = PM.empty(shape, torch.bfloat16, "cuda", contiguous)
        v, vk = PM.empty(shape, torch.bfloat16, "cuda", contiguous)
        st.k_pool, st.v_pool = k, v
        eng = BoundaryEngine(st, gw.B, gw.total_tokens(), Bd.params_from(gw.params))
        steps, moves = [], []
        for _ in range(max(1, args.steps)):
            backup.restore()
            torch.cuda.synchronize()
            ev[0].record()
            eng.scan(req)
            eng.decide(req)
            eng.compact_prepare(req)
            ev[1].record()
            eng.compact_move(req)
            ev[2].record()
            torch.cuda.synchronize()
            steps.append(ev[0].elapsed_time(ev[2]))
            moves.append(ev[1].elapsed_time(ev[2]))
        out.append({"placement": i, "pool_memory": "contiguous" if kk == vk == "contiguous" else "ordinary",
                    "ms_per_step": round(float(np.mean(steps)), 4), "compact_move_ms": round(float(np.mean(moves)), 4)})
        log(f"placement {i}: step {out[-1]['ms_per_step']:.3f} ms, gather {out[-1]['compact_move_ms']:.3f} ms")
        del eng
        st.k_pool = st.v_pool = None
        del k, v
        spacer = None
        torch.cuda.synchronize()
        torch.cuda.empty_cache()  # ordinary pools: return the memory, so the next ones are fresh
        spacer, _ = PM.empty((int(rng.integers(1, 21)) << 29,), torch.bfloat16, "cuda", contiguous)
    print(json.dumps({"metric": "boundary sweep step time per K/V pool placement (ms)", "higher_is_better": False,
                      "config": {"workload": "boundary_sweep: 64 requests x 32 layers, 32q/8kv heads, d128, bf16 "
                                             f"K/V, page 16, fresh {'contiguous' if contiguous else 'ordinary'} "
                                             "pools per placement",
                                 "steps_per_placement": max(1, args.steps), "seed": args.seed},
                      "median_ms_per_step": round(float(np.median([p["ms_per_step"] for p in out])), 4),
                      "min_ms_per_step": min(p["ms_per_step"] for p in out),
                      "max_ms_per_step": max(p["ms_per_step"] for p in out),
                      "placements": out}), flush=True)


def decode_loop(args):
    """The decode loop on the Qwen3-8B shape: 128 requests from 1024-token prompts, 36
    layers, every step updates both summaries and appends one K/V row per request, every
    P-th step (16; 256 with --paper) all 128 requests run a boundary batch.  Input generation is outside the
    timed region; every library call of every step is inside it (HIP events per step).
    With --graphs each step replays a HIP graph of its library calls (one launch); on
    MI355X that measured the same as eager launches (0.611 against 0.607 ms per step):
    the step is bound by its kernels, not by launches."""
    import numpy as np
    import torch

    from demand_paged_kv_amd import binding as Bd
    from demand_paged_kv_amd.engine import BoundaryEngine, DecodeGraph
    from synth.decode_loop import DecodeLoopGen, DecodeSpec

    Bd.load()
    if args.paper:   # the pages' operating point: KV block 256, p 0.99, quota 64
        from synth import workloads as SW
        spec = DecodeSpec(steps=args.decode_steps, P=256, params=dict(SW.PARAMS_PAPER))
    else:
        spec = DecodeSpec(steps=args.decode_steps)
    gen = DecodeLoopGen(spec, "cuda", contiguous=not args.ordinary_pools)
    st = gen.initial_state()
    torch.cuda.synchronize()
    eng = BoundaryEngine(st, spec.B, spec.B * (spec.prompt + spec.steps + spec.P), Bd.params_from(spec.params))
    req = torch.arange(spec.B, dtype=torch.int32, device="cuda")
    graph = None
    if args.graphs:   # one launch per step: every request's boundary falls on the same step
        graph = DecodeGraph(eng, req, spec.B)
        graph.bids.copy_(req)
    acc = torch.zeros(Bd.GP_NUM_COUNTERS, dtype=torch.int64, device="cuda")
    grows = torch.zeros(spec.B, dtype=torch.int64, device="cuda")
    starts, ends, is_boundary = [], [], []
    fill = 0
    scanned = torch.zeros((), dtype=torch.int64, device="cuda")   # candidate slots of every scan
    wall0 = time.time()
    for t in range(spec.steps):
        q, k, v = gen.step(out=(graph.q, graph.k, graph.v) if graph else None)
        st.pos.fill_(spec.prompt + t)
        fill += 1
        boundary = fill == spec.P
        if boundary:   # every write page fills on this step: n = (A + 1) * P per request
            scanned += (st.n_alloc[: spec.B].to(torch.int64).sum() + spec.B) * spec.P
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        if graph:
            out = graph.replay(boundary)
        else:
            out = eng.decode_step(q, k, v, req, req if boundary else None)
        e1.record()
        starts.append(e0)
        ends.append(e1)
        is_boundary.append(boundary)
        if boundary:
            fill = 0
            acc += eng.out.counters.to(torch.int64)
            grows += out.decision[: spec.B].to(torch.int64)
        if (t + 1) % 512 == 0:
            torch.cuda.synchronize()
            log(f"decode step {t + 1}/{spec.steps}: {time.time() - wall0:.1f}s wall")
    torch.cuda.synchronize()
    wall = time.time() - wall0
    ms = [a.elapsed_time(b) for a, b in zip(starts, ends)]
    ms_b = sum(m for m, bd in zip(ms, is_boundary) if bd)
    ms_all = sum(ms)
    c = dict(zip(Bd.COUNTER_NAMES, [int(x) for x in acc.cpu().numpy()]))
    assert c["grow_denied"] == 0 and c["deferred"] == 0, c
    # pool invariant after the run: every page's refcount equals its page-table references
    n_alloc = st.n_alloc[: spec.B].to(torch.int64)
    cols = torch.arange(spec.max_pages, device="cuda")[None, :]
    ref = st.page_table[: spec.B][cols <= n_alloc[:, None]].to(torch.int64)
    refs = torch.bincount(ref, minlength=spec.num_pages)
    assert torch.equal(refs.to(torch.int32), st.refcount), "refcounts do not match the page tables"
    assert int(st.free_top.item()) + int((refs > 0).sum().item()) == spec.num_pages
    L, Hq, Hkv, d = spec.L, spec.Hq, spec.Hkv, spec.d
    n_bound = int(sum(is_boundary))
    ema_bytes = spec.steps * spec.B * L * Hq * d * (2 + 16)
    append_bytes = spec.steps * spec.B * L * Hkv * d * 2 * 2 * 2
    scanned = int(scanned.item())
    scan_bytes = L * Hkv * scanned * d * 2 + n_bound * 2 * spec.B * L * Hq * d * 4
    move_bytes = c["moved_rows"] * 4 * d * 2
    alg = ema_bytes + append_bytes + scan_bytes + move_bytes
    s_all = ms_all / 1e3
    result = {
        "metric": METRIC,
        "value": round(n_bound * spec.B / s_all, 2),
        "unit": "scans/s",
        "n_gpus": 1,
        "steps": spec.steps,
        "warmup": 0,
        "ms_per_step": round(ms_all / spec.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"decode_loop{'_paper' if args.paper else ''}: 128 requests x 36 layers, 32q/8kv "
                               f"heads, d128, bf16 K/V, page {spec.P}, "
                               + ("p 0.99, quota 64, " if args.paper else "")
                               + f"1024-token prompts, {spec.steps} decode steps, boundary every {spec.P} steps",
                   "requests": spec.B, "layers": L, "q_heads": Hq, "kv_heads": Hkv, "head_dim": d,
                   "page_size": spec.P, "prompt": spec.prompt, "pool_pages": spec.num_pages,
                   "top_p": spec.params["top_p"], "n_local": spec.params["n_local"], "seed": spec.seed,
                   "pool_memory": gen.pool_memory, "hip_graphs": graph is not None},
        "boundary_batches": n_bound,
        "scans": n_bound * spec.B,
        "tokens_scanned_per_s": round(L * scanned / s_all, 1),
        "algorithmic_GBps": round(alg / s_all / 1e9, 1),
        "hbm_frac": round(alg / s_all / 1e9 / HBM_PEAK_GBPS, 4),
        "algorithmic_bytes": {"ema": ema_bytes, "append": append_bytes, "scan": scan_bytes,
                              "compact_move": move_bytes},
        "engine_ms": {"all_steps": round(ms_all, 2), "boundary_steps": round(ms_b, 2),
                      "other_steps": round(ms_all - ms_b, 2)},
        "wall_s_including_generation": round(wall, 2),
        "grows": int(grows.sum().item()),
        "counters": c,
    }
    print(json.dumps(result), flush=True)


def policies(args):
    """The decode loop (128 requests x 36 layers from 1024-token prompts, --decode-steps
    steps) under each decision policy: GrowPage's own rule, RANDOM at GrowPage's measured
    grow ratio (same grow frequency, random timing), INVERSE, ALWAYS_COMPACT and SHRINK.  Reports grow (and
    shrink) ratios and pages in use at the end.  For GrowPage's run it also reports how
    the boundary signal delta_t ranks against the change of the recent working set over
    the next h boundaries, sum W_S(t+h) - sum W_L(t) (Spearman rho and sign agreement) --
    a model-free analogue of the pages' demand-prediction check (GrowPage review, "Key
    claims", Fig 6)."""
    import numpy as np
    import torch
    from scipy.stats import spearmanr

    from demand_paged_kv_amd import binding as Bd
    from demand_paged_kv_amd.engine import BoundaryEngine
    from synth.decode_loop import DecodeLoopGen, DecodeSpec

    Bd.load()
    steps = min(args.decode_steps, 2048)
    out = {}
    grow_ratio = None
    sig = None
    for policy in ("growpage", "random", "inverse", "always_compact", "shrink"):
        spec = DecodeSpec(steps=steps)
        gen = DecodeLoopGen(spec, "cuda", contiguous=not args.ordinary_pools)
        st = gen.initial_state()
        eng = BoundaryEngine(st, spec.B, spec.B * (spec.prompt + spec.steps + spec.P),
                             Bd.params_from(dict(spec.params, policy=policy)))
        req = torch.arange(spec.B, dtype=torch.int32, device="cuda")
        rng = np.random.default_rng(spec.seed + 7)
        u = torch.zeros(spec.B, dtype=torch.float32, device="cuda")
        eng.set_policy(policy, u, grow_ratio or 0.0)
        grows = denied = shrinks = boundaries = 0
        ws_s, ws_l, deltas = [], [], []
        t0 = time.time()
        for t in range(spec.steps):
            q, k, v = gen.step()
            st.pos.fill_(spec.prompt + t)
            boundary = (t + 1) % spec.P == 0
            if boundary:
                u.copy_(torch.from_numpy(rng.random(spec.B).astype(np.float32)))
            o = eng.decode_step(q, k, v, req, req if boundary else None)
            if boundary:
                boundaries += 1
                c = o.counters.cpu().numpy()
                grows += int(c[0])
                denied += int(c[2])
                shrinks += int(c[8])
                if policy == "growpage":
                    w = o.ws[: spec.B].to(torch.int64).sum(dim=(1, 2)).cpu().numpy()     # [B][2]
                    ws_s.append(w[:, 0])
                    ws_l.append(w[:, 1])
                    deltas.append(o.delta[: spec.B].cpu().numpy().astype(np.int64))
        torch.cuda.synchronize()
        pages = int(st.n_alloc[: spec.B].sum().item()) + spec.B
        ratio = grows / (boundaries * spec.B)
        out[policy] = {"grow_ratio": round(ratio, 4), "grows": grows, "grow_denied": denied,
                       "pages_in_use_end": pages, "boundaries": boundaries,
                       "wall_s": round(time.time() - t0, 2)}
        if policy == "shrink":
            out[policy]["shrink_ratio"] = round(shrinks / (boundaries * spec.B), 4)
        log(f"policy {policy}: grow ratio {ratio:.4f}, pages {pages}")
        if policy == "growpage":
            grow_ratio = ratio
            S, Lg, D = np.array(ws_s), np.array(ws_l), np.array(deltas)             # [boundaries][B]
            sig = {}
            for h in (1, 2, 4, 8):
                fut = (S[h:] - Lg[:-h]).ravel()
                dd = D[:-h].ravel()
                rho = spearmanr(dd, fut).correlation
                agree = float(np.mean(np.sign(dd) == np.sign(fut)))
                sig[f"h{h}"] = {"spearman": round(float(rho), 4), "sign_agreement": round(agree, 4),
                                "pairs": int(dd.size)}
        del eng, st, gen
        torch.cuda.empty_cache()
    result = {"metric": "decision-policy grow ratios and boundary-signal rank correlation (decode loop)",
              "config": {"workload": f"decode_loop: 128 requests x 36 layers, page 16, 1024-token prompts, "
                                     f"{steps} decode steps"},
              "random_grow_prob": round(grow_ratio, 4), "policies": out, "signal_vs_future": sig,
              "data": "synthetic"}
    print(json.dumps(result), flush=True)


def overlap(args):
    """Boundary-engine cost on a decode loop with decode attention (the reader of the
    pages), boundaries staggered so that every step 1/16 of the requests reach theirs:
    128 requests x 36 layers from 1024-token prompts, page 16.  Two schedules over the
    same steps and the same decisions: serial (the step's boundary batch after its
    attention, one stream; HIP events split the time into decode work and engine work)
    and overlapped (engine.OverlapSchedule: the boundary requests' attention first, then
    their boundary batch on a second stream while the other requests' attention runs;
    the next step waits for it).  The query rows of each subset are gathered by torch
    before the attention."""
    import numpy as np
    import torch

    from demand_paged_kv_amd import binding as Bd
    from demand_paged_kv_amd.engine import BoundaryEngine, OverlapSchedule
    from synth.decode_loop import DecodeLoopGen, DecodeSpec

    Bd.load()
    steps, warm = 256, 32
    res = {}
    for mode in args.schedules.split(","):
        spec = DecodeSpec(steps=steps + warm, stagger=True)
        gen = DecodeLoopGen(spec, "cuda", contiguous=not args.ordinary_pools)
        st = gen.initial_state()
        eng = BoundaryEngine(st, spec.B, spec.B * (spec.prompt + spec.steps + 2 * spec.P),
                             Bd.params_from(spec.params))
        fill = gen.fill0.copy()
        pos0 = torch.from_numpy((spec.prompt + gen.fill0).astype(np.int32)).cuda()
        req = torch.arange(spec.B, dtype=torch.int32, device="cuda")
        out = torch.empty((spec.B, spec.L, spec.Hq, spec.d), dtype=torch.float32, device="cuda")
        sched = OverlapSchedule(eng)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        marks = []
        grows = torch.zeros((), dtype=torch.int64, device="cuda")
        # boundary / other request ids of every step, built before the loop so that building
        # them is outside the timed region
        ids = []
        for t in range(steps + warm):
            fill += 1
            bmask = fill == spec.P
            fill[bmask] = 0
            ids.append((torch.as_tensor(np.flatnonzero(bmask).astype(np.int32), device="cuda"),
                        torch.as_tensor(np.flatnonzero(~bmask).astype(np.int32), device="cuda")))
        torch.cuda.synchronize()
        for t in range(steps + warm):
            q, k, v = gen.step()
            if t == warm:
                torch.cuda.synchronize()
                e0.record()
            torch.add(pos0, t, out=st.pos)
            bids, oids = ids[t]
            nb = int(bids.numel())
            if mode == "serial":
                m = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
                m[0].record()
                eng.update_summaries(q, req)
                eng.append(k, v, req)
                eng.decode_attention(q, req, out)
                m[1].record()
                if nb:
                    o = eng.step(bids)
                    if t >= warm:
                        grows += o.counters[0]
                m[2].record()
                if t >= warm:
                    marks.append(m)
            else:
                sched.step(q, k, v, req, bids, oids, out)
        sched.finish()
        e1.record()
        torch.cuda.synchronize()
        total = e0.elapsed_time(e1) / steps
        res[mode] = {"ms_per_step": round(total, 4)}
        if mode == "serial":
            dec = sum(m[0].elapsed_time(m[1]) for m in marks) / steps
            engm = sum(m[1].elapsed_time(m[2]) for m in marks) / steps
            res[mode].update(decode_ms_per_step=round(dec, 4), engine_ms_per_step=round(engm, 4),
                             grows=int(grows.item()))
        log(f"overlap {mode}: {res[mode]}")
        del eng, st, gen
        torch.cuda.empty_cache()
    ser = res.get("serial")
    hidden = None
    if ser and "overlap" in res:
        hidden = round((ser["ms_per_step"] - res["overlap"]["ms_per_step"]) / max(ser["engine_ms_per_step"], 1e-9), 4)
    result = {"metric": "decode step time with the boundary engine (ms per step)",
              "config": {"workload": "decode loop with decode attention: 128 requests x 36 layers, page 16, "
                                     "1024-token prompts, boundaries staggered (8 requests per step), "
                                     f"{steps} timed steps"},
              "schedules": res,
              "engine_share_serial": round(ser["engine_ms_per_step"] / ser["ms_per_step"], 4) if ser else None,
              "engine_time_hidden_by_overlap": hidden,
              "data": "synthetic"}
    print(json.dumps(result), flush=True)


def prefix_share(args):
    """One boundary batch of the prefix-sharing stress (no room for a state backup, so a
    single timed step): 256 requests x 36 layers, page 32, groups of 16 sharing a 64-page
    prefix, contexts log-uniform in [1024, 32768], pool at 80% of the full-KV demand."""
    import numpy as np
    import torch

    from demand_paged_kv_amd import binding as Bd
    from demand_paged_kv_amd.engine import BoundaryEngine
    from synth import gpu_workloads as GW

    Bd.load()
    t0 = time.time()
    gw = GW.prefix_share(seed=5000, contiguous=not args.ordinary_pools)
    st = gw.st
    torch.cuda.synchronize()
    log(f"workload generated in {time.time() - t0:.1f}s: {gw.B} requests, {gw.total_tokens()} tokens, "
        f"pool {st.num_pages} pages, free {int(st.free_top.item())}")
    eng = BoundaryEngine(st, gw.B, gw.total_tokens(), Bd.params_from(gw.params))
    req = torch.arange(gw.B, dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    names = ("scan", "decide", "compact_prepare", "compact_move")
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
    ev[0].record()
    eng.scan(req)
    ev[1].record()
    eng.decide(req)
    ev[2].record()
    eng.compact_prepare(req)
    ev[3].record()
    eng.compact_move(req)
    ev[4].record()
    torch.cuda.synchronize()
    c = dict(zip(Bd.COUNTER_NAMES, [int(x) for x in eng.out.counters.cpu().numpy()]))
    ms = ev[0].elapsed_time(ev[4])
    L, Hq, Hkv, d = st.L, st.Hq, st.Hkv, st.d
    sum_n = gw.total_tokens()
    scan_bytes = L * Hkv * sum_n * d * 2 + 2 * gw.B * L * Hq * d * 4
    move_bytes = c["moved_rows"] * 4 * d * 2
    cow_bytes = c["copied_rows"] * 2 * 2 * d * 2
    alg = scan_bytes + move_bytes + cow_bytes
    s_ = ms / 1e3
    result = {
        "metric": METRIC, "value": round(gw.B / s_, 2), "unit": "scans/s", "n_gpus": 1, "steps": 1,
        "warmup": 0, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "prefix_share: 256 requests x 36 layers, 32q/8kv heads, d128, bf16 K/V, page 32, "
                               "groups of 16 sharing a 2048-token prefix, contexts log-uniform 1024-32768, "
                               "pool 80% of full-KV demand",
                   "requests": gw.B, "layers": L, "page_size": st.P, "tokens": sum_n,
                   "pool_pages": st.num_pages, "seed": gw.seed, "pool_memory": gw.pool_memory},
        "tokens_scanned_per_s": round(L * sum_n / s_, 1),
        "algorithmic_GBps": round(alg / s_ / 1e9, 1),
        "hbm_frac": round(alg / s_ / 1e9 / HBM_PEAK_GBPS, 4),
        "algorithmic_bytes": {"scan": scan_bytes, "compact_move": move_bytes, "copy_on_write": cow_bytes},
        "breakdown_ms": {k: round(ev[i].elapsed_time(ev[i + 1]), 4) for i, k in enumerate(names)},
        "counters": c,
    }
    print(json.dumps(result), flush=True)


def _oracle_worker(conn, start):
    """One all-cores baseline process: receive a sub-batch, wait for the common start, run
    the oracle's boundary step on it with one BLAS thread, send back the elapsed time."""
    from threadpoolctl import threadpool_limits

    import oracle as O
    wl, params = conn.recv()
    conn.send("ready")
    start.wait()
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        O.boundary_step(wl, wl.sum_s, wl.sum_l, params)
        t = time.perf_counter() - t0
    conn.send(t)
    conn.close()


def _sub_workload(wl, idx):
    """The requests ``idx`` of a host workload over the same pool state (input plumbing)."""
    import dataclasses
    idx = list(idx)
    return dataclasses.replace(wl, page_table=wl.page_table[idx].copy(), n_alloc=wl.n_alloc[idx].copy(),
                               fill=wl.fill[idx].copy(), pos=wl.pos[idx].copy(),
                               k_rows=[wl.k_rows[i] for i in idx], v_rows=[wl.v_rows[i] for i in idx],
                               sum_s=wl.sum_s[idx], sum_l=wl.sum_l[idx],
                               regime=None if wl.regime is None else wl.regime[idx].copy())


def time_oracle(wl, params, max_workers=16):
    """Seconds the oracle's boundary step takes on host workload ``wl``: on one thread, and
    on all cores -- one process per core (at most ``max_workers``; 16 is the GPU machine's CPU
    share), each running the step on its share of the requests (longest first to the
    least loaded), all started together after their data has arrived; the all-cores time
    is the wall time from that start to the last finish.  Returns (t_one, t_all, workers,
    per-process seconds)."""
    import multiprocessing as mp

    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle as O

    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        O.boundary_step(wl, wl.sum_s, wl.sum_l, params)
        t_one = time.perf_counter() - t0
    nproc = os.cpu_count() or 1
    avail = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else nproc
    workers = max(1, min(max_workers, avail, wl.B))
    loads = [0] * workers
    parts = [[] for _ in range(workers)]
    for i in sorted(range(wl.B), key=lambda i: -int(wl.n(i))):
        w = int(np.argmin(loads))
        parts[w].append(i)
        loads[w] += int(wl.n(i))
    ctx = mp.get_context("spawn")       # fresh interpreters: the workers never touch the GPU
    start = ctx.Event()
    procs, conns = [], []
    try:
        for _ in range(workers):
            a, b = ctx.Pipe()
            pr = ctx.Process(target=_oracle_worker, args=(b, start), daemon=True)
            pr.start()
            procs.append(pr)
            conns.append(a)
        for a, part in zip(conns, parts):
            a.send((_sub_workload(wl, sorted(part)), params))
        for a in conns:
            assert a.recv() == "ready"
        t0 = time.perf_counter()
        start.set()
        per = [a.recv() for a in conns]
        t_all = time.perf_counter() - t0
    finally:
        for pr in procs:
            pr.join(timeout=60)
            if pr.is_alive():
                pr.kill()
    return t_one, t_all, workers, per


def cpu_baseline(gw, backup, budget):
    """The oracle, as it stands, on a bounded sample of the same batch (host cores), on one
    thread and on all cores (time_oracle)."""
    import torch

    from synth import gpu_workloads as GW

    backup.restore()
    torch.cuda.synchronize()
    sample, acc = [], 0
    for b in range(gw.B):
        sample.append(b)
        acc += int(gw.n[b]) * gw.st.L
        if acc >= budget:
            break
    wl = GW.to_host_workload(gw, sample)
    t1, tn, workers, per = time_oracle(wl, gw.params)
    log(f"cpu baseline: {len(sample)} requests, {acc} layer-tokens: 1 thread {t1:.1f}s; "
        f"{workers} processes {tn:.1f}s wall (per process {min(per):.1f}-{max(per):.1f}s)")
    desc = (f"first {len(sample)} requests of the same batch ({acc} layer-tokens, all 32 layers), full "
            f"boundary step (scan, decide, keep-sets, compaction) in float64 numpy")
    return {"value": round(len(sample) / tn, 4), "unit": "scans/s", "cores": workers, "kind": "oracle",
            "sample": desc + f"; {workers} processes over requests, one BLAS thread each",
            "seconds": round(tn, 2), "tokens_scanned_per_s": round(acc / tn, 1), "nproc": os.cpu_count(),
            "single_thread": {"value": round(len(sample) / t1, 4), "unit": "scans/s", "cores": 1,
                              "seconds": round(t1, 2), "tokens_scanned_per_s": round(acc / t1, 1)}}


if __name__ == "__main__":
    main()
