"""Bench: paged verify attention on one MI355X.

Prints ONE JSON line. The headline workload is MTP-5 verify with bf16 KV
(8 sequences, query length 6, 16 q / 2 KV heads, D 128, contexts uniform in
[4096, 32768], 16-token pages); a step is one pa_decode_verify call (the
partition kernel and the log-sum-exp reduce) over that batch with its inputs
already in HBM. The metric is the algorithmic KV bytes a call must read
(K + V, plus FP8 scales) divided by the time per call.

Cache hygiene: the MI355X's 256 MiB Infinity Cache would hold a ~150 MB
working set, so consecutive steps rotate over enough copies of the K/V pools
that every call's KV was last touched more than 1 GiB of traffic earlier.
No flush runs inside the timed region.

Timing: the K timed steps are one replay of a HIP graph that captured them
(as a serving engine replays decode steps); the host clock around it, with
device synchronisations on both sides, gives ms_per_step.

Roofline: the partition kernel dominates; its duration is read from HIP
events attached to its launch on the call's stream (pa_set_partition_events:
the events take the kernel's own start and end timestamps) in an eager pass
over the same calls.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import platform
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "KV-read HBM GB/s (% of peak) + µs/call, q=6 verify, bf16 & FP8 KV"
KERNEL_SRC = os.path.join(ROOT, "paged_kv_cache_verify_amd", "csrc", "pa_kernels.hip")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_hash() -> str:
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def load_traffic(workload_key: str):
    """HBM bytes per partition launch from the committed rocprofv3 counter
    summary, if it was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload_key}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_sha256_16") != kernel_hash():
        return None
    return rec.get("bytes_per_launch")


def measure(wl, steps: int, warmup: int, partition_tokens=None, bound_extra=None, warm=False,
            fused=False):
    """Time `steps` calls on rotating pool copies; returns a dict of figures.
    fused: time pa_decode_verify_fused (one launch; its partition kernel
    then includes the merge) instead of the two-launch call.

    The timed region is one replay of a HIP graph holding the `steps` calls
    (the way a serving engine replays its decode steps), bracketed by device
    synchronisations and the host clock; if capture is unavailable the same
    steps run eagerly. A second, eager pass over the same calls records HIP
    events around every partition kernel on its stream, which give that
    kernel's duration per call.
    """
    import torch

    import paged_kv_cache_verify_amd as pav

    dev = wl.to("cuda:0")
    lens_dev = None
    if bound_extra is None:
        plan = pav.plan_for(dev, device=0, partition_tokens=partition_tokens)
        info = plan.info()
        kv = info["kv_bytes"]
    else:
        # A plan on upper bounds (every length + bound_extra) and calls that
        # read the actual lengths from device memory.
        shape = pav.make_shape(
            num_seqs=wl.num_seqs, num_q_heads=wl.num_q_heads, num_kv_heads=wl.num_kv_heads,
            head_dim=wl.head_dim, num_blocks=wl.num_blocks,
            max_blocks_per_seq=wl.max_blocks_per_seq, kv_dtype=wl.kv_dtype,
            out_dtype=wl.out_dtype, softmax_scale=wl.softmax_scale, sinks_mode=wl.sinks_mode,
            partition_tokens=partition_tokens or 0, lengths_are_bounds=1)
        win = None if wl.window is None else wl.window.tolist()
        plan = pav.pa_plan(shape, (wl.ctx_lens + bound_extra).tolist(), wl.q_lens.tolist(), win,
                           device=0)
        info = plan.info()
        kv = wl.kv_bytes()  # the bytes the actual lengths make visible
        lens_dev = wl.ctx_lens.to("cuda:0")
    # Rotating pool copies keep each call's KV out of the caches; `warm`
    # reuses one copy (the KV then sits in the 256 MiB Infinity Cache).
    copies = 1 if (warm or kv >= (1 << 30)) else int(math.ceil((1 << 30) / kv)) + 1
    pools = [(dev.k_pool, dev.v_pool, dev.k_scales, dev.v_scales)]
    for _ in range(copies - 1):
        pools.append(tuple(None if t is None else t.clone() for t in pools[0]))
    dt = torch.float32 if wl.out_dtype == "fp32" else torch.bfloat16
    out = torch.empty((wl.total_q, wl.num_q_heads, wl.head_dim), dtype=dt, device="cuda:0")
    s = torch.cuda.Stream()

    def call(i):
        kp, vp, ks, vs = pools[i % copies]
        if fused:
            pav.pa_decode_verify_fused(plan, lens_dev, dev.q, kp, vp, dev.block_table, ks, vs,
                                       dev.sinks, out, s)
        elif lens_dev is None:
            pav.pa_decode_verify(plan, dev.q, kp, vp, dev.block_table, ks, vs, dev.sinks, out, s)
        else:
            pav.pa_decode_verify_dev(plan, lens_dev, dev.q, kp, vp, dev.block_table, ks, vs,
                                     dev.sinks, out, s)

    ev_b = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ev_a = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        for i in range(warmup):
            call(i)
    torch.cuda.synchronize()

    mode = "hip-graph replay"
    g = None
    try:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            for i in range(steps):
                call(warmup + i)
        with torch.cuda.stream(s):
            g.replay()  # untimed: first replay
        torch.cuda.synchronize()
    except Exception as exc:  # pragma: no cover - depends on the runtime
        log(f"  graph capture unavailable ({exc}); timing eager calls")
        g = None
        mode = "eager launches"
        torch.cuda.synchronize()

    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    with torch.cuda.stream(s):
        t_start.record(s)
        if g is not None:
            g.replay()
        else:
            for i in range(steps):
                call(warmup + i)
        t_end.record(s)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0

    # The same calls launched one by one, with HIP events recorded around
    # every partition kernel on its stream (events inside a replayed graph
    # do not time the node they surround).
    with torch.cuda.stream(s):
        for e in ev_b + ev_a:
            e.record(s)  # creates the HIP events
    torch.cuda.synchronize()
    e0 = time.perf_counter()
    with torch.cuda.stream(s):
        for i in range(steps):
            pav.pa_set_partition_events(plan, ev_b[i], ev_a[i])
            call(i)
    torch.cuda.synchronize()
    eager = time.perf_counter() - e0
    pav.pa_set_partition_events(plan, None, None)
    part_ms = [b.elapsed_time(a) for b, a in zip(ev_b, ev_a)]
    # The streaming floor: the same plan's bytes through the same loads with
    # no compute (pa_stream_floor), timed the same way on the same copies.
    floor_ms = None
    if lens_dev is None and not fused:
        with torch.cuda.stream(s):
            for i in range(steps):
                kp, vp, ks, vs = pools[i % copies]
                pav.pa_set_partition_events(plan, ev_b[i], ev_a[i])
                pav.pa_stream_floor(plan, kp, vp, dev.block_table, ks, vs, s)
        torch.cuda.synchronize()
        pav.pa_set_partition_events(plan, None, None)
        floor_ms = [b.elapsed_time(a) for b, a in zip(ev_b, ev_a)]
    del g
    pav.pa_free(plan)
    return {
        "floor_ms_mean": None if floor_ms is None else statistics.fmean(floor_ms),
        "kv_bytes": kv,
        "copies": copies,
        "plan": info,
        "mode": mode,
        "wall_ms_per_step": 1e3 * wall / steps,
        "event_ms_per_step": t_start.elapsed_time(t_end) / steps,
        "eager_ms_per_step": 1e3 * eager / steps,
        "partition_ms_mean": statistics.fmean(part_ms),
        "partition_ms_median": statistics.median(part_ms),
        "partition_ms_p90": sorted(part_ms)[int(0.9 * (len(part_ms) - 1))],
    }


def measure_append(wl, steps: int, warmup: int):
    """Time pa_kv_append of the workload's new tokens (one call per step,
    `steps` calls in one replayed HIP graph, host clock around the replay).
    Returns the time per call and the call's algorithmic bytes: the bf16 K
    and V rows read plus the pool rows (and FP8 scales) written."""
    import torch

    import paged_kv_cache_verify_amd as pav

    dev = wl.to("cuda:0")
    plan = pav.plan_for(dev, device=0)
    T, Hkv, D = wl.total_q, wl.num_kv_heads, wl.head_dim
    gen = torch.Generator().manual_seed(wl.seed + 1)
    kn = torch.randn((T, Hkv, D), generator=gen).to(torch.bfloat16).to("cuda:0")
    vn = torch.randn((T, Hkv, D), generator=gen).to(torch.bfloat16).to("cuda:0")
    fp8 = wl.kv_dtype == "fp8"
    nbytes = 2 * T * Hkv * (2 * D + (D + 4 if fp8 else 2 * D))
    s = torch.cuda.Stream()

    def call():
        pav.pa_kv_append(plan, kn, vn, dev.block_table, dev.k_pool, dev.v_pool, dev.k_scales,
                         dev.v_scales, s)

    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        for _ in range(warmup):
            call()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for _ in range(steps):
            call()
    with torch.cuda.stream(s):
        g.replay()
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    with torch.cuda.stream(s):
        g.replay()
    torch.cuda.synchronize()
    us = 1e6 * (time.perf_counter() - w0) / steps
    del g
    pav.pa_free(plan)
    return {"us_per_call": round(us, 2), "bytes_per_call": nbytes,
            "GB_s": round(nbytes / (us * 1e-6) / 1e9, 1), "new_tokens": T,
            "timed_as": "hip-graph replay"}


def measure_verdict(q_lens, vocab: int, steps: int, warmup: int):
    """Time pa_verify_greedy over synthetic bf16 logits [T][vocab] (one call
    per step, `steps` calls in one replayed HIP graph). Returns the time per
    call and the logits bytes a call reads."""
    import torch

    import paged_kv_cache_verify_amd as pav

    B, T = len(q_lens), sum(q_lens)
    shape = pav.make_shape(num_seqs=B, num_q_heads=8, num_kv_heads=1, head_dim=128,
                           num_blocks=4 * B, max_blocks_per_seq=4, softmax_scale=0.125)
    plan = pav.pa_plan(shape, [max(q, 1) for q in q_lens], q_lens, None, device=0)
    gen = torch.Generator().manual_seed(77)
    logits = torch.randn((T, vocab), generator=gen).to(torch.bfloat16).to("cuda:0")
    ids = torch.randint(0, vocab, (T,), generator=gen, dtype=torch.int32).to("cuda:0")
    out = torch.empty((T,), dtype=torch.int32, device="cuda:0")
    acc = torch.empty((B,), dtype=torch.int32, device="cuda:0")
    nxt = torch.empty((B,), dtype=torch.int32, device="cuda:0")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        for _ in range(warmup):
            pav.pa_verify_greedy(plan, logits, ids, out, acc, nxt, s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for _ in range(steps):
            pav.pa_verify_greedy(plan, logits, ids, out, acc, nxt, s)
    with torch.cuda.stream(s):
        g.replay()
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    with torch.cuda.stream(s):
        g.replay()
    torch.cuda.synchronize()
    us = 1e6 * (time.perf_counter() - w0) / steps
    del g
    pav.pa_free(plan)
    nbytes = T * vocab * 2
    return {"us_per_call": round(us, 2), "logits_bytes_per_call": nbytes,
            "GB_s": round(nbytes / (us * 1e-6) / 1e9, 1), "rows": T, "vocab": vocab,
            "timed_as": "hip-graph replay (logits resident in the Infinity Cache)"}


def spacing_study(cfg: int, partition_tokens, steps: int):
    """Run the same calls of workload `cfg` four ways, each `steps` calls
    after a synchronisation: eager launches, one replayed HIP graph, and both
    again with a ~20 us spin (torch.cuda._sleep) after every call. Under
    `rocprofv3 --kernel-trace` the partition kernel's durations per phase
    show whether calls run back to back are slower than spaced ones. Prints
    the host time per phase; the kernel durations come from the trace."""
    import torch

    import paged_kv_cache_verify_amd as pav
    import workloads

    wl = workloads.make(cfg)
    dev = wl.to("cuda:0")
    plan = pav.plan_for(dev, device=0, partition_tokens=partition_tokens)
    kv = plan.info()["kv_bytes"]
    copies = 1 if kv >= (1 << 30) else int(math.ceil((1 << 30) / kv)) + 1
    pools = [(dev.k_pool, dev.v_pool, dev.k_scales, dev.v_scales)]
    for _ in range(copies - 1):
        pools.append(tuple(None if t is None else t.clone() for t in pools[0]))
    dt = torch.float32 if wl.out_dtype == "fp32" else torch.bfloat16
    out = torch.empty((wl.total_q, wl.num_q_heads, wl.head_dim), dtype=dt, device="cuda:0")
    s = torch.cuda.Stream()

    def call(i, spin):
        kp, vp, ks, vs = pools[i % copies]
        pav.pa_decode_verify(plan, dev.q, kp, vp, dev.block_table, ks, vs, dev.sinks, out, s)
        if spin:
            torch.cuda._sleep(50000)

    with torch.cuda.stream(s):
        for i in range(3):
            call(i, False)
    torch.cuda.synchronize()
    graphs = {}
    for spin in (False, True):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            for i in range(steps):
                call(i, spin)
        graphs[spin] = g
    torch.cuda.synchronize()
    res = {}
    for spin in (False, True):
        t0 = time.perf_counter()
        with torch.cuda.stream(s):
            for i in range(steps):
                call(i, spin)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        with torch.cuda.stream(s):
            graphs[spin].replay()
        torch.cuda.synchronize()
        t2 = time.perf_counter()
        tag = " + spin" if spin else ""
        res["eager" + tag] = round(1e6 * (t1 - t0) / steps, 2)
        res["graph" + tag] = round(1e6 * (t2 - t1) / steps, 2)
    pav.pa_free(plan)
    print(json.dumps({"spacing_study": wl.name, "steps": steps,
                      "phases_in_order": ["warm-up x3", "eager", "graph", "eager + spin",
                                          "graph + spin"],
                      "host_us_per_call": res}), flush=True)


def stamp_study(cfg: int, partition_tokens, calls: int = 8):
    """Per-workgroup phases of the partition kernel from its stamps
    (pa_set_workgroup_stamps), for the two-launch call and the fused call on
    the same plan: after `calls` calls on rotating pool copies, one stamped
    call of each. Prints one JSON line."""
    import numpy as np
    import torch

    import paged_kv_cache_verify_amd as pav
    import workloads

    wl = workloads.make(cfg)
    dev = wl.to("cuda:0")
    plan = pav.plan_for(dev, device=0, partition_tokens=partition_tokens)
    n = plan.info()["work_items"]
    kv = plan.info()["kv_bytes"]
    copies = 1 if kv >= (1 << 30) else int(math.ceil((1 << 30) / kv)) + 1
    pools = [(dev.k_pool, dev.v_pool, dev.k_scales, dev.v_scales)]
    for _ in range(copies - 1):
        pools.append(tuple(None if t is None else t.clone() for t in pools[0]))
    dt = torch.float32 if wl.out_dtype == "fp32" else torch.bfloat16
    out = torch.empty((wl.total_q, wl.num_q_heads, wl.head_dim), dtype=dt, device="cuda:0")
    st = torch.zeros((n, 8), dtype=torch.int64, device="cuda:0")
    res = {"workload": wl.name, "work_items": n,
           "partition_tokens": plan.info()["partition_tokens"],
           "unit": "us from the first workgroup's start"}
    for mode in ("two-launch", "fused"):
        for i in range(calls + 1):
            if i == calls:
                st.zero_()
                pav.pa_set_workgroup_stamps(plan, st)
            kp, vp, ks, vs = pools[i % copies]
            if mode == "fused":
                pav.pa_decode_verify_fused(plan, None, dev.q, kp, vp, dev.block_table, ks, vs,
                                           dev.sinks, out)
            else:
                pav.pa_decode_verify(plan, dev.q, kp, vp, dev.block_table, ks, vs, dev.sinks, out)
            torch.cuda.synchronize()
        pav.pa_set_workgroup_stamps(plan, None)
        t = st.cpu().numpy()
        T = (t[:, :7] - t[:, 0].min()) / 100.0
        done = np.where(t[:, :7] > 0, T, -1.0).max(axis=1)  # each workgroup's last stamp
        r = {"kernel_span_us": round(float(done.max()), 2),
             "last_start_us": round(float(T[:, 0].max()), 2),
             "chunk_loop_us_median": round(float(np.median(T[:, 1] - T[:, 0])), 2),
             "chunk_loop_us_max": round(float((T[:, 1] - T[:, 0]).max()), 2),
             "loop_end_us_max": round(float(T[:, 1].max()), 2)}
        grid = np.arange(0.0, done.max(), 10.0)
        r["active_workgroups_every_10us"] = [int(((T[:, 0] <= g) & (done > g)).sum()) for g in grid]
        # by the items' packed rows: keys, time from start to loop end, its
        # rate, and when the class's last workgroup finished
        items = plan.items()
        rows = np.array([it[6] for it in items])
        keys = np.array([it[3] - it[2] for it in items])
        loop = T[:, 1] - T[:, 0]
        by = {}
        for rv in np.unique(rows):
            m = rows == rv
            big = m & (keys >= 512)
            by[int(rv)] = {"items": int(m.sum()), "keys_median": int(np.median(keys[m])),
                           "start_to_loop_end_us_median": round(float(np.median(loop[m])), 2),
                           "ns_per_key_median": round(float(np.median(
                               1e3 * loop[big] / keys[big])), 2) if big.any() else None,
                           "done_us_max": round(float(done[m].max()), 2)}
        r["by_rows"] = by
        if mode == "fused":
            split = t[:, 3] > 0
            if split.any():
                r["split_items"] = int(split.sum())
                r["partial_stored_us_median"] = round(
                    float(np.median((T[:, 2] - T[:, 1])[split])), 2)
                r["arrival_us_median"] = round(float(np.median((T[:, 3] - T[:, 2])[split])), 2)
                xcc = (t[:, 7] >> 32) & 0xF
                for lv in range(3):
                    m = t[:, 4 + lv] > 0
                    if not m.any():
                        break
                    d = (T[:, 4 + lv] - T[:, 3 + lv])[m]
                    r[f"level{lv}_merges"] = {
                        "count": int(m.sum()), "us_median": round(float(np.median(d)), 2),
                        "us_max": round(float(d.max()), 2),
                        "per_xcc": np.bincount(xcc[m], minlength=8).tolist()}
        res[mode] = r
    pav.pa_free(plan)
    print(json.dumps({"stamp_study": res}), flush=True)


def cpu_baseline(wl, budget_s: float = 10.0):
    """The oracle as it stands, on the host cores, over the same workload."""
    import oracle

    threads = oracle.default_threads()
    times = []
    t_all = time.perf_counter()
    while True:
        t0 = time.perf_counter()
        oracle.verify(wl, threads=threads)
        times.append(time.perf_counter() - t0)
        if (time.perf_counter() - t_all > budget_s and len(times) >= 3) or len(times) >= 40:
            break
    per_call = statistics.median(times)
    return {
        "value": round(wl.kv_bytes() / per_call / 1e9, 4),
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": (f"the whole workload (all {wl.num_seqs} sequences), fp64 oracle, median of "
                   f"{len(times)} runs: {per_call:.2f} s per call; host "
                   f"{platform.processor() or platform.machine()}, os.cpu_count()="
                   f"{os.cpu_count()}"),
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--partition-tokens", type=int, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-single-launch", action="store_true",
                    help="skip timing pa_decode_verify_fused (kernel traces of one path)")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the FP8, long-context and mixed workloads")
    ap.add_argument("--only", type=int, default=None,
                    help="time just this workload (2..6) and print its figures")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (for counter scaling)")
    ap.add_argument("--spacing", type=int, default=None,
                    help="run the back-to-back vs spaced study on this workload and exit")
    ap.add_argument("--stamps", type=int, default=None,
                    help="print per-workgroup phases of the two-launch and fused calls on this "
                         "workload (with --partition-tokens) and exit")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU; --gpus {args.gpus} is not supported "
              "(the path would shard by KV head, by sequence or by context)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import workloads

    if not torch.cuda.is_available():
        print("bench.py needs an MI355X GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    if args.spacing is not None:
        spacing_study(args.spacing, args.partition_tokens, min(args.steps, 40))
        return
    if args.stamps is not None:
        stamp_study(args.stamps, args.partition_tokens)
        return

    if args.copy_calibration:
        src = torch.empty(1 << 28, dtype=torch.float32, device="cuda:0").fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("copy calibration: 3 x 1 GiB device copies done")
        del src, dst

    main_cfg = args.only or 2
    log(f"generating workload {main_cfg} ...")
    wl = workloads.make(main_cfg)
    log(f"  {wl.name}: L={wl.ctx_lens.tolist()} kv_bytes={wl.kv_bytes()}")
    r = measure(wl, args.steps, args.warmup, args.partition_tokens)
    ms = r["wall_ms_per_step"]
    value = r["kv_bytes"] / (ms * 1e-3) / 1e9
    achieved = r["kv_bytes"] / (r["partition_ms_mean"] * 1e-3) / 1e9
    log(f"  wall {1e3 * ms:.1f} us/step ({value:.0f} GB/s, {r['mode']}), events "
        f"{1e3 * r['event_ms_per_step']:.1f} us/step, partition kernel mean "
        f"{1e3 * r['partition_ms_mean']:.1f} us (median {1e3 * r['partition_ms_median']:.1f}, "
        f"p90 {1e3 * r['partition_ms_p90']:.1f}) = {achieved:.0f} GB/s, eager "
        f"{1e3 * r['eager_ms_per_step']:.1f} us/step; stream floor "
        f"{1e3 * r['floor_ms_mean']:.1f} us; "
        f"plan {r['plan']}, {r['copies']} pool copies")

    key = f"workload{main_cfg}"
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.kv_dtype == "bf16" else "fp8-e4m3 KV, bf16 Q",
        "data": "synthetic",
        "config": {
            "workload": f"{wl.name}, seed {wl.seed}",
            "kv_bytes_per_call": r["kv_bytes"],
            "us_per_call": round(1e3 * ms, 2),
            "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
            "timed_as": r["mode"],
            "us_per_call_eager_launches": round(1e3 * r["eager_ms_per_step"], 2),
            "partition_tokens": r["plan"]["partition_tokens"],
            "work_items": r["plan"]["work_items"],
            "pool_copies_rotated": r["copies"],
            "context_lens": wl.ctx_lens.tolist(),
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "pa_partition_kernel",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": load_traffic(key),
            "partition_us_mean": round(1e3 * r["partition_ms_mean"], 2),
            "partition_us_median": round(1e3 * r["partition_ms_median"], 2),
            "partition_us_p90": round(1e3 * r["partition_ms_p90"], 2),
        },
        "stream_floor": {
            "kernel": "pa_stream_floor_kernel (the plan's KV bytes, same loads, no compute)",
            "us_mean": round(1e3 * r["floor_ms_mean"], 2),
            "GB_s": round(r["kv_bytes"] / (r["floor_ms_mean"] * 1e-3) / 1e9, 1),
            "frac_of_peak": round(r["kv_bytes"] / (r["floor_ms_mean"] * 1e-3) / 1e9
                                  / HBM_PEAK_GBS, 4),
        },
    }
    # The same workload through the single-launch call (pa_decode_verify_fused).
    if not args.no_single_launch:
        rf = measure(wl, args.steps, args.warmup, args.partition_tokens, fused=True)
        log(f"  single launch: wall {1e3 * rf['wall_ms_per_step']:.1f} us/step, fused partition "
            f"kernel mean {1e3 * rf['partition_ms_mean']:.1f} us, eager "
            f"{1e3 * rf['eager_ms_per_step']:.1f} us/step")
        line["single_launch_call"] = {
            "entry_point": "pa_decode_verify_fused",
            "us_per_call": round(1e3 * rf["wall_ms_per_step"], 2),
            "GB_s": round(rf["kv_bytes"] / (rf["wall_ms_per_step"] * 1e-3) / 1e9, 1),
            "us_per_call_eager_launches": round(1e3 * rf["eager_ms_per_step"], 2),
            "kernel_us_mean": round(1e3 * rf["partition_ms_mean"], 2),
            "kernel_us_median": round(1e3 * rf["partition_ms_median"], 2),
        }
    if args.only is None:
        # The same calls on one pool copy: the KV stays in the Infinity Cache
        # between calls, so this is not an HBM figure.
        rw = measure(wl, max(20, args.steps // 4), max(5, args.warmup // 4), args.partition_tokens,
                     warm=True)
        line["config"]["us_per_call_warm_cache_resident"] = round(1e3 * rw["wall_ms_per_step"], 2)

    if not args.no_extra and args.only is None:
        extra = {}
        for cfg, P in ((3, None), (5, None), (4, 512), (4, 0)):
            wlx = workloads.make(cfg)
            log(f"workload {cfg}, partition {P or 'auto'}: {wlx.name}")
            rx = measure(wlx, max(20, args.steps // 4), max(5, args.warmup // 4), P)
            msx = rx["wall_ms_per_step"]
            gbs = rx["kv_bytes"] / (msx * 1e-3) / 1e9
            ach = rx["kv_bytes"] / (rx["partition_ms_mean"] * 1e-3) / 1e9
            log(f"  {1e3 * msx:.1f} us/call = {gbs:.0f} GB/s ({rx['mode']}); partition kernel "
                f"{1e3 * rx['partition_ms_mean']:.1f} us = {ach:.0f} GB/s; eager "
                f"{1e3 * rx['eager_ms_per_step']:.1f} us/call; stream floor "
                f"{1e3 * rx['floor_ms_mean']:.1f} us; plan {rx['plan']}")
            extra[f"workload {cfg}" + ("" if P is None else f" (partition {P or 'auto'})")] = {
                "us_per_call": round(1e3 * msx, 2),
                "us_per_call_eager_launches": round(1e3 * rx["eager_ms_per_step"], 2),
                "GB_s": round(gbs, 1),
                "pct_of_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
                "partition_kernel_GB_s": round(ach, 1),
                "stream_floor_GB_s": round(rx["kv_bytes"] / (rx["floor_ms_mean"] * 1e-3) / 1e9,
                                           1),
                "kv_bytes_per_call": rx["kv_bytes"],
                "work_items": rx["plan"]["work_items"],
                "partition_tokens": rx["plan"]["partition_tokens"],
            }
            rfx = measure(wlx, max(20, args.steps // 4), max(5, args.warmup // 4), P, fused=True)
            log(f"  single launch: {1e3 * rfx['wall_ms_per_step']:.1f} us/call; fused kernel "
                f"{1e3 * rfx['partition_ms_mean']:.1f} us")
            extra[f"workload {cfg}" + ("" if P is None else f" (partition {P or 'auto'})")].update(
                us_per_call_single_launch=round(1e3 * rfx["wall_ms_per_step"], 2),
                single_launch_kernel_us=round(1e3 * rfx["partition_ms_mean"], 2))
            if cfg in (3,) and P is None:
                ra = measure_append(wlx, max(50, args.steps), max(5, args.warmup // 4))
                log(f"  kv append of the {ra['new_tokens']} new tokens (FP8 quantise): "
                    f"{ra['us_per_call']} us/call = {ra['GB_s']} GB/s")
                extra[f"kv append, workload {cfg} shape (per-token FP8 quantise)"] = ra
            del wlx
        # The head-256 FP8 shape of the pages' kernel microbenchmark (8 q /
        # 1 KV head, q 6 = 48 rows, 150,000-token contexts), batch 1/2/4/8,
        # next to the per-layer times the pages print for it on MI355X.
        pages_us = {1: (72.3, 59.4), 2: (74.2, 61.5), 4: (85.7, 68.5), 8: (142.6, 116.7)}
        log("workload 6: generating the head-256 FP8 batch ...")
        wl6 = workloads.make(6)
        for bs in (1, 2, 4, 8):
            wlb = workloads.first_seqs(wl6, bs)
            rx = measure(wlb, max(20, args.steps // 4), max(5, args.warmup // 4))
            msx = rx["wall_ms_per_step"]
            gbs = rx["kv_bytes"] / (msx * 1e-3) / 1e9
            ach = rx["kv_bytes"] / (rx["partition_ms_mean"] * 1e-3) / 1e9
            log(f"  batch {bs}: {1e3 * msx:.1f} us/call = {gbs:.0f} GB/s; partition kernel "
                f"{1e3 * rx['partition_ms_mean']:.1f} us = {ach:.0f} GB/s; pages: "
                f"{pages_us[bs][0]} us generic, {pages_us[bs][1]} us pipe; plan {rx['plan']}")
            extra[f"workload 6, batch {bs} (head 256, FP8, 48 rows, 150k context)"] = {
                "us_per_call": round(1e3 * msx, 2),
                "us_per_call_eager_launches": round(1e3 * rx["eager_ms_per_step"], 2),
                "GB_s": round(gbs, 1),
                "pct_of_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
                "partition_kernel_GB_s": round(ach, 1),
                "stream_floor_GB_s": round(rx["kv_bytes"] / (rx["floor_ms_mean"] * 1e-3) / 1e9,
                                           1),
                "kv_bytes_per_call": rx["kv_bytes"],
                "work_items": rx["plan"]["work_items"],
                "pages_us_generic_kernel": pages_us[bs][0],
                "pages_us_tuned_pipe": pages_us[bs][1],
            }
            del wlb
        del wl6
        # The headline workload through the device-length call: a plan built
        # on bounds 64 tokens past every length, the lengths read at run time.
        wlb = workloads.make(main_cfg, extra_max_blocks=5)
        rb = measure(wlb, max(20, args.steps // 4), max(5, args.warmup // 4), bound_extra=64)
        msb = rb["wall_ms_per_step"]
        log(f"workload {main_cfg}, lengths read on the device (plan on bounds +64): "
            f"{1e3 * msb:.1f} us/call; partition kernel {1e3 * rb['partition_ms_mean']:.1f} us")
        extra[f"workload {main_cfg}, lengths read on the device (plan on bounds L + 64)"] = {
            "us_per_call": round(1e3 * msb, 2),
            "GB_s": round(rb["kv_bytes"] / (msb * 1e-3) / 1e9, 1),
            "partition_kernel_us": round(1e3 * rb["partition_ms_mean"], 2),
            "work_items": rb["plan"]["work_items"],
        }
        del wlb
        rv = measure_verdict([6] * 8, 131072, max(50, args.steps), max(5, args.warmup // 4))
        log(f"greedy verdict, 8 x 6 verify rows over a 131,072-entry vocabulary (bf16 logits): "
            f"{rv['us_per_call']} us/call = {rv['GB_s']} GB/s")
        extra["greedy verdict, 8 sequences x 6 rows, vocab 131072, bf16 logits"] = rv
        ra = measure_append(wl, max(50, args.steps), max(5, args.warmup // 4))
        log(f"kv append of workload {main_cfg}'s {ra['new_tokens']} new tokens (bf16): "
            f"{ra['us_per_call']} us/call = {ra['GB_s']} GB/s")
        extra[f"kv append, workload {main_cfg} shape (bf16 copy)"] = ra
        line["other_workloads"] = extra

    if not args.no_cpu_baseline and args.only is None:
        log("timing the CPU oracle ...")
        line["cpu_baseline"] = cpu_baseline(wl)
        log(f"  {line['cpu_baseline']}")

    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
