#!/usr/bin/env python3
"""Dispatch + combine throughput of libep.so on one MI355X.

One step is one pass of the whole hot path over one batch of synthetic
input already resident in HBM:
    ep_get_dispatch_layout -> ep_dispatch -> ep_combine -> ep_dispatch_fp8
with the combine fed the dispatched rows (identity experts).  Extra phases,
reported beside the headline and not part of it: the rank-deduplicated pair
ep_dispatch_ht -> ep_combine (unweighted, over the per-rank rows), the padded
expert-major (low-latency) layout ep_dispatch_ll -> ep_combine (over the slot
map) -> ep_dispatch_ll_fp8 with the capacity set to the busiest expert's load
rounded up to 64 rows (nothing dropped), ep_dispatch_cached (the copy
kernel alone, reusing token_row) and ep_dispatch_fp8_cached (the FP8 cast and
copy alone).  Before each
phase (outside its events) a 512 MiB write followed by a 512 MiB read of
another buffer evicts L2 and the 256 MB Infinity Cache: the phase's inputs
are then only in HBM and the caches hold clean, unrelated lines, so no
write-back of earlier data lands inside a timed phase.  This stands in for
the expert computation that separates dispatch from combine in a model.

Each phase is bracketed by HIP events recorded on the stream the kernels are
launched on (torch's current stream, which the binding passes to the C ABI).
The headline `value` is

    (algorithmic bytes of ep_dispatch + ep_combine) / (t_dispatch + t_combine)

in GB/s, summed over the timed steps, and `ms_per_step` is that
t_dispatch + t_combine per step; the layout and FP8 dispatch of each step are
timed as phases of their own.  Secondary figures: `full_path` adds the layout
call, and `payload_convention` counts bytes as the pages' own benchmark does
(one bf16 row per dispatched (token, expert) pair in each direction, over the
same times).  `roofline` reports the combine kernel (one kernel per
ep_combine call) against the 8 TB/s HBM3E peak; `traffic` comes from
committed rocprofv3 FETCH_SIZE / WRITE_SIZE counters when they were taken on
the current kernel source, else null.  `cpu_baseline` times the C oracle
(single thread) on the same workload on this host.  `per_config` then repeats
the measurement (fewer steps) on each of the five workloads -- tiny, dsv3,
skewed, ll_fp8, large -- each with its own oracle timing on this host.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload dsv3]
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "dispatch+combine effective GB/s and % of HBM peak at T=4096,H=7168,k=8"
HBM_PEAK_GBS = 8000.0
FLUSH_BYTES = 512 << 20           # written, then as much again read
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "combine_dsv3_traffic.json")
# The combine kernel is defined by these two sources; counters taken on other
# versions of them are not reported.
COMBINE_SRCS = [os.path.join(ROOT, "combine_get_dispatch_02_amd", "csrc", f)
                for f in ("combine.hip", "ep_device.h")]


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def ht_rows(wl, idx):
    """Rows of the rank-deduplicated dispatch: one per (token, rank it reaches)."""
    import numpy as np
    valid = (idx >= 0) & (idx < wl.E)
    hit = np.zeros((wl.T, wl.R), dtype=bool)
    t, j = np.nonzero(valid)
    hit[t, idx[t, j] // (wl.E // wl.R)] = True
    return int(hit.sum())


def ll_capacity(wl, idx):
    """Capacity that drops nothing: the busiest expert's load rounded up to a
    multiple of 64 rows, the M-tile of a grouped GEMM over [capacity, H]."""
    import numpy as np
    valid = idx[(idx >= 0) & (idx < wl.E)]
    busiest = int(np.bincount(valid, minlength=wl.E).max()) if valid.size else 1
    return (max(busiest, 1) + 63) // 64 * 64


def algorithmic_bytes(wl, n_ht=None, n_ll=None):
    """Bytes each call must move at least (read once, write once)."""
    T, H, k, E, R, G = wl.T, wl.H, wl.k, wl.E, wl.R, wl.G
    N = T * k
    n = T * R if n_ht is None else n_ht
    m = N if n_ll is None else n_ll                                  # slots kept by the padded layout
    ht_maps = 4 * T * R + 4 * n + 8 * n * k + 4 * n * k + 4 * (R + 1)   # token_rank_row, src, ids, w
    maps = 4 * N + 4 * N + 4 * T * k + 4 * (E + 1) + 4 * (R + 1)   # src, recv_w, token_row, offsets
    reads = 8 * T * k + 4 * T * k                                  # topk_idx, topk_weights
    return dict(
        layout=8 * T * k + T * R + 4 * (E + R + G),
        dispatch=reads + 2 * T * H + 2 * N * H + maps,
        dispatch_fp8=reads + 2 * T * H + N * H + 4 * N * (H // 128) + maps,
        combine=4 * T * k + 4 * T * k + 2 * N * H + 2 * T * H,
        # the copy alone, driven by a saved token_row (x read, rows written, map read)
        dispatch_cached=2 * T * H + 2 * N * H + 4 * T * k,
        # the FP8 cast-and-copy alone (x read, codes and scales written, map read)
        dispatch_fp8_cached=2 * T * H + N * H + 4 * N * (H // 128) + 4 * T * k,
        dispatch_ht=8 * T * k + 4 * T * k + 2 * T * H + 2 * n * H + ht_maps,
        combine_ht=4 * T * R + 2 * n * H + 2 * T * H,
        # padded layout, m slots kept: token_slot, src and weight per kept
        # slot, the E counts
        dispatch_ll=reads + 2 * T * H + 2 * m * H + 4 * T * k + 8 * m + 4 * E,
        combine_ll=4 * T * k + 4 * T * k + 2 * m * H + 2 * T * H,
        dispatch_ll_fp8=reads + 2 * T * H + m * H + 4 * m * (H // 128) + 4 * T * k + 8 * m + 4 * E,
    )


def sources_sha256(paths):
    h = hashlib.sha256()
    for path in paths:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def load_traffic(per_launch_alg_bytes):
    """Counter-derived HBM bytes of one combine launch, if taken on this source."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as f:
        t = json.load(f)
    if t.get("kernel_source_sha256") != sources_sha256(COMBINE_SRCS):
        return None
    return t.get("hbm_bytes_per_launch")


def cpu_baseline(wl, x, idx, w, budget_s):
    """Single-threaded C oracle on the same workload: dispatch + combine
    (identity experts), repeated until the time budget is used."""
    import ctypes

    import numpy as np
    import oracle

    L = oracle._load()
    T, H, k, E, R = wl.T, wl.H, wl.k, wl.E, wl.R
    N = T * k
    recv = np.empty((N, H), np.uint16)
    src = np.empty(N, np.int32)
    rw = np.empty(N, np.float32)
    eoff = np.empty(E + 1, np.int32)
    roff = np.empty(R + 1, np.int32)
    trow = np.empty((T, k), np.int32)
    out = np.empty((T, H), np.uint16)
    G = wl.G
    per_rank = np.empty(R, np.int32)
    per_group = np.empty(G, np.int32)
    per_expert = np.empty(E, np.int32)
    in_rank = np.empty((T, R), np.uint8)
    p = lambda a: a.ctypes.data_as(ctypes.c_void_p)  # noqa: E731
    t_d = t_c = t_l = 0.0
    passes = 0
    t_start = time.perf_counter()
    while passes == 0 or time.perf_counter() - t_start < budget_s:
        t0 = time.perf_counter()
        rc = L.oracle_dispatch(p(x), p(idx), p(w), T, H, k, E, R, p(recv), p(src), p(rw), p(eoff),
                               p(roff), p(trow))
        t1 = time.perf_counter()
        rc |= L.oracle_combine(p(recv), N, p(trow), p(w), T, H, k, p(out))
        t2 = time.perf_counter()
        rc |= L.oracle_layout(p(idx), T, k, E, R, wl.P, p(per_rank), p(per_group), p(per_expert),
                              p(in_rank))
        t3 = time.perf_counter()
        if rc:
            raise RuntimeError("oracle failed")
        t_d += t1 - t0
        t_c += t2 - t1
        t_l += t3 - t2
        passes += 1
    # The FP8 oracle encodes by a search over the code table: timed on the
    # first 64 tokens only and reported per token.
    ts = min(T, 64)
    ns = ts * k
    q8 = np.empty((ns, H), np.uint8)
    s8 = np.empty((ns, H // 128), np.float32)
    src8, rw8 = np.empty(ns, np.int32), np.empty(ns, np.float32)
    eoff8, roff8, trow8 = np.empty(E + 1, np.int32), np.empty(R + 1, np.int32), np.empty((ts, k), np.int32)
    x8, idx8, w8 = (np.ascontiguousarray(a[:ts]) for a in (x, idx, w))
    t4 = time.perf_counter()
    if L.oracle_dispatch_fp8(p(x8), p(idx8), p(w8), ts, H, k, E, R, p(q8), p(s8), p(src8), p(rw8),
                             p(eoff8), p(roff8), p(trow8)):
        raise RuntimeError("oracle failed")
    fp8_us_per_token = 1e6 * (time.perf_counter() - t4) / ts
    b = algorithmic_bytes(wl)
    gbs = (b["dispatch"] + b["combine"]) * passes / (t_d + t_c) / 1e9
    # All cores: the same oracle combine called on disjoint token ranges from
    # one thread per available core (ctypes releases the GIL during the call);
    # dispatch stays one call (its counting sort is sequential by definition).
    from concurrent.futures import ThreadPoolExecutor
    threads = max(1, len(os.sched_getaffinity(0)))
    bounds = [T * i // threads for i in range(threads + 1)]

    def part(i):
        t0_, t1_ = bounds[i], bounds[i + 1]
        if t1_ <= t0_:
            return 0
        return L.oracle_combine(p(recv), N, p(trow[t0_:]), p(w[t0_:]), t1_ - t0_, H, k, p(out[t0_:]))

    out_ref = out.copy()
    reps, t_par = 0, 0.0
    with ThreadPoolExecutor(max_workers=threads) as pool:
        t_start = time.perf_counter()
        while reps == 0 or time.perf_counter() - t_start < max(1.0, budget_s / 5):
            t5 = time.perf_counter()
            if any(pool.map(part, range(threads))):
                raise RuntimeError("oracle failed")
            t_par += time.perf_counter() - t5
            reps += 1
    if not np.array_equal(out, out_ref):
        raise RuntimeError("threaded oracle combine differs from the single-threaded one")
    par_combine_s = t_par / reps
    gbs_all = (b["dispatch"] + b["combine"]) / (t_d / passes + par_combine_s) / 1e9
    try:
        model = next(l.split(":", 1)[1].strip() for l in open("/proc/cpuinfo") if l.startswith("model name"))
    except Exception:
        model = "unknown"
    return {
        "value": round(gbs, 3),
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "sample": (f"{wl.describe()}: {passes} full passes of oracle dispatch + combine (+ layout) "
                   f"(identity experts), {t_d + t_c:.1f} s, 1 thread"),
        "dispatch_ms": round(1e3 * t_d / passes, 2),
        "combine_ms": round(1e3 * t_c / passes, 2),
        "layout_ms": round(1e3 * t_l / passes, 3),
        "dispatch_fp8_us_per_token": round(fp8_us_per_token, 1),
        "dispatch_fp8_note": f"timed on the first {ts} tokens (the FP8 oracle searches the code table)",
        "host_cores_available": len(os.sched_getaffinity(0)),
        "host_cpu": model,
        "all_cores": {"value": round(gbs_all, 3), "unit": "GB/s", "cores": threads,
                      "combine_ms": round(1e3 * par_combine_s, 2),
                      "note": "oracle combine split over token ranges, one thread per available "
                              "core; oracle dispatch single-threaded as above"},
    }


def oracle_entry(cpu):
    """The per-workload part of a cpu_baseline record."""
    return {"GBps": cpu["value"], "cores": cpu["cores"], "dispatch_ms": cpu["dispatch_ms"],
            "combine_ms": cpu["combine_ms"], "layout_ms": cpu["layout_ms"],
            "dispatch_fp8_us_per_token": cpu["dispatch_fp8_us_per_token"], "sample": cpu["sample"],
            "all_cores_GBps": cpu["all_cores"]["value"], "all_cores_threads": cpu["all_cores"]["cores"]}


def graph_mode(args, wl, ep, torch, np, idxd, xd, wd, lay, ws_l, disp, ws_d, comb, fp8):
    """Eager vs HIP-graph replay of one whole step, caches left warm."""
    E, R, P, N = wl.E, wl.R, wl.P, wl.T * wl.k

    def body():
        ep.ep_get_dispatch_layout(idxd, E, R, P, out=lay, workspace=ws_l)
        ep.ep_dispatch(xd, idxd, wd, E, R, out=disp, workspace=ws_d)
        ep.ep_combine(disp["recv_x"], disp["token_row"], wd, num_rows=N, out=comb)
        ep.ep_dispatch_fp8(xd, idxd, wd, E, R, out=fp8, workspace=ws_d)

    for _ in range(max(args.warmup, 3)):
        body()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            body()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()

    def timed(fn):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(args.steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return 1e3 * e0.elapsed_time(e1) / args.steps

    eager_us = timed(body)
    graph_us = timed(g.replay)
    print(json.dumps({"mode": "graph", "workload": wl.describe(), "steps": args.steps,
                      "eager_us_per_step": round(eager_us, 2), "graph_us_per_step": round(graph_us, 2),
                      "speedup": round(eager_us / graph_us, 3),
                      "note": "layout + dispatch + combine + FP8 dispatch back to back, caches warm"}),
          flush=True)


def drain_check(args, wl, ep, torch, np, idxd, xd, wd, disp, ws_d, comb, flush):
    """Whether a timed phase leaves write-backs for later: each of ep_dispatch
    and ep_combine is timed alone, then followed inside the same events by a
    512 MiB read of unrelated memory, which is also timed alone.  If the
    phase's stores were still in the caches at its end event, the read would
    have to write them back and the pair would take longer than the two
    parts."""
    N = wl.T * wl.k
    drain = torch.ones(64 << 20, dtype=torch.int64, device=xd.device)

    def timed(fn):
        ts = []
        for i in range(args.warmup + args.steps):
            flush(i)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            if i >= args.warmup:
                ts.append(a.elapsed_time(b) * 1e3)
        return float(np.median(ts))

    def d():
        ep.ep_dispatch(xd, idxd, wd, wl.E, wl.R, out=disp, workspace=ws_d)

    def c():
        ep.ep_combine(disp["recv_x"], disp["token_row"], wd, num_rows=N, out=comb)

    r = timed(lambda: drain.sum())
    res = {"mode": "drain_check", "workload": wl.describe(), "steps": args.steps,
           "read_512MiB_us": round(r, 2)}
    for name, fn in (("ep_dispatch", d), ("ep_combine", c)):
        t1 = timed(fn)
        t2 = timed(lambda: (fn(), drain.sum()))
        res[name] = {"alone_us": round(t1, 2), "then_read_us": round(t2, 2),
                     "deferred_us": round(t2 - r - t1, 2)}
    print(json.dumps(res), flush=True)


def scatter_check(args, wl, ep, torch, np, xd, disp, fp8, cached, cached8, flush):
    """The copy kernels alone (ep_dispatch_cached / ep_dispatch_fp8_cached),
    caches evicted before each call, on the real receive map and on an
    identity map that sends token t's slots to rows t*k .. t*k+k-1: the same
    bytes read and written, but one sequential write stream instead of one
    per expert."""
    T, k = wl.T, wl.k
    N = T * k
    ident = torch.arange(N, dtype=torch.int32, device=xd.device).view(T, k)

    def timed(fn):
        ts = []
        for i in range(args.warmup + args.steps):
            flush(i)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            if i >= args.warmup:
                ts.append(a.elapsed_time(b) * 1e3)
        return round(float(np.median(ts)), 2)

    res = {"mode": "scatter_check", "workload": wl.describe(), "steps": args.steps}
    for name, fn in (("bf16", lambda m: ep.ep_dispatch_cached(xd, m, N, out=cached)),
                     ("fp8", lambda m: ep.ep_dispatch_fp8_cached(xd, m, N, out=cached8))):
        for mname, m in (("real_map", disp["token_row"]), ("identity_map", ident)):
            res[f"{name}_{mname}_us"] = timed(lambda: fn(m))
    print(json.dumps(res), flush=True)


# Steps of the per-workload measurements that follow the headline (latency-
# bound batches take more steps: each costs a few microseconds).
PER_CONFIG_STEPS = {"tiny": 1000, "ll_fp8": 1000}
PER_CONFIG_DEFAULT_STEPS = 100
PER_CONFIG_WARMUP = 5
PER_CONFIG_CPU_SECONDS = 2.0


def measure(wl, steps, warmup, args, ep, torch, np, mode=None):
    """Time every phase of `steps` steps of workload wl (after `warmup`
    untimed steps).  Returns the phase times (ms arrays), algorithmic bytes
    and derived figures; with mode = "graph" / "drain" / "scatter" it runs that
    measurement instead and returns None."""
    from combine_get_dispatch_02_amd.workloads import make_workload

    dev = torch.device("cuda:0")
    x, idx, w = make_workload(wl)
    xd = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev)
    idxd = torch.from_numpy(idx).to(dev)
    wd = torch.from_numpy(w).to(dev)
    T, H, k, E, R, P, G = wl.T, wl.H, wl.k, wl.E, wl.R, wl.P, wl.G
    N = T * k

    # All outputs and workspaces allocated once, outside the timed region.
    lay = dict(num_tokens_per_rank=torch.empty(R, dtype=torch.int32, device=dev),
               num_tokens_per_group=torch.empty(G, dtype=torch.int32, device=dev),
               num_tokens_per_expert=torch.empty(E, dtype=torch.int32, device=dev),
               is_token_in_rank=torch.empty((T, R), dtype=torch.uint8, device=dev))
    ws_l = torch.empty(ep.ep_layout_workspace_bytes(T, E, R, P), dtype=torch.uint8, device=dev)

    def maps():
        return dict(recv_src_idx=torch.empty(N, dtype=torch.int32, device=dev),
                    recv_topk_weights=torch.empty(N, dtype=torch.float32, device=dev),
                    recv_expert_offset=torch.empty(E + 1, dtype=torch.int32, device=dev),
                    recv_rank_offset=torch.empty(R + 1, dtype=torch.int32, device=dev),
                    token_row=torch.empty((T, k), dtype=torch.int32, device=dev))
    disp = maps()
    disp["recv_x"] = torch.empty((N, H), dtype=torch.bfloat16, device=dev)
    fp8 = maps()
    fp8["recv_x_fp8"] = torch.empty((N, H), dtype=torch.uint8, device=dev)
    fp8["recv_scales"] = torch.empty((N, H // 128), dtype=torch.float32, device=dev)
    ws_d = torch.empty(ep.ep_dispatch_workspace_bytes(T, k, E), dtype=torch.uint8, device=dev)
    comb = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    n_ht = ht_rows(wl, idx)
    cap_ht = T * R
    ht = dict(recv_x=torch.empty((cap_ht, H), dtype=torch.bfloat16, device=dev),
              recv_src_idx=torch.empty(cap_ht, dtype=torch.int32, device=dev),
              recv_topk_idx=torch.empty((cap_ht, k), dtype=torch.int64, device=dev),
              recv_topk_weights=torch.empty((cap_ht, k), dtype=torch.float32, device=dev),
              recv_rank_offset=torch.empty(R + 1, dtype=torch.int32, device=dev),
              token_rank_row=torch.empty((T, R), dtype=torch.int32, device=dev))
    ws_ht = torch.empty(ep.ep_dispatch_ht_workspace_bytes(T, R), dtype=torch.uint8, device=dev)
    comb_ht = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    cap_ll = args.ll_capacity or ll_capacity(wl, idx)
    n_ll = int(np.minimum(np.bincount(idx[(idx >= 0) & (idx < E)], minlength=E), cap_ll).sum())
    ll = dict(recv_x=torch.empty((E, cap_ll, H), dtype=torch.bfloat16, device=dev),
              recv_count=torch.empty(E, dtype=torch.int32, device=dev),
              recv_src_idx=torch.empty((E, cap_ll), dtype=torch.int32, device=dev),
              recv_topk_weights=torch.empty((E, cap_ll), dtype=torch.float32, device=dev),
              token_slot=torch.empty((T, k), dtype=torch.int32, device=dev))
    ll8 = dict(recv_x_fp8=torch.empty((E, cap_ll, H), dtype=torch.uint8, device=dev),
               recv_scales=torch.empty((E, cap_ll, H // 128), dtype=torch.float32, device=dev),
               recv_count=torch.empty(E, dtype=torch.int32, device=dev),
               recv_src_idx=torch.empty((E, cap_ll), dtype=torch.int32, device=dev),
               recv_topk_weights=torch.empty((E, cap_ll), dtype=torch.float32, device=dev),
               token_slot=torch.empty((T, k), dtype=torch.int32, device=dev))
    ws_ll = torch.empty(ep.ep_dispatch_ll_workspace_bytes(T, k, E), dtype=torch.uint8, device=dev)
    comb_ll = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    cached = torch.empty((N, H), dtype=torch.bfloat16, device=dev)
    cached8 = dict(recv_x_fp8=torch.empty((N, H), dtype=torch.uint8, device=dev),
                   recv_scales=torch.empty((N, H // 128), dtype=torch.float32, device=dev))
    flush_buf = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)
    flush_src = torch.ones(FLUSH_BYTES // 8, dtype=torch.int64, device=dev)

    def flush(i):
        if not args.no_flush:
            flush_buf.fill_(i & 0xFF)
            flush_src.sum()

    calls = [
        ("layout", lambda: ep.ep_get_dispatch_layout(idxd, E, R, P, out=lay, workspace=ws_l)),
        ("dispatch", lambda: ep.ep_dispatch(xd, idxd, wd, E, R, out=disp, workspace=ws_d)),
        ("combine", lambda: ep.ep_combine(disp["recv_x"], disp["token_row"], wd, num_rows=N, out=comb)),
        ("dispatch_fp8", lambda: ep.ep_dispatch_fp8(xd, idxd, wd, E, R, out=fp8, workspace=ws_d)),
        ("dispatch_ht", lambda: ep.ep_dispatch_ht(xd, idxd, wd, E, R, out=ht, workspace=ws_ht)),
        ("combine_ht", lambda: ep.ep_combine(ht["recv_x"], ht["token_rank_row"], None, num_rows=n_ht,
                                             out=comb_ht)),
        ("dispatch_ll", lambda: ep.ep_dispatch_ll(xd, idxd, wd, E, cap_ll, out=ll, workspace=ws_ll)),
        ("combine_ll", lambda: ep.ep_combine(ll["recv_x"].view(E * cap_ll, H), ll["token_slot"], wd,
                                             out=comb_ll)),
        ("dispatch_ll_fp8", lambda: ep.ep_dispatch_ll_fp8(xd, idxd, wd, E, cap_ll, out=ll8,
                                                          workspace=ws_ll)),
        ("dispatch_cached", lambda: ep.ep_dispatch_cached(xd, disp["token_row"], N, out=cached)),
        ("dispatch_fp8_cached", lambda: ep.ep_dispatch_fp8_cached(xd, fp8["token_row"], N, out=cached8)),
    ]
    phases = [name for name, _ in calls]

    if mode == "graph":
        graph_mode(args, wl, ep, torch, np, idxd, xd, wd, lay, ws_l, disp, ws_d, comb, fp8)
        return None
    if mode == "drain":
        drain_check(args, wl, ep, torch, np, idxd, xd, wd, disp, ws_d, comb, flush)
        return None
    if mode == "scatter":
        ep.ep_dispatch(xd, idxd, wd, E, R, out=disp, workspace=ws_d)
        ep.ep_dispatch_fp8(xd, idxd, wd, E, R, out=fp8, workspace=ws_d)
        scatter_check(args, wl, ep, torch, np, xd, disp, fp8, cached, cached8, flush)
        return None

    def step(i, ev):
        # every phase starts from evicted caches; its events bracket only its call
        for p_i, (_, fn) in enumerate(calls):
            flush(i + p_i)
            ev[2 * p_i].record()
            fn()
            ev[2 * p_i + 1].record()

    def events():
        return [torch.cuda.Event(enable_timing=True) for _ in range(2 * len(calls))]

    for i in range(warmup):
        step(i, events())
    torch.cuda.synchronize()
    if disp["recv_expert_offset"][-1].item() != N:
        raise RuntimeError("dispatch filled an unexpected number of rows")
    if ht["recv_rank_offset"][-1].item() != n_ht:
        raise RuntimeError("rank-deduplicated dispatch filled an unexpected number of rows")
    if ll["recv_count"].sum().item() != n_ll or ll8["recv_count"].sum().item() != n_ll:
        raise RuntimeError("padded dispatch filled an unexpected number of slots")

    evs = [events() for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = {p: np.array([e[2 * i].elapsed_time(e[2 * i + 1]) for e in evs]) for i, p in enumerate(phases)}

    res = dict(wl=wl, x=x, idx=idx, w=w, ms=ms, wall=wall, steps=steps, n_ht=n_ht, cap_ll=cap_ll,
               n_ll=n_ll, B=algorithmic_bytes(wl, n_ht, n_ll), phases=phases)
    if mode == "headline":
        # Secondary: the same dispatch and combine with warm caches (no eviction).
        warm_ev = []
        for i in range(max(steps // 5, 5)):
            e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
            e[0].record()
            calls[1][1]()
            e[1].record()
            calls[2][1]()
            e[2].record()
            warm_ev.append(e)
        torch.cuda.synchronize()
        res["warm_d"] = np.array([e[0].elapsed_time(e[1]) for e in warm_ev[1:]]) * 1e3
        res["warm_c"] = np.array([e[1].elapsed_time(e[2]) for e in warm_ev[1:]]) * 1e3
        if args.calibration_copy:
            cal_src = torch.empty(256 << 20, dtype=torch.uint8, device=dev).fill_(1)
            cal_dst = torch.empty_like(cal_src)
            torch.cuda.synchronize()
            for _ in range(4):
                cal_dst.copy_(cal_src)
            torch.cuda.synchronize()
        # An event pair with nothing between it, after the same eviction: the
        # part of every phase time that is the events' own cost, not the kernel's.
        empty = []
        for i in range(20):
            flush(i)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            b.record()
            torch.cuda.synchronize()
            empty.append(a.elapsed_time(b) * 1e3)
        res["pair_us"] = float(np.median(empty))
    return res


def phase_summary(res, np):
    """Per phase: mean / median / p10 / p90 event time, algorithmic bytes,
    GB/s and fraction of the HBM peak."""
    out = {}
    for p in res["phases"]:
        us = res["ms"][p] * 1e3
        gbs = res["B"][p] / (us.mean() * 1e-6) / 1e9
        out[p] = {"us_mean": round(float(us.mean()), 2), "us_median": round(float(np.median(us)), 2),
                  "us_p10": round(float(np.percentile(us, 10)), 2),
                  "us_p90": round(float(np.percentile(us, 90)), 2),
                  "alg_bytes": int(res["B"][p]), "GBps": round(gbs, 1),
                  "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)}
    return out


def pair_gbs(res, a, b):
    """Algorithmic bytes of phases a + b over their summed event times (GB/s)."""
    t = float(res["ms"][a].sum() + res["ms"][b].sum()) / 1e3
    return (res["B"][a] + res["B"][b]) * res["steps"] / t / 1e9


def config_entry(res, np, cpu):
    """Compact per-workload record of the bench line."""
    ms = res["ms"]
    wl = res["wl"]
    v = pair_gbs(res, "dispatch", "combine")
    us = lambda p: round(float(ms[p].mean()) * 1e3, 2)  # noqa: E731
    pct = lambda p: {"median": round(float(np.median(ms[p])) * 1e3, 2),  # noqa: E731
                     "p10": round(float(np.percentile(ms[p], 10)) * 1e3, 2),
                     "p90": round(float(np.percentile(ms[p], 90)) * 1e3, 2)}
    frac = lambda p: round(res["B"][p] / (ms[p].mean() * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)  # noqa: E731
    e = {"workload": wl.describe(), "steps": res["steps"],
         "dispatch_plus_combine_GBps": round(v, 1), "frac_of_hbm_peak": round(v / HBM_PEAK_GBS, 4),
         "dispatch_us": us("dispatch"), "dispatch_frac": frac("dispatch"),
         "combine_us": us("combine"), "combine_frac": frac("combine"),
         "dispatch_fp8_us": us("dispatch_fp8"), "dispatch_fp8_frac": frac("dispatch_fp8"),
         "layout_us": us("layout"),
         "us_percentiles": {p: pct(p) for p in ("dispatch", "combine", "dispatch_fp8")},
         "ht_pair_frac": round(pair_gbs(res, "dispatch_ht", "combine_ht") / HBM_PEAK_GBS, 4),
         "ll_pair_frac": round(pair_gbs(res, "dispatch_ll", "combine_ll") / HBM_PEAK_GBS, 4),
         "dispatch_copy_frac": frac("dispatch_cached"), "fp8_copy_frac": frac("dispatch_fp8_cached"),
         "oracle": cpu}
    if wl.T * wl.H * 2 < (64 << 20):
        e["note"] = ("latency-bound: the whole path fits the 256 MB Infinity Cache and each call "
                     "lasts a few launch latencies, so the HBM fraction is not a roofline here")
    return e


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="dsv3")
    ap.add_argument("--no-flush", action="store_true", help="do not evict caches between phases")
    ap.add_argument("--cpu-baseline-seconds", type=float, default=10.0)
    ap.add_argument("--skip-cpu-baseline", action="store_true")
    ap.add_argument("--skip-per-config", action="store_true",
                    help="time the headline workload only (no per_config records)")
    ap.add_argument("--graph", action="store_true",
                    help="instead of the headline: time one whole step (layout, dispatch, combine, "
                         "FP8 dispatch; no cache eviction) replayed from a captured HIP graph "
                         "against the same step launched eagerly")
    ap.add_argument("--drain-check", action="store_true",
                    help="instead of the headline: check that ep_dispatch and ep_combine leave no "
                         "write-backs behind their end events (each timed alone and followed by "
                         "a 512 MiB read)")
    ap.add_argument("--scatter-check", action="store_true",
                    help="instead of the headline: time the dispatch copy kernels alone on the real "
                         "receive map and on an identity map (one sequential write stream)")
    ap.add_argument("--ll-capacity", type=int, default=0,
                    help="capacity (rows per expert) of the padded-layout phases; default: the "
                         "busiest expert's load rounded up to 64 rows")
    ap.add_argument("--calibration-copy", action="store_true",
                    help="after the timed steps, run 4 plain 256 MiB device copies (a known-size "
                         "reference for rocprofv3 FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE={world}): "
              "every destination rank is a partition of one GPU's HBM here; run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from combine_get_dispatch_02_amd import ep
    from combine_get_dispatch_02_amd.workloads import CONFIGS

    wl = CONFIGS[args.workload]
    torch.cuda.set_device(torch.device("cuda:0"))
    log(f"[bench] {wl.describe()} steps={args.steps} warmup={args.warmup} ({ep.version()})")
    if args.graph or args.drain_check or args.scatter_check:
        measure(wl, args.steps, args.warmup, args, ep, torch, np,
                mode="graph" if args.graph else "drain" if args.drain_check else "scatter")
        return

    res = measure(wl, args.steps, args.warmup, args, ep, torch, np, mode="headline")
    ms, B, N, H = res["ms"], res["B"], wl.T * wl.k, wl.H
    T, k, E, R, P = wl.T, wl.k, wl.E, wl.R, wl.P
    t_dc = float(ms["dispatch"].sum() + ms["combine"].sum()) / 1e3
    value = (B["dispatch"] + B["combine"]) * args.steps / t_dc / 1e9
    phase_info = phase_summary(res, np)
    full_us = float(sum(ms[p].mean() for p in ("layout", "dispatch", "combine"))) * 1e3
    full_b = B["layout"] + B["dispatch"] + B["combine"]
    payload_b = 2 * 2 * N * H
    c_us = float(ms["combine"].mean()) * 1e3
    achieved = B["combine"] / (c_us * 1e-6) / 1e9
    traffic = load_traffic(B["combine"])
    k_us = float(ms["dispatch_cached"].mean()) * 1e3
    k_gbs = B["dispatch_cached"] / (k_us * 1e-6) / 1e9
    roofline_copy = {"kernel": "copy_bf16_kernel (ep_dispatch_cached: the dispatch copy alone, "
                               "x read from HBM)", "bound": "hbm", "achieved": round(k_gbs, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(k_gbs / HBM_PEAK_GBS, 4),
                     "alg_bytes_per_launch": int(B["dispatch_cached"]), "avg_launch_us": round(k_us, 2)}
    q_us = float(ms["dispatch_fp8_cached"].mean()) * 1e3
    q_gbs = B["dispatch_fp8_cached"] / (q_us * 1e-6) / 1e9
    roofline_fp8 = {"kernel": "copy_fp8_kernel (ep_dispatch_fp8_cached: the FP8 cast and copy alone, "
                              "x read from HBM)", "bound": "hbm", "achieved": round(q_gbs, 1),
                    "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(q_gbs / HBM_PEAK_GBS, 4),
                    "alg_bytes_per_launch": int(B["dispatch_fp8_cached"]), "avg_launch_us": round(q_us, 2)}
    roofline = {"kernel": "combine_kernel<1, true> (ep_combine)", "bound": "hbm",
                "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                "alg_bytes_per_launch": int(B["combine"]), "avg_launch_us": round(c_us, 2),
                "empty_event_pair_us": round(res["pair_us"], 2),
                "note": "avg_launch_us is the HIP-event time of the one-kernel ep_combine call, so it "
                        "includes one event pair; the kernel-trace average is lower by about that"}

    cpu = None
    if not args.skip_cpu_baseline:
        log(f"[bench] cpu baseline (oracle, ~{args.cpu_baseline_seconds:.0f} s)")
        cpu = cpu_baseline(wl, res["x"], res["idx"], res["w"], args.cpu_baseline_seconds)

    per_config = {}
    if not args.skip_per_config:
        for name, other in CONFIGS.items():
            if name == wl.name:
                per_config[name] = config_entry(res, np, cpu and oracle_entry(cpu))
                continue
            st = PER_CONFIG_STEPS.get(name, PER_CONFIG_DEFAULT_STEPS)
            log(f"[bench] per-config {other.describe()} steps={st}")
            r = measure(other, st, PER_CONFIG_WARMUP, args, ep, torch, np)
            torch.cuda.empty_cache()
            c = None
            if not args.skip_cpu_baseline:
                c = oracle_entry(cpu_baseline(other, r["x"], r["idx"], r["w"], PER_CONFIG_CPU_SECONDS))
            per_config[name] = config_entry(r, np, c)
            del r
            torch.cuda.empty_cache()

    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(1e3 * t_dc / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.describe(), "T": T, "H": H, "k": k, "num_experts": E,
                   "num_ranks": R, "ranks_per_group": P, "global_batch": T, "parallelism": "none (1 GPU)"},
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "ms_per_step_note": "ep_dispatch + ep_combine, the time value is computed from; the layout "
                            "and FP8 dispatch of each step are timed separately (phases)",
        "layout_ms_per_step": round(float(ms["layout"].mean()), 4),
        "dispatch_fp8_ms_per_step": round(float(ms["dispatch_fp8"].mean()), 4),
        "caches_flushed_between_phases": not args.no_flush,
        "wall_ms_per_step_incl_flush": round(1e3 * res["wall"] / args.steps, 4),
        "phases": phase_info,
        "warm": {"dispatch_us": round(float(np.median(res["warm_d"])), 2),
                 "combine_us": round(float(np.median(res["warm_c"])), 2),
                 "value": round((B["dispatch"] + B["combine"]) /
                                ((np.median(res["warm_d"]) + np.median(res["warm_c"])) * 1e-6) / 1e9, 1),
                 "note": "secondary: dispatch then combine back to back, no cache eviction "
                         "(x and part of the rows may be served from the 256 MB Infinity Cache)"},
        "rank_dedup": {"rows": res["n_ht"], "rows_per_token": round(res["n_ht"] / max(T, 1), 4),
                       "dispatch_plus_combine_GBps": round(pair_gbs(res, "dispatch_ht", "combine_ht"), 1),
                       "pct_of_hbm_peak": round(100 * pair_gbs(res, "dispatch_ht", "combine_ht") / HBM_PEAK_GBS, 2),
                       "us_per_pair": round(1e3 * float(ms["dispatch_ht"].mean() + ms["combine_ht"].mean()), 2),
                       "note": "ep_dispatch_ht + unweighted ep_combine; not part of value or ms_per_step"},
        "ll_padded": {"capacity": res["cap_ll"], "slots_filled": res["n_ll"], "slots_dropped": N - res["n_ll"],
                      "slots_allocated": E * res["cap_ll"],
                      "dispatch_plus_combine_GBps": round(pair_gbs(res, "dispatch_ll", "combine_ll"), 1),
                      "pct_of_hbm_peak": round(100 * pair_gbs(res, "dispatch_ll", "combine_ll") / HBM_PEAK_GBS, 2),
                      "us_per_pair": round(1e3 * float(ms["dispatch_ll"].mean() + ms["combine_ll"].mean()), 2),
                      "note": "ep_dispatch_ll + ep_combine over token_slot, capacity = busiest "
                              "expert's load rounded up to 64 rows (nothing dropped); not part of "
                              "value or ms_per_step"},
        "full_path": {"us_per_step": round(full_us, 2), "alg_bytes": int(full_b),
                      "GBps": round(full_b / (full_us * 1e-6) / 1e9, 1),
                      "pct_of_hbm_peak": round(100 * full_b / (full_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 2),
                      "note": "layout + dispatch + combine, mean event times"},
        "payload_convention": {"bytes_per_pair": int(payload_b),
                               "GBps": round(payload_b * args.steps / t_dc / 1e9, 1),
                               "note": "the pages' benchmark byte count: one bf16 row per dispatched "
                                       "(token, expert) pair in each direction (2 N H 2 bytes), without "
                                       "the x read, the output write or the index bytes; same times "
                                       "as value"},
        "roofline": roofline,
        "roofline_dispatch_copy": roofline_copy,
        "roofline_fp8_copy": roofline_fp8,
        "cpu_baseline": cpu,
        "per_config": per_config,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
