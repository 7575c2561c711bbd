#!/usr/bin/env python3
"""Benchmark of the Adamas decode step on one MI355X.

Workload: one Llama-3.1-8B-shaped attention layer at decode time -- batch 1,
32 query heads / 8 KV heads, head_dim 128, 32768 cached positions, token budget
128 (budget 1024 is reported alongside) -- synthetic seeded data (workloads.py).

One step = the whole hot path, one adamas_append_decode_step call: encode the
newly appended key of every KV head (transform + bucketize + pack, position
len-1), encode the queries, scan every packed key code (Manhattan distance),
select the top-k, gather the original K/V rows and run exact softmax attention.
The same step issued as adamas_encode_keys + adamas_decode_step is reported too.  Steps are replayed from a HIP graph (the launch
sequence of each step is captured once), over R rotating copies of the cache so
that successive steps do not hit data left in the 256 MB last-level cache by
the previous ones ("cold"); a warm figure (one copy) is reported as well.

Printed: one JSON line.  `value` is the mean decode-step latency in microseconds
(lower is better).  `roofline` covers the dominant kernel of the step: its
algorithmic bytes per launch divided by its mean duration, measured with HIP
events recorded by the kernel dispatch itself (adamas_profile_events).
`cpu_baseline` is the CPU oracle (oracle/) timed on this host for a bounded
number of steps of the same workload.
"""
import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "decode-step sparse-attn latency (us) and achieved HBM GB/s vs peak, 32K ctx"
HBM_PEAK_GBS = 8000.0
# The secondary workloads: name -> (workload maker, rotating cache copies).
OTHER_WORKLOADS = {
    "batched16_ragged16k-32k_b256": (lambda W, seed: W.batched(seed), 3),
    "long512k_b1024": (lambda W, seed: W.llama(seed, cap=524288, budget=1024, name="long512k"), 2),
}
PROFILE_DIR = os.path.join(ROOT, "profiles")


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=640, help="timed steps (exactly)")
    ap.add_argument("--warmup", type=int, default=64, help="untimed steps before them (exactly)")
    ap.add_argument("--budget", type=int, default=128)
    ap.add_argument("--context", type=int, default=32768)
    ap.add_argument("--copies", type=int, default=64, help="rotating cache copies (cold-cache timing)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-extra", action="store_true", help="skip the secondary measurements")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-sweep", action="store_true",
                    help="skip the context x budget sweep (4K..128K x 64..1024) in the extras")
    ap.add_argument("--no-e2e", action="store_true",
                    help="skip the end-to-end decode of the 32-layer Llama-3.1-8B-shaped stack (random weights)")
    ap.add_argument("--e2e-steps", type=int, default=16, help="timed tokens per end-to-end variant")
    ap.add_argument("--sweep", action="store_true",
                    help="instead of the headline: step latency over contexts 4K..128K x budgets 64..1024 on the "
                         "32/8-head layer (one JSON line per context), with the dense baseline")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="first run a plain device-to-device copy of this many MiB, three times (the reference "
                         "kernel that scales the HBM byte counters of a rocprofv3 --pmc run)")
    ap.add_argument("--summarize-counters", nargs=3, metavar=("WORKLOAD", "FETCH_DIR", "WRITE_DIR"),
                    help="no GPU: write the HBM byte counter summaries of the step's kernels on WORKLOAD "
                         "(llama32k_b128 or a secondary workload's name) under profiles/ from the CSV output of "
                         "two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of PMC_COMMAND")
    ap.add_argument("--only-launch-modes", action="store_true",
                    help="instead of the headline: the 32K step in both launch modes (two kernels, single "
                         "launch) on the same cold rotation, one JSON line (the program TRACE_COMMAND traces "
                         "for the launch-mode comparison)")
    ap.add_argument("--only-workload", choices=sorted(OTHER_WORKLOADS),
                    help="instead of the headline: only this secondary workload's step and dense baseline, one "
                         "JSON line (the program SQ_COMMAND profiles)")
    ap.add_argument("--only-prefill-encode", action="store_true",
                    help="instead of the headline: only the full-cache key encode (prefill) of the 32K layer, "
                         "graph replay over 16 rotating cold copies, one JSON line (profiled by SQ_COMMAND)")
    ap.add_argument("--summarize-sq", nargs=3, metavar=("WORKLOAD", "DIR_A", "DIR_B"),
                    help="no GPU: write the SQ counter summary (occupancy, VALU, LDS bank conflicts per kernel) "
                         "under profiles/ from the CSV output of the two SQ_COMMAND passes on WORKLOAD "
                         "(llama32k_b128 or a secondary workload's name)")
    ap.add_argument("--summarize-trace", nargs=3, metavar=("NAME", "TRACE_DIR", "BENCH_JSON"),
                    help="no GPU: write the kernel-trace summary NAME (a key of TRACE_ARGS) under profiles/ from "
                         "the CSV output of TRACE_COMMAND and the JSON line of the same bench.py command run "
                         "without the profiler on the same box and sources")
    return ap.parse_args()


class Hip:
    """Raw HIP events through libamdhip64 (the library's kernels are timed by
    events its own dispatches record)."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def event(self):
        e = ctypes.c_void_p()
        assert self.lib.hipEventCreate(ctypes.byref(e)) == 0
        return e.value

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        rc = self.lib.hipEventElapsedTime(ctypes.byref(ms), a, b)
        assert rc == 0, "hipEventElapsedTime failed (%d)" % rc
        return ms.value


def main():
    args = parse()
    if args.summarize_counters:
        return summarize_counters(*args.summarize_counters)
    if args.summarize_trace:
        return summarize_trace(*args.summarize_trace)
    if args.summarize_sq:
        return summarize_sq(*args.summarize_sq)
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the Adamas decode step runs and is timed on a single MI355X; "
              "runs over several GPUs are not supported (requested --gpus %d, WORLD_SIZE %d)" % (args.gpus, world),
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import sparse_attention_long_fwht_amd as A
    import workloads as W

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)
    hip = Hip()
    log = lambda *a: print(*a, file=sys.stderr, flush=True)
    if args.sweep:
        return sweep(A, W, np, torch, dev, log)
    if args.calibrate_copy_mib > 0:
        n = args.calibrate_copy_mib << 20
        src = torch.randint(0, 255, (n,), dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("[bench] calibration copy: %d MiB x 3" % args.calibrate_copy_mib)
        del src, dst
    if args.only_prefill_encode:
        print(json.dumps(prefill_encode_only(A, W, np, torch, dev, args.seed, log)), flush=True)
        return
    if args.only_launch_modes:
        print(json.dumps(launch_modes_only(A, W, np, torch, dev, args.seed, log)), flush=True)
        return
    if args.only_workload:
        make, ncopy = OTHER_WORKLOADS[args.only_workload]
        r = other_workload(A, np, torch, dev, make(W, args.seed), ncopy, hip, name=args.only_workload)
        print(json.dumps(dict(r, workload=args.only_workload)), flush=True)
        return

    cap = args.context
    budget = args.budget
    t0 = time.time()
    wl = W.llama(args.seed, cap=cap, budget=budget)
    B, Hq, Hkv = wl.B, wl.Hq, wl.Hkv
    log("[bench] generated %s in %.1fs" % (wl.name, time.time() - t0))

    def up(a):
        return torch.from_numpy(np.ascontiguousarray(a.view(np.int16) if a.dtype == np.uint16 else a)).to(dev)

    q0, k0, v0 = up(wl.q), up(wl.k), up(wl.v)
    kv_len = up(wl.kv_len)
    start = up(wl.kv_len - 1)
    codes0 = torch.zeros((B, Hkv, cap, 32), dtype=torch.uint8, device=dev)
    A.encode_keys(k0, kv_len, codes0)
    R = max(1, args.copies)
    copies = [(q0, k0, v0, codes0)] + [(q0.clone(), k0.clone(), v0.clone(), codes0.clone()) for _ in range(R - 1)]
    out = torch.empty((B, Hq, 128), dtype=torch.float32, device=dev)
    ws = A.alloc_workspace(A.decode_workspace_size(B, Hq, Hkv, cap, budget), dev)
    ws_dense = A.alloc_workspace(A.dense_workspace_size(B, Hq, Hkv, cap), dev)
    torch.cuda.synchronize()
    log("[bench] %d cache copies resident (%.1f GiB)" % (R, R * (2 * k0.numel() * 2 + codes0.numel()) / 2 ** 30))

    def step(c, bud=budget, work=ws):
        # append the key at len-1 and decode, one call (adamas_append_decode_step)
        q, k, v, codes = c
        A.decode_step(q, k, v, codes, kv_len, bud, wl.scale, out, work, append=True)

    def step_unfused(c):
        q, k, v, codes = c
        A.encode_keys(k, kv_len, codes, start=start, max_rows=1)
        A.decode_step(q, k, v, codes, kv_len, budget, wl.scale, out, ws)

    def dense_step(c):
        q, k, v, _ = c
        A.dense_decode_attention(q, k, v, kv_len, wl.scale, out, ws_dense)

    def graph_of(fn, cs):
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            for c in cs:  # eager pass on the capture stream first
                fn(c)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            for c in cs:
                fn(c)
        torch.cuda.synchronize()
        return g

    def time_graph(g, n_per_replay, steps, warmup):
        reps = max(1, (steps + n_per_replay - 1) // n_per_replay)
        wreps = max(1, (warmup + n_per_replay - 1) // n_per_replay)
        for _ in range(wreps):
            g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / (reps * n_per_replay), reps * n_per_replay

    # ---- headline: exactly --warmup untimed steps, then exactly --steps timed
    # steps, each a graph of that many steps over the rotating copies (step i
    # reads copy i mod R)
    K, Wu = max(1, args.steps), max(0, args.warmup)
    g_main = graph_of(step, [copies[i % R] for i in range(K)])
    g_wu = graph_of(step, [copies[(K + i) % R] for i in range(Wu)]) if Wu else None
    torch.cuda.synchronize()
    if g_wu is not None:
        g_wu.replay()
        torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    g_main.replay()
    e1.record()
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / K
    steps_done = K
    del g_main, g_wu
    log("[bench] decode step (adamas_append_decode_step), cold: %.2f us over exactly %d steps after %d warm-up"
        % (ms_step * 1e3, K, Wu))
    def replay_spread(fn, n_replays=24, per_graph=16):
        """Mean step time of each of n_replays timed replays of 16-step graphs
        that together cycle through every copy (so the rotation stays cold):
        median, p10, p90, min, max over the replays."""
        gs = [graph_of(fn, [copies[(j * per_graph + i) % R] for i in range(per_graph)])
              for j in range(max(1, R // per_graph))]
        for g in gs:
            g.replay()
        torch.cuda.synchronize()
        per = []
        for i in range(n_replays):
            e0.record()
            gs[i % len(gs)].replay()
            e1.record()
            torch.cuda.synchronize()
            per.append(e0.elapsed_time(e1) * 1e3 / per_graph)
        del gs
        per.sort()
        return {"steps": n_replays * per_graph, "replay_steps": per_graph, "median_us": round(per[len(per) // 2], 3),
                "p10_us": round(per[int(0.1 * (len(per) - 1))], 3),
                "p90_us": round(per[int(0.9 * (len(per) - 1))], 3), "min_us": round(per[0], 3),
                "max_us": round(per[-1], 3)}

    # the spread: 24 timed replays of 16-step graphs (384 steps)
    spread = replay_spread(step)
    log("[bench] spread over 24 x 16 steps: %s" % spread)
    g_cold = None

    # ---- kernel-by-kernel durations (dispatch-recorded HIP events), cold rotation
    names = ["scan", "select_attend"]
    evs = [hip.event() for _ in range(2 * len(names))]
    ev_enc = [hip.event() for _ in range(2)]
    sums = [0.0] * len(names)
    enc_sum = 0.0
    n_prof = max(2 * R, 64)
    for i in range(n_prof + 8):
        q, k, v, codes = copies[i % R]
        A.profile_events(ev_enc)
        A.encode_keys(k, kv_len, codes, start=start, max_rows=1)
        A.profile_events(evs)
        A.decode_step(q, k, v, codes, kv_len, budget, wl.scale, out, ws, append=True)
        A.profile_events(None)
        torch.cuda.synchronize()
        if i >= 8:
            for j in range(len(names)):
                sums[j] += hip.elapsed_ms(evs[2 * j], evs[2 * j + 1])
            enc_sum += hip.elapsed_ms(ev_enc[0], ev_enc[1])
    kern_us = {names[j]: sums[j] / n_prof * 1e3 for j in range(len(names))}
    kern_us["append_encode"] = enc_sum / n_prof * 1e3
    log("[bench] kernel means (us): %s" % kern_us)

    # algorithmic bytes (what the method must move), per launch
    lens = wl.kv_len.astype(np.int64)
    code_bytes = int(Hkv * lens.sum() * 32)
    q_bytes = B * Hq * 128 * 2
    out_bytes = B * Hq * 128 * 4
    # unique gathered rows per (b, kv head): union of the group's selections
    sel = torch.empty((B, Hq, budget), dtype=torch.int32, device=dev)
    A.decode_step(q0, k0, v0, codes0, kv_len, budget, wl.scale, out, ws, sel_idx=sel)
    torch.cuda.synchronize()
    sel_np = sel.cpu().numpy()
    grp = Hq // Hkv
    uniq = sum(len(np.unique(sel_np[b, g * grp:(g + 1) * grp][sel_np[b, g * grp:(g + 1) * grp] >= 0]))
               for b in range(B) for g in range(Hkv))
    nodedup = int((sel_np >= 0).sum())
    gather_bytes = uniq * 512
    algo = {"scan": code_bytes + q_bytes, "select_attend": gather_bytes + q_bytes + out_bytes,
            "append_encode": B * Hkv * (256 + 32)}
    dominant = max(kern_us, key=kern_us.get)
    achieved = algo[dominant] / (kern_us[dominant] * 1e-6) / 1e9 if algo[dominant] else 0.0
    step_bytes = code_bytes + gather_bytes + q_bytes + out_bytes + B * Hkv * (256 + 32)

    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": read_traffic(dominant),
                "kernel": dominant + "_kernel", "kernel_us": round(kern_us[dominant], 3),
                "algorithmic_bytes_per_launch": algo[dominant]}

    step_gbs = step_bytes / (ms_step * 1e-3) / 1e9
    extra = {"kernel_us": {k: round(v, 3) for k, v in kern_us.items()},
             "step_algorithmic_bytes": step_bytes,
             "step_achieved_GBps": round(step_gbs, 1),
             "step_hbm_frac": round(step_gbs / HBM_PEAK_GBS, 4),
             "step_spread": spread,
             "gathered_rows_unique": uniq, "gathered_rows_no_dedup": nodedup,
             "cache_copies": R}

    if not args.no_extra:
        extra["selection_quality"] = selection_quality(torch, wl, q0, k0, v0, kv_len, sel, out, ws_dense, A)
        log("[bench] selection quality (informational): %s" % extra["selection_quality"])
        # the same step as two library calls: adamas_encode_keys + adamas_decode_step
        g_unf = graph_of(step_unfused, copies)
        ms_unf, _ = time_graph(g_unf, R, args.steps, args.warmup)
        extra["step_us_unfused_encode_then_decode"] = round(ms_unf * 1e3, 3)
        log("[bench] encode_keys + decode_step (two calls): %.2f us" % (ms_unf * 1e3))
        del g_unf
        # warm: one copy
        g_warm = graph_of(step, [copies[0]] * 8)
        ms_warm, _ = time_graph(g_warm, 8, args.steps, args.warmup)
        extra["step_us_warm"] = round(ms_warm * 1e3, 3)
        # dense baseline, cold rotation
        g_dense = graph_of(dense_step, copies)
        ms_dense, _ = time_graph(g_dense, R, max(R, args.steps // 4), R)
        dense_bytes = int(Hkv * lens.sum() * 512 + q_bytes + out_bytes)
        extra["dense_us"] = round(ms_dense * 1e3, 3)
        extra["dense_GBps"] = round(dense_bytes / (ms_dense * 1e-3) / 1e9, 1)
        extra["speedup_vs_dense"] = round(ms_dense / ms_step, 3)
        log("[bench] dense decode baseline: %.2f us (%.0f GB/s); speedup %.2fx"
            % (ms_dense * 1e3, extra["dense_GBps"], extra["speedup_vs_dense"]))
        # budget 1024 on the same data
        if budget != 1024:
            ws1k = A.alloc_workspace(A.decode_workspace_size(B, Hq, Hkv, cap, 1024), dev)
            g_1k = graph_of(lambda c: step(c, 1024, ws1k), copies)
            ms_1k, _ = time_graph(g_1k, R, args.steps, args.warmup)
            extra["step_us_budget1024"] = round(ms_1k * 1e3, 3)
            log("[bench] budget 1024: %.2f us" % (ms_1k * 1e3))
            del g_1k
        # forced positions: 4 sinks and a 64-token window (same budget, same data)
        if budget > 68:
            def forced_step(c):
                q, k, v, codes = c
                A.decode_step(q, k, v, codes, kv_len, budget, wl.scale, out, ws, append=True, sink=4, recent=64)
            g_f = graph_of(forced_step, copies)
            ms_f, _ = time_graph(g_f, R, args.steps, args.warmup)
            extra["step_us_forced_sink4_recent64"] = round(ms_f * 1e3, 3)
            log("[bench] forced (4 sinks, 64 recent): %.2f us" % (ms_f * 1e3))
            del g_f
        # paged caches: the same data in shuffled pages of 16 and 64 positions
        # (16 rotating copies, one block table shared by all)
        for page in (16, 64):
            mp = cap // page
            perm = torch.randperm(B * mp, device=dev).view(B, mp).to(torch.int32)

            def to_pages(t):  # [B][Hkv][cap][D] -> pool [B*mp][Hkv][page][D], logical page (b, j) at perm[b][j]
                src = t.view(B, Hkv, mp, page, t.shape[-1]).permute(0, 2, 1, 3, 4).reshape(B * mp, Hkv, page, -1)
                pool = torch.empty(src.shape, dtype=src.dtype, device=src.device)
                pool[perm.view(-1).long()] = src
                return pool

            pages = A.Pages(perm, page, capacity=cap)
            pcopies = [(c[0], to_pages(c[1]), to_pages(c[2]), to_pages(c[3])) for c in copies[:16]]

            def paged_step(c):
                q, kp, vp, cp = c
                A.decode_step(q, kp, vp, cp, kv_len, budget, wl.scale, out, ws, append=True, pages=pages)
            g_p = graph_of(paged_step, pcopies)
            ms_p, _ = time_graph(g_p, 16, args.steps, args.warmup)
            extra["step_us_paged_page%d" % page] = round(ms_p * 1e3, 3)
            log("[bench] paged (page %d): %.2f us" % (page, ms_p * 1e3))
            del g_p, pcopies
        # the single-launch step (adamas_decode_launch_mode(1)) beside the
        # two-kernel one, same rotation and replays
        A.decode_launch_mode(1)
        sl = replay_spread(step)
        assert A.last_launch_count() == 1
        A.decode_launch_mode(0)
        extra["step_us_single_launch_median"] = sl["median_us"]
        extra["step_us_two_kernels_median"] = spread["median_us"]
        log("[bench] single-launch step: median %.2f us (two kernels %.2f)" % (sl["median_us"], spread["median_us"]))
        # full-cache key encode (prefill) pass, cold rotation
        g_enc = graph_of(lambda c: A.encode_keys(c[1], kv_len, c[3]), copies[:16])
        ms_enc, _ = time_graph(g_enc, 16, 64, 16)
        enc_bytes = int(Hkv * lens.sum() * (256 + 32))
        extra["prefill_encode_us"] = round(ms_enc * 1e3, 3)
        extra["prefill_encode_GBps"] = round(enc_bytes / (ms_enc * 1e-3) / 1e9, 1)
        log("[bench] prefill key encode: %.2f us (%.0f GB/s)" % (ms_enc * 1e3, extra["prefill_encode_GBps"]))
        del copies, g_cold, g_warm, g_dense, g_enc
        torch.cuda.empty_cache()
        # budget 1024 on the same layer: kernels, deduplicated bytes, fractions
        extra["llama32k_b1024"] = other_workload(A, np, torch, dev, W.llama(args.seed, cap=cap, budget=1024), 8,
                                                 hip)
        log("[bench] budget 1024: %s" % extra["llama32k_b1024"])
        torch.cuda.empty_cache()
        # the batched and long-context workloads
        for name, (make, ncopy) in OTHER_WORKLOADS.items():
            extra[name] = other_workload(A, np, torch, dev, make(W, args.seed), ncopy, hip, name=name)
            log("[bench] %s: %s" % (name, extra[name]))
            torch.cuda.empty_cache()
        if not args.no_sweep:
            extra["sweep_context_x_budget"] = sweep_rows(A, W, np, torch, dev, log, hip)
            torch.cuda.empty_cache()

    if not args.no_extra and not args.no_e2e:
        extra["e2e_llama31_8b_shaped_b1"] = e2e(torch, dev, log, [args.context], budget, args.e2e_steps)
        torch.cuda.empty_cache()
        lens16 = W.batched_lengths(np.random.default_rng(args.seed))
        extra["e2e_llama31_8b_shaped_b16_ragged16k-32k"] = e2e(torch, dev, log, [int(x) for x in lens16], 256,
                                                               args.e2e_steps)
        torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(wl, budget, args.cpu_seconds, log)

    res = {"metric": METRIC, "value": round(ms_step * 1e3, 3), "unit": "us", "n_gpus": 1, "steps": steps_done,
           "warmup": Wu, "ms_per_step": round(ms_step, 6), "higher_is_better": False,
           "scaling": "weak", "vs_baseline": None, "dtype": "u8+fp32", "data": "synthetic",
           "config": {"workload": "llama3.1-8b-shaped decode layer: batch 1, 32 q / 8 kv heads, head_dim 128, "
                                  "%d cached positions, budget %d; append-encode + decode per step; cold cache"
                                  % (cap, budget),
                      "batch": B, "seq_len": cap, "budget": budget, "q_heads": Hq, "kv_heads": Hkv,
                      "head_dim": 128, "parallelism": "single GPU"},
           "roofline": roofline, "cpu_baseline": cpu, "extra": extra}
    print(json.dumps(res), flush=True)


# Source files that make up each kernel of the step; a counter summary counts
# only while the sha256 of these files is the one it was taken on.
CSRC = os.path.join(ROOT, "sparse_attention_long_fwht_amd", "csrc")
KERNEL_SOURCES = {
    "scan": ["decode.hip", "device_common.h", "plan.h"],
    "select_attend": ["decode.hip", "device_common.h", "plan.h"],
    "append_encode": ["kernels.hip", "device_common.h", "plan.h"],
}
WORKLOAD_TAG = "llama32k_b128"
# bench.py arguments of the program each HBM byte counter run profiles
PMC_ARGS = {WORKLOAD_TAG: "--steps 8 --warmup 2 --copies 4 --no-extra --no-cpu --calibrate-copy-mib 64"}
PMC_ARGS.update({name: "--only-workload %s --calibrate-copy-mib 64" % name for name in OTHER_WORKLOADS})
PMC_COMMAND = ("cd /tmp && export TMPDIR=/tmp && cd $GRAFT_REPO_ROOT && timeout -s KILL 120 rocprofv3 --pmc {counter} "
               "--output-format csv -d gpurun_out/pmc_{workload}_{tag} -o pmc -- python3 bench.py {args}")
# bench.py arguments of the program each kernel trace covers
TRACE_ARGS = {WORKLOAD_TAG: "--no-extra",
              "llama32k_b128_launch_modes": "--only-launch-modes",
              "batched16_ragged16k-32k_b256": "--only-workload batched16_ragged16k-32k_b256"}
TRACE_COMMAND = ("cd /tmp && export TMPDIR=/tmp && cd $GRAFT_REPO_ROOT && timeout -k 10 300 rocprofv3 --kernel-trace "
                 "--stats --output-format csv -d gpurun_out/trace_{name} -o trace -- python3 bench.py {args}")
WORKLOAD_TEXT = {
    WORKLOAD_TAG: "Llama-3.1-8B-shaped decode layer (batch 1, 32 q / 8 kv heads, head_dim 128, 32768 cached "
                  "positions, budget 128)",
    "batched16_ragged16k-32k_b256": "batch 16, 32 q / 8 kv heads, head_dim 128, ragged 16K-32K cached positions, "
                                    "budget 256",
    "long512k_b1024": "batch 1, 32 q / 8 kv heads, head_dim 128, 524288 cached positions, budget 1024",
}
COPY_KIB = 64 * 1024  # the calibration copy: reads and writes 64 MiB


def source_hash(kernel):
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        h.update(open(os.path.join(CSRC, f), "rb").read())
    return h.hexdigest()[:16]


def counters_path(kernel, workload=WORKLOAD_TAG):
    return os.path.join(PROFILE_DIR, "%s_kernel_%s_counters.txt" % (kernel, workload))


def read_traffic(kernel, workload=WORKLOAD_TAG):
    """HBM bytes per launch of `kernel` on `workload` from the committed
    rocprofv3 counter summary, if it was taken on the current kernel source;
    otherwise None."""
    path = counters_path(kernel, workload)
    if not os.path.exists(path):
        return None
    recorded, hbm = None, None
    for line in open(path):
        if line.startswith("source sha256[:16]:"):  # "<hash>  (files)"
            recorded = line[len("source sha256[:16]:"):].split()[0]
        elif line.startswith("hbm_bytes_per_launch:"):
            hbm = int(float(line.split(":", 1)[1]))
    if recorded != source_hash(kernel) or hbm is None:
        return None
    return hbm


def _csv_rows(d, suffix):
    import csv
    import glob
    files = sorted(glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True))
    if not files:
        raise SystemExit("no *%s under %s" % (suffix, d))
    rows = []
    for f in files:
        with open(f, newline="") as fh:
            rows.extend(csv.DictReader(fh))
    return rows


def _per_dispatch(rows, counter, with_ids=False):
    """{kernel name: [value per dispatch]} for one counter (summed over the
    dimensions rocprofv3 reports it in); with_ids: [(dispatch id, value)] in
    dispatch order."""
    acc = {}
    for r in rows:
        if r.get("Counter_Name") != counter:
            continue
        key = (r["Kernel_Name"], int(r.get("Dispatch_Id", r.get("Correlation_Id"))))
        acc[key] = acc.get(key, 0.0) + float(r["Counter_Value"])
    out = {}
    for (name, did), v in sorted(acc.items(), key=lambda kv: kv[0][1]):
        out.setdefault(name, []).append((did, v) if with_ids else v)
    return out


def _calibration_kib(table):
    """The counter value of the calibration copy: the first device copies of
    the program (--calibrate-copy-mib runs three before anything else), their
    largest reading."""
    copies = sorted((did, v) for name, vals in table.items() if "copyBuffer" in name for did, v in vals)
    if len(copies) < 3:
        raise SystemExit("fewer than three copyBuffer dispatches (was --calibrate-copy-mib given?)")
    return max(v for _, v in copies[:3])


def summarize_counters(workload, fetch_dir, write_dir):
    """Counter summaries of the step's two kernels on one workload: FETCH_SIZE
    and WRITE_SIZE (KiB per dispatch), each scaled by calibration against a copy
    of known size."""
    import statistics
    if workload not in PMC_ARGS:
        raise SystemExit("unknown workload %r (one of %s)" % (workload, sorted(PMC_ARGS)))
    fetch = _per_dispatch(_csv_rows(fetch_dir, "counter_collection.csv"), "FETCH_SIZE", with_ids=True)
    write = _per_dispatch(_csv_rows(write_dir, "counter_collection.csv"), "WRITE_SIZE", with_ids=True)

    def pick(table, sub):
        names = [n for n in table if sub in n]
        if not names:
            raise SystemExit("no kernel matching %r in %s" % (sub, sorted(table)))
        vals = [v for n in names for _, v in table[n]]
        return names, vals

    cf, cw = _calibration_kib(fetch), _calibration_kib(write)
    # scale: the copy reads and writes COPY_KIB
    f_scale = COPY_KIB / cf
    w_scale = COPY_KIB / cw
    lines = []
    for kernel in ("select_attend", "scan"):
        nf, vf = pick(fetch, kernel + "_kernel")
        _, vw = pick(write, kernel + "_kernel")
        fk, wk = statistics.mean(vf), statistics.mean(vw)
        hbm = (fk * f_scale + wk * w_scale) * 1024
        text = [
            "rocprofv3 HBM byte counters: %s_kernel, %s" % (kernel, WORKLOAD_TEXT[workload]),
            "",
            "command (FETCH_SIZE): " + PMC_COMMAND.format(counter="FETCH_SIZE", workload=workload, tag="fetch",
                                                          args=PMC_ARGS[workload]),
            "command (WRITE_SIZE): " + PMC_COMMAND.format(counter="WRITE_SIZE", workload=workload, tag="write",
                                                          args=PMC_ARGS[workload]),
            "kernel: " + nf[0],
            "dispatches: %d (FETCH_SIZE run), %d (WRITE_SIZE run)" % (len(vf), len(vw)),
            "FETCH_SIZE KiB/dispatch mean: %.1f  (min %.1f, max %.1f)" % (fk, min(vf), max(vf)),
            "WRITE_SIZE KiB/dispatch mean: %.1f  (min %.1f, max %.1f)" % (wk, min(vw), max(vw)),
            "calibration copy (%d KiB read + written, the first copies of the program): FETCH_SIZE %.1f KiB, "
            "WRITE_SIZE %.1f KiB" % (COPY_KIB, cf, cw),
            "scale: FETCH_SIZE x %.3f, WRITE_SIZE x %.3f" % (f_scale, w_scale),
            "hbm_bytes_per_launch: %d" % int(hbm),
            "source sha256[:16]: %s  (%s)" % (source_hash(kernel), ", ".join(KERNEL_SOURCES[kernel])),
        ]
        os.makedirs(PROFILE_DIR, exist_ok=True)
        with open(counters_path(kernel, workload), "w") as fh:
            fh.write("\n".join(text) + "\n")
        lines.append("%s: %.0f bytes/launch" % (kernel, hbm))
    print("\n".join(lines))


# Two SQ counter passes per workload (each within one pass's limits: at most
# 8 SQ and 2 GRBM counters); GRBM_GUI_ACTIVE in both, for the normalisation.
SQ_PASSES = {
    "a": "SQ_WAVES,SQ_WAVE_CYCLES,SQ_BUSY_CU_CYCLES,SQ_ACTIVE_INST_VALU,SQ_ACTIVE_INST_ANY,SQ_WAIT_INST_ANY,"
         "GRBM_GUI_ACTIVE",
    "b": "SQ_INSTS_VALU,SQ_INSTS_LDS,SQ_LDS_BANK_CONFLICT,SQ_LDS_IDX_ACTIVE,GRBM_GUI_ACTIVE",
}
SQ_ARGS = {WORKLOAD_TAG: "--steps 8 --warmup 2 --copies 4 --no-extra --no-cpu"}
SQ_ARGS.update({name: "--only-workload " + name for name in OTHER_WORKLOADS})
SQ_ARGS["prefill_encode32k"] = "--only-prefill-encode"
SQ_COMMAND = ("cd /tmp && export TMPDIR=/tmp && cd $GRAFT_REPO_ROOT && timeout -s KILL 120 rocprofv3 --pmc {counters} "
              "--output-format csv -d gpurun_out/sq_{workload}_{p} -o pmc -- python3 bench.py {args}")
CU_NUM = 256


def summarize_sq(workload, dir_a, dir_b):
    """Per-kernel SQ counter summary of the step's kernels (and the dense
    baseline's) on one workload, with rocprofv3's own derived metrics."""
    import csv
    import glob
    if workload not in SQ_ARGS:
        raise SystemExit("unknown workload %r (one of %s)" % (workload, sorted(SQ_ARGS)))
    per = {}    # (kernel, pass, dispatch) -> {counter: value}
    wpb = {}    # kernel -> waves per block
    dur = {}    # kernel -> [us per dispatch, under the profiler]
    for p, d in (("a", dir_a), ("b", dir_b)):
        files = sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True))
        if not files:
            raise SystemExit("no counter_collection.csv under " + d)
        for f in files:
            for r in csv.DictReader(open(f, newline="")):
                name = r["Kernel_Name"]
                if "adamas::" not in name:
                    continue
                k = name.split("(")[0].replace("void adamas::", "")
                c, v = r["Counter_Name"], float(r["Counter_Value"])
                acc = per.setdefault((k, p, r["Dispatch_Id"]), {})
                # GRBM_GUI_ACTIVE: the busy cycles of the device (the largest
                # instance); SQ counters: summed over shader engines and XCDs
                acc[c] = max(acc.get(c, 0.0), v) if c == "GRBM_GUI_ACTIVE" else acc.get(c, 0.0) + v
                wpb[k] = int(r["Workgroup_Size"]) // 64
                if p == "a" and c == "SQ_WAVES":
                    dur.setdefault(k, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)

    def mean(k, p, c):
        vals = [a[c] for (kk, pp, _), a in per.items() if kk == k and pp == p and c in a]
        return sum(vals) / len(vals) if vals else float("nan"), len(vals)

    cmd = {p: SQ_COMMAND.format(counters=SQ_PASSES[p], workload=workload, p=p, args=SQ_ARGS[workload])
           for p in SQ_PASSES}
    text = ["rocprofv3 SQ counters per kernel, workload %s (the step's kernels and the dense baseline's)" % workload,
            "", "command (pass a): " + cmd["a"], "command (pass b): " + cmd["b"], "",
            "Under --pmc every dispatch runs alone and GRBM_GUI_ACTIVE also counts the profiler's own time around",
            "it, so nothing below is normalised by it.  SQ_WAVE_CYCLES, SQ_BUSY_CU_CYCLES and SQ_ACTIVE_INST_VALU",
            "are quad-cycles summed over SIMDs; per kernel, means over its dispatches:",
            "  us      = End - Start timestamp of the dispatch under the profiler",
            "  w/SIMD  = SQ_WAVE_CYCLES / SQ_BUSY_CU_CYCLES: waves resident per SIMD while its CU has work (of 8)",
            "  VALU/cy = SQ_ACTIVE_INST_VALU / SQ_BUSY_CU_CYCLES: wave-cycles on VALU instructions per busy SIMD",
            "            cycle (the issue share of the SIMD when at most one wave's VALU instruction is in flight)",
            "  ANY/cy  = SQ_ACTIVE_INST_ANY / SQ_BUSY_CU_CYCLES: the same for instructions of any kind",
            "  wait    = SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES: share of resident wave-cycles spent waiting on a",
            "            dependency (s_waitcnt on memory, LDS or a VALU result)",
            "  VALU/w, LDS/w = SQ_INSTS_VALU, SQ_INSTS_LDS per wave",
            "  cf/LDS  = SQ_LDS_BANK_CONFLICT / SQ_INSTS_LDS: bank-conflict stall cycles per LDS instruction",
            "  cf/act  = SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE: share of LDS-busy cycles lost to bank conflicts",
            "",
            "%-32s %5s %7s %5s %8s %7s %7s %7s %6s %9s %7s %7s %7s" % (
                "kernel", "disp", "waves", "w/blk", "us", "w/SIMD", "VALU/cy", "ANY/cy", "wait", "VALU/w", "LDS/w",
                "cf/LDS", "cf/act")]
    for k in sorted({kk for kk, _, _ in per}):
        waves, n = mean(k, "a", "SQ_WAVES")
        wcyc, _ = mean(k, "a", "SQ_WAVE_CYCLES")
        busy, _ = mean(k, "a", "SQ_BUSY_CU_CYCLES")
        valu_act, _ = mean(k, "a", "SQ_ACTIVE_INST_VALU")
        any_act, _ = mean(k, "a", "SQ_ACTIVE_INST_ANY")
        wait, _ = mean(k, "a", "SQ_WAIT_INST_ANY")
        valu, _ = mean(k, "b", "SQ_INSTS_VALU")
        lds, _ = mean(k, "b", "SQ_INSTS_LDS")
        conf, _ = mean(k, "b", "SQ_LDS_BANK_CONFLICT")
        lact, _ = mean(k, "b", "SQ_LDS_IDX_ACTIVE")
        us = sum(dur[k]) / len(dur[k])
        text.append("%-32s %5d %7.0f %5d %8.2f %7.2f %7.3f %7.3f %6.3f %9.1f %7.1f %7.2f %7.3f" % (
            k[:32], n, waves, wpb[k], us, wcyc / busy, valu_act / busy, any_act / busy, wait / wcyc, valu / waves,
            lds / waves,
            conf / lds if lds else 0.0, conf / lact if lact else 0.0))
    src = "append_encode" if workload == "prefill_encode32k" else "scan"
    text += ["", "source sha256[:16]: %s  (%s)" % (source_hash(src), ", ".join(KERNEL_SOURCES[src]))]
    os.makedirs(PROFILE_DIR, exist_ok=True)
    path = os.path.join(PROFILE_DIR, "sq_counters_%s.txt" % workload)
    with open(path, "w") as fh:
        fh.write("\n".join(text) + "\n")
    print(path)


def summarize_trace(name, trace_dir, bench_json):
    """Kernel-trace statistics of one TRACE_COMMAND beside the JSON line of the
    same bench.py command run without the profiler."""
    if name not in TRACE_ARGS:
        raise SystemExit("unknown trace %r (one of %s)" % (name, sorted(TRACE_ARGS)))
    stats = _csv_rows(trace_dir, "kernel_stats.csv")
    res = None
    for line in open(bench_json):
        line = line.strip()
        if line.startswith("{"):
            res = json.loads(line)
    if res is None:
        raise SystemExit("no JSON line in " + bench_json)
    what = WORKLOAD_TEXT.get(name, WORKLOAD_TEXT[WORKLOAD_TAG])
    text = ["rocprofv3 kernel trace (%s): Adamas decode step, %s" % (name, what), "",
            "command: " + TRACE_COMMAND.format(name=name, args=TRACE_ARGS[name]), "",
            "%-60s %7s %10s %10s %10s" % ("kernel", "calls", "avg_us", "min_us", "max_us")]
    for r in sorted(stats, key=lambda r: -float(r["TotalDurationNs"])):
        nm = r["Name"].split("(")[0]
        text.append("%-60s %7s %10.3f %10.3f %10.3f" % (nm[-60:], r["Calls"], float(r["AverageNs"]) / 1e3,
                                                       float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3))
    text += ["", "python3 bench.py %s without the profiler, same box and sources, just before (under the profiler" %
             TRACE_ARGS[name], "the library's dispatch-recorded events read high, so they are not used):"]
    if "extra" in res:  # the headline line
        text += ["kernel_us: " + json.dumps(res["extra"]["kernel_us"]),
                 "step us (graph replay, cold): %s" % res["value"]]
    else:
        text += ["result: " + json.dumps(res)]
    text += ["source sha256[:16]: %s  (%s)" % (source_hash("select_attend"),
                                             ", ".join(KERNEL_SOURCES["select_attend"]))]
    os.makedirs(PROFILE_DIR, exist_ok=True)
    path = os.path.join(PROFILE_DIR, "decode_step_%s_kernel_trace.txt" % name)
    with open(path, "w") as fh:
        fh.write("\n".join(text) + "\n")
    print(path)


def launch_modes_only(A, W, np, torch, dev, seed, log, ncopy=16, steps=64):
    """The 32K step (append-encode + decode) as graphs of `steps` steps over
    rotating copies, in launch mode 0 (two kernels) and 1 (single launch)."""
    wl = W.llama(seed, cap=32768, budget=128)
    up = lambda a: torch.from_numpy(np.ascontiguousarray(a.view(np.int16) if a.dtype == np.uint16 else a)).to(dev)
    q, k, v, kv_len = up(wl.q), up(wl.k), up(wl.v), up(wl.kv_len)
    codes = torch.zeros((wl.B, wl.Hkv, wl.cap, 32), dtype=torch.uint8, device=dev)
    A.encode_keys(k, kv_len, codes)
    cases = [(q, k, v, codes)] + [tuple(t.clone() for t in (q, k, v, codes)) for _ in range(ncopy - 1)]
    out = torch.empty((wl.B, wl.Hq, 128), dtype=torch.float32, device=dev)
    ws = A.alloc_workspace(A.decode_workspace_size(wl.B, wl.Hq, wl.Hkv, wl.cap, wl.budget), dev)
    step = lambda c: A.decode_step(c[0], c[1], c[2], c[3], kv_len, wl.budget, wl.scale, out, ws, append=True)
    res = {"workload": "llama32k_b128_launch_modes", "steps_per_mode": 2 * steps}
    for mode, key in ((0, "two_kernels"), (1, "single_launch")):
        A.decode_launch_mode(mode)
        us = timed_graph_steps(torch, step, [cases[i % ncopy] for i in range(steps)], 2)
        res[key + "_us"] = round(us, 3)
        res[key + "_launches_per_step"] = A.last_launch_count()
        log("[bench] launch mode %d: %.2f us per step (%d launches)" % (mode, us, A.last_launch_count()))
    A.decode_launch_mode(0)
    return res


def prefill_encode_only(A, W, np, torch, dev, seed, log, ncopy=16, reps=8):
    """Key encode of every cached position of the 32K layer (8 KV heads), as a
    HIP graph of `ncopy` calls over rotating copies of K and the codes."""
    wl = W.llama(seed, cap=32768, budget=128)
    up = lambda a: torch.from_numpy(np.ascontiguousarray(a.view(np.int16) if a.dtype == np.uint16 else a)).to(dev)
    k0, kv_len = up(wl.k), up(wl.kv_len)
    cases = [(k0 if i == 0 else k0.clone(), torch.zeros((wl.B, wl.Hkv, wl.cap, 32), dtype=torch.uint8, device=dev))
             for i in range(ncopy)]
    us = timed_graph_steps(torch, lambda c: A.encode_keys(c[0], kv_len, c[1]), cases, reps)
    ref = cases[0][1]
    assert all(torch.equal(c[1], ref) for c in cases[1:])
    nbytes = int(wl.Hkv * wl.kv_len.sum()) * (256 + 32)
    log("[bench] prefill key encode: %.2f us (%.0f GB/s)" % (us, nbytes / (us * 1e-6) / 1e9))
    return {"workload": "prefill_encode32k", "us": round(us, 3), "bytes": nbytes,
            "GBps": round(nbytes / (us * 1e-6) / 1e9, 1), "hbm_frac": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}


def timed_graph_steps(torch, fn, cases, reps):
    """Mean microseconds per call of fn(case), from a HIP graph holding one call
    per case (rotating copies), replayed `reps` times after one untimed replay."""
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for c in cases:
            fn(c)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        for c in cases:
            fn(c)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / (reps * len(cases))


def selection_quality(torch, wl, q, k, v, kv_len, sel, out, ws_dense, A):
    """Informational, never a pass/fail criterion (no page fixes a target on
    synthetic data): how much of the exact attention the selection keeps, on the
    headline workload.  Per query head: recall of the exact top-k by q.K (fp32
    scores), recall of the planted positions the query was built from, the
    softmax mass of the selected rows, and the output's relative L2 distance to
    dense attention.  `sel` and `out` hold the Adamas step's selection and output
    for (q, k, v) (bf16 bit patterns, any 2-byte dtype)."""
    import numpy as np
    B, Hq, budget = sel.shape
    qb, kb = q.view(torch.bfloat16), k.view(torch.bfloat16)
    grp = Hq // wl.Hkv
    dense = torch.empty_like(out)
    A.dense_decode_attention(q, k, v, kv_len, wl.scale, dense, ws_dense)
    torch.cuda.synchronize()
    rec, planted, mass, err = [], [], [], []
    for b in range(B):
        L = int(wl.kv_len[b])
        for h in range(Hq):
            kf = kb[b, h // grp, :L].float().contiguous()
            s = (kf @ qb[b, h].float().contiguous()) * wl.scale
            top = set(torch.topk(s, min(budget, L)).indices.cpu().tolist())
            chosen = sel[b, h]
            chosen = set(chosen[chosen >= 0].cpu().tolist())
            rec.append(len(top & chosen) / max(1, len(top)))
            pl = set(int(x) for x in wl.planted[b * Hq + h])
            planted.append(len(pl & chosen) / max(1, len(pl)))
            p = torch.softmax(s, 0)
            mass.append(float(p[torch.tensor(sorted(chosen), device=p.device)].sum()))
            d = dense[b, h]
            err.append(float((out[b, h] - d).norm() / d.norm()))
    return {"recall_vs_exact_qk_topk": round(float(np.mean(rec)), 4),
            "planted_recall": round(float(np.mean(planted)), 4),
            "softmax_mass_kept": round(float(np.mean(mass)), 4),
            "out_rel_l2_vs_dense": round(float(np.mean(err)), 4)}


def e2e(torch, dev, log, lengths, budget, steps):
    """Per-token latency of a 32-layer Llama-3.1-8B-shaped decode (random bf16
    weights; torch GEMMs and the fused elementwise kernels for the dense parts)
    with Adamas attention, with the last 3 layers dense (blog section 3.2), and
    with dense attention everywhere; each step is one HIP graph replay (blog
    section 5.1: graph capture at small batch), plus the Adamas step run
    eagerly.  Sequence b holds lengths[b] positions when each variant starts;
    every timed token appends one."""
    import time
    from sparse_attention_long_fwht_amd.llama_decode import LLAMA31_8B, LlamaShapedDecoder
    t0 = time.time()
    batch, context = len(lengths), max(lengths)
    m = LlamaShapedDecoder(LLAMA31_8B, batch, context + 4 * steps + 64, attention="adamas", budget=budget)
    m.fill_cache(lengths)
    torch.cuda.synchronize()
    log("[bench] e2e model and caches (batch %d, up to %d positions) ready (%.1f s)"
        % (batch, context, time.time() - t0))
    start = m.state()

    def timed(fn, n):
        m.restore(start)
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    res = {"model": "llama3.1-8b-shaped, 32 layers, random weights", "batch": batch, "max_context": context,
           "positions": int(sum(lengths)), "budget": budget}
    for name, mode, dense_last in (("adamas", "adamas", 0), ("adamas_last3_dense", "adamas", 3),
                                   ("dense", "dense", 0)):
        m.use(mode, dense_last)
        g = m.capture(1)
        res[name + "_ms_per_token"] = round(timed(g.replay, steps), 4)
        del g
        log("[bench] e2e %s: %.3f ms/token" % (name, res[name + "_ms_per_token"]))
    m.use("adamas", 0)
    res["adamas_eager_ms_per_token"] = round(timed(m.step, steps), 4)
    res["speedup_vs_dense"] = round(res["dense_ms_per_token"] / res["adamas_ms_per_token"], 3)
    res["speedup_vs_dense_last3_dense"] = round(res["dense_ms_per_token"] / res["adamas_last3_dense_ms_per_token"], 3)
    res["graph_gain_vs_eager"] = round(1 - res["adamas_ms_per_token"] / res["adamas_eager_ms_per_token"], 3)
    log("[bench] e2e: %s" % res)
    del m
    return res


def upload(np, torch, dev, a):
    return torch.from_numpy(np.ascontiguousarray(a.view(np.int16) if a.dtype == np.uint16 else a)).to(dev)


def kernel_means(A, torch, hip, fn, cases, names):
    """Mean duration (us) of each kernel of fn(case), from HIP events recorded
    by the kernels' own dispatches (adamas_profile_events), over the cases."""
    evs = [hip.event() for _ in range(2 * len(names))]
    sums = [0.0] * len(names)
    n = 0
    for i in range(len(cases) + 2):
        A.profile_events(evs)
        fn(cases[i % len(cases)])
        A.profile_events(None)
        torch.cuda.synchronize()
        if i >= 2:
            for j in range(len(names)):
                sums[j] += hip.elapsed_ms(evs[2 * j], evs[2 * j + 1])
            n += 1
    return {names[j]: sums[j] / n * 1e3 for j in range(len(names))}


def unique_rows(np, sel, Hkv):
    """K/V rows one step must read: the union of the selections of each (b, kv
    head)'s query heads (int32 [B][Hq][budget], -1 padded)."""
    B, Hq, _ = sel.shape
    grp = Hq // Hkv
    return sum(len(np.unique(s[s >= 0])) for b in range(B) for g in range(Hkv)
               for s in (sel[b, g * grp:(g + 1) * grp],))


def other_workload(A, np, torch, dev, wl, ncopy, hip=None, name=None):
    """Step latency (append-encode + decode, rotating `ncopy` copies of q, K, V
    and codes) and the dense baseline on one workload; with `hip`, also the
    kernels' durations, the deduplicated algorithmic bytes and the fractions of
    the HBM peak they reach."""
    kv_len = upload(np, torch, dev, wl.kv_len)
    q, k, v = upload(np, torch, dev, wl.q), upload(np, torch, dev, wl.k), upload(np, torch, dev, wl.v)
    codes = torch.zeros((wl.B, wl.Hkv, wl.cap, 32), dtype=torch.uint8, device=dev)
    A.encode_keys(k, kv_len, codes)
    cases = [(q, k, v, codes)] + [tuple(t.clone() for t in (q, k, v, codes)) for _ in range(ncopy - 1)]
    out = torch.empty((wl.B, wl.Hq, 128), dtype=torch.float32, device=dev)
    ws = A.alloc_workspace(A.decode_workspace_size(wl.B, wl.Hq, wl.Hkv, wl.cap, wl.budget), dev)
    wsd = A.alloc_workspace(A.dense_workspace_size(wl.B, wl.Hq, wl.Hkv, wl.cap), dev)
    step = lambda c: A.decode_step(c[0], c[1], c[2], c[3], kv_len, wl.budget, wl.scale, out, ws, append=True)
    step_us = timed_graph_steps(torch, step, cases * max(1, 16 // ncopy), 5)
    dense_us = timed_graph_steps(torch, lambda c: A.dense_decode_attention(c[0], c[1], c[2], kv_len, wl.scale,
                                                                           out, wsd), cases, 5)
    L = int(wl.kv_len.astype(np.int64).sum())
    code_bytes = L * wl.Hkv * 32
    gathered_max = wl.B * wl.Hq * wl.budget * 512  # no-dedup upper bound
    res = {"batch": wl.B, "context": wl.cap, "positions": L, "budget": wl.budget, "cache_copies": ncopy,
           "step_us": round(step_us, 3), "dense_us": round(dense_us, 3),
           "speedup_vs_dense": round(dense_us / step_us, 3),
           "dense_GBps": round(L * wl.Hkv * 512 / (dense_us * 1e3), 1),
           "dense_hbm_frac": round(L * wl.Hkv * 512 / (dense_us * 1e3) / HBM_PEAK_GBS, 4),
           "step_GBps_codes_plus_gather_upper_bound": round((code_bytes + gathered_max) / (step_us * 1e3), 1)}
    if hip is None:
        return res
    sel = torch.empty((wl.B, wl.Hq, wl.budget), dtype=torch.int32, device=dev)
    A.decode_step(q, k, v, codes, kv_len, wl.budget, wl.scale, out, ws, sel_idx=sel)
    torch.cuda.synchronize()
    uniq = unique_rows(np, sel.cpu().numpy(), wl.Hkv)
    qo = wl.B * wl.Hq * (256 + 512)
    algo = {"scan": code_bytes + wl.B * wl.Hq * 256 + wl.B * wl.Hkv * 288, "select_attend": uniq * 512 + qo}
    step_bytes = code_bytes + uniq * 512 + qo + wl.B * wl.Hkv * 288
    kus = kernel_means(A, torch, hip, step, cases, ["scan", "select_attend"])
    res.update({"gathered_rows_unique": uniq, "step_algorithmic_bytes": step_bytes,
                "step_GBps": round(step_bytes / (step_us * 1e3), 1),
                "step_hbm_frac": round(step_bytes / (step_us * 1e3) / HBM_PEAK_GBS, 4),
                "kernel_us": {n: round(t, 3) for n, t in kus.items()},
                "kernel_GBps": {n: round(algo[n] / (kus[n] * 1e3), 1) for n in kus},
                "kernel_hbm_frac": {n: round(algo[n] / (kus[n] * 1e3) / HBM_PEAK_GBS, 4) for n in kus}})
    if name is not None:
        # HBM bytes per launch from the committed counter summaries (None when
        # absent or taken on other sources)
        res["kernel_traffic_bytes"] = {n: read_traffic(n, name) for n in kus}
    return res


SWEEP_CONTEXTS = (4096, 8192, 16384, 32768, 65536, 131072)
SWEEP_BUDGETS = (64, 128, 256, 512, 1024)


def sweep_rows(A, W, np, torch, dev, log, hip=None):
    """Contexts 4K..128K x budgets 64..1024 on the 32/8-head layer: step latency
    (4 rotating copies) and the dense baseline, one row per context."""
    rows = []
    for cap in SWEEP_CONTEXTS:
        wl = W.llama(0, cap=cap, budget=64)
        row = {"context": cap, "step_us": {}}
        for budget in SWEEP_BUDGETS:
            wl.budget = budget
            r = other_workload(A, np, torch, dev, wl, 4)
            row["step_us"][budget] = r["step_us"]
            row["dense_us"] = r["dense_us"]
            log("[sweep] context %d budget %d: %.2f us (dense %.2f us)" % (cap, budget, r["step_us"], r["dense_us"]))
            torch.cuda.empty_cache()
        rows.append(row)
    return rows


def sweep(A, W, np, torch, dev, log):
    for row in sweep_rows(A, W, np, torch, dev, log):
        print(json.dumps(row), flush=True)


def host_cpu():
    """(logical CPUs this process may run on, CPU model name) of the host."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return n, model


def cpu_baseline(wl, budget, seconds, log):
    """The oracle as it stands, timed on this host for a bounded number of full
    decode steps of the same workload: on all the host's CPUs (OpenMP over
    (b, q head)) and on one thread."""
    import oracle
    ncpu, model = host_cpu()
    codes = oracle.encode_keys(wl.k, wl.kv_len, threads=ncpu)

    def timed(threads, budget_s):
        t0 = time.time()
        oracle.decode_step(wl.q, wl.k, wl.v, codes, wl.kv_len, budget, wl.scale, threads=threads, want_dist=False)
        one = time.time() - t0
        n = max(1, int(budget_s / max(one, 1e-3)))
        t0 = time.time()
        for _ in range(n):
            oracle.decode_step(wl.q, wl.k, wl.v, codes, wl.kv_len, budget, wl.scale, threads=threads,
                               want_dist=False)
        return (time.time() - t0) / n, n

    dt_all, n_all = timed(ncpu, seconds)
    dt_one, n_one = timed(1, seconds)
    log("[bench] cpu oracle: %.1f us/step with %d threads (%d steps), %.1f us/step on one thread (%d steps); %s"
        % (dt_all * 1e6, ncpu, n_all, dt_one * 1e6, n_one, model))
    return {"value": round(dt_all * 1e6, 1), "unit": "us", "cores": ncpu, "kind": "oracle",
            "sample": "%d full decode steps (query encode, distances, top-%d, fp64 attention) of the same "
                      "32K-context layer on %d threads, then %d on one thread; key codes precomputed"
                      % (n_all, budget, ncpu, n_one),
            "value_single_thread": round(dt_one * 1e6, 1), "host_logical_cpus": ncpu, "cpu_model": model}


if __name__ == "__main__":
    main()
