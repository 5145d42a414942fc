"""Benchmark of the LSA decode hot path on one MI355X.

One step = score (every compressed indexer key of the source layer) -> select
-> per sparse layer: ratio map -> LRU stage + fetch of missed rows -> attend.
Default workload: 1M-token context, ratio-4 source layer of 262144 entries,
4 x (ratio-4 + ratio-128) sparse layers with pinned host cold pools and
1024-slot LRU pools, top-512, 3 indexers x 8 heads x 128.

Two schedules are timed: "lookahead" (lsa_lookahead_step: the current step's
row copy and attention share launches with the next step's score and
selection) and "sync" (lsa_decode_step: all of it in order).  `value` is the
--schedule one (default lookahead); the other is reported beside it, and so is
the lookahead schedule with a periodic indexer (one prediction per window of
2, 4 or 8 steps).  With a 1M workload the run also times the 256K threshold
workload (batch 4, bf16 rows) in both schedules with a sampled parity check
(`ctx_256k`) and the KVSwap step at its 32K shape (`kvswap_32k`).

`roofline` is fm_score's with its keys read from HBM: back-to-back launches
rotate over copies of the keys that together exceed the 256 MiB last-level
cache twice over.  The back-to-back figure on one copy, where part of the
134 MB of keys comes from that cache, is reported beside it as
`cache_assisted`.

Prints ONE JSON line.  Per-kernel times come from HIP events recorded on the
launch stream inside the timed region; the CPU baseline is the plain oracle
timed on a bounded sample of the same steps.

    python bench.py [--steps K] [--warmup W] [--workload swap_1m|swap_1m_fp8|swap_1m_mxfp4|swap_1m_mxint8|thresh_256k|ens_8k|tiny_8k]
                    [--no-cpu-baseline] [--copy-calibration]
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "LSA decode steps/s (score+select+attend) at 256K/1M ctx; % of HBM peak"
HBM_PEAK_GBS = 8000.0
KERNELS = ["score", "select", "stage", "attend", "combine"]


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def kernel_source_hash(*names):
    """sha256[:16] over the named csrc files."""
    h = hashlib.sha256()
    for name in names:
        with open(os.path.join(ROOT, "learned_sparse_kv_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def stored_traffic(profile, src, src_hash):
    """HBM bytes per launch of the roofline kernel from the committed rocprofv3
    counter summary profiles/<profile>, or None when absent or taken on a
    different version of its source file `src`."""
    path = os.path.join(ROOT, "profiles", profile)
    if not os.path.exists(path):
        return None
    txt = open(path).read()
    m_hash = re.search(re.escape(src) + r" sha256\[:16\]:\s*([0-9a-f]+)", txt)
    m_bytes = re.search(r"hbm_bytes_per_dispatch:\s*([0-9.eE+]+)", txt)
    if not m_hash or not m_bytes or m_hash.group(1) != src_hash:
        return None
    return float(m_bytes.group(1))


def cpu_info():
    """(CPU model from /proc/cpuinfo, logical CPUs, CPUs this process may run on)."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count() or 1
    return model, os.cpu_count(), avail


def oracle_threads():
    """Threads for the CPU baseline: the CPUs this process may use, at most 16 (the
    host share of one GPU on the box)."""
    return max(1, min(16, cpu_info()[2]))


def run_threads(fn, n):
    """Runs fn(i) on n threads (the oracle's ctypes calls release the GIL); returns wall seconds."""
    import threading
    errs = []

    def body(i):
        try:
            fn(i)
        except BaseException as e:   # re-raised in the caller
            errs.append(e)
    ths = [threading.Thread(target=body, args=(i,)) for i in range(n)]
    t0 = time.perf_counter()
    for t in ths:
        t.start()
    for t in ths:
        t.join()
    if errs:
        raise errs[0]
    return time.perf_counter() - t0


def copy_calibration():
    """A plain device copy of known size, for scaling FETCH_SIZE / WRITE_SIZE."""
    import torch
    n = 256 << 20
    a = torch.empty(n // 4, dtype=torch.float32, device="cuda:0").fill_(1.0)
    b = torch.empty_like(a)
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    log(f"copy calibration: 5 copies of {n} bytes (read {n}, write {n} per dispatch)")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=32)
    ap.add_argument("--workload", default="swap_1m")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-steps", type=int, default=28)
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--no-kvswap", action="store_true", help="skip the KVSwap leg of the 1M run")
    ap.add_argument("--graph", type=int, default=0,
                    help="time eager launches (0, the default: faster here, the host keeps ahead of the GPU) "
                         "or HIP-graph replays, one graph per step (1)")
    ap.add_argument("--schedule", choices=["lookahead", "sync"], default="lookahead",
                    help="lookahead: each step's row copy and attention share launches with the next step's "
                         "score and selection; sync: score, select, stage and attend one after another")
    ap.add_argument("--cold", choices=["host", "hbm"], default=None,
                    help="override where the workload's cold pools live (diagnostic; default: the workload's)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this build runs the decode path on a single MI355X "
              "(the multi-GPU sharding is a design, not code); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if args.copy_calibration:
        copy_calibration()
        return

    import lsa_inputs as L
    from learned_sparse_kv_amd import lsa
    from learned_sparse_kv_amd.workload import DeviceWorkload

    if args.workload in L.KVSWAP_WORKLOADS:
        return bench_kvswap(args)
    wl = L.WORKLOADS[args.workload]
    if args.cold:
        wl = wl.replace(cold=args.cold)
    K, Wm = args.steps, args.warmup
    log(f"workload {wl.name}: ctx={wl.ctx} B={wl.batch} N={wl.n_src} layers={wl.layer_ratios} "
        f"k={wl.k} S={wl.gpu_chunks} cold={wl.cold} keys={wl.key_dtype} kv={wl.kv_dtype}")
    t0 = time.time()
    dw = DeviceWorkload(wl, keep_host=not args.no_cpu_baseline, log=log)
    dw.make_steps(Wm + K + 2)
    log(f"set-up {time.time() - t0:.1f}s")

    def periodic_region(period):
        """The lookahead schedule with one prediction per window of `period` steps:
        lsa_lookahead_step on the last step of a window, lsa_lookahead_attend on the
        others (eager launches, pools start empty).  Returns ms per step."""
        dw.reset_pools()
        dw.lookahead_prime(0)

        def run(t):
            if (t + 1) % period == 0:
                dw.lookahead_step(t, t_next=t + 1)
            else:
                dw.lookahead_attend(t)
        for t in range(Wm):
            run(t)
        # descriptors marshalled before the timed region, as in timed_region
        dw.prepare_periodic(range(Wm, Wm + K), period)
        torch.cuda.synchronize()
        t_start = time.perf_counter()
        for t in range(Wm, Wm + K):
            dw.run_prepared(t)
        t_enq = time.perf_counter()
        torch.cuda.synchronize()
        t_end = time.perf_counter()
        ms = (t_end - t_start) * 1e3 / K
        log(f"lookahead, period {period} (eager): host enqueue {(t_enq - t_start) * 1e6 / K:.1f} us/step, "
            f"wall {ms * 1e3:.1f} us/step")
        return ms

    def timed_region(schedule, use_graph):
        """Warm up, then time K steps of the schedule, launched eagerly or as HIP-graph
        replays (one graph per step); the pools start empty.  Returns (ms per step, LRU
        stats before, after)."""
        dw.reset_pools()
        la = schedule == "lookahead"
        if la:
            dw.lookahead_prime(0)
        eager = dw.lookahead_step if la else dw.step
        for t in range(Wm):
            eager(t)
        torch.cuda.synchronize()
        if use_graph:
            if la:
                dw.capture_lookahead(range(Wm, Wm + K))
            else:
                dw.capture(range(Wm, Wm + K))
            run = dw.replay
        else:
            # descriptors marshalled before the timed region
            if la:
                dw.prepare_lookahead(range(Wm, Wm + K))
            else:
                dw.prepare_steps(range(Wm, Wm + K))
            run = dw.run_prepared
        s0 = [p.stats() for p in dw.pools]
        torch.cuda.synchronize()
        t_start = time.perf_counter()
        for t in range(Wm, Wm + K):
            run(t)
        t_enq = time.perf_counter()
        torch.cuda.synchronize()
        t_end = time.perf_counter()
        log(f"{schedule} ({'graph' if use_graph else 'eager'}): host enqueue {(t_enq - t_start) * 1e6 / K:.1f} "
            f"us/step, wall {(t_end - t_start) * 1e6 / K:.1f} us/step")
        s1 = [p.stats() for p in dw.pools]
        dw.graphs = {}
        return (t_end - t_start) * 1e3 / K, s0, s1

    # ---- timed regions: K steps of each schedule, launched as --graph says; the
    # chosen schedule is also timed with the other launch mode, for context.
    # `value` is the chosen schedule's
    other = "sync" if args.schedule == "lookahead" else "lookahead"
    use_graph = args.graph != 0
    other_ms, _, _ = timed_region(other, use_graph)
    alt_ms, _, _ = timed_region(args.schedule, not use_graph)
    ms_per_step, stats0, stats1 = timed_region(args.schedule, use_graph)
    value = 1e3 / ms_per_step
    periodic = {str(d): {"value": round(1e3 / m, 2), "ms_per_step": round(m, 5)}
                for d, m in ((d, periodic_region(d)) for d in (2, 4, 8))}
    # the same steps with the keys loaded non-temporally (lsa_ctx_set_key_policy):
    # in this loop the one indexer layer's keys would otherwise stay in the
    # last-level cache from step to step
    dw.ctx.set_key_policy(True)
    nt_ms = {sch: timed_region(sch, use_graph)[0] for sch in ("lookahead", "sync")}
    dw.ctx.set_key_policy(False)

    # ---- kernel-timed region: the same K steps of the synchronous schedule
    # launched eagerly with HIP events around every kernel on the launch stream
    dw.reset_pools()
    for t in range(Wm):
        dw.step(t)
    dw.ctx.set_timing(True)
    dw.ctx.timing_read()
    for t in range(Wm, Wm + K):
        dw.step(t)
    ktimes = dw.ctx.timing_read()
    dw.ctx.set_timing(False)
    # the attention with every row resident: after the last step once more (all rows
    # are in their slots now, so the attention reads HBM only), RA attention-only
    # calls (lsa_decode_attend) back to back between two HIP events
    t_last_step = Wm + K - 1
    dw.step(t_last_step)
    RA = 64
    st_a = torch.cuda.current_stream()
    ea0, ea1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    dw.attend(t_last_step)
    ea0.record(st_a)
    for _ in range(RA):
        dw.attend(t_last_step)
    ea1.record(st_a)
    torch.cuda.synchronize()
    att_res_ms = ea0.elapsed_time(ea1) / RA

    # ---- roofline region: the dominant kernel (fm_score) alone, R launches back to
    # back on the launch stream (torch's current stream, which lsa calls use)
    # between two HIP events, so no per-launch event overhead enters its time
    R = 64
    st = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_last = Wm + K - 1
    lsa.score(dw.keys, dw.q_idx[t_last], dw.w_idx[t_last], dw.scores, ensemble=wl.ensemble, key_scales=dw.key_scales)
    ev0.record(st)
    for _ in range(R):
        lsa.score(dw.keys, dw.q_idx[t_last], dw.w_idx[t_last], dw.scores, ensemble=wl.ensemble, key_scales=dw.key_scales)
    ev1.record(st)
    torch.cuda.synchronize()
    score_ms = ev0.elapsed_time(ev1) / R

    # the same launch with its keys in HBM: the keys are copied until the other
    # copies hold at least 512 MiB (twice the 256 MiB last-level cache), and R
    # launches rotate over the copies back to back between two HIP events, so
    # every launch finds its keys evicted by the launches before it and no
    # per-launch event overhead enters the average
    key_bytes = dw.keys.numel() * dw.keys.element_size() + \
        (dw.key_scales.numel() if dw.key_scales is not None else 0)
    n_copies = 1 + -(-(512 << 20) // key_bytes)
    copies = [(dw.keys, dw.key_scales)] + [
        (dw.keys.clone(), dw.key_scales.clone() if dw.key_scales is not None else None) for _ in range(n_copies - 1)]
    for i in range(2 * n_copies):
        kc, ks = copies[i % n_copies]
        lsa.score(kc, dw.q_idx[t_last], dw.w_idx[t_last], dw.scores, ensemble=wl.ensemble, key_scales=ks)
    RC = max(R, 4 * n_copies)
    ev0.record(st)
    for i in range(RC):
        kc, ks = copies[i % n_copies]
        lsa.score(kc, dw.q_idx[t_last], dw.w_idx[t_last], dw.scores, ensemble=wl.ensemble, key_scales=ks)
    ev1.record(st)
    torch.cuda.synchronize()
    cold_ms = ev0.elapsed_time(ev1) / RC
    del copies

    # single launches, each bracketed by its own HIP events after a 512 MiB read
    # (a sum, so no dirty lines are left to write back) that evicts the keys
    flush = torch.zeros(64 << 20, dtype=torch.int64, device="cuda")
    RS = 16
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(RS)]
    for e0, e1 in evs:
        flush.sum()
        e0.record(st)
        lsa.score(dw.keys, dw.q_idx[t_last], dw.w_idx[t_last], dw.scores, ensemble=wl.ensemble, key_scales=dw.key_scales)
        e1.record(st)
    torch.cuda.synchronize()
    single_all = sorted(e0.elapsed_time(e1) for e0, e1 in evs)
    single_ms = sum(single_all) / RS

    # ---- the indexers' query/weight projection (hidden[4096] -> q, w) at this
    # workload's indexer shape, bf16 weights: back to back behind a GPU sleep that
    # covers the host's launch calls, and after the cache-evicting read
    proj = project_timing(wl, flush)
    del flush

    # ---- adaptive staging capacity (synchronous steps): the swapping pools start at
    # top-k slots and adapt every 8 steps toward an 80 % hit rate (the page's own
    # alarm levels, 50 % misses or 10 MB of H2D per step, never fire on this
    # workload); and the time of one shrink of every swapping pool
    adaptive = adaptive_capacity(dw, wl, Wm + K)

    # ---- the metric's other context length: the 256K threshold workload (batch 4,
    # bf16 rows), both schedules launched eagerly, K steps each
    ctx256 = other_context("thresh_256k", K, Wm, parity_steps=0 if args.no_cpu_baseline else 2) \
        if wl.name.startswith("swap_1m") else None
    # the pages' whole sparse-layer stack at 1M: 41 layers (20 ratio-4, 21 ratio-128)
    # on one selection per step, 11.1 GB of pinned-host cold pools
    stack41 = other_context("stack_1m_41", min(K, 64), min(Wm, 16), parity_steps=0 if args.no_cpu_baseline else 1) \
        if wl.name == "swap_1m" else None
    kvs = kvswap_measure(L.KVSWAP_WORKLOADS["kvswap_32k"], min(K, 32), min(Wm, 8),
                         parity_steps=0 if args.no_cpu_baseline else 2) \
        if wl.name.startswith("swap_1m") and not args.no_kvswap else None
    # the rolling buffer of the KVSwap article's section 3.2 (400 slots, top 200,
    # recency and importance weighed equally, 70 % high-water mark)
    kvs_wr = kvswap_measure(L.KVSWAP_WORKLOADS["kvswap_32k_wr"], min(K, 32), min(Wm, 8),
                            parity_steps=0 if args.no_cpu_baseline else 2) \
        if wl.name.startswith("swap_1m") and not args.no_kvswap else None

    # ---- algorithmic bytes (per launch)
    # a key row (plus its E8M0 block scales for the MX dtypes) read, a score written
    key_row = wl.dk * L.DTYPE_BYTES[wl.key_dtype] + (wl.dk // 32 if wl.key_dtype in L.MX_DTYPES else 0)
    kv_b = L.DTYPE_BYTES[wl.kv_dtype]
    score_bytes = int(wl.batch * wl.n_src * (key_row + 4))
    avg = {k: (ktimes[k][0] / ktimes[k][1] if ktimes[k][1] else 0.0) for k in KERNELS}
    score_gbs = score_bytes / (score_ms * 1e-3) / 1e9
    hits = sum(s1["hits"] - s0["hits"] for s0, s1 in zip(stats0, stats1))
    misses = sum(s1["misses"] - s0["misses"] for s0, s1 in zip(stats0, stats1))
    # rows copied from the cold pools into slots per timed step (over PCIe when
    # the cold pools are in pinned host memory)
    fetch_bytes = sum(s1["h2d_bytes"] - s0["h2d_bytes"] for s0, s1 in zip(stats0, stats1)) / K
    # attention bytes: window + staged rows of every layer and sequence, read once
    n_rows = dw.n_rows.cpu().numpy()
    attend_bytes = float(n_rows.sum()) * wl.kv_dim * kv_b
    # fm_score with its keys from HBM (the rotating launches) + the attention over
    # resident rows (back to back); also with the cache-assisted score time (inside a
    # decode loop one layer's keys stay in the last-level cache from step to step)
    sa_ms = cold_ms + att_res_ms
    sa_frac = (score_bytes + attend_bytes) / (sa_ms * 1e-3) / 1e9 / HBM_PEAK_GBS
    sa_frac_warm = (score_bytes + attend_bytes) / ((score_ms + att_res_ms) * 1e-3) / 1e9 / HBM_PEAK_GBS

    src_hash = kernel_source_hash("fm_score.hip")
    traffic = stored_traffic(f"fm_score_{wl.name}_pmc.txt", "fm_score.hip", src_hash)
    cold_gbs = score_bytes / (cold_ms * 1e-3) / 1e9
    roofline = {"bound": "hbm", "achieved": round(cold_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(cold_gbs / HBM_PEAK_GBS, 4), "traffic": traffic, "kernel": "fm_score",
                "algorithmic_bytes_per_launch": score_bytes, "avg_launch_us": round(cold_ms * 1e3, 2),
                "timing": f"{RC} back-to-back launches between HIP events on the launch stream, rotating over "
                          f"{n_copies} copies of the keys ({n_copies * key_bytes / 1e6:.0f} MB): each launch reads "
                          "its keys from HBM, the copies read since its last use having evicted them",
                "single_launch_after_evict": {
                    "avg_launch_us": round(single_ms * 1e3, 2), "median_launch_us": round(single_all[RS // 2] * 1e3, 2),
                    "timing": f"{RS} launches, each bracketed by its own HIP events after a 512 MiB read; the "
                              "events add their own overhead to each launch"},
                "cache_assisted": {"avg_launch_us": round(score_ms * 1e3, 2), "achieved": round(score_gbs, 1),
                                   "frac": round(score_gbs / HBM_PEAK_GBS, 4),
                                   "timing": f"{R} back-to-back launches between HIP events: part of the keys "
                                             "stay in the 256 MiB last-level cache between launches"}}

    # ---- CPU baseline: the oracle on a bounded sample of the same steps, and a
    # parity check of the GPU on those steps (pools reset on both sides)
    cpu = None
    parity = None
    if not args.no_cpu_baseline:
        import oracle
        n_s = max(1, min(args.cpu_sample_steps, Wm + K))
        ref = oracle.DecodeState(wl, dw.windows, dw.stores)
        dw.reset_pools()
        sel_ok, max_err = True, 0.0
        outs_ref = []
        tc0 = time.perf_counter()
        cpu_s = 0.0
        for t in range(n_s):
            dw.step(t)
            torch.cuda.synchronize()
            c0 = time.perf_counter()
            want = ref.step(dw.keys_np, dw.q_idx_np[t], dw.w_idx_np[t], dw.q_attn_np[t])
            cpu_s += time.perf_counter() - c0
            outs_ref.append(want["out"])
            cnt = dw.count.cpu().numpy()
            sel = dw.sel.cpu().numpy()
            out = dw.out.cpu().numpy()
            phys = dw.phys.cpu().numpy()
            for b in range(wl.batch):
                sel_ok &= bool(np.array_equal(sel[b, :cnt[b]], want["sel"][b]))
                for l in range(wl.n_layers):
                    w_ = want["out"][l][b]
                    den = np.maximum(np.abs(w_).max(axis=1), 1e-30)
                    max_err = max(max_err, float((np.abs(out[l, b] - w_).max(axis=1) / den).max()))
                    n = want["phys"][l][b].size
                    sel_ok &= bool(np.array_equal(phys[l, b, :n], want["phys"][l][b]))
        # the lookahead schedule over the same steps (the oracle's outputs above)
        dw.reset_pools()
        dw.lookahead_prime(0)
        la_err = 0.0
        for t in range(n_s):
            dw.lookahead_step(t)
            torch.cuda.synchronize()
            out = dw.out.cpu().numpy()
            for b in range(wl.batch):
                for l in range(wl.n_layers):
                    w_ = outs_ref[t][l][b]
                    den = np.maximum(np.abs(w_).max(axis=1), 1e-30)
                    la_err = max(la_err, float((np.abs(out[l, b] - w_).max(axis=1) / den).max()))
        tol = 1e-5 if wl.kv_dtype == "f32" else 2e-2
        parity = {"steps": n_s, "selected_sets_and_rows_identical": sel_ok, "max_rel_err": max_err,
                  "lookahead_max_rel_err": la_err, "tolerance": tol,
                  "pass": bool(sel_ok and max_err <= tol and la_err <= tol)}
        log(f"cpu baseline (1 thread) {n_s / cpu_s:.3f} steps/s over {n_s} steps "
            f"({time.perf_counter() - tc0:.1f}s incl. GPU replay)")
        # throughput on the host's cores: independent oracle instances (fresh pools,
        # the same steps), one per thread
        T = oracle_threads()
        n_t = 3

        def one(i):
            st = oracle.DecodeState(wl, dw.windows, dw.stores)
            for t in range(n_t):
                st.step(dw.keys_np, dw.q_idx_np[t], dw.w_idx_np[t], dw.q_attn_np[t])
        wall = run_threads(one, T)
        model, n_cpu, avail = cpu_info()
        cpu = {"value": round(T * n_t / wall, 4), "unit": "steps/s", "cores": T, "kind": "oracle",
               "sample": f"{T} threads, each an independent oracle over steps 0..{n_t - 1} of {wl.name} (score of "
                         f"all {wl.batch}x{wl.n_src} entries, select, {wl.n_layers} layers of stage + attend), "
                         f"{wall:.1f}s wall; unchanged C++ oracle, its calls release the GIL",
               "single_thread": {"value": round(n_s / cpu_s, 4), "steps": n_s, "seconds": round(cpu_s, 1)},
               "cpu_model": model, "cpus": n_cpu, "cpus_available": avail}
        log(f"cpu baseline ({T} threads) {cpu['value']} steps/s, {wall:.1f}s wall")

    res = {
        "metric": METRIC, "value": round(value, 2), "unit": "steps/s", "n_gpus": 1, "steps": K, "warmup": Wm,
        "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": wl.kv_dtype if wl.kv_dtype == wl.key_dtype else f"{wl.key_dtype}/{wl.kv_dtype}",
        "data": "synthetic (seeded 1/8-grid values)",
        "config": {"workload": wl.name, "ctx": wl.ctx, "batch": wl.batch, "src_entries": wl.n_src,
                   "sparse_layer_ratios": list(wl.layer_ratios), "indexers": f"{wl.n_idx}x{wl.heads}x{wl.dk}",
                   "select": f"{wl.mode} k={wl.k}", "gpu_chunks": wl.gpu_chunks, "cold_pool": wl.cold,
                   "window": wl.window, "kv_dim": wl.kv_dim, "attn_heads": wl.hq,
                   "step": "score+select+stage+fetch+attend",
                   "schedule": args.schedule,
                   "launch": "hip graph per step" if use_graph else "eager"},
        other + "_schedule": {"value": round(1e3 / other_ms, 2), "ms_per_step": round(other_ms, 5)},
        ("graph" if not use_graph else "eager") + "_launch": {"value": round(1e3 / alt_ms, 2),
                                                             "ms_per_step": round(alt_ms, 5)},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "project": proj,
        "adaptive_capacity": adaptive,
        "ctx_256k": ctx256,
        "stack_41_layers": stack41,
        "kvswap_32k": kvs,
        "kvswap_32k_wr": kvs_wr,
        "key_policy_non_temporal": {
            sch: {"value": round(1e3 / m, 2), "ms_per_step": round(m, 5)} for sch, m in nt_ms.items()},
        "periodic_indexer": {"schedule": "lookahead, eager; one prediction per window of `period` steps "
                                         "(lsa_lookahead_step on a window's last step, lsa_lookahead_attend "
                                         "on the others)", "by_period": periodic},
        "kernels_us_events": {k: round(avg[k] * 1e3, 2) for k in KERNELS},
        "score_attend_hbm_frac": round(sa_frac, 4),
        "score_attend_frac_cache_assisted": round(sa_frac_warm, 4),
        "attend_resident": {"us": round(att_res_ms * 1e3, 2), "bytes": int(attend_bytes),
                            "achieved": round(attend_bytes / (att_res_ms * 1e-3) / 1e9, 1),
                            "timing": f"{RA} attention-only calls (lsa_decode_attend) over the last step's "
                                      "rows, all resident, back to back between two HIP events"},
        "hit_rate": round(hits / max(1, hits + misses), 4),
        "fetch": {"bytes_per_step": round(fetch_bytes), "cold_pool": wl.cold,
                  "gbs_over_the_step": round(fetch_bytes / (ms_per_step * 1e-3) / 1e9, 2),
                  "note": "missed rows copied from the cold pools into their slots per timed step; in the "
                          "lookahead schedule the score launch carries the copy, so a step takes at least the "
                          "copy at the link's rate"},
        "parity": parity,
        "fm_score_src": src_hash,
    }
    print(json.dumps(res), flush=True)


def other_context(name, K, Wm, parity_steps=0):
    """Decode steps/s of another workload (its own set-up; pools start empty; eager
    launches; the lookahead schedule with descriptors marshalled beforehand), and a
    parity check of `parity_steps` synchronous steps against the oracle."""
    import numpy as np
    import torch

    import lsa_inputs as L
    from learned_sparse_kv_amd.workload import DeviceWorkload

    wl = L.WORKLOADS[name]
    dw = DeviceWorkload(wl, keep_host=parity_steps > 0, log=log)
    dw.make_steps(Wm + K + 2)
    res = {"workload": name, "ctx": wl.ctx, "batch": wl.batch, "src_entries": wl.n_src,
           "sparse_layer_ratios": list(wl.layer_ratios), "select": f"{wl.mode} cap {wl.k}", "kv_dtype": wl.kv_dtype,
           "key_dtype": wl.key_dtype, "cold_pool": wl.cold}
    for schedule in ("lookahead", "sync"):
        dw.reset_pools()
        la = schedule == "lookahead"
        if la:
            dw.lookahead_prime(0)
        eager = dw.lookahead_step if la else dw.step
        for t in range(Wm):
            eager(t)
        if la:
            dw.prepare_lookahead(range(Wm, Wm + K))
        else:
            dw.prepare_steps(range(Wm, Wm + K))
        eager = dw.run_prepared
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for t in range(Wm, Wm + K):
            eager(t)
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / K
        res[schedule] = {"value": round(1e3 / ms, 2), "unit": "steps/s", "ms_per_step": round(ms, 5)}
        log(f"{name} {schedule} (eager): {ms * 1e3:.1f} us/step")
    if parity_steps:
        import oracle
        ref = oracle.DecodeState(wl, dw.windows, dw.stores)
        dw.reset_pools()
        ok, err = True, 0.0
        for t in range(parity_steps):
            dw.step(t)
            torch.cuda.synchronize()
            want = ref.step(dw.keys_np, dw.q_idx_np[t], dw.w_idx_np[t], dw.q_attn_np[t])
            cnt, sel, out = dw.count.cpu().numpy(), dw.sel.cpu().numpy(), dw.out.cpu().numpy()
            for b in range(wl.batch):
                ok &= bool(np.array_equal(sel[b, :cnt[b]], want["sel"][b]))
                for l in range(wl.n_layers):
                    w_ = want["out"][l][b]
                    den = np.maximum(np.abs(w_).max(axis=1), 1e-30)
                    err = max(err, float((np.abs(out[l, b] - w_).max(axis=1) / den).max()))
        tol = 1e-5 if wl.kv_dtype == "f32" else 2e-2
        res["parity"] = {"steps": parity_steps, "selected_sets_identical": ok, "max_rel_err": err,
                         "tolerance": tol, "pass": bool(ok and err <= tol),
                         "note": f"both sides read the same {wl.kv_dtype} rows and accumulate in fp32 / double; "
                                 "max_rel_err is the observed difference"}
        log(f"{name} parity over {parity_steps} steps: sets {ok}, max rel err {err:.3g}")
    del dw
    torch.cuda.empty_cache()
    return res


def adaptive_capacity(dw, wl, n_steps):
    """lsa_pool_adapt over the synchronous schedule; None when no pool swaps."""
    import torch
    sw = [p for p in dw.pools if p.swap]
    if not sw:
        return None
    full = sw[0].capacity()
    every, n = 8, min(n_steps, 64)
    dw.reset_pools()
    for p in sw:
        p.set_capacity(wl.k)
    caps, rates = [], []
    s_prev = [p.stats() for p in sw]
    for t in range(n):
        dw.step(t)
        if t % every == every - 1:
            s_now = [p.stats() for p in sw]
            h = sum(b["hits"] - a["hits"] for a, b in zip(s_prev, s_now))
            m = sum(b["misses"] - a["misses"] for a, b in zip(s_prev, s_now))
            rates.append(round(h / max(1, h + m), 4))
            s_prev = s_now
            caps.append([p.adapt(every, wl.k, full, 128, 0.2, 10e6, 0.05) for p in sw][0])
    # one shrink of every swapping pool (full -> k + k/4: evictions and moved rows;
    # its kernel time is in the kernel trace as pool_shrink_kernel)
    for p in sw:
        p.set_capacity(full)
    dw.reset_pools()
    for t in range(8):
        dw.step(t)
    for p in sw:
        p.set_capacity(wl.k + wl.k // 4)
    torch.cuda.synchronize()
    for p in sw:
        p.set_capacity(full)
    dw.reset_pools()
    return {"policy": f"start at {wl.k} slots; every {every} sync steps: +128 above 20 % misses or 10 MB "
                      f"H2D per step, -128 below 5 % misses, within [{wl.k}, {full}]",
            "hit_rate_per_window": rates, "capacity_after_window": caps,
            "shrink": f"{len(sw)} pools, {full} -> {wl.k + wl.k // 4} slots after 8 steps, one launch each"}


def project_timing(wl, flush):
    """lsa_project at the workload's indexer shape from d_model 4096, bf16 weights."""
    import torch
    import lsa_inputs as L
    from learned_sparse_kv_amd import lsa
    from learned_sparse_kv_amd.workload import to_device
    wq, ww = L.projection_weights(wl)
    twq = to_device(L.encode(wq, "bf16"), "bf16", "cuda")
    tww = to_device(L.encode(ww, "bf16"), "bf16", "cuda")
    hid = torch.from_numpy(__import__("numpy").stack([L.hidden_state(wl, b, 0) for b in range(wl.batch)])).cuda()
    q = torch.empty((wl.batch, wl.n_idx, wl.heads, wl.dk), device="cuda")
    w = torch.empty((wl.batch, wl.n_idx, wl.heads), device="cuda")
    lsa.project(hid, twq, tww, q, w)
    R = 32
    st = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    sleep = getattr(torch.cuda, "_sleep", None)
    if sleep is not None:
        sleep(2_000_000)   # keeps the GPU busy while the launches are enqueued
    e0.record(st)
    for _ in range(R):
        lsa.project(hid, twq, tww, q, w)
    e1.record(st)
    torch.cuda.synchronize()
    warm_ms = e0.elapsed_time(e1) / R
    cold = []
    for _ in range(8):
        flush.sum()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(st)
        lsa.project(hid, twq, tww, q, w)
        b.record(st)
        torch.cuda.synchronize()
        cold.append(a.elapsed_time(b))
    cold_ms = sorted(cold)[len(cold) // 2]
    nbytes = (wq.size + ww.size) * 2 + hid.numel() * 4 + (q.numel() + w.numel()) * 4
    gbs = lambda ms: nbytes / (ms * 1e-3) / 1e9
    return {"shape": f"{wl.batch}x4096 -> {wl.n_idx}x{wl.heads}x({wl.dk}+1), bf16 weights",
            "algorithmic_bytes_per_launch": int(nbytes),
            "avg_launch_us": round(warm_ms * 1e3, 2), "achieved": round(gbs(warm_ms), 1),
            "frac": round(gbs(warm_ms) / HBM_PEAK_GBS, 4),
            "cold_cache": {"avg_launch_us": round(cold_ms * 1e3, 2), "achieved": round(gbs(cold_ms), 1),
                           "frac": round(gbs(cold_ms) / HBM_PEAK_GBS, 4)},
            "timing": f"{R} back-to-back launches between HIP events (queued behind a GPU sleep); "
                      "cold: median of 8 single launches after the 512 MiB read"}


def kvswap_segments(wl, n=16):
    """n segments spread over layers, groups and sequences (distinct; pool indices
    l * groups + g above 16 included)."""
    segs = []
    i = 0
    while len(segs) < min(n, wl.n_seg):
        l = (i * 7 + 3) % wl.layers
        g = (i * 3 + 1) % wl.groups
        b = (i * 5 + 2) % wl.batch
        s_ = wl.seg(l, g, b)
        if s_ not in segs:
            segs.append(s_)
        i += 1
    return sorted(segs)


def kvswap_measure(wl, K, Wm, parity_steps=2, n_parity_segs=16):
    """KVSwap step at its workload: eager steps/s, per-kernel event times, the
    score+attention HBM fraction, and (parity_steps > 0) the GPU's selections and
    outputs of n_parity_segs sampled segments against the oracle, one thread per
    segment, which also gives the CPU baseline."""
    import numpy as np
    import torch

    from learned_sparse_kv_amd.kvswap_workload import DeviceKVSwap

    log(f"workload {wl.name}: ctx={wl.ctx} B={wl.batch} layers={wl.layers} groups={wl.groups}x{wl.group_heads}x"
        f"{wl.head_dim} rank={wl.rank} k={wl.k} slots={wl.slots} segments={wl.n_seg}")
    t0 = time.time()
    dw = DeviceKVSwap(wl, log=log)
    dw.make_steps(max(Wm + K, parity_steps))
    # pools that weigh importance read the step's scores; otherwise the step gets
    # no scores buffer and scores and selects each segment in one launch
    fused = wl.recency_w >= 100
    log(f"set-up {time.time() - t0:.1f}s")
    for t in range(Wm):
        dw.step(t, fused=fused)
    torch.cuda.synchronize()
    stats0 = [p.stats() for p in dw.pools]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for t in range(Wm, Wm + K):
        dw.step(t, fused=fused)
    torch.cuda.synchronize()
    t_end = time.perf_counter()
    ms_per_step = (t_end - t_start) * 1e3 / K
    stats1 = [p.stats() for p in dw.pools]
    # per-kernel times: the same steps again with HIP events on the launch stream
    dw.ctx.set_timing(True)
    dw.ctx.timing_read()
    stats_e0 = [p.stats() for p in dw.pools]
    for t in range(Wm, Wm + K):
        dw.step(t, fused=fused)
    kt = dw.ctx.timing_read()
    stats_e1 = [p.stats() for p in dw.pools]
    dw.ctx.set_timing(False)
    names = ["score", "select", "stage", "attend"]
    avg = {k: (kt[k][0] / kt[k][1] if kt[k][1] else 0.0) for k in names}
    n_seg, T, r = wl.n_seg, wl.ctx, wl.rank
    # U, V and q read; the scores written (not when fused)
    scan_bytes = n_seg * T * (2 * r + (0 if fused else 4)) + n_seg * (wl.C * r * 2 + wl.C * 4)
    n_rows = dw.n_rows.cpu().numpy()
    attend_bytes = float(n_rows.sum()) * wl.row_elems * 2
    hits = sum(b["hits"] - a["hits"] for a, b in zip(stats0, stats1))
    misses = sum(b["misses"] - a["misses"] for a, b in zip(stats0, stats1))
    # rows that missed in the event-timed steps are read from the cold store and
    # also written into their slots: that write is part of the attention's traffic
    misses_ev = sum(b["misses"] - a["misses"] for a, b in zip(stats_e0, stats_e1)) / K
    attend_written = misses_ev * wl.row_elems * 2
    score_gbs = scan_bytes / (avg["score"] * 1e-3) / 1e9
    attend_gbs = attend_bytes / (avg["attend"] * 1e-3) / 1e9
    attend_rw_gbs = (attend_bytes + attend_written) / (avg["attend"] * 1e-3) / 1e9
    sa_frac = (scan_bytes + attend_bytes + attend_written) / ((avg["score"] + avg["attend"]) * 1e-3) / 1e9 / HBM_PEAK_GBS
    roofline = {"bound": "hbm", "achieved": round(score_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(score_gbs / HBM_PEAK_GBS, 4),
                "traffic": (stored_traffic(f"{wl.name}_pmc.txt", "lowrank.hip", kernel_source_hash("lowrank.hip"))
                            if fused else None),
                "kernel": ("lowrank_select (p, U scan and top-k in one launch, no scores written)" if fused
                           else "lowrank_p + lowrank_scan"),
                "algorithmic_bytes_per_launch": scan_bytes, "avg_launch_us": round(avg["score"] * 1e3, 2)}
    cpu = parity = None
    if parity_steps:
        import oracle
        segs = kvswap_segments(wl, n_parity_segs)
        ref = oracle.KVSwapState(wl, segs)
        dw.reset_pools()
        inputs = {}

        def load(i):
            inputs[segs[i]] = dw.host_inputs(segs[i], 0)
        run_threads(load, len(segs))
        ok, max_err, cpu_wall, seg_steps = True, 0.0, 0.0, 0
        errs = {}
        for t in range(parity_steps):
            dw.step(t, fused=fused)
            torch.cuda.synchronize()
            sel, cnt, out = dw.sel.cpu().numpy(), dw.count.cpu().numpy(), dw.out.cpu().numpy()
            wants = {}

            def one(i):
                sg = segs[i]
                U, S, V, _, cold = inputs[sg]
                wants[sg] = ref.step(sg, U, S, V, dw.q_np[t, sg], cold)
            cpu_wall += run_threads(one, len(segs))
            seg_steps += len(segs)
            for sg in segs:
                want = wants[sg]
                ok &= bool(cnt[sg] == want["sel"].size and np.array_equal(sel[sg, :cnt[sg]], want["sel"]))
                den = np.maximum(np.abs(want["out"]).max(axis=1), 1e-30)
                errs[sg] = max(errs.get(sg, 0.0), float((np.abs(out[sg] - want["out"]).max(axis=1) / den).max()))
        max_err = max(errs.values())
        pool_ids = sorted({sg // wl.batch for sg in segs})
        parity = {"steps": parity_steps, "segments": segs, "pools": pool_ids, "selected_sets_identical": ok,
                  "max_rel_err": max_err, "tolerance": 2e-2, "pass": bool(ok and max_err <= 2e-2),
                  "note": "f16 K/V on both sides; the tolerance is the f16 storage bound, max_rel_err the "
                          "observed difference"}
        model, n_cpu, avail = cpu_info()
        per_seg = cpu_wall / seg_steps * len(segs)   # seconds per segment-step on one thread
        cpu = {"value": round(len(segs) / (per_seg * wl.n_seg), 6), "unit": "steps/s", "cores": len(segs),
               "kind": "oracle",
               "sample": f"{parity_steps} steps x {len(segs)} of the {wl.n_seg} group segments (score over {T} "
                         f"positions, top-{wl.k}, LRU, {wl.group_heads}-head attention), one thread per segment, "
                         f"{cpu_wall:.1f}s wall; scaled to a whole step; unchanged C++ oracle",
               "cpu_model": model, "cpus": n_cpu, "cpus_available": avail}
        log(f"{wl.name} parity over {parity_steps} steps x {len(segs)} segments: sets {ok}, max rel err {max_err:.3g}")
    res = {
        "metric": f"KVSwap decode steps/s (32K ctx, batch 16, 32 layers x 8 groups of 4 heads, top-{wl.k})",
        "value": round(1e3 / ms_per_step, 3), "unit": "steps/s", "steps": K, "warmup": Wm,
        "ms_per_step": round(ms_per_step, 4),
        "config": {"workload": wl.name, "ctx": T, "batch": wl.batch, "layers": wl.layers, "groups": wl.groups,
                   "group_heads": wl.group_heads, "head_dim": wl.head_dim, "rank": r, "k": wl.k,
                   "slots": wl.slots, "segments": n_seg, "launch": "eager",
                   "score_and_select": "one launch per step, no scores written" if fused else "two launches",
                   "stage_and_attend": ("one launch per step (each segment's stage, then its attention, in one "
                                        "workgroup); the attend figures include the stage"
                                        if avg["stage"] == 0.0 else "two launches"),
                   "replacement": {"recency_weight": wl.recency_w, "high_water": wl.high_water}},
        "roofline": roofline,
        "attend": {"achieved_gbs": round(attend_gbs, 1), "bytes_per_launch": attend_bytes,
                   "bytes_written_per_launch": round(attend_written), "achieved_gbs_read_and_written": round(attend_rw_gbs, 1),
                   "avg_launch_us": round(avg["attend"] * 1e3, 2)},
        "score_attend_hbm_frac": round(sa_frac, 4),
        "cpu_baseline": cpu,
        "kernels_us": {k: round(avg[k] * 1e3, 2) for k in names},
        "hit_rate": round(hits / max(1, hits + misses), 4),
        "parity": parity,
    }
    log(f"{wl.name}: {ms_per_step:.3f} ms/step")
    del dw
    torch.cuda.empty_cache()
    return res


def bench_kvswap(args):
    """KVSwap variant as the headline: one step = low-rank score of every group over
    all positions, top-k per group, LRU staging of every pool, per-head attention."""
    import lsa_inputs as L
    wl = L.KVSWAP_WORKLOADS[args.workload]
    res = kvswap_measure(wl, args.steps, args.warmup, parity_steps=0 if args.no_cpu_baseline else 2)
    line = {"metric": res.pop("metric"), "value": res.pop("value"), "unit": res.pop("unit"), "n_gpus": 1}
    line.update({"steps": res.pop("steps"), "warmup": res.pop("warmup"), "ms_per_step": res.pop("ms_per_step"),
                 "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
                 "data": "synthetic (seeded 1/8-grid values)"})
    line.update(res)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
