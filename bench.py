"""Benchmark of one paged decode step on one MI355X.

A step is the whole hot path over one batch: copy-on-write of shared blocks
(when the batch has any), append of each sequence's new token, then decode
attention through the block tables.  The append and the decode run as one
launch (pa_decode_append); `--separate` times them as two (pa_reshape_and_cache,
then pa_decode).  Inputs are synthetic and seeded (the
generator in paged_kv_cache_59_amd.workloads) and resident in HBM before the
timed region.  The pools are cloned into several replicas totalling at least
2 GB and the steps rotate over them, so the 256 MB Infinity Cache cannot
serve a step from the previous one's reads.

Prints one JSON line:
  value        bytes the step must move / step time, GB/s (the steps launched
               one by one from the host)
  graph_value  the same for the same steps replayed from one captured HIP
               graph (`graph_ms_per_step`), with no host dispatch between them
  roofline     the decode kernel (one launch: balanced persistent workers with
               the merge of cut sequences and the append fused) timed with HIP
               events bound to the kernel on its stream: its algorithmic bytes
               (decode, plus the append's writes) / mean kernel duration vs
               8 TB/s, over a second pass of the same steps
               (`call_mean_us`: events recorded around the call, in a pass of
               their own, which add queueing and dispatch latency; the
               wall-clock region records no events, since on this stack each
               record costs the step several microseconds);
               `traffic` is the HBM bytes per launch from the committed
               rocprofv3 counter summary (profiles/), null if the kernel changed
  cpu_baseline the CPU oracle on this host on one whole step of the same batch
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "paged decode attention: achieved HBM GB/s (fraction of peak) + sequences/s"
HBM_PEAK_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    # default: 20 for decode; 300 (about 100 ms) for the compute-bound prefill,
    # whose clock settles only after tens of milliseconds of sustained load
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", default="llama8b_b64")
    ap.add_argument("--num-workers", type=int, default=0)
    ap.add_argument("--separate", action="store_true",
                    help="append and decode as two launches instead of one")
    ap.add_argument("--replica-gb", type=float, default=2.0)
    ap.add_argument("--placement", default="shuffled", choices=["shuffled", "sequential"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the pass that replays the timed steps from one captured HIP graph")
    ap.add_argument("--cpu-budget-s", type=float, default=20.0)
    ap.add_argument("--probe-gib", type=float, default=4.0,
                    help="read-bandwidth probe size (0: skip the probe)")
    ap.add_argument("--flush-mb", type=int, default=1024,
                    help="decode: a third pass of kernel timings, each step preceded by a write "
                         "of this many MB of scratch (flushes L2 and the Infinity Cache); 0 = skip")
    ap.add_argument("--block-size", type=int, default=16, choices=[8, 16, 32])
    ap.add_argument("--swap-blocks", type=int, default=0,
                    help="only measure swapping this many blocks (Llama-3.1-8B layer shape) "
                         "out to pinned host memory and back in")
    ap.add_argument("--trace", action="store_true",
                    help="decode: per-worker timeline from the measurement build "
                         "(libpagedkv_trace.so, `python -m paged_kv_cache_59_amd.build --trace`), "
                         "one launch per step with a synchronisation after each; prints a summary")
    ap.add_argument("--decode-variant", default=None, choices=["valu"],
                    help="decode: time the measurement build libpagedkv_<variant>.so "
                         "(`python -m paged_kv_cache_59_amd.build --valu`: q.K and P.V on the "
                         "vector ALUs with v_dot2_f32_f16 instead of the 4x4x4 MFMA)")
    ap.add_argument("--trace-dump", default=None,
                    help="with --trace: also save every step's raw per-worker stamps (.npy)")
    ap.add_argument("--copy-probe-mb", type=int, default=0,
                    help="only run `steps` plain device copies of this many MiB (an elementwise "
                         "kernel reading and writing known bytes, to calibrate HBM counters)")
    return ap.parse_args()


def copy_probe(args):
    import torch
    n = args.copy_probe_mb << 20
    src = torch.ones(n // 2, dtype=torch.float16, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(args.steps):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_read": n, "copy_probe_bytes_written": n,
                      "launches": args.steps}), flush=True)


def measured_traffic(workload, fused, shared):
    """HBM bytes per step of the timed kernels (the decode kernel, and the
    prefix pass before it on a shared-blocks batch) from the committed
    rocprofv3 counter runs (FETCH_SIZE and WRITE_SIZE, calibrated against a
    plain copy), or None when there are none for this workload and variant
    (append fused or not, shared-blocks flag) or a kernel source changed
    since."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"decode_{workload}_hbm_counters.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if bool(rec.get("append_fused", False)) != bool(fused):
        return None
    if bool(rec.get("shared_blocks_flag", False)) != bool(shared):
        return None
    digests = rec.get("source_sha256")
    if not isinstance(digests, dict):  # (a record of one kernel source, from before)
        return None
    for src, digest in digests.items():
        if hashlib.sha256(open(os.path.join(ROOT, src), "rb").read()).hexdigest() != digest:
            return None
    return int(round(rec["traffic_bytes_per_step"]))


def achievable_read(torch, pk, gib, reps=5):
    """HBM read rates the probe reaches on this device (GB/s): a sequential
    read of `gib` GiB, and the same bytes as 4 KiB tiles in a shuffled
    order (the gather pattern of the block tables); kernel-bound events,
    mean over `reps` launches each."""
    n = int(gib * (1 << 30))
    buf = torch.full((n,), 1, dtype=torch.uint8, device="cuda")  # pages written once before
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    order = torch.from_numpy(np.random.default_rng(5).permutation(n // 4096).astype(np.int32)).cuda()
    rates = []
    for tiles in (None, order):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(reps + 1)]
        for a, b in ev:
            a.record()
            b.record()
        torch.cuda.synchronize()
        for e in ev:  # the first launch warms up
            pk.pa_read_probe(buf, sink, tiles, 4096, kernel_events=e)
        torch.cuda.synchronize()
        ms = np.mean([a.elapsed_time(b) for a, b in ev[1:]])
        rates.append(n / (ms * 1e-3) / 1e9)
    del buf, order
    torch.cuda.empty_cache()
    return rates


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:  # pragma: no cover
        pass
    return None


# Oracle repetitions per batch: 3 on the small and the gated batch, 1 on the
# large ones (each of those takes seconds); a single-thread step on the two
# small ones as well.
CPU_REPS = {"tiny_d64": 3, "llama8b_b64": 3}
CPU_ONE_THREAD = ("tiny_d64", "llama8b_b64")


def cpu_baseline(w, budget_s, step_bytes):
    """The oracle (as it is) on whole steps of the same batch, on this host:
    at least the planned repetitions, more while they fit half the budget (at
    most 20); then, for the small batches, one step with BLAS on one thread.
    ``step_bytes`` is the numerator the GPU line uses."""
    import oracle
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        blas = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas, threadpool_limits = 1, None
    planned = CPU_REPS.get(w.name, 1)
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.decode_step(w.q, w.k_new, w.v_new, w.k_cache, w.v_cache, w.block_tables,
                           w.context_lens, w.slot_mapping, w.block_mapping, w.scale,
                           w.num_kv_heads, block_size=w.block_size)
        reps += 1
        el = time.perf_counter() - t0
        if reps >= planned and (el >= budget_s * 0.5 or reps >= 20):
            break
    sec = el / reps
    one = None
    if threadpool_limits is not None and w.name in CPU_ONE_THREAD:
        with threadpool_limits(limits=1):
            t1 = time.perf_counter()
            oracle.decode_step(w.q, w.k_new, w.v_new, w.k_cache, w.v_cache, w.block_tables,
                               w.context_lens, w.slot_mapping, w.block_mapping, w.scale,
                               w.num_kv_heads, block_size=w.block_size)
            one = time.perf_counter() - t1
    return {"value": step_bytes / sec / 1e9, "unit": "GB/s", "cores": int(blas),
            "kind": "oracle", "seconds_per_step": sec, "seqs_per_s": w.num_seqs / sec,
            "one_thread_seconds_per_step": one,
            "host_cpus": len(os.sched_getaffinity(0)), "os_cpu_count": os.cpu_count(),
            "cpu_model": cpu_model(),
            "sample": f"{reps} whole step(s) of {w.name} (copy, append, fp64 decode of all "
                      f"{w.num_seqs} sequences), NumPy"}


PREFILL_METRIC = "multi-query paged attention (chunked prefill): achieved TFLOP/s (fraction of peak)"
MFMA_F16_PEAK_TFLOPS = 2500.0


def prefill_cpu_baseline(w, budget_s):
    """The prefill oracle (as it is) on whole sequences of the same batch, as
    many as fit about half the budget, scaled to TFLOP/s."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas = 1
    kc, vc = oracle.reshape_and_cache(w.k_new, w.v_new, w.k_cache, w.v_cache, w.slot_mapping)
    flops, seqs, t0 = 0, 0, time.perf_counter()
    for s in range(w.num_seqs):
        a, b = int(w.query_start[s]), int(w.query_start[s + 1])
        oracle.prefill(w.q[a:b], kc, vc, w.block_tables[s:s + 1], w.context_lens[s:s + 1],
                       np.array([0, b - a], np.int32), w.scale, w.num_kv_heads)
        flops += oracle.prefill_flops(w.context_lens[s:s + 1], [0, b - a], w.num_q_heads,
                                      w.head_dim)
        seqs += 1
        if time.perf_counter() - t0 >= budget_s * 0.5:
            break
    el = time.perf_counter() - t0
    return {"value": flops / el / 1e12, "unit": "TFLOP/s", "cores": int(blas), "kind": "oracle",
            "seconds": el, "host_cpus": len(os.sched_getaffinity(0)),
            "sample": f"{seqs} of {w.num_seqs} sequences' chunks of {w.name} (fp64 NumPy, "
                      "append excluded)"}


def bench_prefill(args):
    """One step = append of every chunk's K/V + multi-query attention.  The
    attention is MFMA-bound (4 Hq D flops per query-key pair against 4 Hkv D
    bytes per key), so it is priced against the fp16 MFMA peak.  Its duration
    follows the chip's clock, which under sustained load dips and then settles
    over about 35 ms: the default warm-up (300 steps) runs past that."""
    import torch
    from paged_kv_cache_59_amd import binding as pk
    from paged_kv_cache_59_amd import workloads as wl

    assert torch.cuda.is_available()
    torch.cuda.set_device(0)
    w = wl.make_named_prefill(args.workload, block_size=args.block_size)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    q, tab, lens, qs = t(w.q), t(w.block_tables), t(w.context_lens), t(w.query_start)
    k_new, v_new, slots = t(w.k_new), t(w.v_new), t(w.slot_mapping)
    kc, vc = t(w.k_cache), t(w.v_cache)
    out = torch.empty_like(q)
    stream = torch.cuda.current_stream()
    flops = w.flops()

    def step(ev=None):
        pk.pa_reshape_and_cache(k_new, v_new, kc, vc, slots)
        if ev is not None:
            ev[0].record(stream)
        pk.pa_prefill(out, q, kc, vc, tab, lens, qs, float(w.scale), w.num_kv_heads,
                      max_context_len=w.max_context_len, max_query_len=w.max_query_len)
        if ev is not None:
            ev[1].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # wall clock over exactly `steps` steps, no events in between; then the
    # same steps with events around each prefill call
    t0 = time.perf_counter()
    for i in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    ms = np.array([a.elapsed_time(b) for a, b in evs])
    ms_per_step = wall * 1e3 / args.steps
    mean_s = float(ms.mean()) * 1e-3
    achieved = flops / mean_s / 1e12
    res = {
        "metric": PREFILL_METRIC,
        "value": round(flops / (ms_per_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f16", "data": "synthetic",
        "tokens_per_s": round(w.num_tokens / (ms_per_step * 1e-3), 1),
        "config": {
            "workload": w.name, "num_seqs": w.num_seqs, "num_tokens": w.num_tokens,
            "num_q_heads": w.num_q_heads, "num_kv_heads": w.num_kv_heads,
            "head_dim": w.head_dim, "block_size": w.block_size, "max_context_len": w.max_context_len,
            "max_query_len": w.max_query_len, "seed": w.seed, "accumulate": "f32",
            "flops": flops,
        },
        "roofline": {
            "bound": "mfma", "achieved": round(achieved, 2), "peak": MFMA_F16_PEAK_TFLOPS,
            "unit": "TFLOP/s", "frac": round(achieved / MFMA_F16_PEAK_TFLOPS, 4),
            "traffic": None, "kernel": "prefill_kernel",
            "mean_us": round(mean_s * 1e6, 3),
            "median_us": round(float(np.median(ms)) * 1e3, 3),
            "p10_us": round(float(np.percentile(ms, 10)) * 1e3, 3),
            "p90_us": round(float(np.percentile(ms, 90)) * 1e3, 3),
            "timing": "HIP events recorded around each prefill call on its stream",
        },
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = prefill_cpu_baseline(w, args.cpu_budget_s)
    print(json.dumps(res), flush=True)


HOST_LINK_PEAK_GBS = 64.0   # PCIe 5.0 x16, one direction


def bench_swap(args):
    """Preemption by swap: copy N blocks of the Llama-3.1-8B layer shape (8 KV
    heads, head dim 128) from the device pool to pinned host memory and back,
    one pa_swap_blocks call per direction, timed with HIP events.  Bound by
    the host link."""
    import torch
    from paged_kv_cache_59_amd import binding as pk
    assert torch.cuda.is_available()
    torch.cuda.set_device(0)
    bs, hkv, d, n = args.block_size, 8, 128, args.swap_blocks
    nb = 2 * n
    rng = np.random.default_rng(7)
    kd = torch.from_numpy(rng.standard_normal((nb, hkv, d // 8, bs, 8), dtype=np.float32)
                          .astype(np.float16)).cuda()
    vd = torch.from_numpy(rng.standard_normal((nb, hkv, bs // 8, d, 8), dtype=np.float32)
                          .astype(np.float16)).cuda()
    hk = torch.empty((n, hkv, d // 8, bs, 8), dtype=torch.float16).pin_memory()
    hv = torch.empty((n, hkv, bs // 8, d, 8), dtype=torch.float16).pin_memory()
    src = torch.from_numpy(rng.permutation(nb)[:n].astype(np.int64))
    out_map = torch.stack([src, torch.arange(n)], 1).contiguous().cuda()
    in_map = torch.stack([torch.arange(n), torch.from_numpy(rng.permutation(nb)[:n].astype(np.int64))],
                         1).contiguous().cuda()
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        pk.pa_swap_blocks(kd, vd, hk, hv, out_map)
        pk.pa_swap_blocks(hk, hv, kd, vd, in_map)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    t_out, t_in = [], []
    t0 = time.perf_counter()
    for _ in range(args.steps):
        ev[0].record(stream)
        pk.pa_swap_blocks(kd, vd, hk, hv, out_map)
        ev[1].record(stream)
        pk.pa_swap_blocks(hk, hv, kd, vd, in_map)
        ev[2].record(stream)
        torch.cuda.synchronize()
        t_out.append(ev[0].elapsed_time(ev[1]))
        t_in.append(ev[1].elapsed_time(ev[2]))
    wall = time.perf_counter() - t0
    nbytes = n * 2 * hkv * d * bs * 2
    out_gbs = nbytes / (np.mean(t_out) * 1e-3) / 1e9
    in_gbs = nbytes / (np.mean(t_in) * 1e-3) / 1e9
    res = {"metric": "block swap over the host link: GB/s per direction", "unit": "GB/s",
           "value": round(2 * nbytes * args.steps / wall / 1e9, 2), "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "f16", "data": "synthetic",
           "config": {"workload": f"swap_llama_{n}", "blocks": n, "block_size": bs,
                      "num_kv_heads": hkv, "head_dim": d, "bytes_per_direction": nbytes},
           "roofline": {"bound": "host link", "peak": HOST_LINK_PEAK_GBS, "unit": "GB/s",
                        "swap_out": round(out_gbs, 2), "swap_in": round(in_gbs, 2),
                        "frac_out": round(out_gbs / HOST_LINK_PEAK_GBS, 4),
                        "frac_in": round(in_gbs / HOST_LINK_PEAK_GBS, 4),
                        "out_ms": round(float(np.mean(t_out)), 4),
                        "in_ms": round(float(np.mean(t_in)), 4)},
           "cpu_baseline": None}
    print(json.dumps(res), flush=True)


def trace_decode(args):
    """Per-worker timeline of the decode kernel, from the stamps the
    measurement build writes at the start of the workspace (100 MHz clock,
    the same on every CU).  Each step is synchronised and its stamps read
    back; times are relative to the step's earliest worker entry."""
    import torch
    from paged_kv_cache_59_amd import binding as pk
    pk.use_trace_library()
    from paged_kv_cache_59_amd import workloads as wl
    assert torch.cuda.is_available()
    torch.cuda.set_device(0)
    w = wl.make_named(args.workload, placement=args.placement, block_size=args.block_size)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    q, tab, lens = t(w.q), t(w.block_tables), t(w.context_lens)
    k_new, v_new, slots, pairs = t(w.k_new), t(w.v_new), t(w.slot_mapping), t(w.block_mapping)
    kc0, vc0 = t(w.k_cache), t(w.v_cache)
    pool_bytes = kc0.numel() * 2 + vc0.numel() * 2
    R = max(1, int(np.ceil(args.replica_gb * 1e9 / pool_bytes)))
    replicas = [(kc0, vc0)] + [(kc0.clone(), vc0.clone()) for _ in range(R - 1)]
    out = torch.empty_like(q)
    workers = args.num_workers or pk.pa_decode_num_workers()
    ws = pk.new_workspace(w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim, w.max_context_len,
                          workers)
    shared = w.shares_blocks()
    S = pk.TRACE_SLOTS
    runs = []
    kev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    for a, b in kev:
        a.record()
        b.record()
    torch.cuda.synchronize()
    for i in range(args.warmup + args.steps):
        kc, vc = replicas[i % R]
        if pairs.shape[0]:
            pk.pa_copy_blocks(kc, vc, pairs)
        ws[:workers * S * 8].zero_()
        pk.pa_decode_append(out, q, k_new, v_new, slots, kc, vc, tab, lens, float(w.scale),
                            w.num_kv_heads, max_context_len=w.max_context_len,
                            num_workers=workers, workspace=ws, shared_blocks=shared,
                            kernel_events=kev[i - args.warmup] if i >= args.warmup else None)
        torch.cuda.synchronize()
        if i >= args.warmup:
            runs.append(ws[:workers * S * 8].view(torch.int64).view(workers, S).cpu().numpy())
    kern_us = np.array([a.elapsed_time(b) * 1e3 for a, b in kev])
    if args.trace_dump:
        np.save(args.trace_dump, np.stack(runs))
    names = ["entry", "tables", "first_unit", "stream_end", "stores_issued", "helper_end"]
    rel = {n: [] for n in names}
    spans = []
    per_xcd_end = []
    per_xcd_rate = []
    for tr in runs:
        tr = tr[tr[:, 0] > 0]
        t0 = tr[:, 0].min()
        for j, n in enumerate(names):
            rel[n].append((tr[:, j] - t0) * 0.01)  # 100 MHz -> us
        spans.append(((tr[:, 5].max() - t0) * 0.01, (tr[:, 3].max() - t0) * 0.01))
        xcc = tr[:, 6] & 15
        rate = (tr[:, 3] - tr[:, 2]) * 0.01 / np.maximum(tr[:, 7] - 1, 1)
        per_xcd_end.append([float(np.median((tr[xcc == x, 3] - t0) * 0.01)) for x in range(8)])
        per_xcd_rate.append([float(np.median(rate[xcc == x])) for x in range(8)])
    pct = lambda a: {"min": round(float(np.min(a)), 2), "p10": round(float(np.percentile(a, 10)), 2),
                     "median": round(float(np.median(a)), 2),
                     "p90": round(float(np.percentile(a, 90)), 2), "max": round(float(np.max(a)), 2)}
    allw = np.concatenate([r[r[:, 0] > 0] for r in runs])
    merges = allw[:, 9]
    t_end = np.concatenate(rel["stream_end"])
    res = {
        "trace": w.name, "workers": workers, "steps": args.steps, "warmup": args.warmup,
        "kernel_us_events": pct(kern_us),
        "stamp_us_from_first_entry": {n: pct(np.concatenate(rel[n])) for n in names},
        "last_helper_end_us": pct([a for a, _ in spans]),
        "last_stream_end_us": pct([b for _, b in spans]),
        "median_stream_end_by_xcd_us": [round(float(np.median([p[x] for p in per_xcd_end])), 2)
                                        for x in range(8)],
        "us_per_unit_by_xcd": [round(float(np.median([p[x] for p in per_xcd_rate])), 3)
                               for x in range(8)],
        "stream_end_us_by_merges": {int(m): round(float(np.median(t_end[merges == m])), 2)
                                    for m in np.unique(merges) if (merges == m).sum() >= 20},
        "units_per_worker": pct(allw[:, 7]), "pieces_per_worker": pct(allw[:, 8]),
        "merges_per_worker": pct(merges),
        "helper_busy_us_per_worker": pct(allw[:, 12] * 0.01),
        "ring_wait_us_per_worker": pct(allw[:, 11] * 0.01),
        "note": "one launch per step, synchronised after each; stamps in us from the step's "
                "earliest worker entry (s_memrealtime, 100 MHz); us_per_unit = (stream end - "
                "first unit) / (units - 1)",
    }
    print(json.dumps(res), flush=True)


def main():
    args = parse()
    from paged_kv_cache_59_amd import workloads as wl_names
    prefill = args.workload in wl_names.PREFILL_WORKLOADS and not (args.swap_blocks or args.copy_probe_mb)
    if args.warmup is None:
        args.warmup = 300 if prefill else 20
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); "
              "the library has no multi-GPU path", file=sys.stderr)
        sys.exit(2)
    if args.copy_probe_mb:
        copy_probe(args)
        return
    if args.swap_blocks:
        bench_swap(args)
        return
    if args.trace:
        trace_decode(args)
        return
    if prefill:
        bench_prefill(args)
        return
    import torch
    from paged_kv_cache_59_amd import binding as pk
    from paged_kv_cache_59_amd import workloads as wl

    if args.decode_variant:
        pk.use_variant_library(args.decode_variant)
    assert torch.cuda.is_available()
    torch.cuda.set_device(0)
    w = wl.make_named(args.workload, placement=args.placement, block_size=args.block_size)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    q, tab, lens = t(w.q), t(w.block_tables), t(w.context_lens)
    k_new, v_new, slots = t(w.k_new), t(w.v_new), t(w.slot_mapping)
    pairs = t(w.block_mapping)
    kc0, vc0 = t(w.k_cache), t(w.v_cache)
    pool_bytes = kc0.numel() * 2 + vc0.numel() * 2
    R = max(1, int(np.ceil(args.replica_gb * 1e9 / pool_bytes)))
    replicas = [(kc0, vc0)] + [(kc0.clone(), vc0.clone()) for _ in range(R - 1)]
    out = torch.empty_like(q)
    workers = args.num_workers or pk.pa_decode_num_workers()
    ws = pk.new_workspace(w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim, w.max_context_len,
                          workers)
    stream = torch.cuda.current_stream()
    has_copy = w.block_mapping.shape[0] > 0
    # the caller's knowledge that sequences share blocks (prefix caching):
    # some physical block appears in more than one table row
    shared = w.shares_blocks()

    def step(i, ev=None, kernel_ev=None):
        kc, vc = replicas[i % R]
        if has_copy:
            pk.pa_copy_blocks(kc, vc, pairs)
        if args.separate:
            pk.pa_reshape_and_cache(k_new, v_new, kc, vc, slots)
        if ev is not None:
            ev[0].record(stream)
        if args.separate:
            pk.pa_decode(out, q, kc, vc, tab, lens, float(w.scale), w.num_kv_heads,
                         max_context_len=w.max_context_len, num_workers=workers, workspace=ws,
                         kernel_events=kernel_ev)
        else:
            pk.pa_decode_append(out, q, k_new, v_new, slots, kc, vc, tab, lens, float(w.scale),
                                w.num_kv_heads, max_context_len=w.max_context_len,
                                num_workers=workers, workspace=ws, kernel_events=kernel_ev,
                                shared_blocks=shared)
        if ev is not None:
            ev[1].record(stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # timed region: exactly `steps` steps, synchronised on both sides and
    # nothing else enqueued between them
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    # the same steps again with events recorded around each decode call (they
    # include queueing and dispatch latency)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    for i in range(args.steps):
        step(args.steps + i, evs[i])
    torch.cuda.synchronize()
    call_ms = np.array([a.elapsed_time(b) for a, b in evs])

    # kernel durations: the same `steps` steps again, right after, with events
    # bound to the decode kernel itself (pa_decode_timed: its own start and
    # end, the duration rocprofv3's kernel trace reports).  Binding costs the
    # launch a few microseconds of host-side dispatch, so it stays out of the
    # wall-clock region above.  torch creates an event at its first record.
    kev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    for a, b in kev:
        a.record(stream)
        b.record(stream)
    torch.cuda.synchronize()
    for i in range(args.steps):
        step(2 * args.steps + i, kernel_ev=kev[i])
    torch.cuda.synchronize()
    dec_ms = np.array([a.elapsed_time(b) for a, b in kev])

    # cross-check of the cache hygiene: the same steps once more, each
    # preceded (outside the kernel-bound events) by a write of flush_mb MB of
    # scratch, which evicts L2 and the Infinity Cache; with the replicas
    # rotating, the kernel should take as long as above
    flushed_ms = None
    if args.flush_mb > 0:
        scratch = torch.empty(args.flush_mb << 20, dtype=torch.uint8, device="cuda")
        fev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        for a, b in fev:
            a.record(stream)
            b.record(stream)
        torch.cuda.synchronize()
        for i in range(args.steps):
            scratch.fill_(i & 255)
            step(3 * args.steps + i, kernel_ev=fev[i])
        torch.cuda.synchronize()
        flushed_ms = np.array([a.elapsed_time(b) for a, b in fev])
        del scratch

    # The same `steps` steps captured once in a HIP graph (torch.cuda.CUDAGraph:
    # the library enqueues only kernels) and replayed between two
    # synchronisations: no host dispatch between the launches, as in a serving
    # loop that replays captured decode steps.  Reported beside the value.
    graph_ms_per_step = None
    if not args.no_graph:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(args.steps):
                step(4 * args.steps + i)
        torch.cuda.synchronize()
        graph.replay()  # (first replay: warm)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        graph.replay()
        torch.cuda.synchronize()
        graph_ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
        del graph

    probe = achievable_read(torch, pk, args.probe_gib) if args.probe_gib > 0 else None
    ms_per_step = wall * 1e3 / args.steps
    # Bytes the method must move.  A block several sequences share is counted
    # once (its repeat reads are reported as the logical figures below).  One
    # launch reads each new row once (for the attention and the store) and
    # writes it once; two launches read it twice.
    fused = not args.separate
    append_part = w.append_bytes() // 2 if fused else w.append_bytes()
    kernel_bytes = w.unique_decode_bytes() + (append_part if fused else 0)
    step_bytes = w.unique_decode_bytes() + w.copy_bytes() + append_part
    logical_kernel_bytes = w.decode_bytes() + (append_part if fused else 0)
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    dec_mean_s = float(dec_ms.mean()) * 1e-3
    achieved = kernel_bytes / dec_mean_s / 1e9
    logical_achieved = logical_kernel_bytes / dec_mean_s / 1e9
    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "seqs_per_s": round(w.num_seqs / (ms_per_step * 1e-3), 1),
        "frac_of_peak": round(value / HBM_PEAK_GBS, 4),
        # the same steps replayed from one captured HIP graph
        "graph_ms_per_step": (None if graph_ms_per_step is None
                              else round(graph_ms_per_step, 5)),
        "graph_value": (None if graph_ms_per_step is None
                        else round(step_bytes / (graph_ms_per_step * 1e-3) / 1e9, 2)),
        "config": {
            "workload": w.name, "num_seqs": w.num_seqs, "num_q_heads": w.num_q_heads,
            "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim, "block_size": w.block_size,
            "max_context_len": w.max_context_len, "mean_context_len": float(w.context_lens.mean()),
            "seed": w.seed, "num_workers": workers, "replicas": R, "accumulate": "f32",
            "copies_per_step": int(w.block_mapping.shape[0]), "placement": args.placement,
            "step_bytes": step_bytes, "decode_bytes": w.unique_decode_bytes(),
            "logical_decode_bytes": w.decode_bytes(),
            "kernel_bytes": kernel_bytes, "append": "fused" if fused else "separate launch",
            "shared_blocks_flag": bool(shared and fused),
            "decode_variant": args.decode_variant or "mfma",
        },
        "roofline": {
            "bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": (measured_traffic(w.name, fused, shared and fused)
                        if w.block_size == 16 and not args.decode_variant else None),
            "kernel": ("prefix_kernel + " if shared and fused else "")
                      + "decode_kernel" + (" (append fused)" if fused else ""),
            "mean_us": round(dec_mean_s * 1e6, 3),
            "median_us": round(float(np.median(dec_ms)) * 1e3, 3),
            "p10_us": round(float(np.percentile(dec_ms, 10)) * 1e3, 3),
            "p90_us": round(float(np.percentile(dec_ms, 90)) * 1e3, 3),
            "timing": ("HIP events bound to the start of the prefix pass and the end of "
                       "the decode kernel" if shared and fused else
                       "HIP events bound to the decode kernel")
                      + " (hipExtLaunchKernel), over the timed steps run again right after "
                        "the wall-clock region",
            "call_mean_us": round(float(call_ms.mean()) * 1e3, 3),
            "flushed_mean_us": (None if flushed_ms is None
                                else round(float(flushed_ms.mean()) * 1e3, 3)),
            "flush_mb": args.flush_mb,
            "achievable": (None if probe is None else {
                "sequential_gbs": round(probe[0], 1), "tiles_4k_gbs": round(probe[1], 1),
                "probe": f"pa_read_probe over {args.probe_gib:g} GiB, 16-byte non-temporal "
                         "loads; 4 KiB tiles in a shuffled order for the second rate"}),
            "frac_of_achievable": (None if probe is None else round(achieved / probe[1], 4)),
            "call_frac": round(kernel_bytes / (float(call_ms.mean()) * 1e-3) / 1e9
                               / HBM_PEAK_GBS, 4),
            # every holder's reads of shared blocks counted (equal to the above
            # when no block is shared)
            "logical_achieved": round(logical_achieved, 2),
            "logical_frac": round(logical_achieved / HBM_PEAK_GBS, 4),
        },
        "cpu_baseline": None,
    }
    if shared:
        res["config"]["unique_kv_bytes"] = w.unique_kv_bytes()
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, args.cpu_budget_s, step_bytes)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
