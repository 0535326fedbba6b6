#!/usr/bin/env python3
"""Benchmark of the CSA2 decode hot path on one MI355X.

One step = the whole hot path over one batch: for the default workload (16
requests x 131,072 cached entries, 64 heads, Full layer) that is the MXFP4
indexer scan with block maxima, the 2,048-block pool, the top-512 positions,
the sparse attention and the sliding-window merge, for all 16 requests.

Inputs are resident in HBM before the timed region; the KV caches rotate
over several identical copies so that the 256 MB Infinity Cache cannot serve
the 143 MB key stream from one step to the next.

Prints one JSON line: the whole-step throughput in (request x head) decodes
per second, the per-kernel breakdown, the roofline object of the indexer scan
(algorithmic bytes per launch over its event-timed average duration, and the
HBM bytes the counter runs measured for it), the rate of a plain streaming
read of the same key bytes on the same buffers (the ceiling the indexer is
compared with) and the oracle's CPU rate on a bounded sample of the same
workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
PEAK_F16_TFLOPS = 2500.0          # MI355X dense fp16/bf16 matrix peak
LLC_BYTES = 256 << 20             # MI355X Infinity Cache
METRIC = "CSA2 decode steps/s (batch×heads) at 128K ctx; achieved HBM GB/s vs peak"
DOMINANT = "index_score"          # the kernel the roofline object describes
DOMINANT_SRC = os.path.join(ROOT, "long_context_sparse_amd", "csrc", "index_score.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "index_score_{workload}_traffic.json")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="c1",
                    help="c0..c4, stack (20 decoder layers), hca (dense 8,192-entry attention), write (the write "
                         "path); the JSON line is for c1 by default")
    ap.add_argument("--copies", type=int, default=4, help="rotated KV-cache copies")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--cpu-rows", type=int, default=16, help="requests in the oracle sample")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="repeat the oracle sample until this much time has passed")
    ap.add_argument("--breakdown-steps", type=int, default=50,
                    help="steps of the separate per-kernel pass (at least 25): HIP events around every call of "
                         "every step, the stream kept busy; the roofline averages its indexer launches")
    ap.add_argument("--no-overlap", action="store_true",
                    help="skip the second timed pass (two independent batches on two streams)")
    ap.add_argument("--calib-copy", action="store_true",
                    help="after the timed steps, run a 1 GiB device copy (counter calibration)")
    return ap.parse_args()


def source_hash(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic(workload):
    """HBM bytes per launch of the dominant kernel from the committed counter
    runs, only for the workload and the kernel source they were taken on."""
    try:
        with open(TRAFFIC_FILE.format(workload=workload)) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    if d.get("source_sha256_16") != source_hash(DOMINANT_SRC) or d.get("workload") != workload:
        return None
    return d.get("bytes_per_launch")


def cpu_model():
    """The host CPU's model name (first 'model name' line of /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(cfg, rows, thread_counts, min_seconds):
    """The oracle as it stands, on a bounded sample of the same workload: the
    first `rows` requests, full rows (scoring every position, the pool, the
    top-512, attention over 512 + 128 entries for all heads), one request per
    thread, repeated until `min_seconds` have passed, for each thread count.
    Inputs are drawn and packed once, before any clock starts, as on the GPU.
    Returns [(seconds, rows done)] per thread count."""
    import numpy as np
    import oracle
    from tests.ref import RowRef

    refs = [RowRef(cfg, r) for r in range(rows)]
    packed = [r.packed_index(np.arange(r.n_vis)) for r in refs]

    def run(i):
        r = refs[i]
        kc, ks = packed[i]
        sc = oracle.index_score(r.qc, r.qs, r.w, kc, ks)
        _, idx = oracle.full_select(sc)
        return r.attend(idx)

    res = []
    for threads in thread_counts:
        done = 0
        t0 = time.perf_counter()
        while True:
            if threads > 1:
                oracle.map_rows(run, list(range(rows)), threads=threads)
                done += rows
            else:
                run(done % rows)
                done += 1
            dt = time.perf_counter() - t0
            if dt >= min_seconds:
                break
        res.append((dt, done))
    return res


def bench_write(args):
    """The write path alone (csa2_compress_pack): the prefill of a
    262,144-token context at 2 tokens per entry (131,072 entries, overlapping
    compression), latent entries with RMSNorm and RoPE packed to the 288-B
    format and indexer keys to the 68-B one.  HBM-bound: each launch reads its
    four fp32 token streams once and writes the packed entries."""
    import numpy as np
    import torch

    import long_context_sparse_amd as lib
    from long_context_sparse_amd.hip_events import HipEvent
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    n_tok, m = 262144, 2
    n_ent = n_tok // m
    res = {}
    for kind, width, norm in ((lib.MAIN_FP4, 512, True), (lib.INDEX_MXFP4, 128, False)):
        st = [torch.empty((n_tok, width), dtype=torch.float32, device=dev) for _ in range(4)]
        for k, t in enumerate(st):
            lib.csa2_synth_normal(7, 40 + k, 0, t)
        b = [torch.empty((m, width), dtype=torch.float32, device=dev) for _ in range(2)]
        for k, t in enumerate(b):
            lib.csa2_synth_normal(7, 50 + k, 0, t)
        w = torch.ones(width, dtype=torch.float32, device=dev) if norm else None
        codes = torch.empty((n_ent, 256 if width == 512 else 64), dtype=torch.uint8, device=dev)
        scales = torch.empty((n_ent, 32 if width == 512 else 4), dtype=torch.uint8, device=dev)

        def call():
            lib.csa2_compress_pack(kind, m, st[0], st[1], b[0], codes, scales, cb=st[2], zb=st[3], bb=b[1],
                                   norm_weight=w, rope=norm, pos0=0)
        for _ in range(args.warmup):
            call()
        n = max(25, args.steps)
        evs = [(HipEvent(), HipEvent()) for _ in range(n)]
        torch.cuda.synchronize()
        for a, e in evs:
            a.record()
            call()
            e.record()
        torch.cuda.synchronize()
        us = float(np.mean([a.elapsed_ms(e) for a, e in evs])) * 1e3
        nbytes = 4 * n_tok * width * 4 + n_ent * (288 if width == 512 else 68) + 2 * m * width * 4
        res["latent_512" if width == 512 else "index_128"] = {
            "entries": n_ent, "avg_launch_us": round(us, 2), "algorithmic_bytes": nbytes,
            "gbs": round(nbytes / us / 1e3, 1), "frac_of_hbm_peak": round(nbytes / us / 1e3 / PEAK_HBM_GBS, 4)}
        del st, b, codes, scales
        torch.cuda.empty_cache()
    lat = res["latent_512"]
    out = {
        "metric": "write path: compressed entries written/s (compression + RMSNorm + RoPE + FP4 packing)",
        "value": round(n_ent / (lat["avg_launch_us"] * 1e-6), 1),
        "unit": "entries/s",
        "n_gpus": 1, "steps": max(25, args.steps), "warmup": args.warmup, "higher_is_better": True,
        "dtype": "fp32 in, FP4/MXFP4 out", "data": "synthetic (seeded N(0,1) streams)",
        "config": {"workload": "write_prefill_262144_tokens_m2", "tokens": n_tok, "tokens_per_entry": m},
        "kernels": res,
        "roofline": {"kernel": "compress_pack_kernel<512>", "bound": "hbm", "achieved": lat["gbs"],
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": lat["frac_of_hbm_peak"], "traffic": None},
    }
    print(json.dumps(out), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); requests are independent, so "
              f"N GPUs would each run this same step on their own requests.", file=sys.stderr)
        sys.exit(2)
    if args.workload == "write":
        bench_write(args)
        return
    import numpy as np
    import torch

    import long_context_sparse_amd as lib
    from long_context_sparse_amd.hip_events import HipEvent
    from long_context_sparse_amd.workload import Workload
    from synth import configs

    lib.lib()        # raises if the HIP library is missing: there is no other path
    cfg = configs.ALL[args.workload]()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl = Workload(cfg, copies=args.copies)
    B, H = wl.n_rows, cfg.heads
    algo = wl.algorithmic_bytes()

    for i in range(args.warmup):
        wl.step(copy=i)
    torch.cuda.synchronize()

    # ---- timed region: exactly K steps, nothing else on the stream
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        wl.step(copy=args.warmup + i)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0

    # ---- second timed pass: two independent batches of the same workload in
    # flight on two streams of equal (default) priority, steps alternating
    # between them; each stream runs its batch's steps in order.  The
    # latency-bound selection and attention of one batch then run beside the
    # bandwidth-bound indexer scan of the other.  Reported beside the value,
    # which is the single-batch figure above.
    overlap = None
    if not args.no_overlap:
        mbs = [wl, wl.micro_batch()]
        streams = [torch.cuda.Stream(), torch.cuda.Stream()]
        main = torch.cuda.current_stream()
        for s_ in streams:
            s_.wait_stream(main)
        for i in range(2 * args.warmup):
            with torch.cuda.stream(streams[i % 2]):
                mbs[i % 2].step(copy=i)
        torch.cuda.synchronize()
        n2 = 2 * args.steps
        t0 = time.perf_counter()
        for i in range(n2):
            with torch.cuda.stream(streams[i % 2]):
                mbs[i % 2].step(copy=args.warmup + i)
        torch.cuda.synchronize()
        dt2 = time.perf_counter() - t0
        overlap = {
            "what": "two independent batches of this workload in flight on two streams (default priority), "
                    "their steps alternating; each batch's steps in order on its own stream",
            "steps": n2,
            "us_per_step": round(dt2 * 1e6 / n2, 2),
            "value": round(n2 / dt2 * B * H, 1),
            "step_frac_of_hbm_peak": round(algo["total"] / (dt2 / n2) / 1e9 / PEAK_HBM_GBS, 4),
        }
        # The same pass once more, each step bracketed by HIP events on its
        # own stream (after the timed pass, so that its host calls do not
        # touch the figure above): the share of a step's interval during which
        # a step of the other batch is also in flight.  A kernel trace cannot
        # show this: the profiler runs the two streams' dispatches one after
        # another.
        n_ev = 50
        evs = [(HipEvent(), HipEvent()) for _ in range(n_ev)]
        ref = HipEvent()
        torch.cuda.synchronize()
        ref.record(main)
        for s_ in streams:
            s_.wait_stream(main)
        for i in range(n_ev):
            st_ = streams[i % 2]
            with torch.cuda.stream(st_):
                evs[i][0].record(st_)
                mbs[i % 2].step(copy=args.warmup + i)
                evs[i][1].record(st_)
        torch.cuda.synchronize()
        iv = [(ref.elapsed_ms(a_) * 1e3, ref.elapsed_ms(b_) * 1e3) for a_, b_ in evs]
        shares = []
        for i, (lo, hi) in enumerate(iv):
            other = [iv[j] for j in range(i % 2 ^ 1, n_ev, 2)]
            beside = sum(max(0.0, min(hi, h2) - max(lo, l2)) for l2, h2 in other)
            shares.append(beside / max(hi - lo, 1e-9))
        overlap["event_pass"] = {
            "steps": n_ev,
            "mean_step_interval_us": round(sum(h - l for l, h in iv) / n_ev, 2),
            "span_us_per_step": round((iv[-1][1] - iv[0][0]) / n_ev, 2),
            "mean_share_beside_other_batch": round(sum(shares) / n_ev, 3),
        }
        del mbs

    if args.calib_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()

    # ---- per-kernel pass (separate from the timed region): every call of
    # every step bracketed by HIP events (no system fence), steps enqueued back
    # to back with no synchronisation in between, so each interval holds its
    # kernels' execution on a busy stream and not the host's launch latency.
    # The dominant kernel's roofline averages this pass's launches.  (Events
    # around one call only per pass measure worse: the bracketed interval
    # then also holds the end-of-kernel write-back of the call before it.)
    names = ["index_score", "select", "attention"]
    if cfg.mode == "reindex":
        names = ["index_score", "select_positions", "attention"]
    elif cfg.mode == "dense":
        names = ["attention"]
    dominant = "attention" if cfg.mode == "dense" else DOMINANT
    nb = max(25, args.breakdown_steps)
    marks_all = [{n: (HipEvent(), HipEvent()) for n in names} for _ in range(nb)]
    torch.cuda.synchronize()
    tb0 = time.perf_counter()
    for i, marks in enumerate(marks_all):
        wl.step(copy=i, marks=marks)
    torch.cuda.synchronize()
    breakdown_step_us = (time.perf_counter() - tb0) * 1e6 / nb
    per = {n: np.array([m[n][0].elapsed_ms(m[n][1]) * 1e3 for m in marks_all]) for n in names}
    kernels_us = {n: round(float(np.mean(v)), 2) for n, v in per.items()}
    k2_ms = float(np.mean(per[dominant])) * 1e-3

    # ---- streaming-read ceiling (separate, untimed): the plain non-temporal
    # read of the indexer's key-code plane, the same rotated buffers, one
    # launch each, HIP events as for the indexer
    planes = [idx[0] for (_, idx) in wl.kv_copies]      # (codes, scales) of each copy's INDEX entries
    xo = torch.zeros(lib.STREAM_XOR_WORDS, dtype=torch.int32, device=dev)
    for i in range(4):
        lib.csa2_stream_xor(planes[i % len(planes)], xo)
    rd = []
    for i in range(20):
        a, b = HipEvent(), HipEvent()
        a.record()
        lib.csa2_stream_xor(planes[i % len(planes)], xo)
        b.record()
        rd.append((a, b))
    torch.cuda.synchronize()
    rd_us = float(np.mean([a.elapsed_ms(b) for a, b in rd])) * 1e3
    rd_bytes = planes[0].numel() * planes[0].element_size()
    rd_gbs = rd_bytes / (rd_us * 1e-6) / 1e9
    # a ceiling of HBM only when the rotated planes exceed the 256 MB
    # last-level cache (the small workloads' planes are served from it)
    rd_hbm = sum({p.data_ptr(): p.numel() * p.element_size() for p in planes}.values()) > LLC_BYTES

    ms = dt * 1e3 / args.steps
    steps_s = args.steps / dt
    k2_bytes = algo.get("index_keys_full", algo.get("index_keys_pool", 0))
    k2_gbs = k2_bytes / (k2_ms * 1e-3) / 1e9
    step_gbs = algo["total"] / (ms * 1e-3) / 1e9
    traffic = measured_traffic(cfg.name)
    if cfg.mode == "dense":
        # every entry of every row against every head: two products of 2 x 512
        # flops per (head, entry) pair; the matrix cores' fp16 dense peak
        entries = int(wl.n_vis_host.sum()) + B * cfg.window
        flops = 4 * H * 512 * entries
        roofline = {
            "kernel": "attention (dense: attn_kernel + attn_merge_kernel)",
            "bound": "mfma",
            "achieved": round(flops / k2_ms / 1e9, 2),
            "peak": PEAK_F16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(flops / k2_ms / 1e9 / PEAK_F16_TFLOPS, 4),
            "traffic": None,
            "algorithmic_flops_per_launch": flops,
            "avg_launch_us": round(k2_ms * 1e3, 2),
            "launches_timed": nb,
        }
    else:
        roofline = {
            "kernel": DOMINANT,
            "bound": "hbm",
            "achieved": round(k2_gbs, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(k2_gbs / PEAK_HBM_GBS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": k2_bytes,
            "avg_launch_us": round(k2_ms * 1e3, 2),
            "launches_timed": nb,
            "frac_of_read_ceiling": round(k2_gbs / rd_gbs, 4) if rd_hbm else None,
        }

    out = {
        "metric": METRIC,
        "value": round(steps_s * B * H, 1),
        "unit": "(request x head) decodes/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp4 (indexer MFMA, exact) + bf16/fp16 (attention MFMA), fp32 accumulate",
        "data": "synthetic (seeded counter-based N(0,1)/U(0,1), packed on the GPU)",
        "config": {"workload": cfg.name, "requests": B, "context_entries": int(wl.max_vis), "heads": H,
                   "idx_heads": cfg.idx_heads,
                   "pool_blocks": {"dense": None, "prefill": 512, "csa": 512}.get(cfg.mode, 2048), "topk": 512, "window": cfg.window,
                   "kv_copies_rotated": args.copies},
        "steps_per_s": round(steps_s, 2),
        "step_algorithmic_bytes": algo["total"],
        "step_gbs": round(step_gbs, 1),
        "step_frac_of_hbm_peak": round(step_gbs / PEAK_HBM_GBS, 4),
        "two_batches_in_flight": overlap,
        "kernels_us": kernels_us,
        "kernels_us_note": f"means over the {nb}-step per-kernel pass (events around each call, stream kept busy; "
                           f"that pass ran at {breakdown_step_us:.1f} us per step); consecutive kernels overlap at "
                           f"their boundaries (the next one is dispatched during the previous one's end-of-kernel "
                           f"write-back), so the durations of one step can add up to slightly more than the step",
        "roofline": roofline,
        "read_ceiling": None if not rd_hbm else {
            "kernel": "stream_xor_kernel",
            "what": "plain streaming read (16-B non-temporal loads) of the indexer's key-code plane, same rotated buffers",
            "bytes_per_launch": rd_bytes,
            "avg_launch_us": round(rd_us, 2),
            "gbs": round(rd_gbs, 1),
            "frac_of_peak": round(rd_gbs / PEAK_HBM_GBS, 4),
        },
    }
    if not args.no_cpu:
        import oracle
        rows = min(args.cpu_rows, B)
        threads = min(rows, oracle.default_threads())
        (cdt, done), (cdt1, done1) = cpu_baseline(cfg, rows, [threads, 1], args.cpu_seconds)
        try:
            affinity = len(os.sched_getaffinity(0))
        except (AttributeError, OSError):
            affinity = None
        out["cpu_baseline"] = {
            "value": round(done * H / cdt, 3),
            "unit": "(request x head) decodes/s",
            "cores": threads,
            "kind": "oracle",
            "sample": f"{rows} of {B} requests of the same workload, whole rows ({int(wl.max_vis)} entries "
                      f"scored, pool, top-512, {H}-head attention), one request per thread: {done} rows in "
                      f"{cdt:.1f} s on {threads} threads; {done1} rows in {cdt1:.1f} s on 1 thread",
            "value_1thread": round(done1 * H / cdt1, 3),
            "host_cpus": os.cpu_count(),
            "host_cpus_usable": affinity,
            "cpu_model": cpu_model(),
        }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
