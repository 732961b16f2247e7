"""Benchmark: fused float_moment + float_psnr over 16-bit 3840x2160 frames.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 4]

One step = the whole hot path (per-row exact sums, plan, walk with its
fallbacks, PSNR row chain, divisions) over one batch of the workload's
frames already resident in HBM.  Batches rotate through a ring of device
copies larger than the 256 MB Infinity Cache, so every step reads its
frames from HBM.  Prints ONE JSON line.

value          frames per second over K timed pipelined steps
               (bef_pipe_submit, then one bef_pipe_join; torch events on the
               submitting stream, bracketed by synchronisations), after
               their own warm-up; each step is one batch through the whole
               path, and a batch's ordered part overlaps the next batches'
               row passes on the library's streams
config         the run's figures, among them the one-stream figures
               (bef_frames_async, every kernel of a step after the one
               before on one stream: one_stream_*); for the 16-bit
               3840x2160 full-range workload (the default) also
               config.halfrange, the half-range workload (8 frames a step)
               measured the same way in the same run
roofline       the row-sum kernel (the dominant one): algorithmic bytes per
               launch (2 planes x w x h x 2 B x frames) over its average
               duration, measured over a pass of K one-stream steps with HIP
               events that each dispatch records on the launch stream (one
               launch at a time: pipelined row passes overlap in pairs);
               peak = MI355X HBM3E 8 TB/s
cpu_baseline   the CPU oracle (plain loops) on host copies of the same frames:
               one core (frames one after another, warm) and all of this
               process's CPUs (one frame per thread), with nproc and the
               CPU model
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0

# The row kernel's HBM traffic comes from rocprofv3 counter runs recorded in
# this file (FETCH_SIZE and WRITE_SIZE per dispatch, each scaled by what the
# same counter reads for an elementwise kernel of known size).  It is
# reported only while the sources that make the kernel are the ones the
# counters were taken on.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "k_rows16_16bit_3840x2160_traffic.txt")
ROW_KERNEL_SOURCES = ["rows.hip", "wave.h", "ordsum.h", "bef_internal.h"]


def row_kernel_fingerprint():
    import hashlib
    h = hashlib.sha256()
    for name in ROW_KERNEL_SOURCES:
        h.update(name.encode())
        with open(os.path.join(ROOT, "bit_exact_frame_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def recorded_traffic(workload_name):
    """HBM bytes per launch of the row kernel, or None when the record is
    missing, for another workload, or older than the kernel's sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = dict(line.split(":", 1) for line in f if ":" in line and not line.startswith("#"))
    except OSError:
        return None
    rec = {k.strip(): v.strip() for k, v in rec.items()}
    if rec.get("sources_sha256") != row_kernel_fingerprint():
        return None
    if rec.get("workload") != workload_name:
        return None
    return int(rec["hbm_bytes_per_launch"])


def cpu_facts():
    """Host CPU count (nproc), the CPUs this process may run on, and the
    model string /proc/cpuinfo gives."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")),
                         None)
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = os.cpu_count() or 1
    return os.cpu_count() or 1, usable, model


def cpu_baseline(ref, dis, bpc, w, bytes_per_frame, budget_s=20.0, one_core_frames=8):
    """The oracle (plain loops) on host copies of the batch: (1) one core,
    frames one after another, warm, over ``one_core_frames`` frames; (2) all
    cores, one frame per thread (each frame's loop stays serial) with as many
    threads as this process has CPUs, over about ``budget_s`` of CPU work."""
    import concurrent.futures as cf

    import oracle

    orc = oracle.Oracle()
    nproc, usable, model = cpu_facts()
    frames = ref.shape[0]

    def one(k):
        k %= frames
        return orc.frames(ref[k:k + 1], dis[k:k + 1], bpc, w=w)

    one(0)  # warm: library loaded, pages touched
    t0 = time.perf_counter()
    for k in range(one_core_frames):
        one(k)
    t1 = time.perf_counter() - t0
    per_frame = t1 / one_core_frames
    threads = usable
    n = max(frames, int(math.ceil(budget_s / max(per_frame, 1e-6))))
    n = int(math.ceil(n / threads) * threads)
    t0 = time.perf_counter()
    with cf.ThreadPoolExecutor(max_workers=threads) as ex:
        list(ex.map(one, range(n)))
    dt = time.perf_counter() - t0
    fps_all = n / dt
    fps_one = one_core_frames / t1
    return {"value": round(fps_all, 2), "unit": "frames/s", "cores": threads, "kind": "oracle",
            "sample": f"all cores: {n} frames of the batch ({frames} distinct), one frame per "
                      f"thread, {threads} threads, {dt:.2f} s wall; one core: {one_core_frames} "
                      f"frames one after another after a warm-up frame, {t1:.2f} s",
            "GBps": round(fps_all * bytes_per_frame / 1e9, 3),
            "one_core_value": round(fps_one, 2),
            "one_core_GBps": round(fps_one * bytes_per_frame / 1e9, 3),
            "one_core_ms_per_frame": round(1e3 * per_frame, 2),
            "nproc": nproc, "usable_cpus": usable, "cpu_model": model}


def measure(api, key, steps, warmup, ring=0, ceiling=True, pipe=True):
    """Whole-path throughput of workload ``key``: batches rotate through a
    ring of device copies of at least 1 GB, W warm-up steps (plus settle
    steps until the warm-up has lasted 50 ms), K timed steps bracketed by
    events on the launch stream, then K more steps with per-kernel events
    for the kernels' averages; before those (``pipe``), K pipelined steps
    after their own warm-up.  Returns a dict of figures and the frames."""
    import numpy as np
    import torch

    from bit_exact_frame_amd import synth

    wl = synth.WORKLOADS[key]
    ref_h, dis_h = synth.make_frames(key)
    F = ref_h.shape[0]
    batch_bytes = F * wl.bytes_per_frame
    ring = ring or max(2, int(math.ceil(1e9 / batch_bytes)))
    refs = [torch.from_numpy(ref_h).cuda() for _ in range(ring)]
    diss = [torch.from_numpy(dis_h).cuda() for _ in range(ring)]
    out = torch.empty((F, 6), dtype=torch.float64, device="cuda")
    stream = torch.cuda.current_stream()

    # correctness of this very configuration, outside the timed region
    api.bef_debug_set(0)
    want_mom, want_ps = api.bef_frames(refs[0], diss[0], wl.bpc, w=wl.w)

    # Pipelined batches (bef_pipe_submit): the same K steps, each one batch
    # through the whole path, with a batch's ordered part overlapping the
    # next batches' row passes on the library's own streams.  Submitted from
    # a stream of torch's pool (non-blocking: the legacy NULL stream would
    # wait for the library's streams), joined at the end, timed by events on
    # that stream.
    pipe_ms = None
    pipe_settle = 0
    if pipe:
        pstream = torch.cuda.Stream()
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        # the warm-up writes pwarm, the timed steps pout (filled beforehand:
        # any host pause between the warm-up and the timed steps lets the
        # clocks drop, and the next few hundred steps run up to 25% slower)
        pwarm = torch.empty((F, 6), dtype=torch.float64, device="cuda")
        pout = torch.full((F, 6), -1.0, dtype=torch.float64, device="cuda")

        def prun(n, o):
            for k in range(n):
                api.bef_pipe_submit(refs[k % ring], diss[k % ring], wl.bpc, o, w=wl.w,
                                    stream=pstream)
            api.bef_pipe_join(0, pstream)

        # Warm-up, then settle: chunks of 100 pipelined steps, each timed,
        # until two in a row agree within 1% after at least 100 ms, at most
        # 2 s.
        torch.cuda.synchronize()
        t_warm = time.perf_counter()
        prun(warmup, pwarm)
        torch.cuda.synchronize()
        last = None
        while True:
            ev0.record(pstream)
            prun(100, pwarm)
            ev1.record(pstream)
            torch.cuda.synchronize()
            pipe_settle += 100
            rate = ev0.elapsed_time(ev1)
            waited = time.perf_counter() - t_warm
            if waited > 2.0 or (waited > 0.1 and last is not None and
                                abs(rate - last) <= 0.01 * last):
                break
            last = rate
        ev0.record(pstream)
        prun(steps, pout)
        ev1.record(pstream)
        torch.cuda.synchronize()
        pipe_ms = ev0.elapsed_time(ev1)
        got = pout.cpu().numpy()
        assert (got[:, :4].view(np.uint64) == want_mom.view(np.uint64)).all()
        assert (got[:, 4:].view(np.uint64) == want_ps.view(np.uint64)).all()
        del pout, pwarm

    def run(n):
        for k in range(n):
            api.bef_frames_async(refs[k % ring], diss[k % ring], wl.bpc, out, w=wl.w,
                                 stream=stream)

    # The GPU's clocks take about 20-25 ms of sustained load to settle (the
    # row kernel runs up to 25% slower before that).
    t_warm = time.perf_counter()
    run(warmup)
    torch.cuda.synchronize()
    settle = 0
    while time.perf_counter() - t_warm < 0.05:
        run(20)
        torch.cuda.synchronize()
        settle += 20

    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    run(steps)
    ev1.record(stream)
    torch.cuda.synchronize()
    clean_ms = ev0.elapsed_time(ev1)
    got = out.cpu().numpy()
    assert (got[:, :4].view(np.uint64) == want_mom.view(np.uint64)).all()
    assert (got[:, 4:].view(np.uint64) == want_ps.view(np.uint64)).all()

    # the same K steps again, each kernel timed by HIP events that its own
    # dispatch records on the launch stream
    api.bef_timing_enable(True)
    api.bef_timing_reset()
    ev0.record(stream)
    run(steps)
    ev1.record(stream)
    torch.cuda.synchronize()
    api.bef_timing_enable(False)
    total_ms = ev0.elapsed_time(ev1)
    kern = {}
    for name in ("rows", "plan", "pairs", "walk"):
        ms, n = api.bef_timing_read(name)
        if n:
            kern[name] = 1e3 * ms / n  # microseconds per launch

    ceil_gbps = None
    if ceiling and wl.bpc != 8:
        cout = torch.empty(F * wl.h, dtype=torch.int32, device="cuda")
        for k in range(10):
            api.bef_read_ceiling(refs[k % ring], diss[k % ring], cout, w=wl.w, stream=stream)
        torch.cuda.synchronize()
        api.bef_timing_enable(True)
        api.bef_timing_reset()
        for k in range(max(20, steps // 2)):
            api.bef_read_ceiling(refs[k % ring], diss[k % ring], cout, w=wl.w, stream=stream)
        torch.cuda.synchronize()
        api.bef_timing_enable(False)
        c_ms, c_n = api.bef_timing_read("ceiling")
        ceil_gbps = batch_bytes / (c_ms / c_n / 1e3) / 1e9

    del refs, diss
    gbps = batch_bytes * steps / (clean_ms / 1e3) / 1e9
    res = {"wl": wl, "F": F, "ring": ring, "settle": settle, "clean_ms": clean_ms,
           "total_ms": total_ms, "kern": kern, "ceiling": ceil_gbps, "batch_bytes": batch_bytes,
           "fps": F * steps / (clean_ms / 1e3), "gbps": gbps, "ref_h": ref_h, "dis_h": dis_h,
           "pipe_ms": pipe_ms, "pipe_settle": pipe_settle}
    if pipe_ms is not None:
        res["pipe_fps"] = F * steps / (pipe_ms / 1e3)
        res["pipe_gbps"] = batch_bytes * steps / (pipe_ms / 1e3) / 1e9
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=500)
    ap.add_argument("--workload", type=int, default=4)
    ap.add_argument("--ring", type=int, default=0, help="device copies of the batch (0 = auto)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the cpu_baseline leg")
    ap.add_argument("--no-host", action="store_true",
                    help="skip the host-memory pipeline figure (PCIe-inclusive context)")
    ap.add_argument("--no-half", action="store_true",
                    help="skip the 16-bit 3840x2160 half-range leg reported under config")
    ap.add_argument("--calib-copy", type=int, default=0, metavar="MIB",
                    help="only run device-to-device copies of MIB MiB (HBM counter "
                         "calibration) and exit")
    args = ap.parse_args()
    if args.calib_copy:
        import torch
        n = args.calib_copy << 20
        # an elementwise kernel (not a DMA copy) that reads n bytes and writes n
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        print(json.dumps({"calib_copy_bytes_read": n, "calib_copy_bytes_written": n,
                          "launches": 5}), flush=True)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}): this path is a "
              "per-frame reduction with no cross-GPU exchange; frames shard with no "
              "communication, so one GPU's throughput is the figure.", file=sys.stderr)
        sys.exit(2)

    import torch

    from bit_exact_frame_amd import api

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    m = measure(api, args.workload, args.steps, args.warmup, ring=args.ring)
    wl, F, batch_bytes = m["wl"], m["F"], m["batch_bytes"]
    ref_h, dis_h = m["ref_h"], m["dis_h"]

    # context: the same frames from pinned host memory through the library's
    # two-slot upload pipeline (PCIe-inclusive rate; never the value)
    host_fps = None
    if not args.no_host:
        rp, dp = torch.from_numpy(ref_h).pin_memory(), torch.from_numpy(dis_h).pin_memory()
        api.bef_frames_host(rp, dp, wl.bpc, w=wl.w)
        t0 = time.perf_counter()
        for _ in range(3):
            api.bef_frames_host(rp, dp, wl.bpc, w=wl.w)
        host_fps = 3 * F / (time.perf_counter() - t0)
        del rp, dp

    # the half-range 16-bit 3840x2160 workload (8 frames a step), measured
    # the same way in the same run
    half = None
    if args.workload == 4 and not args.no_half:
        h5 = measure(api, 5, args.steps, args.warmup)
        r5 = h5["kern"].get("rows")
        half = {"workload": h5["wl"].name, "frames_per_step": h5["F"],
                "recipe": h5["wl"].recipe, "ring_copies": h5["ring"],
                "fps": round(h5["pipe_fps"], 1),
                "ms_per_step": round(h5["pipe_ms"] / args.steps, 5),
                "whole_path_GBps": round(h5["pipe_gbps"], 1),
                "whole_path_frac": round(h5["pipe_gbps"] / PEAK_HBM_GBS, 4),
                "one_stream_fps": round(h5["fps"], 1),
                "one_stream_ms_per_step": round(h5["clean_ms"] / args.steps, 5),
                "one_stream_whole_path_frac": round(h5["gbps"] / PEAK_HBM_GBS, 4),
                "rows_avg_us": None if r5 is None else round(r5, 2),
                "rows_frac": None if r5 is None else
                round(h5["batch_bytes"] / (r5 / 1e6) / 1e9 / PEAK_HBM_GBS, 4),
                "walk_avg_us": round(h5["kern"].get("walk", 0.0), 2),
                "read_ceiling_GBps": None if h5["ceiling"] is None else round(h5["ceiling"], 1),
                "settle_steps_after_warmup": h5["settle"],
                "pipelined_settle_steps_after_warmup": h5["pipe_settle"]}

    rows_us = m["kern"]["rows"]
    achieved = batch_bytes / (rows_us / 1e6) / 1e9
    ceiling = m["ceiling"]
    config = {"workload": wl.name, "frames_per_step": F, "w": wl.w, "h": wl.h,
              "bpc": wl.bpc, "recipe": wl.recipe, "ring_copies": m["ring"],
              "path": f"bef_pipe_submit, {api.bef_pipe_walk_cus()} walk CUs",
              "whole_path_GBps": round(m["pipe_gbps"], 1),
              "whole_path_frac": round(m["pipe_gbps"] / PEAK_HBM_GBS, 4),
              "one_stream_fps": round(m["fps"], 1),
              "one_stream_ms_per_step": round(m["clean_ms"] / args.steps, 5),
              "one_stream_whole_path_frac": round(m["gbps"] / PEAK_HBM_GBS, 4),
              "walk_avg_us": round(m["kern"].get("walk", 0.0), 2)}
    for name in ("plan", "pairs"):  # only where a plane can pass 2^55
        if name in m["kern"]:
            config[f"{name}_avg_us"] = round(m["kern"][name], 2)
    config.update({
        "read_ceiling_GBps": None if ceiling is None else round(ceiling, 1),
        "host_pipeline_fps_pcie_inclusive": None if host_fps is None else round(host_fps, 1),
        "rows_over_read_ceiling": None if ceiling is None else round(achieved / ceiling, 4),
        "timed_with_events_ms_per_step": round(m["total_ms"] / args.steps, 5),
        "settle_steps_after_warmup": m["settle"],
        "pipelined_settle_steps_after_warmup": m["pipe_settle"]})
    if half is not None:
        config["halfrange"] = half
    rec = {
        "metric": "frames/sec and achieved HBM GB/s (% of peak), 16-bit 3840x2160, 1 MI355X",
        "value": round(m["pipe_fps"], 1),
        "unit": "frames/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(m["pipe_ms"] / args.steps, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u16 in, u64/f64 sums",
        "data": "synthetic",
        "config": config,
        "roofline": {"bound": "hbm", "kernel": "k_rows16", "achieved": round(achieved, 1),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": recorded_traffic(wl.name),
                     "bytes_per_launch": batch_bytes,
                     "avg_launch_us": round(rows_us, 2)},
    }
    if not args.no_cpu:
        rec["cpu_baseline"] = cpu_baseline(ref_h, dis_h, wl.bpc, wl.w, wl.bytes_per_frame)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
