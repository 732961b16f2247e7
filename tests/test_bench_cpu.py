"""bench.py's host-side contract, without a GPU: the one-GPU guard, the
traffic record lookup, and the workload table (CPU only)."""
from __future__ import annotations

import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from bit_exact_frame_amd import synth  # noqa: E402


def test_more_than_one_gpu_is_refused():
    """--gpus N > 1 exits with a message and status 2 before touching a GPU."""
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr
    assert res.stdout == ""


def test_traffic_record_lookup():
    """The HBM record is returned only for its own workload, and only while
    the row kernel's sources match the fingerprint it was taken on."""
    fp = bench.row_kernel_fingerprint()
    assert len(fp) == 16 and int(fp, 16) >= 0
    assert bench.recorded_traffic("no_such_workload") is None
    rec = {}
    with open(bench.TRAFFIC_FILE) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                rec[k.strip()] = v.strip()
    got = bench.recorded_traffic(rec["workload"])
    if rec["sources_sha256"] == fp:
        assert got == int(rec["hbm_bytes_per_launch"])
        # the record's own arithmetic: counters times their calibration scales
        # (the file prints the scales to four places, hence the tolerance)
        hbm = (float(rec["fetch_kib_per_dispatch"]) * float(rec["fetch_scale"]) +
               float(rec["write_kib_per_dispatch"]) * float(rec["write_scale"])) * 1024
        assert abs(hbm - got) <= 1e-4 * got
    else:
        assert got is None


def test_workload_table():
    """Every workload names its shape consistently; the small parity
    workload draws frames of that shape, padded past w with the container's
    top value."""
    for key, wl in synth.WORKLOADS.items():
        assert wl.key == key
        assert wl.stride >= wl.w and wl.h > 0 and wl.frames > 0
        assert 8 <= wl.bpc <= 16
    wl = synth.WORKLOADS[1]
    ref, dis = synth.make_frames(1)
    assert ref.shape == (wl.frames, wl.h, wl.stride) == dis.shape
    assert ref.dtype == dis.dtype == (np.uint8 if wl.bpc == 8 else np.uint16)
    assert int(ref[:, :, :wl.w].max()) < (1 << wl.bpc)


def test_cpu_baseline_fields():
    """The oracle leg reports a warm one-core rate over several frames, an
    all-cores rate with one thread per usable CPU, nproc and the CPU model
    (small frames and a short budget here)."""
    wl = synth.WORKLOADS[1]
    ref, dis = synth.make_frames(1)
    rec = bench.cpu_baseline(ref, dis, wl.bpc, wl.w, wl.bytes_per_frame, budget_s=0.2,
                             one_core_frames=8)
    nproc, usable, _ = bench.cpu_facts()
    assert rec["kind"] == "oracle" and rec["unit"] == "frames/s"
    assert rec["cores"] == usable and rec["nproc"] == nproc == os.cpu_count()
    assert rec["value"] > 0 and rec["one_core_value"] > 0
    assert abs(rec["GBps"] - rec["value"] * wl.bytes_per_frame / 1e9) < 1e-3
    assert "8 frames one after another" in rec["sample"]
