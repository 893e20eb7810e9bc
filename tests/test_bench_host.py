"""Host-side logic of bench.py, on the CPU: the one-GPU guard, the algorithmic
byte counts of the memory-bound stages and the traffic figure taken from the
committed counter summary."""
import json
import os
import subprocess
import sys
from types import SimpleNamespace

import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402
import synth  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and "one GPU" in line["error"]


def test_algorithmic_bytes_at_720p():
    # 720p: 40 heads, d = 128, 75,600 real tokens, 1,440 cubes of 64 (92,160 slots)
    wl = synth.WORKLOADS[2]
    kept = 4_150_000
    path = SimpleNamespace(wl=wl, nblk=1440, n_real=75600, n_pad=92160,
                           counts=torch.tensor([kept], dtype=torch.int64))
    got = bench.algorithmic_bytes(path)
    # reorder, per head: Q, K, V each read (75,600 rows) and written (92,160 rows) at
    # 256 B a row = 128,839,680 B, plus the float64 means of Q and K (2 x 1,440 x 128 x 8
    # = 2,949,120 B)
    assert got["reorder"] == 40 * (128_839_680 + 2_949_120)
    # mask, per head: the means read back (2,949,120 B), the float32 scores written and
    # read (2 x 1,440^2 x 4 = 16,588,800 B) and the counts (5,760 B); 4 B per kept id
    assert got["mask"] == 40 * (2_949_120 + 16_588_800 + 5_760) + 4 * kept


def test_recorded_traffic_only_for_the_profiled_kernel_and_workload():
    assert bench.recorded_traffic("480p") is None
    vals = {}
    with open(os.path.join(ROOT, "profiles", "kernels_720p-hybrid95_hbm_traffic.txt")) as f:
        for line in f:
            parts = line.split()
            if len(parts) == 2:
                vals[parts[0]] = parts[1]
    got = bench.recorded_traffic("720p-hybrid95")
    if vals["fwd_source_sha256"] == bench.fwd_source_hash():
        assert got == int(vals["traffic_bytes_per_launch"])
    else:   # the forward changed since the counters were taken: no figure
        assert got is None
