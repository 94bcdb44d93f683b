"""Host-side logic of bench.py (no GPU): the one-GPU guard, the L2-miss
traffic figure read from the committed counter summary (and dropped once the
contraction kernel's source differs from the one the counters were taken
on), the measured ceilings read from the committed peaks summary, the
bytes-per-pair figures per storage type, and the oracle host description."""

import os
import shutil
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
K2_SRC = os.path.join(ROOT, "pair_representation_amd", "csrc", "k2_contract.hip")


def test_more_than_one_gpu_is_refused():
    for argv, env in ((["--gpus", "2"], {}), ([], {"WORLD_SIZE": "4"})):
        r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + argv, cwd=ROOT,
                           env={**os.environ, **env}, capture_output=True, text=True, timeout=60)
        assert r.returncode == 2
        assert "exactly one GPU" in r.stderr
        assert r.stdout == ""


def test_traffic_follows_the_kernel_source(tmp_path):
    t = bench.traffic_from_profile(K2_SRC)
    # the committed summary was taken on the committed source: a figure of
    # the order of the 2.8x-algorithmic traffic it records
    assert t is not None and 1e10 < t < 1e11
    changed = tmp_path / "k2_contract.hip"
    shutil.copy(K2_SRC, changed)
    with open(changed, "a") as f:
        f.write("\n")
    assert bench.traffic_from_profile(str(changed)) is None


def test_host_description():
    h = bench.host_cpu(3)
    assert h["blas_threads"] == 3
    assert h["os_cpu_count"] == os.cpu_count()
    assert h["usable_cpus"] is None or 1 <= h["usable_cpus"] <= os.cpu_count()
    assert bench.blas_threads() >= 1


def test_measured_ceilings_and_bytes_per_pair():
    c = bench.measured_ceilings()
    # a matrix-core loop near the published 2.5 PFLOP/s; streaming rates
    # below the published 8 TB/s
    assert 2000 < c["mfma_bf16"] <= 2520
    for k in ("k1_mix_1r_2w", "k3_mix_3r_2w", "copy"):
        assert 3000 < c[k] < 8000
    # bf16: z 256 + mask 1 + a, b 512; fp32 doubles the z and operand bytes
    assert bench.k1_bytes_per_pair(2) == 769 and bench.k1_bytes_per_pair(4) == 1537
    assert bench.k3_bytes_per_pair(2) == 1281 and bench.k3_bytes_per_pair(4) == 1537
