"""Host logic of bench.py (CPU only): the one-GPU refusal, the algorithmic work accounting
behind the roofline, and the traffic lookup in the committed rocprofv3 summaries."""

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from workloads import CONFIGS  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0 and "one GPU" in r.stderr and r.stdout == ""


def test_assign_accounting_by_hand():
    # acausal_8k: B=4 H=8 N=8192 D=64 bf16, Cq 32, Ck 128. One launch assigns both tensors:
    # reads Q and K once (2 bytes per element) and writes two int32 labels per position.
    cfg = CONFIGS["acausal_8k"]
    nbytes, flops = bench.kernel_work("kmeans_assign_mfma", cfg)
    assert nbytes == 2 * (32 * 8192 * 64 * 2) + 2 * 32 * 8192 * 4
    # one multiply-add per (point, centroid, dimension) for each tensor
    assert flops == 2.0 * 32 * 8192 * (32 + 128) * 64


def test_moments_accounting_by_hand():
    # sum_m w_m v_m k_m^T for every (query centroid, key): 2 Cq N D^2 flops per head
    cfg = CONFIGS["causal_64k_d128"]
    _, flops = bench.kernel_work("s1_moments_f16", cfg)
    assert flops == 2.0 * 16 * 32 * 65536 * 128 * 128


def test_hierarchical_stage2_reads_by_hand():
    # 32 blocks: block b reads popcount(b) table entries, 80 reads over blocks 1..31
    cfg = CONFIGS["causal_64k_d128"]
    base, fl = bench.kernel_work("s2_mfma", cfg)
    hb, hfl = bench.kernel_work("s2_mfma", cfg, hier=True)
    # in 5 launches per call (the bit length of 31), each reading the queries and writing
    # the far field; the figure is per call
    assert sum(bin(b).count("1") for b in range(32)) == 80
    x = 16 * 65536 * 128 * 2
    assert hb == pytest.approx(5 * 2 * x + (base - 2 * x) * 80 / 31)
    assert hfl == pytest.approx(fl * 80 / 31)


def test_roofline_classification_and_fraction():
    cfg = CONFIGS["acausal_8k"]
    nbytes, flops = bench.kernel_work("kmeans_assign_mfma", cfg)
    r = bench.roofline_entry("kmeans_assign_mfma", cfg, 40e-6)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == 8000.0
    assert r["achieved"] == pytest.approx(nbytes / 40e-6 / 1e9)
    assert r["frac"] == pytest.approx(r["achieved"] / 8000.0)
    m = bench.roofline_entry("s1_moments_f16", cfg, 80e-6)
    assert m["bound"] == "mfma" and m["unit"] == "TFLOP/s" and m["peak"] == 2500.0
    assert m["frac"] == pytest.approx(bench.kernel_work("s1_moments_f16", cfg)[1] / 80e-6 / 1e12 / 2500.0)
    assert bench.roofline_entry("no_such_kernel", cfg, 1e-6) is None


def _profile_record(workload):
    with open(os.path.join(ROOT, "profiles", f"muse_fwd_{workload}.md")) as fh:
        for line in fh:
            if line.startswith("traffic-json: "):
                return json.loads(line[len("traffic-json: "):])
    raise AssertionError("no traffic-json line")


@pytest.mark.parametrize("workload,kernel", [("acausal_8k", "kmeans_assign_mfma"),
                                             ("causal_64k_d128", "s1_causal_scan")])
def test_traffic_lookup_follows_the_source_hash(workload, kernel, monkeypatch):
    rec = _profile_record(workload)
    k = rec["kernels"][kernel]
    # the bench reports the profile's bytes only while the kernel sources hash to the profile's
    monkeypatch.setattr(bench, "csrc_sha", lambda: rec["csrc_sha"])
    assert bench.measured_traffic(workload, kernel) == k["fetch_bytes"] + k["write_bytes"]
    monkeypatch.setattr(bench, "csrc_sha", lambda: "0" * 16)
    assert bench.measured_traffic(workload, kernel) is None
    assert bench.measured_traffic("no_such_workload", kernel) is None
