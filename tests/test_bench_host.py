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
    # 32 blocks of 2048 queries: block b >= 1 sees popcount(b) squares (80 over blocks 1..31).
    # Each square's launch reads the block's bf16 queries and one table entry and writes the
    # fp32 far field (o_far and l_far); every launch after a block's first also reads it.
    cfg = CONFIGS["causal_64k_d128"]
    hb, hfl = bench.kernel_work("s2_mfma", cfg, hier=True)
    assert sum(bin(b).count("1") for b in range(32)) == 80
    BH, blk, D, Cq, Ck = 16, 2048, 128, 32, 128
    q_blk = blk * D * 2
    entry = Cq * Ck * 4 + 4 * Cq * Ck * D * 2 + Cq * D * D * 2  # log Z, K hi/lo, V hi/lo, s D_i
    far = blk * (D + 1) * 4
    assert hb == BH * (80 * (q_blk + entry + far) + (80 - 31) * far)
    assert hfl == BH * 80 * blk * 2.0 * (2 * Ck * D + D * D)
    # the prefix form: every block b >= 1 once
    pb, pfl = bench.kernel_work("s2_mfma", cfg)
    assert pb == BH * 31 * (q_blk + entry + far)
    assert pfl == BH * 31 * blk * 2.0 * (2 * Ck * D + D * D)


def test_retrieval_accounting_by_hand():
    # one head, 3 blocks, Cq = 2, Ck = 2, k1 = 1, k2 = 1: the retrieved key counts come from
    # the selections and the bucket sizes
    import numpy as np
    import torch
    from workloads import scaled_config
    cfg = scaled_config("retrieval_16k", B=1, H=1, N=12, block=4, Cq=2, Ck=2, topk_clusters=1, topk_blocks=1)
    sel = -np.ones((1, 1, 3, 2, 1, 2), np.int32)
    sel[0, 0, 1, 0, 0] = [1, 0]   # block 1, query cluster 0: key cluster 1 in block 0
    sel[0, 0, 2, 1, 0] = [0, 1]   # block 2, query cluster 1: key cluster 0 in block 1
    offs_k = np.array([[[0, 1, 4, 6, 6, 8, 12]]], np.int32)   # buckets (b, j): 1,3 | 2,0 | 2,4
    offs_q = np.array([[[0, 2, 4, 7, 8, 9, 12]]], np.int32)   # queries (b, i): 2,2 | 3,1 | 1,3
    ex = {"retrieval_trace": torch.from_numpy(sel), "offs_k": torch.from_numpy(offs_k),
          "offs_q": torch.from_numpy(offs_q)}
    c = bench.retrieval_counts(cfg, ex)
    # (b=1, i=0): 3 keys for 3 queries; (b=2, i=1): 2 keys for 3 queries
    assert c == {"nR": 5, "nqR": 3 * 3 + 2 * 3}
    nbytes, flops = bench.kernel_work("retr_exact_mfma", cfg, ctx=c)
    assert flops == 4.0 * 64 * 15
    assert bench.kernel_work("retr_exact_mfma", cfg) is None  # needs the counts


def test_cpu_info_fields():
    info = bench.host_cpu_info()
    assert info["host_cpus"] == os.cpu_count() and info["affinity_cpus"] >= 1 and info["blas_threads"] >= 1


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


def test_backward_accounting_by_hand():
    # acausal_8k: 32 heads x 8192 queries, Ck 128, D 64: per query 5 Ck D + 2 D^2 fp32
    # multiply-adds in the stage-2 backward; priced against the vector-ALU peak
    import bench
    from workloads import CONFIGS
    cfg = CONFIGS["acausal_8k"]
    nbytes, flops = bench.kernel_work("bw_refine", cfg)
    assert flops == 2.0 * 32 * 8192 * (5 * 128 * 64 + 2 * 64 * 64)
    x = 32 * 8192 * 64 * 2
    ftab = 32 * 32 * 128 * (1 + 2 * 64) * 4
    dip = 32 * 32 * 64 * 64 * 4
    assert nbytes == 2 * x + 32 * 8192 * 64 * 4 + 2 * (ftab + dip)
    r = bench.roofline_entry("bw_refine", cfg, 1e-3)
    assert r["bound"] == "alu" and r["peak"] == bench.PEAK_FP32_VALU_TFLOPS
    assert abs(r["achieved"] - flops / 1e-3 / 1e12) < 1e-9
    # the matrix-core key pass is priced against the bf16 peak (above the ridge point)
    assert bench.roofline_entry("bw_keys_a", cfg, 1e-3)["bound"] == "mfma"
