"""Throughput of the MuSe forward pass on one MI355X, with roofline and CPU-oracle baseline.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload acausal_8k] [--no-cpu]
                [--no-exact] [--no-secondary] [--no-peaks] [--no-backward] [--hierarchy]
                [--single-stream]

A step is one muse_attn_fwd call over the whole workload batch (K-means, stage 1,
stage 2 and, when causal, the exact diagonal blocks), with inputs resident in HBM and
the workspace allocated beforehand. Prints ONE JSON line: `value` is the 8k workload's
tokens/s (or the chosen workload's). Extra fields: the in-library exact attention time
on the same shape (speedup), the relative squared error of MuSe against it, per-kernel
average durations measured with HIP events on the stream the kernels run on, the
untilted-dipole run and the paper's speed setting (key clusters capped at 1.5 N / Ck
members, one Lloyd iteration) of a workload without retrieval, the hierarchical-decomposition
run of a causal one without retrieval, the backward pass of a D = 64 one without
retrieval (`backward`: dq, dk, dv for an upstream gradient with the forward's labels
fixed), `measured_peaks` (a
device copy and a bf16
GEMM on this GPU, beside the published peaks the roofline uses) and, with the default
workload, `secondary`: the same figures for the 64k causal configuration.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# MI355X published peaks
PEAK_HBM_GBS = 8000.0
PEAK_BF16_MFMA_TFLOPS = 2500.0
PEAK_FP32_VALU_TFLOPS = 157.3

WORKLOAD_TEXT = {
    "acausal_1k_f32": "acausal MuSe fwd, B=1 H=1 N=1024 D=64 fp32, Cq=8 Ck=32, 5 Lloyd iterations",
    "acausal_8k": "acausal MuSe fwd, B=4 H=8 N=8192 D=64 bf16 (fp32 accumulate), Cq=32 Ck=128, 5 Lloyd iterations",
    "causal_16k": "causal MuSe fwd, B=8 H=8 N=16384 D=64 bf16, block 1024, Cq=16 Ck=64, 5 Lloyd iterations",
    "causal_64k_d128": "causal MuSe fwd, B=1 H=16 N=65536 D=128 bf16, block 2048, Cq=32 Ck=128, 5 Lloyd iterations",
    "retrieval_16k": "causal MuSe fwd with retrieval k1=4 k2=2, B=2 H=8 N=16384 D=64 bf16, block 1024, Cq=16 Ck=64",
}


RIDGE = PEAK_BF16_MFMA_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)  # flop/byte where the two roofs meet
METRIC = "MuSe fwd tokens/s at 8k and 64k; speedup vs exact attn; % MFMA/HBM roofline"
SECONDARY = "causal_64k_d128"  # the 64k configuration reported beside the 8k one


def retrieval_counts(cfg, ex) -> dict:
    """Per-call sums over (head, query cluster i, block b >= 1) of the retrieved key count
    nR(i, b) and of nq(i, b) * nR(i, b) (queries of cluster i in block b times the keys they
    attend exactly), from a traced call's selections and bucket offsets (integer outputs of
    the library: [B,H,nb,Cq,k1,1+k2] cluster ids then block ids, -1 = none)."""
    sel = ex["retrieval_trace"].cpu().numpy()
    offs_k = ex["offs_k"].cpu().numpy().astype(np.int64)
    offs_q = ex["offs_q"].cpu().numpy().astype(np.int64)
    Ck, Cq = cfg.Ck, cfg.Cq
    nr_sum = nqr_sum = 0
    B, H, nb = sel.shape[:3]
    for b_ in range(B):
        for h in range(H):
            bucket = np.diff(offs_k[b_, h])          # [nb*Ck] keys per (block, cluster)
            qcount = np.diff(offs_q[b_, h])          # [nb*Cq]
            for b in range(1, nb):
                for i in range(Cq):
                    nr = 0
                    for row in sel[b_, h, b, i]:
                        j = int(row[0])
                        if j < 0:
                            continue
                        for bp in row[1:]:
                            if bp >= 0:
                                nr += int(bucket[int(bp) * Ck + j])
                    nr_sum += nr
                    nqr_sum += nr * int(qcount[b * Cq + i])
    return {"nR": nr_sum, "nqR": nqr_sum}


def kernel_work(name: str, cfg, hier: bool = False, ctx: dict = None):
    """(algorithmic bytes, algorithmic flops) of ONE launch of a library kernel on this
    workload, or None when the kernel is not listed. Bytes count every tensor a launch
    must read or write at least once (inputs read once, outputs written once); flops count
    the arithmetic the method defines (multiply-add = 2), not the extra products of the
    bf16 hi/lo splits. Causal tables have one entry per block (nbS = nb); a causal far
    field exists for blocks b >= 1 only and is an fp32 partial result (o_far, l_far).

    Hierarchical decomposition (hier): block b >= 1 sees popcount(b) squares; stage 2 runs
    one launch per chain level, and the launch that adds a square to block b reads the
    block's queries and the square's table entry and writes the fp32 far field, which
    every launch after the first also reads. The figure is per call, as the library's
    HIP-event scope covers those launches together.

    Retrieval kernels need ctx = retrieval_counts(...): the retrieved key counts are
    data-dependent."""
    BH, N, D, Cq, Ck = cfg.B * cfg.H, cfg.N, cfg.D, cfg.Cq, cfg.Ck
    e = 2 if cfg.dtype == "bf16" else 4
    nb = cfg.N // cfg.block if cfg.causal else 1
    blk = cfg.block if cfg.causal else N
    if cfg.causal or cfg.dtype != "bf16":
        mbk = cfg.block if cfg.causal else N
    else:  # the library's acausal moment slices: about 256 workgroups, multiples of 128 keys
        groups = -(-Cq // (16 if D == 64 else 4))
        want = max(1, -(-256 // (groups * BH)))
        mbk = min(-(-(-(-N // want)) // 128) * 128, 8192)
    nmb = (N + mbk - 1) // mbk
    x = BH * N * D * e                      # one [B, H, N, D] input tensor
    table = BH * nb * Cq * Ck               # (entry, i, j) cells
    tbytes = table * (4 + 8 * D)            # log Z + bf16 hi/lo of K_ij and of V_ij
    ftab = table * (1 + 2 * D) * 4          # fp32 log Z, K_ij, V_ij
    dip32 = BH * nb * Cq * D * D * 4         # fp32 dipole (or E[v k^T]) per table entry
    far_rows = BH * (N - blk) if cfg.causal else 0   # rows with a far field
    far = far_rows * (D + 1) * 4            # fp32 o_far + l_far of those rows
    s2_flops_row = 2.0 * (2 * Ck * D + D * D)
    if cfg.causal:
        # one entry per block b >= 1: bf16 tables and s D_i
        entry = Cq * Ck * (4 + 8 * D) + Cq * D * D * 2 if e == 2 else Cq * Ck * (1 + 2 * D) * 4 + Cq * D * D * 4
        if hier and nb > 1:
            pc = [bin(b).count("1") for b in range(nb)]
            per_head = sum(c * (blk * D * e + entry + blk * (D + 1) * 4) + (c - 1) * blk * (D + 1) * 4
                           for c in pc[1:])
            s2 = (BH * per_head, BH * s2_flops_row * blk * sum(pc[1:]))
        else:
            s2 = (far_rows * D * e + far + BH * (nb - 1) * entry, s2_flops_row * far_rows)
    else:
        s2 = (2 * x + tbytes + BH * Cq * D * D * 2, s2_flops_row * BH * N)
    w = {
        "kmeans_assign_mfma": (2 * x + 2 * BH * N * 4, 2.0 * BH * N * (Cq + Ck) * D),
        "kmeans_assign": (2 * x + 2 * BH * N * 4, 2.0 * BH * N * (Cq + Ck) * D),
        "s1_scores": (x + BH * Cq * N * 4, 2.0 * BH * Cq * N * D),
        "s1_atoms_mfma": (2 * x + table * (2 + 2 * D) * 4, 6.0 * BH * Cq * N * D),
        "s1_atoms": (2 * x + table * (2 + 2 * D) * 4, 6.0 * BH * Cq * N * D),
        "s1_moments_f16": (2 * x + BH * Cq * N * 4 + BH * nmb * Cq * (D * D + 1) * 4, 2.0 * BH * Cq * N * D * D),
        "s1_moments": (2 * x + BH * nmb * Cq * (D * D + 1) * 4, 2.0 * BH * Cq * N * D * D),
        "s1_finalize": (table * (2 + 2 * D) * 4 + BH * nmb * Cq * (D * D + 1) * 4 + tbytes + BH * Cq * D * D * 2,
                        2.0 * BH * Cq * Ck * D * D),
        "s1_prefix": (table * (2 + 2 * D) * 4 + ftab, 0.0),
        "s1_mom_prefix": (BH * nmb * Cq * (D * D + 1) * 4 + dip32, 0.0),
        # fp32 tables: read K, V, E and write D_i; bf16 (matrix cores): read K, V, E and write the
        # bf16 hi/lo tables and s D_i
        "s1_dip_final": ((ftab + dip32 + tbytes + dip32 // 2) if e == 2 else (ftab + 2 * dip32),
                         2.0 * BH * nb * Cq * Ck * D * D),
        "s1_pack": (ftab + dip32 + tbytes + dip32 // 2, 0.0),
        "s1_causal_scan": (table * (2 + 2 * D) * 4 + BH * nmb * Cq * (D * D + 1) * 4 + tbytes + BH * nb * Cq * D * D * 2,
                           2.0 * BH * nb * Cq * Ck * D * D),
        "s2_mfma": s2,
        "s2_refine": (x + (far if cfg.causal else x) + table * (1 + 2 * D) * 4 + BH * nb * Cq * D * D * 4,
                      s2_flops_row * (far_rows if cfg.causal else BH * N)),
        # the diagonal blocks: Q, K, V and the far field read, the output written
        "local_block_mfma": (4 * x + far, 4.0 * BH * N * (blk / 2) * D),
        "exact_mfma": (4 * x, (2.0 if cfg.causal else 4.0) * BH * N * N * D),
        "exact_valu": (4 * x, (2.0 if cfg.causal else 4.0) * BH * N * N * D),
        # untilted dipole: per key cluster covariance (keys and values read once), then
        # D_i = sum_j P_ij Cov_j (covariances and log Z read, s D_i written)
        "s1_cluster_cov": (2 * x + BH * Ck * D * D * 4, 2.0 * BH * N * D * D),
        "s1_untilted_dip": (BH * Ck * D * D * 4 + BH * Cq * Ck * 4 + BH * Cq * D * D * e, 2.0 * BH * Cq * Ck * D * D),
        # causal untilted: bucket statistics folded into prefix counts and means; per block
        # the running centred sums take the block's buckets and D_i = sum_j P_ij Cov_j^{<b}
        "s1_untilted_prefix": (2 * BH * nb * Ck * (1 + 2 * D) * 4, 0.0),
        "s1_untilted_causal": (BH * nb * Ck * (D * D + 2 + 4 * D) * 4 + BH * nb * Cq * Ck * 4 + BH * nb * Cq * D * D * e,
                               2.0 * BH * nb * Cq * Ck * D * D + 2.0 * BH * nb * Ck * D * D),
        # acausal general-path tables from whole atoms
        "s1_tables": (table * (2 + 2 * D) * 4 + ftab, 0.0),
        # backward: stage 2 per query cluster (q and dout read, causal: the far field's fp32
        # share of dout; dq written; tables read; summary gradients written), q.K, g.V, p g,
        # dl q, dl K, g D, g q per query
        "bw_refine": (x + (BH * N * (D + 1) * 4 if cfg.causal else x) + BH * N * D * 4 + 2 * (ftab + dip32),
                      2.0 * BH * N * (5 * Ck * D + 2 * D * D)),
        # the same on the matrix cores (bf16 inputs)
        "bw_refine_mfma": (x + (BH * N * (D + 1) * 4 if cfg.causal else x) + BH * N * D * 4 + 2 * (ftab + dip32),
                           2.0 * BH * N * (5 * Ck * D + 2 * D * D)),
        # tilted: per (query cluster, key) G k and G^T v on the matrix cores; keys, values,
        # a_im and G (bf16 hi/lo, both layouts) read, Q and w Q written, the dk and dv terms written
        "bw_keys_a": (2 * x + (2 if cfg.causal else 3) * BH * Cq * N * 4 + BH * nb * Cq * 4 * D * D * 2
                      + 2 * BH * N * D * 4, 4.0 * BH * Cq * (N - blk if cfg.causal else N) * D * D),
        # per (query cluster, key): a_im, dL/dw, the dk and dv updates and the tile partials
        "bw_keys_b": (2 * x + 4 * BH * N * D * 4 + 2 * table * D * 4 + 4 * table * 4 + BH * Cq * N * 4
                      + BH * (-(-N // 64)) * Cq * D * 4, 14.0 * BH * N * Cq * D),
        # causal backward: the merge (both partial outputs and the upstream gradient read,
        # their gradients written in place), the suffix sums (dK', dV' of every entry read,
        # sdk, sdv written; G_Dip of every entry read, its four bf16 copies written)
        "bw_merge": (x + 4 * BH * N * D * 4 + 4 * BH * N * 4, 0.0),
        "bw_suffix": (4 * table * D * 4 + 3 * table * 4, 0.0),
        "bw_suffix_dip": (BH * nb * Cq * D * D * (4 + 8), 0.0),
        # exact in-block backward over the 64 x 64 tile pairs on or below the diagonal:
        # q.k, g.v, p g, dS q per pair (keys' pass) and q.k, g.v, dS k (queries' pass); inputs,
        # dL/do_loc and the gradients read once, dk, dv (dq) updated
        "bw_local_kv": (3 * x + BH * N * D * 4 + 4 * BH * N * D * 4 + 2 * BH * N * 4,
                        8.0 * 64 ** 3 * BH * nb * (blk // 64) * (blk // 64 + 1) // 2),
        "bw_local_q": (3 * x + BH * N * D * 4 + 2 * BH * N * D * 4 + 2 * BH * N * 4,
                       6.0 * 64 ** 3 * BH * nb * (blk // 64) * (blk // 64 + 1) // 2),
    }
    # the matrix-core versions of the in-block backward (bf16 inputs) do the same work
    w["bw_local_kv_mfma"] = w["bw_local_kv"]
    w["bw_local_q_mfma"] = w["bw_local_q"]
    if cfg.topk_clusters and ctx is not None:
        k1, k2 = cfg.topk_clusters, cfg.topk_blocks
        cells = BH * (nb - 1) * Cq                   # (head, i, b >= 1)
        w.update({
            # prefix log Z and every atom's log mass read once, the selections written
            "retr_select": (BH * nb * Cq * Ck * 4 * 3 + cells * k1 * (1 + k2) * 4, 0.0),
            # per (i, b): the chosen clusters' prefix entries and retrieved atoms read, their
            # remainder entries written
            "retr_tables": (cells * (k1 * (1 + k2) * (2 + 2 * D) * 4 + k1 * (1 + 2 * D) * 4), 0.0),
            # per (i, b): the retrieved rows of K and V, the entry's moment read and written;
            # sum over retrieved keys of w v k^T
            "retr_moment_mfma": (ctx["nR"] * 2 * D * e + cells * D * D * 8, 2.0 * D * D * ctx["nR"]),
            # queries with a far field, the retrieved rows (once per (i, b)), the far field
            # read and written; q.k and p v for every (query, retrieved key)
            "retr_exact_mfma": (far_rows * D * e + ctx["nR"] * 2 * D * e + 2 * far, 4.0 * D * ctx["nqR"]),
            "retr_exact": (far_rows * D * e + ctx["nR"] * 2 * D * e + 2 * far, 4.0 * D * ctx["nqR"]),
        })
    return w.get(name)


# kernels whose arithmetic runs on the vector ALUs in fp32 (priced against the vector peak)
ALU_KERNELS = ("bw_refine", "bw_keys_b", "bw_local_kv", "bw_local_q")


def roofline_entry(name: str, cfg, avg_s: float, hier: bool = False, ctx: dict = None):
    """Roofline of one kernel from its measured average launch duration: memory-bound when
    its arithmetic intensity is below the ridge point, else matrix-core-bound (vector-ALU
    bound for the fp32 vector kernels of ALU_KERNELS above their own ridge point)."""
    wk = kernel_work(name, cfg, hier, ctx)
    if wk is None:
        return None
    nbytes, flops = wk
    if name in ALU_KERNELS and flops / nbytes >= PEAK_FP32_VALU_TFLOPS * 1e3 / PEAK_HBM_GBS:
        return {"bound": "alu", "achieved": flops / avg_s / 1e12, "peak": PEAK_FP32_VALU_TFLOPS, "unit": "TFLOP/s",
                "frac": flops / avg_s / 1e12 / PEAK_FP32_VALU_TFLOPS, "bytes_per_launch": nbytes,
                "flops_per_launch": flops}
    if flops / nbytes < RIDGE or flops == 0:
        return {"bound": "hbm", "achieved": nbytes / avg_s / 1e9, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": nbytes / avg_s / 1e9 / PEAK_HBM_GBS, "bytes_per_launch": nbytes, "flops_per_launch": flops}
    return {"bound": "mfma", "achieved": flops / avg_s / 1e12, "peak": PEAK_BF16_MFMA_TFLOPS, "unit": "TFLOP/s",
            "frac": flops / avg_s / 1e12 / PEAK_BF16_MFMA_TFLOPS, "bytes_per_launch": nbytes, "flops_per_launch": flops}


def csrc_sha() -> str:
    """Hash of the library sources (kernels, launchers, public header)."""
    import hashlib
    h = hashlib.sha1()
    d = os.path.join(ROOT, "clustered_softmax_attention_amd", "csrc")
    for f in sorted(os.listdir(d)):
        if f.endswith((".hip", ".hpp")):
            h.update(f.encode())
            with open(os.path.join(d, f), "rb") as fh:
                h.update(fh.read())
    with open(os.path.join(ROOT, "include", "muse.h"), "rb") as fh:
        h.update(fh.read())
    return h.hexdigest()[:16]


def profile_record(workload: str, kernel: str, kind: str = "fwd"):
    """The per-launch figures of `kernel` in the rocprofv3 summary profiles/muse_<kind>_<workload>.md
    (kind fwd: the forward step; bwd: the run with the backward pass), i.e. bytes read and
    written at the L2-to-memory interface from the raw EA request counters, matrix-core busy
    fraction, counted matrix-core flops; None when absent or taken on other kernel sources."""
    path = os.path.join(ROOT, "profiles", f"muse_{kind}_{workload}.md")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        for line in fh:
            if line.startswith("traffic-json: "):
                rec = json.loads(line[len("traffic-json: "):])
                if rec.get("csrc_sha") != csrc_sha() or kernel not in rec["kernels"]:
                    return None
                return rec["kernels"][kernel]
    return None


def measured_traffic(workload: str, kernel: str, kind: str = "fwd"):
    """HBM bytes per launch (read + written) from the profile summary, or None."""
    k = profile_record(workload, kernel, kind)
    return None if k is None else k["fetch_bytes"] + k["write_bytes"]


def timed(fn, steps: int, warmup: int):
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(s)
    for _ in range(steps):
        fn()
    e1.record(s)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return e0.elapsed_time(e1) / steps, wall


def host_cpu_info() -> dict:
    """The host the CPU baseline ran on: logical CPUs, those this process may use, the CPU
    model (from /proc/cpuinfo) and the BLAS thread pool size (threadpoolctl, else
    OMP_NUM_THREADS)."""
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        affinity = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        affinity = os.cpu_count() or 1
    blas = None
    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        blas = max([i.get("num_threads", 1) for i in info if i.get("user_api") == "blas"] or [0]) or None
    except Exception:
        pass
    if blas is None:
        blas = int(os.environ.get("OMP_NUM_THREADS", "1"))
    return {"host_cpus": os.cpu_count(), "affinity_cpus": affinity, "cpu_model": model, "blas_threads": blas}


def cpu_baseline(cfg, q, k, v, budget_s: float):
    """The CPU oracle (unchanged) on whole heads of the same workload until the time budget
    is used; tokens/s scaled to the whole job (every token needs all H heads). `cores` is
    the number of threads the oracle computes with: its matrix products run on the BLAS
    thread pool, everything else on one thread."""
    from oracle import muse_acausal, muse_causal
    host = host_cpu_info()
    heads = [(b, h) for b in range(cfg.B) for h in range(cfg.H)]
    t0 = time.perf_counter()
    done = 0
    for b, h in heads:
        if cfg.causal:
            muse_causal(q[b, h], k[b, h], v[b, h], cfg.Cq, cfg.Ck, cfg.iters, cfg.block)
        else:
            muse_acausal(q[b, h], k[b, h], v[b, h], cfg.Cq, cfg.Ck, cfg.iters)
        done += 1
        if time.perf_counter() - t0 > budget_s:
            break
    t = time.perf_counter() - t0
    tok_s = cfg.N * done / (t * cfg.H)
    return {"value": tok_s, "unit": "tokens/s", "cores": int(host["blas_threads"]), "kind": "oracle",
            "sample": f"{done} of {cfg.B * cfg.H} heads of the same workload ({t:.1f} s), "
                      f"scaled as N*heads_done/(t*H)", **host}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="acausal_8k", choices=sorted(WORKLOAD_TEXT))
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    ap.add_argument("--no-exact", action="store_true", help="skip the exact-attention comparator")
    ap.add_argument("--no-secondary", action="store_true",
                    help="with the default workload, skip the 64k causal configuration reported beside it")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--no-peaks", action="store_true", help="skip the copy and GEMM reference measurements")
    ap.add_argument("--no-backward", action="store_true", help="skip the backward-pass record")
    ap.add_argument("--single-stream", action="store_true",
                    help="run every library kernel on one stream (no side stream), e.g. to profile each alone")
    ap.add_argument("--hierarchy", action="store_true",
                    help="time the hierarchical causal decomposition instead of the prefix form "
                         "(causal workloads without retrieval)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run K device-to-device copies of MIB MiB (to scale HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(heads are independent, so a multi-GPU run would shard (b, h) heads with no communication).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_calibration:
        n = args.copy_calibration * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": 4 * n, "copy_calibration_bytes_written": 4 * n,
                          "launches": args.steps}))
        return
    from clustered_softmax_attention_amd import binding

    binding.load()
    res = measure(args.workload, args.steps, args.warmup, not args.no_exact, args.hierarchy, args.single_stream,
                  backward=not args.no_backward)
    cfg = res["cfg"]
    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(cfg, *res["host_inputs"], args.cpu_budget)
    secondary = None
    if args.workload == "acausal_8k" and not args.no_secondary:
        # the metric is quoted at 8k and at 64k: the 64k causal configuration alongside
        del res["host_inputs"]
        torch.cuda.empty_cache()
        sec = measure(SECONDARY, args.steps, args.warmup, not args.no_exact)
        secondary = {"workload": WORKLOAD_TEXT[SECONDARY], "name": SECONDARY, "value": sec["value"],
                     "unit": "tokens/s", "ms_per_step": sec["ms"], "roofline": sec["roofline"], **sec["extra"]}

    peaks = None if args.no_peaks else measured_peaks()

    line = {
        "metric": METRIC,
        "value": res["value"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": res["ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic Gaussian-mixture Q/K/V (seeded), no dataset",
        "config": {"workload": WORKLOAD_TEXT[args.workload], "name": args.workload, "global_batch": cfg.B,
                   "seq_len": cfg.N, "heads": cfg.H, "head_dim": cfg.D, "Cq": cfg.Cq, "Ck": cfg.Ck,
                   "kmeans_iters": cfg.iters, "causal": cfg.causal, "block": cfg.block,
                   "hierarchy": bool(args.hierarchy), "single_stream": bool(args.single_stream)},
        "roofline": res["roofline"],
        "cpu_baseline": cpu,
        "kernels": res["kernels"],
        "wall_s_timed": res["wall"],
        **res["extra"],
        "secondary": secondary,
        "measured_peaks": peaks,
    }
    if peaks is not None:
        # the dominant kernel against what this GPU reaches for plain streaming / GEMM work
        for rf in [res["roofline"]] + ([secondary["roofline"]] if secondary else []):
            ref = peaks["copy_GBps"] if rf["bound"] == "hbm" else peaks["bf16_gemm_TFLOPs"]
            rf["frac_of_measured_peak"] = rf["achieved"] / ref
    print(json.dumps(line), flush=True)


def measured_peaks() -> dict:
    """What this GPU reaches on plain work, as context for the published peaks: a 1 GiB
    device-to-device copy (bytes read + written per second) and a bf16 8192^3 GEMM
    (torch.matmul, contiguous operands; 2 flops per multiply-add), 10 timed runs each."""
    import torch

    def timed_events(fn, reps=10):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps / 1e3  # seconds per run

    n = 1 << 28  # floats: 1 GiB
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    t_copy = timed_events(lambda: dst.copy_(src))
    del src, dst
    m = 8192
    a = torch.randn(m, m, device="cuda", dtype=torch.bfloat16)
    b = torch.randn(m, m, device="cuda", dtype=torch.bfloat16)
    c = torch.empty(m, m, device="cuda", dtype=torch.bfloat16)
    t_gemm = timed_events(lambda: torch.matmul(a, b, out=c))
    del a, b, c
    torch.cuda.empty_cache()
    return {"copy_GBps": 2 * 4 * n / t_copy / 1e9, "bf16_gemm_TFLOPs": 2 * m ** 3 / t_gemm / 1e12,
            "published_hbm_GBps": PEAK_HBM_GBS, "published_bf16_TFLOPs": PEAK_BF16_MFMA_TFLOPS}


def measure(name: str, steps: int, warmup: int, exact: bool, hierarchy: bool = False,
            single_stream: bool = False, backward: bool = True) -> dict:
    """Time `steps` MuSe forward calls of workload `name` after `warmup` (whole step on
    the GPU, inputs resident), then the per-kernel HIP-event durations over a second pass,
    the roofline of the dominant kernel and, with `exact`, the in-library exact attention."""
    import torch
    from clustered_softmax_attention_amd import binding
    from workloads import CONFIGS, make_inputs

    cfg = CONFIGS[name]
    if hierarchy and (not cfg.causal or cfg.topk_clusters > 0):
        raise SystemExit(f"--hierarchy needs a causal workload without retrieval, not {name}")
    q, k, v = make_inputs(cfg)
    tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    Q, K, V = (torch.from_numpy(t).cuda().to(tdt) for t in (q, k, v))
    ws = torch.empty(binding.workspace_bytes(cfg.B, cfg.H, cfg.N, cfg.D, cfg.Cq, cfg.Ck, cfg.causal,
                                             cfg.block, 1 if cfg.dtype == "bf16" else 0,
                                             cfg.topk_clusters, cfg.topk_blocks, hierarchy=hierarchy),
                     dtype=torch.uint8, device="cuda")
    out = torch.empty_like(Q)

    def muse_step():
        binding.attn_fwd(Q, K, V, cfg.Cq, cfg.Ck, cfg.iters, causal=cfg.causal, block=cfg.block, out=out,
                         topk_clusters=cfg.topk_clusters, topk_blocks=cfg.topk_blocks, workspace=ws,
                         hierarchy=hierarchy, single_stream=single_stream)

    print(f"# timing {name}: {warmup} warmup + {steps} steps", file=sys.stderr, flush=True)
    ms, wall = timed(muse_step, steps, warmup)
    value = cfg.B * cfg.N / (ms / 1e3)

    # per-kernel durations, HIP events on the launch stream, over a second pass of K steps
    binding.prof_reset()
    binding.prof_enable(True)
    for _ in range(steps):
        muse_step()
    torch.cuda.synchronize()
    prof = binding.prof_collect()
    binding.prof_enable(False)
    kernels = {n: {"avg_us": 1e3 * t / c, "launches_per_step": c / steps} for n, (t, c) in prof.items()}
    ctx = None
    if cfg.topk_clusters:
        # retrieved key counts (data-dependent) from one traced call: selections and buckets
        _, ex_r = binding.attn_fwd(Q, K, V, cfg.Cq, cfg.Ck, cfg.iters, causal=cfg.causal, block=cfg.block,
                                   topk_clusters=cfg.topk_clusters, topk_blocks=cfg.topk_blocks,
                                   return_trace=True, return_buckets=True)
        torch.cuda.synchronize()
        ctx = retrieval_counts(cfg, ex_r)
        del ex_r
    # dominant kernel: the largest share of the step among those with a defined roofline
    ranked = sorted(prof.items(), key=lambda kv: -kv[1][0])
    dom = next(n for n, _ in ranked if kernel_work(n, cfg, hierarchy, ctx) is not None)
    avg_s = prof[dom][0] / prof[dom][1] / 1e3
    profile = name + ("_hierarchy" if hierarchy else "")
    # with the hierarchy, stage 2 is several dispatches per call (one per chain level) while
    # the counters are per dispatch: no per-call traffic figure for it
    traffic = None if (hierarchy and dom == "s2_mfma") else measured_traffic(profile, dom)
    rec = profile_record(profile, dom)
    roofline = {"kernel": dom, **roofline_entry(dom, cfg, avg_s, hierarchy, ctx), "traffic": traffic,
                "mfma_busy_counter": None if rec is None else rec.get("mfma_busy"),
                "share_of_step": prof[dom][0] / sum(t for t, _ in prof.values())}
    for n, d in kernels.items():
        r = roofline_entry(n, cfg, prof[n][0] / prof[n][1] / 1e3, hierarchy, ctx)
        if r is not None:
            d.update({"bound": r["bound"], "frac": r["frac"]})
    print(f"# kernels: " + ", ".join(f"{n} {d['avg_us']:.1f}us x{d['launches_per_step']:.0f}"
                                     for n, d in sorted(kernels.items(), key=lambda kv: -prof[kv[0]][0])),
          file=sys.stderr, flush=True)

    extra = {}
    if exact:
        out_ex = torch.empty_like(Q)

        def exact_step():
            binding.exact_attn_fwd(Q, K, V, causal=cfg.causal, out=out_ex)

        ex_steps = max(1, min(steps, 3))
        ms_ex, _ = timed(exact_step, ex_steps, 1)
        muse_step()
        torch.cuda.synchronize()
        o_m, o_e = out.double(), out_ex.double()
        rse = float(((o_m - o_e) ** 2).sum() / (o_e ** 2).sum())
        extra = {"exact_ms_per_step": ms_ex, "speedup_vs_exact": ms_ex / ms, "rse_vs_exact": rse}
        print(f"# exact {ms_ex:.3f} ms/step, MuSe {ms:.3f} ms/step, speedup {ms_ex / ms:.2f}x, RSE {rse:.3e}",
              file=sys.stderr, flush=True)
        def variant(label: str, iters: int, kernel_filter, **kw):
            # the same workload with other options, timed like the main step; RSE against
            # exact attention and the per-kernel durations of one profiled call
            ws_x = torch.empty(binding.workspace_bytes(cfg.B, cfg.H, cfg.N, cfg.D, cfg.Cq, cfg.Ck, cfg.causal,
                                                       cfg.block, 1 if cfg.dtype == "bf16" else 0, **kw),
                               dtype=torch.uint8, device="cuda")

            def step():
                binding.attn_fwd(Q, K, V, cfg.Cq, cfg.Ck, iters, causal=cfg.causal, block=cfg.block, out=out,
                                 workspace=ws_x, **kw)

            ms_x, _ = timed(step, steps, warmup)
            binding.prof_reset()
            binding.prof_enable(True)
            step()
            torch.cuda.synchronize()
            prof_x = binding.prof_collect()
            binding.prof_enable(False)
            o_x = out.double()
            rse_x = float(((o_x - o_e) ** 2).sum() / (o_e ** 2).sum())
            extra[label] = {
                "ms_per_step": ms_x, "value": cfg.B * cfg.N / (ms_x / 1e3), "speedup_vs_exact": ms_ex / ms_x,
                "rse_vs_exact": rse_x,
                "kernels_us": {n: round(1e3 * t / c, 2) for n, (t, c) in sorted(prof_x.items(), key=lambda kv: -kv[1][0])
                               if kernel_filter(n)}}
            print(f"# {label}: {ms_x:.3f} ms/step, speedup {ms_ex / ms_x:.2f}x, RSE {rse_x:.3e}, "
                  f"{extra[label]['kernels_us']}", file=sys.stderr, flush=True)

        if cfg.topk_clusters == 0 and not hierarchy:
            # the untilted (per key cluster) dipole
            variant("untilted_dipole", cfg.iters, lambda n: "untilted" in n or "cov" in n, dipole="untilted")
            # the paper's speed setting: key clusters capped at 1.5 N / Ck members, one
            # Lloyd iteration
            variant("cap1.5_iters1", 1, lambda n: True, cap_ratio=1.5)
        if cfg.topk_clusters > 0:
            # the same workload with retrieval off (k1 = 0): what retrieval changes in time
            # and in error against exact attention
            variant("retrieval_off", cfg.iters, lambda n: True)
        if cfg.causal and cfg.topk_clusters == 0 and not hierarchy:
            # the hierarchical block decomposition (one two-stage approximation per square
            # below the diagonal, log-sum-exp merged)
            variant("hierarchy", cfg.iters, lambda n: True, hierarchy=True)
    if backward and cfg.D == 64 and cfg.topk_clusters == 0 and not hierarchy:
        # the backward pass (dq, dk, dv for an upstream gradient, labels of one forward call
        # held fixed), timed like the forward step
        _, ex_b = binding.attn_fwd(Q, K, V, cfg.Cq, cfg.Ck, cfg.iters, causal=cfg.causal, block=cfg.block,
                                   return_trace=True)
        lq = ex_b["labels_q_trace"][-1].contiguous()
        lk = ex_b["labels_k_trace"][-1].contiguous()
        del ex_b
        gen = torch.Generator(device="cuda").manual_seed(11)
        dO = torch.randn(Q.shape, generator=gen, device="cuda", dtype=torch.float32).to(Q.dtype)
        ws_b = torch.empty(binding.bwd_workspace_bytes(cfg.B, cfg.H, cfg.N, cfg.D, cfg.Cq, cfg.Ck, cfg.causal,
                                                       cfg.block, 1 if cfg.dtype == "bf16" else 0),
                           dtype=torch.uint8, device="cuda")

        def bwd_step():
            binding.attn_bwd(Q, K, V, dO, lq, lk, cfg.Cq, cfg.Ck, causal=cfg.causal, block=cfg.block, workspace=ws_b)

        ms_b, _ = timed(bwd_step, steps, warmup)
        binding.prof_reset()
        binding.prof_enable(True)
        bwd_step()
        torch.cuda.synchronize()
        prof_b = binding.prof_collect()
        binding.prof_enable(False)
        dom_b = next((n for n, _ in sorted(prof_b.items(), key=lambda kv: -kv[1][0])
                      if kernel_work(n, cfg) is not None), None)
        rec_b = None if dom_b is None else profile_record(name, dom_b, "bwd")
        extra["backward"] = {
            "ms_per_step": ms_b, "value": cfg.B * cfg.N / (ms_b / 1e3), "unit": "tokens/s",
            "roofline": None if dom_b is None else {
                "kernel": dom_b, **roofline_entry(dom_b, cfg, prof_b[dom_b][0] / prof_b[dom_b][1] / 1e3),
                "traffic": measured_traffic(name, dom_b, "bwd"),
                "mfma_busy_counter": None if rec_b is None else rec_b.get("mfma_busy")},
            "kernels_us": {n: round(1e3 * t / c, 2) for n, (t, c) in sorted(prof_b.items(), key=lambda kv: -kv[1][0])}}
        print(f"# backward: {ms_b:.3f} ms/step, {extra['backward']['kernels_us']}", file=sys.stderr, flush=True)
        del ws_b
    if ctx is not None:
        extra["retrieved_keys"] = ctx
    return {"cfg": cfg, "ms": ms, "wall": wall, "value": value, "kernels": kernels, "roofline": roofline,
            "extra": extra, "host_inputs": (q, k, v)}


if __name__ == "__main__":
    main()
