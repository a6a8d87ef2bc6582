"""Throughput of the MuSe forward pass on one MI355X, with roofline and CPU-oracle baseline.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload acausal_8k] [--no-cpu]
                [--no-exact] [--no-secondary] [--no-peaks] [--hierarchy]

A step is one muse_attn_fwd call over the whole workload batch (K-means, stage 1,
stage 2 and, when causal, the exact diagonal blocks), with inputs resident in HBM and
the workspace allocated beforehand. Prints ONE JSON line: `value` is the 8k workload's
tokens/s (or the chosen workload's). Extra fields: the in-library exact attention time
on the same shape (speedup), the relative squared error of MuSe against it, per-kernel
average durations measured with HIP events on the stream the kernels run on, the
untilted-dipole run of an acausal workload, the hierarchical-decomposition run of a causal
one without retrieval, `measured_peaks` (a device copy and a bf16
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


def kernel_work(name: str, cfg, hier: bool = False):
    """(algorithmic bytes, algorithmic flops) of ONE launch of a library kernel on this
    workload, or None when the kernel is not listed. Bytes count every tensor a launch
    must read or write at least once (inputs read once, outputs written once); flops count
    the arithmetic the method defines (multiply-add = 2), not the extra products of the
    bf16 hi/lo splits. Causal tables have one entry per block (nbS = nb). With the
    hierarchical decomposition (hier) stage 2 of block b reads popcount(b) entries, so
    entry e is read lowbit(e) times: its table reads scale by sum_b popcount(b) / (nb - 1);
    stage 2 then runs one launch per chain level (the bit length of nb - 1), each reading
    the queries and writing the far field; the figure is per call, as the library's
    HIP-event scope covers those launches together."""
    BH, N, D, Cq, Ck = cfg.B * cfg.H, cfg.N, cfg.D, cfg.Cq, cfg.Ck
    e = 2 if cfg.dtype == "bf16" else 4
    nb = cfg.N // cfg.block if cfg.causal else 1
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
    reads = (sum(bin(b).count("1") for b in range(nb)) / (nb - 1)) if (hier and nb > 1) else 1.0
    levels = (nb - 1).bit_length() if (hier and nb > 1) else 1
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
        "s2_mfma": (levels * 2 * x + reads * (tbytes + BH * nb * Cq * D * D * 2),
                    2.0 * BH * N * (2 * Ck * D + D * D) * reads),
        "s2_refine": (x + x + table * (1 + 2 * D) * 4 + BH * nb * Cq * D * D * 4, 2.0 * BH * N * (2 * Ck * D + D * D)),
        "local_block_mfma": (3 * x + BH * N * D * 4, 4.0 * BH * N * (cfg.block / 2) * D),
        "exact_mfma": (4 * x, (2.0 if cfg.causal else 4.0) * BH * N * N * D),
        "exact_valu": (4 * x, (2.0 if cfg.causal else 4.0) * BH * N * N * D),
    }
    return w.get(name)


def roofline_entry(name: str, cfg, avg_s: float, hier: bool = False):
    """Roofline of one kernel from its measured average launch duration: memory-bound when
    its arithmetic intensity is below the ridge point, else matrix-core-bound."""
    wk = kernel_work(name, cfg, hier)
    if wk is None:
        return None
    nbytes, flops = wk
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


def measured_traffic(workload: str, kernel: str):
    """HBM bytes per launch (scaled FETCH_SIZE + WRITE_SIZE) recorded in the rocprofv3 summary
    profiles/muse_fwd_<workload>.md, or None when absent or taken on other kernel sources."""
    path = os.path.join(ROOT, "profiles", f"muse_fwd_{workload}.md")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        for line in fh:
            if line.startswith("traffic-json: "):
                rec = json.loads(line[len("traffic-json: "):])
                if rec.get("csrc_sha") != csrc_sha() or kernel not in rec["kernels"]:
                    return None
                k = rec["kernels"][kernel]
                return k["fetch_bytes"] + k["write_bytes"]
    return None


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


def cpu_baseline(cfg, q, k, v, budget_s: float):
    """The CPU oracle (unchanged) on whole heads of the same workload until the time budget
    is used; tokens/s scaled to the whole job (every token needs all H heads)."""
    from oracle import muse_acausal, muse_causal
    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        threads = max([i.get("num_threads", 1) for i in info] or [os.cpu_count() or 1])
    except Exception:
        threads = os.cpu_count() or 1
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
    return {"value": tok_s, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{done} of {cfg.B * cfg.H} heads of the same workload ({t:.1f} s), "
                      f"scaled as N*heads_done/(t*H)"}


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
    res = measure(args.workload, args.steps, args.warmup, not args.no_exact, args.hierarchy)
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
                   "hierarchy": bool(args.hierarchy)},
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


def measure(name: str, steps: int, warmup: int, exact: bool, hierarchy: bool = False) -> dict:
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
                         hierarchy=hierarchy)

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
    # dominant kernel: the largest share of the step among those with a defined roofline
    ranked = sorted(prof.items(), key=lambda kv: -kv[1][0])
    dom = next(n for n, _ in ranked if kernel_work(n, cfg, hierarchy) is not None)
    avg_s = prof[dom][0] / prof[dom][1] / 1e3
    profile = name + ("_hierarchy" if hierarchy else "")
    # with the hierarchy, stage 2 is several dispatches per call (one per chain level) while
    # the counters are per dispatch: no per-call traffic figure for it
    traffic = None if (hierarchy and dom == "s2_mfma") else measured_traffic(profile, dom)
    roofline = {"kernel": dom, **roofline_entry(dom, cfg, avg_s, hierarchy), "traffic": traffic,
                "share_of_step": prof[dom][0] / sum(t for t, _ in prof.values())}
    for n, d in kernels.items():
        r = roofline_entry(n, cfg, prof[n][0] / prof[n][1] / 1e3, hierarchy)
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
        if not cfg.causal:
            # the same workload with the untilted (per key cluster) dipole
            ws_u = torch.empty(binding.workspace_bytes(cfg.B, cfg.H, cfg.N, cfg.D, cfg.Cq, cfg.Ck, False, 0,
                                                       1 if cfg.dtype == "bf16" else 0, dipole="untilted"),
                               dtype=torch.uint8, device="cuda")

            def untilted_step():
                binding.attn_fwd(Q, K, V, cfg.Cq, cfg.Ck, cfg.iters, out=out, dipole="untilted", workspace=ws_u)

            ms_u, _ = timed(untilted_step, steps, warmup)
            binding.prof_reset()
            binding.prof_enable(True)
            untilted_step()
            torch.cuda.synchronize()
            prof_u = binding.prof_collect()
            binding.prof_enable(False)
            o_u = out.double()
            rse_u = float(((o_u - o_e) ** 2).sum() / (o_e ** 2).sum())
            extra["untilted_dipole"] = {
                "ms_per_step": ms_u, "value": cfg.B * cfg.N / (ms_u / 1e3), "speedup_vs_exact": ms_ex / ms_u,
                "rse_vs_exact": rse_u,
                "kernels_us": {n: round(1e3 * t / c, 2) for n, (t, c) in prof_u.items() if "untilted" in n or "cov" in n}}
            print(f"# untilted dipole: {ms_u:.3f} ms/step, speedup {ms_ex / ms_u:.2f}x, RSE {rse_u:.3e}, "
                  f"{extra['untilted_dipole']['kernels_us']}", file=sys.stderr, flush=True)
        elif cfg.topk_clusters == 0 and not hierarchy:
            # the same workload with the hierarchical block decomposition (one two-stage
            # approximation per square below the diagonal, log-sum-exp merged)
            ws_h = torch.empty(binding.workspace_bytes(cfg.B, cfg.H, cfg.N, cfg.D, cfg.Cq, cfg.Ck, True, cfg.block,
                                                       1 if cfg.dtype == "bf16" else 0, hierarchy=True),
                               dtype=torch.uint8, device="cuda")

            def hier_step():
                binding.attn_fwd(Q, K, V, cfg.Cq, cfg.Ck, cfg.iters, causal=True, block=cfg.block, out=out,
                                 workspace=ws_h, hierarchy=True)

            ms_h, _ = timed(hier_step, steps, warmup)
            binding.prof_reset()
            binding.prof_enable(True)
            hier_step()
            torch.cuda.synchronize()
            prof_h = binding.prof_collect()
            binding.prof_enable(False)
            o_h = out.double()
            rse_h = float(((o_h - o_e) ** 2).sum() / (o_e ** 2).sum())
            extra["hierarchy"] = {
                "ms_per_step": ms_h, "value": cfg.B * cfg.N / (ms_h / 1e3), "speedup_vs_exact": ms_ex / ms_h,
                "rse_vs_exact": rse_h,
                "kernels_us": {n: round(1e3 * t / c, 2) for n, (t, c) in sorted(prof_h.items(), key=lambda kv: -kv[1][0])}}
            print(f"# hierarchy: {ms_h:.3f} ms/step, speedup {ms_ex / ms_h:.2f}x, RSE {rse_h:.3e}, "
                  f"{extra['hierarchy']['kernels_us']}", file=sys.stderr, flush=True)
    return {"cfg": cfg, "ms": ms, "wall": wall, "value": value, "kernels": kernels, "roofline": roofline,
            "extra": extra, "host_inputs": (q, k, v)}


if __name__ == "__main__":
    main()
