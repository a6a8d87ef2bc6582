"""Throughput of the MuSe forward pass on one MI355X, with roofline and CPU-oracle baseline.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c2] [--no-cpu]

A step is one muse_attn_fwd call over the whole workload batch (K-means, stage 1,
stage 2 and, when causal, the exact diagonal blocks), with inputs resident in HBM and
the workspace allocated beforehand. Prints ONE JSON line. Extra fields: the in-library
exact attention time on the same shape (speedup), the relative squared error of MuSe
against it, and per-kernel average durations measured with HIP events on the stream the
kernels run on.
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
    "c1": "acausal MuSe fwd, B=1 H=1 N=1024 D=64 fp32, Cq=8 Ck=32, 5 Lloyd iterations",
    "c2": "acausal MuSe fwd, B=4 H=8 N=8192 D=64 bf16 (fp32 accumulate), Cq=32 Ck=128, 5 Lloyd iterations",
    "c3": "causal MuSe fwd, B=8 H=8 N=16384 D=64 bf16, block 1024, Cq=16 Ck=64, 5 Lloyd iterations",
    "c4": "causal MuSe fwd, B=1 H=16 N=65536 D=128 bf16, block 2048, Cq=32 Ck=128, 5 Lloyd iterations",
    "c5": "causal MuSe fwd with retrieval k1=4 k2=2, B=2 H=8 N=16384 D=64 bf16, block 1024, Cq=16 Ck=64",
}


def kernel_work(name: str, cfg) -> tuple:
    """(bound, algorithmic amount per launch, unit, peak) of a library kernel on this workload.

    Flop counts are multiply-add = 2 flops, per head, times B*H heads."""
    BH, N, D, Cq, Ck = cfg.B * cfg.H, cfg.N, cfg.D, cfg.Cq, cfg.Ck
    nb = cfg.N // cfg.block if cfg.causal else 1
    e = 2 if cfg.dtype == "bf16" else 4
    valu = ("alu", "TFLOP/s", PEAK_FP32_VALU_TFLOPS)
    mfma = ("mfma", "TFLOP/s", PEAK_BF16_MFMA_TFLOPS)
    tbl = {
        "kmeans_assign": (valu, 2.0 * N * (Cq + Ck) * D * BH),
        "kmeans_assign_mfma": (mfma, 2.0 * N * (Cq + Ck) * D * BH),
        "s1_atoms": (valu, 6.0 * Cq * N * D * BH),
        "s1_moments": (valu, (2.0 * Cq * N * D * D + 2.0 * Cq * N * D) * BH),
        "s1_moments_mfma": (mfma, (2.0 * Cq * N * D * D + 2.0 * Cq * N * D) * BH),
        "s1_dip_final": (valu, 2.0 * nb * Cq * Ck * D * D * BH),
        "s2_refine": (valu, 2.0 * N * (2 * Ck * D + D * D) * BH),
        "exact_valu": (valu, (2.0 if cfg.causal else 4.0) * N * N * D * BH),
        "local_block_exact": (valu, 2.0 * N * cfg.block * D * BH),
    }
    if name in tbl:
        (bound, unit, peak), amount = tbl[name]
        return bound, amount / 1e12, unit, peak
    # streaming kernels: minimum bytes (inputs read once, outputs written once)
    return "hbm", 2.0 * N * D * e * BH / 1e9, "GB/s", PEAK_HBM_GBS


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
    ap.add_argument("--workload", default="c2", choices=sorted(WORKLOAD_TEXT))
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    ap.add_argument("--no-exact", action="store_true", help="skip the exact-attention comparator")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run K device-to-device copies of MIB MiB (to scale HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported by this build "
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
    from workloads import CONFIGS, make_inputs

    binding.load()
    cfg = CONFIGS[args.workload]
    q, k, v = make_inputs(cfg)
    tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    Q, K, V = (torch.from_numpy(t).cuda().to(tdt) for t in (q, k, v))
    ws = torch.empty(binding.workspace_bytes(cfg.B, cfg.H, cfg.N, cfg.D, cfg.Cq, cfg.Ck, cfg.causal,
                                             cfg.block, 1 if cfg.dtype == "bf16" else 0,
                                             cfg.topk_clusters, cfg.topk_blocks),
                     dtype=torch.uint8, device="cuda")
    out = torch.empty_like(Q)

    def muse_step():
        binding.attn_fwd(Q, K, V, cfg.Cq, cfg.Ck, cfg.iters, causal=cfg.causal, block=cfg.block, out=out,
                         topk_clusters=cfg.topk_clusters, topk_blocks=cfg.topk_blocks, workspace=ws)

    print(f"# timing {args.workload}: {args.warmup} warmup + {args.steps} steps", file=sys.stderr, flush=True)
    ms, wall = timed(muse_step, args.steps, args.warmup)
    tokens = cfg.B * cfg.N
    value = tokens / (ms / 1e3)

    # per-kernel durations, HIP events on the launch stream, over a second pass of K steps
    binding.prof_reset()
    binding.prof_enable(True)
    for _ in range(args.steps):
        muse_step()
    torch.cuda.synchronize()
    prof = binding.prof_collect()
    binding.prof_enable(False)
    kernels = {n: {"avg_us": 1e3 * t / c, "launches_per_step": c / args.steps} for n, (t, c) in prof.items()}
    dom = max(prof.items(), key=lambda kv: kv[1][0])[0]
    bound, amount, unit, peak = kernel_work(dom, cfg)
    avg_s = prof[dom][0] / prof[dom][1] / 1e3
    achieved = amount / avg_s
    roofline = {"bound": bound, "kernel": dom, "achieved": achieved, "peak": peak, "unit": unit,
                "frac": achieved / peak, "traffic": None}
    print(f"# kernels: " + ", ".join(f"{n} {d['avg_us']:.1f}us x{d['launches_per_step']:.0f}"
                                     for n, d in sorted(kernels.items(), key=lambda kv: -prof[kv[0]][0])),
          file=sys.stderr, flush=True)

    extra = {}
    if not args.no_exact:
        out_ex = torch.empty_like(Q)

        def exact_step():
            binding.exact_attn_fwd(Q, K, V, causal=cfg.causal, out=out_ex)

        ex_steps = max(1, min(args.steps, 3))
        ms_ex, _ = timed(exact_step, ex_steps, 1)
        muse_step()
        torch.cuda.synchronize()
        o_m, o_e = out.double(), out_ex.double()
        rse = float(((o_m - o_e) ** 2).sum() / (o_e ** 2).sum())
        extra = {"exact_ms_per_step": ms_ex, "speedup_vs_exact": ms_ex / ms, "rse_vs_exact": rse}
        print(f"# exact {ms_ex:.3f} ms/step, MuSe {ms:.3f} ms/step, speedup {ms_ex / ms:.2f}x, RSE {rse:.3e}",
              file=sys.stderr, flush=True)

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(cfg, q, k, v, args.cpu_budget)

    line = {
        "metric": "MuSe fwd tokens/s",
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic Gaussian-mixture Q/K/V (seeded), no dataset",
        "config": {"workload": WORKLOAD_TEXT[args.workload], "name": args.workload, "global_batch": cfg.B,
                   "seq_len": cfg.N, "heads": cfg.H, "head_dim": cfg.D, "Cq": cfg.Cq, "Ck": cfg.Ck,
                   "kmeans_iters": cfg.iters, "causal": cfg.causal, "block": cfg.block},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "kernels": kernels,
        "wall_s_timed": wall,
        **extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
