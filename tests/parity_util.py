"""Helpers shared by the GPU parity tests: move seeded inputs to the device, run the
library through its C-ABI binding, and compare with the CPU oracle head by head."""

from __future__ import annotations

import dataclasses
import sys
import time
from typing import List, Optional, Sequence, Tuple

import numpy as np
import torch

from oracle import bucket_order, cap_key_labels, exact_attention, lloyd_kmeans, muse_acausal, muse_causal
from workloads import WorkloadConfig, make_inputs

# Tolerances on relative L2 error (whole checked tensor) for fp32 and bf16 inputs with
# fp32 accumulation.
TOL = {"f32": 1e-5, "bf16": 3e-3}


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def to_device(x: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x)).cuda()
    return t.to(torch.bfloat16) if dtype == "bf16" else t


def rel_l2(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


@dataclasses.dataclass
class HeadCheck:
    b: int
    h: int
    rel: float
    near_ties_q: int
    near_ties_k: int
    dropped_k: int = 0   # keys left out of the stage-1 summaries by a cluster size cap


def run_gpu(cfg: WorkloadConfig, q, k, v, out_dtype=torch.float32, dipole=True, labels_q_in=None,
            labels_k_in=None, topk=None, hierarchy=False, scale: float = 0.0, extra_returns: bool = False,
            cap_ratio: float = 0.0, plain: bool = False):
    """plain: the output only (no traces, log-sum-exp or other extra outputs), as the
    benchmark calls it."""
    if topk is None:
        topk = (cfg.topk_clusters, cfg.topk_blocks)
    from clustered_softmax_attention_amd import attn_fwd
    Q, K, V = (to_device(t, cfg.dtype) for t in (q, k, v))
    if plain:
        out = attn_fwd(Q, K, V, cfg.Cq, cfg.Ck, cfg.iters, causal=cfg.causal, block=cfg.block,
                       out_dtype=out_dtype, dipole=dipole, labels_q_in=labels_q_in, labels_k_in=labels_k_in,
                       topk_clusters=topk[0], topk_blocks=topk[1], hierarchy=hierarchy, scale=scale,
                       cap_ratio=cap_ratio)
        torch.cuda.synchronize()
        return out, {}
    out, ex = attn_fwd(Q, K, V, cfg.Cq, cfg.Ck, cfg.iters, causal=cfg.causal, block=cfg.block,
                       out_dtype=out_dtype, dipole=dipole, return_trace=True, return_lse=True,
                       return_centroids=extra_returns, return_buckets=extra_returns,
                       labels_q_in=labels_q_in, labels_k_in=labels_k_in,
                       topk_clusters=topk[0], topk_blocks=topk[1], hierarchy=hierarchy, scale=scale,
                       cap_ratio=cap_ratio)
    torch.cuda.synchronize()
    return out, ex


def oracle_head(cfg: WorkloadConfig, q, k, v, trace_q, trace_k, dipole="tilted",
                blocks: Optional[Sequence[int]] = None, rows: Optional[np.ndarray] = None,
                retrieval_trace: Optional[np.ndarray] = None, hierarchy: bool = False,
                scale: Optional[float] = None, cap_ratio: Optional[float] = None):
    """Oracle of one head in follow mode (near-tie labels adopted from the GPU traces).
    Retrieval selections must equal the GPU's exactly (no near-tie adoption)."""
    kq = lloyd_kmeans(q, cfg.Cq, cfg.iters, follow_trace=trace_q)
    kk = lloyd_kmeans(k, cfg.Ck, cfg.iters, follow_trace=trace_k)
    assert kq.mismatches == 0, f"query labels differ beyond near-ties: {kq.mismatch_info}"
    assert kk.mismatches == 0, f"key labels differ beyond near-ties: {kk.mismatch_info}"
    if cfg.causal:
        r = muse_causal(q, k, v, cfg.Cq, cfg.Ck, cfg.iters, cfg.block, dipole=dipole, scale=scale,
                        topk_clusters=cfg.topk_clusters, topk_blocks=cfg.topk_blocks,
                        labels_q=kq.labels, labels_k=kk.labels, blocks_to_eval=blocks,
                        retrieval_follow=retrieval_trace, hierarchical=hierarchy, cap_ratio=cap_ratio)
        assert r.retrieval_mismatches == 0, "retrieval selections differ beyond near-ties"
        assert r.retrieval_near_ties == 0, "retrieval selections adopted from the GPU at near-ties"
    else:
        r = muse_acausal(q, k, v, cfg.Cq, cfg.Ck, cfg.iters, dipole=dipole, scale=scale,
                         labels_q=kq.labels, labels_k=kk.labels, rows=rows, cap_ratio=cap_ratio)
    return r, kq, kk


def check_centroids_and_buckets(cfg: WorkloadConfig, ex: dict, b: int, h: int, kq, kk):
    """Final centroids against the oracle's member means, and the bucket order (the
    stable grouping by (block, cluster)) bit-exactly against the oracle's definition
    applied to the same final labels."""
    blk = cfg.block if cfg.causal else 0
    for name, km, C in (("q", kq, cfg.Cq), ("k", kk, cfg.Ck)):
        c_gpu = ex["centroids_" + name][b, h].cpu().numpy()
        rel = rel_l2(c_gpu, km.centroids)
        assert rel <= 1e-5, f"{name} centroids rel-L2 {rel}"
        perm, offs = bucket_order(km.labels, C, blk)
        assert np.array_equal(ex["perm_" + name][b, h].cpu().numpy(), perm), f"{name} bucket permutation"
        assert np.array_equal(ex["offs_" + name][b, h].cpu().numpy(), offs), f"{name} bucket offsets"


def oracle_dipole(dipole) -> str:
    """The oracle's dipole mode for a binding dipole argument (True, False or a mode name)."""
    if isinstance(dipole, bool):
        return "tilted" if dipole else "none"
    return str(dipole)


def check_config(cfg: WorkloadConfig, heads: List[Tuple[int, int]], tol: Optional[float] = None,
                 blocks: Optional[Sequence[int]] = None, out_dtype=torch.float32, dipole=True,
                 rows: Optional[np.ndarray] = None, hierarchy: bool = False, scale: Optional[float] = None,
                 inputs=None, cap_ratio: Optional[float] = None) -> List[HeadCheck]:
    """Run the whole [B,H,N,D] workload on the GPU and compare the listed heads.

    scale: softmax scale passed to both sides (None: the library's and the oracle's
    default 1/sqrt(D)). inputs: (q, k, v) to use instead of the workload's generator.
    cap_ratio: key cluster size cap passed to both sides (None: no cap).
    Besides the output and LSE, the final centroids (relative L2 <= 1e-5 per head: fp32
    member means against float64 ones) and the bucket order (bit-exact) are compared.
    The output of a second call that asks for nothing else (the benchmark's launches:
    no traces and no log-sum-exp output) is compared at the same tolerance."""
    t0 = time.time()
    q, k, v = make_inputs(cfg) if inputs is None else inputs
    out, ex = run_gpu(cfg, q, k, v, out_dtype=out_dtype, dipole=dipole, hierarchy=hierarchy,
                      scale=0.0 if scale is None else scale, extra_returns=True,
                      cap_ratio=0.0 if cap_ratio is None else cap_ratio)
    o_gpu = out.float().cpu().numpy()
    out2, _ = run_gpu(cfg, q, k, v, out_dtype=out_dtype, dipole=dipole, hierarchy=hierarchy,
                      scale=0.0 if scale is None else scale, cap_ratio=0.0 if cap_ratio is None else cap_ratio,
                      plain=True)
    o_plain = out2.float().cpu().numpy()
    del out2
    tq = ex["labels_q_trace"].cpu().numpy()
    tk = ex["labels_k_trace"].cpu().numpy()
    lse = ex["lse"].cpu().numpy()
    rtr = ex["retrieval_trace"].cpu().numpy() if "retrieval_trace" in ex else None
    log(f"[{cfg.name}] gpu done in {time.time() - t0:.1f}s; checking heads {heads}")
    res = []
    tol = TOL[cfg.dtype] if tol is None else tol
    for b, h in heads:
        r, kq, kk = oracle_head(cfg, q[b, h], k[b, h], v[b, h], tq[:, b, h], tk[:, b, h],
                                dipole=oracle_dipole(dipole), blocks=blocks, rows=rows,
                                retrieval_trace=None if rtr is None else rtr[b, h], hierarchy=hierarchy,
                                scale=scale, cap_ratio=cap_ratio)
        assert np.array_equal(kq.labels, tq[-1, b, h]) and np.array_equal(kk.labels, tk[-1, b, h])
        check_centroids_and_buckets(cfg, ex, b, h, kq, kk)
        sel = np.isfinite(r.o[:, 0])
        rel = rel_l2(o_gpu[b, h][sel], r.o[sel])
        rel_plain = rel_l2(o_plain[b, h][sel], r.o[sel])
        lse_err = float(np.max(np.abs(lse[b, h][sel] - r.lse[sel])))
        log(f"[{cfg.name}] head ({b},{h}): rel-L2 {rel:.3e} (plain call {rel_plain:.3e}, tol {tol:.0e}), "
            f"max |dLSE| {lse_err:.2e}, "
            f"near-ties q={kq.near_ties} k={kk.near_ties} retrieval={r.retrieval_near_ties}, "
            f"rows checked {int(sel.sum())}")
        assert rel <= tol, f"rel-L2 {rel} > {tol}"
        assert rel_plain <= tol, f"rel-L2 of the plain call {rel_plain} > {tol}"
        assert lse_err <= (1e-4 if cfg.dtype == "f32" else 2e-3)
        dropped = int((cap_key_labels(kk.labels, cfg.Ck, cap_ratio) < 0).sum())
        if cap_ratio is not None:
            log(f"[{cfg.name}] head ({b},{h}): cap ratio {cap_ratio}: {dropped} keys left out")
        res.append(HeadCheck(b, h, rel, kq.near_ties, kk.near_ties, dropped))
    return res
