"""Helpers shared by the GPU parity tests: move seeded inputs to the device, run the
library through its C-ABI binding, and compare with the CPU oracle head by head."""

from __future__ import annotations

import dataclasses
import sys
import time
from typing import List, Optional, Sequence, Tuple

import numpy as np
import torch

from oracle import exact_attention, lloyd_kmeans, muse_acausal, muse_causal
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


def run_gpu(cfg: WorkloadConfig, q, k, v, out_dtype=torch.float32, dipole=True, labels_q_in=None,
            labels_k_in=None, topk=None, hierarchy=False):
    if topk is None:
        topk = (cfg.topk_clusters, cfg.topk_blocks)
    from clustered_softmax_attention_amd import attn_fwd
    Q, K, V = (to_device(t, cfg.dtype) for t in (q, k, v))
    out, ex = attn_fwd(Q, K, V, cfg.Cq, cfg.Ck, cfg.iters, causal=cfg.causal, block=cfg.block,
                       out_dtype=out_dtype, dipole=dipole, return_trace=True, return_lse=True,
                       labels_q_in=labels_q_in, labels_k_in=labels_k_in,
                       topk_clusters=topk[0], topk_blocks=topk[1], hierarchy=hierarchy)
    torch.cuda.synchronize()
    return out, ex


def oracle_head(cfg: WorkloadConfig, q, k, v, trace_q, trace_k, dipole="tilted",
                blocks: Optional[Sequence[int]] = None, rows: Optional[np.ndarray] = None,
                retrieval_trace: Optional[np.ndarray] = None, hierarchy: bool = False):
    """Oracle of one head in follow mode (near-tie labels adopted from the GPU traces)."""
    kq = lloyd_kmeans(q, cfg.Cq, cfg.iters, follow_trace=trace_q)
    kk = lloyd_kmeans(k, cfg.Ck, cfg.iters, follow_trace=trace_k)
    assert kq.mismatches == 0, f"query labels differ beyond near-ties: {kq.mismatch_info}"
    assert kk.mismatches == 0, f"key labels differ beyond near-ties: {kk.mismatch_info}"
    if cfg.causal:
        r = muse_causal(q, k, v, cfg.Cq, cfg.Ck, cfg.iters, cfg.block, dipole=dipole,
                        topk_clusters=cfg.topk_clusters, topk_blocks=cfg.topk_blocks,
                        labels_q=kq.labels, labels_k=kk.labels, blocks_to_eval=blocks,
                        retrieval_follow=retrieval_trace, hierarchical=hierarchy)
        assert r.retrieval_mismatches == 0, "retrieval selections differ beyond near-ties"
    else:
        r = muse_acausal(q, k, v, cfg.Cq, cfg.Ck, cfg.iters, dipole=dipole,
                         labels_q=kq.labels, labels_k=kk.labels, rows=rows)
    return r, kq, kk


def oracle_dipole(dipole) -> str:
    """The oracle's dipole mode for a binding dipole argument (True, False or a mode name)."""
    if isinstance(dipole, bool):
        return "tilted" if dipole else "none"
    return str(dipole)


def check_config(cfg: WorkloadConfig, heads: List[Tuple[int, int]], tol: Optional[float] = None,
                 blocks: Optional[Sequence[int]] = None, out_dtype=torch.float32, dipole=True,
                 rows: Optional[np.ndarray] = None, hierarchy: bool = False) -> List[HeadCheck]:
    """Run the whole [B,H,N,D] workload on the GPU and compare the listed heads."""
    t0 = time.time()
    q, k, v = make_inputs(cfg)
    out, ex = run_gpu(cfg, q, k, v, out_dtype=out_dtype, dipole=dipole, hierarchy=hierarchy)
    o_gpu = out.float().cpu().numpy()
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
                                retrieval_trace=None if rtr is None else rtr[b, h], hierarchy=hierarchy)
        assert np.array_equal(kq.labels, tq[-1, b, h]) and np.array_equal(kk.labels, tk[-1, b, h])
        sel = np.isfinite(r.o[:, 0])
        rel = rel_l2(o_gpu[b, h][sel], r.o[sel])
        lse_err = float(np.max(np.abs(lse[b, h][sel] - r.lse[sel])))
        log(f"[{cfg.name}] head ({b},{h}): rel-L2 {rel:.3e} (tol {tol:.0e}), max |dLSE| {lse_err:.2e}, "
            f"near-ties q={kq.near_ties} k={kk.near_ties} retrieval={r.retrieval_near_ties}, "
            f"rows checked {int(sel.sum())}")
        assert rel <= tol, f"rel-L2 {rel} > {tol}"
        assert lse_err <= (1e-4 if cfg.dtype == "f32" else 2e-3)
        res.append(HeadCheck(b, h, rel, kq.near_ties, kk.near_ties))
    return res
