"""Plain float64 CPU oracle of the MuSe backward pass (gradients of the forward output).

TEST INFRASTRUCTURE ONLY, like muse_ref.py: imported by the tests, never by the GPU
library; it shares no code with the HIP path.

What is differentiated. The reviews note that the paper's backward pass "uses the same
approximations" as its forward and that its error was never measured ([REVIEW] "Reading
between the lines"; "Referee Report", Section 7.2 / Q4). The reading taken here: the
gradient of the MuSe forward output o(q, k, v) of muse_ref.py with the K-means labels
held fixed (the clustering is piecewise constant in q and k, so it has no gradient);
the query centroids are the member means of the fixed labels and carry gradient to
every member. Given an upstream gradient dO = dLoss/do, the functions return
dq, dk, dv (vector-Jacobian products), written out stage by stage in reverse:

  stage 2  o_n = sum_j p_nj V_ij + s D_i qt_n,  p_n = softmax_j(l_n),
           l_nj = log Z_ij + s qt_n . K_ij,  qt_n = q_n - qbar_i
  stage 1  D_i = sum_j P_ij C_ij,  P_i = softmax_j(log Z_i.),
           per key cluster j: a_m = s qbar_i . k_m, w = softmax_m(a), log Z_ij = lse_m a_m,
           K_ij = sum w k, V_ij = sum w v, C_ij = sum w v k^T - V_ij K_ij^T
  centroid qbar_i = mean of the queries labelled i
  causal   o = exp(L_far - L) o_far + exp(L_loc - L) o_loc, L = logaddexp(L_far, L_loc)
           (or over the squares of the hierarchy), with the local part exact attention.

Pins (tests/test_oracle_bwd.py, CPU): central finite differences of muse_acausal and
muse_causal (tilted, untilted and no dipole; prefix and hierarchical causal forms; scale
1/sqrt(D) and 1); exact attention's backward against torch autograd of scaled dot-product
attention in float64; reductions: singleton clusters give exact attention's gradients;
with keys (queries) equal to their centroids so do the gradients of the other inputs, and
with degenerate queries also dq under the tilted dipole, not without it.
"""

from __future__ import annotations

from typing import List, Optional, Sequence, Tuple

import numpy as np

from .muse_ref import (NEG_INF, Summaries, _attend, _cluster, cap_key_labels, default_scale, hierarchy_squares,
                       lse_merge, refine, tilted_summaries)


# --------------------------------------------------------------------------------------
# exact softmax attention
# --------------------------------------------------------------------------------------

def attend_bwd(qrows, keys, vals, scale: float, allowed, dO, dL=None):
    """Backward of _attend: o = softmax_m(s q.k_m) v over allowed keys, L = lse.
    da = p * (dp - sum_m p dp) + p dL with dp = dO . v_m; dq = s da k, dk = s da^T q."""
    qrows = np.asarray(qrows, np.float64)
    keys = np.asarray(keys, np.float64)
    vals = np.asarray(vals, np.float64)
    a = scale * (qrows @ keys.T)
    if allowed is not None:
        a = np.where(allowed, a, NEG_INF)
    mx = a.max(axis=1, keepdims=True) if a.shape[1] else np.full((a.shape[0], 1), NEG_INF)
    mx_safe = np.where(np.isfinite(mx), mx, 0.0)
    e = np.where(np.isfinite(a), np.exp(a - mx_safe), 0.0)
    z = e.sum(axis=1, keepdims=True)
    p = np.divide(e, z, out=np.zeros_like(e), where=z > 0)
    dv = p.T @ dO
    dp = dO @ vals.T
    da = p * (dp - (p * dp).sum(axis=1, keepdims=True))
    if dL is not None:
        da += p * np.asarray(dL)[:, None]
    return scale * (da @ keys), scale * (da.T @ qrows), dv


def exact_attention_bwd(q, k, v, dO, scale: Optional[float] = None, causal: bool = False,
                        row_block: int = 512):
    """dq, dk, dv of exact softmax attention (o of muse_ref.exact_attention) for dO."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    dO = np.asarray(dO, np.float64)
    s = default_scale(q.shape[1]) if scale is None else scale
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    cols = np.arange(k.shape[0])
    for r0 in range(0, q.shape[0], row_block):
        r1 = min(q.shape[0], r0 + row_block)
        allowed = (cols[None, :] <= np.arange(r0, r1)[:, None]) if causal else None
        gq, gk, gv = attend_bwd(q[r0:r1], k, v, s, allowed, dO[r0:r1])
        dq[r0:r1] += gq
        dk += gk
        dv += gv
    return dq, dk, dv


# --------------------------------------------------------------------------------------
# log-sum-exp merge of partial results over disjoint key sets
# --------------------------------------------------------------------------------------

def lse_merge_bwd(parts: Sequence[Tuple[np.ndarray, np.ndarray]], dO, dL=None):
    """Backward of o = sum_s exp(L_s - L) o_s, L = logsumexp_s L_s. Returns per part
    (do_s, dL_s): do_s = alpha_s dO, dL_s = alpha_s (dO . (o_s - o) + dL)."""
    Ls = np.stack([L for _, L in parts])
    L = np.logaddexp.reduce(Ls, axis=0)
    alphas = [np.where(np.isfinite(Lp), np.exp(Lp - L), 0.0) for _, Lp in parts]
    o = sum(al[:, None] * op for al, (op, _) in zip(alphas, parts))
    out = []
    for al, (op, _) in zip(alphas, parts):
        dLs = al * ((dO * (op - o)).sum(axis=1) + (0.0 if dL is None else dL))
        out.append((al[:, None] * dO, dLs))
    return out


# --------------------------------------------------------------------------------------
# stage 2 and stage 1 backward
# --------------------------------------------------------------------------------------

class SummaryGrads:
    """Gradients with respect to the stage-1 summaries (shapes as Summaries)."""

    def __init__(self, Cq: int, Ck: int, D: int, Dv: int):
        self.logZ = np.zeros((Cq, Ck))
        self.K = np.zeros((Cq, Ck, D))
        self.V = np.zeros((Cq, Ck, Dv))
        self.Dip = np.zeros((Cq, Dv, D))


def refine_bwd(q, q_labels, qbar, S: Summaries, scale: float, dipole: bool, dO, dL=None,
               rows: Optional[np.ndarray] = None):
    """Backward of muse_ref.refine over the listed rows (all rows when None). Returns
    (dq of the rows through the residuals, dqbar, SummaryGrads)."""
    q = np.asarray(q, np.float64)
    q_labels = np.asarray(q_labels)
    N, D = q.shape
    Cq, Ck = S.logZ.shape
    Dv = S.V.shape[2]
    dq = np.zeros_like(q)
    dqbar = np.zeros((Cq, D))
    G = SummaryGrads(Cq, Ck, D, Dv)
    sel = np.arange(N) if rows is None else np.asarray(rows)
    for i in np.unique(q_labels[sel]):
        idx = sel[q_labels[sel] == i]
        qt = q[idx] - qbar[i]
        l = S.logZ[i][None, :] + scale * (qt @ S.K[i].T)
        mx = l.max(axis=1, keepdims=True)
        mx_safe = np.where(np.isfinite(mx), mx, 0.0)
        e = np.where(np.isfinite(l), np.exp(l - mx_safe), 0.0)
        z = e.sum(axis=1, keepdims=True)
        p = np.divide(e, z, out=np.zeros_like(e), where=z > 0)
        g = np.asarray(dO)[idx]
        G.V[i] += p.T @ g
        dp = g @ S.V[i].T
        dl = p * (dp - (p * dp).sum(axis=1, keepdims=True))
        if dL is not None:
            dl += p * np.asarray(dL)[idx][:, None]
        G.logZ[i] += dl.sum(axis=0)
        dqt = scale * (dl @ S.K[i])
        G.K[i] += scale * (dl.T @ qt)
        if dipole:
            dqt += scale * (g @ S.Dip[i])
            G.Dip[i] += scale * (g.T @ qt)
        dq[idx] += dqt
        dqbar[i] -= dqt.sum(axis=0)
    return dq, dqbar, G


def tilted_summaries_bwd(qbar, k, v, key_labels, Ck: int, scale: float, dipole: str, G: SummaryGrads):
    """Backward of muse_ref.tilted_summaries: (dqbar, dk, dv) for the summary gradients G."""
    qbar = np.asarray(qbar, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    key_labels = np.asarray(key_labels)
    S = tilted_summaries(qbar, k, v, key_labels, Ck, scale, dipole)
    Cq, D = qbar.shape
    dqbar = np.zeros_like(qbar)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    dlogZ = G.logZ.copy()
    members = [np.nonzero(key_labels == j)[0] for j in range(Ck)]
    finite = np.isfinite(S.logZ)
    mx = S.logZ.max(axis=1, keepdims=True)
    P = np.where(finite, np.exp(S.logZ - mx), 0.0)
    P /= P.sum(axis=1, keepdims=True)
    # per-cluster covariances C_ij (as the forward forms them) and their gradients
    Cmat = {}
    if dipole != "none":
        dP = np.zeros_like(P)
        for j, idx in enumerate(members):
            if idx.size == 0:
                continue
            if dipole == "tilted":
                a = scale * (qbar @ k[idx].T)
                w = np.exp(a - S.logZ[:, j][:, None])
                vc = v[idx][None] - S.V[:, j][:, None, :]
                kc = k[idx][None] - S.K[:, j][:, None, :]
                Cij = np.matmul((vc * w[:, :, None]).transpose(0, 2, 1), kc)
            else:
                vc = v[idx] - v[idx].mean(axis=0)
                kc = k[idx] - k[idx].mean(axis=0)
                Cij = np.broadcast_to((vc.T @ kc) / idx.size, (Cq,) + (v.shape[1], D))
            Cmat[j] = Cij
            dP[:, j] = (G.Dip * Cij).sum(axis=(1, 2))
        # D_i = sum_j P_ij C_ij: softmax backward into log Z
        dlogZ += np.where(finite, P * (dP - (P * dP).sum(axis=1, keepdims=True)), 0.0)
    for j, idx in enumerate(members):
        if idx.size == 0:
            continue
        kj, vj = k[idx], v[idx]
        a = scale * (qbar @ kj.T)                          # [Cq, n]
        w = np.exp(a - S.logZ[:, j][:, None])              # tilted weights
        dK = G.K[:, j].copy()                              # [Cq, D]
        dV = G.V[:, j].copy()                              # [Cq, Dv]
        dw = np.zeros_like(w)
        if dipole == "tilted":
            dC = P[:, j, None, None] * G.Dip               # [Cq, Dv, D]
            # C = M - V K^T with M = sum_m w_m v_m k_m^T
            dV -= np.einsum("ivd,id->iv", dC, S.K[:, j])
            dK -= np.einsum("ivd,iv->id", dC, S.V[:, j])
            dw += np.einsum("mv,ivd,md->im", vj, dC, kj)
            dk[idx] += np.einsum("im,ivd,mv->md", w, dC, vj)
            dv[idx] += np.einsum("im,ivd,md->mv", w, dC, kj)
        elif dipole == "untilted":
            dCov = (P[:, j, None, None] * G.Dip).sum(axis=0)   # [Dv, D]
            n = idx.size
            dv[idx] += ((kj - kj.mean(axis=0)) @ dCov.T) / n
            dk[idx] += ((vj - vj.mean(axis=0)) @ dCov) / n
        # K = sum w k, V = sum w v
        dw += dK @ kj.T + dV @ vj.T
        dk[idx] += w.T @ dK
        dv[idx] += w.T @ dV
        # softmax over the cluster's keys, and log Z = lse(a)
        da = w * (dw - (w * dw).sum(axis=1, keepdims=True)) + w * dlogZ[:, j][:, None]
        dqbar += scale * (da @ kj)
        dk[idx] += scale * (da.T @ qbar)
    return dqbar, dk, dv


def _centroid_bwd(dq, dqbar, labels, Cq: int):
    """qbar_i = mean of the queries labelled i: each member gets dqbar_i / n_i."""
    labels = np.asarray(labels)
    for i in range(Cq):
        m = labels == i
        if m.any():
            dq[m] += dqbar[i] / m.sum()
    return dq


# --------------------------------------------------------------------------------------
# whole backward passes
# --------------------------------------------------------------------------------------

def muse_acausal_bwd(q, k, v, Cq: int, Ck: int, labels_q, labels_k, dO, scale: Optional[float] = None,
                     dipole: str = "tilted", cap_ratio: Optional[float] = None):
    """dq, dk, dv of muse_ref.muse_acausal's output with the labels fixed. cap_ratio: key
    clusters capped as in the forward (cap_key_labels): the keys left out of the summaries
    get no gradient through them."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    s = default_scale(q.shape[1]) if scale is None else scale
    _, lq, qbar = _cluster(q, Cq, 1, labels_q, None, 0.0)
    _, lk, _ = _cluster(k, Ck, 1, labels_k, None, 0.0)
    lk = cap_key_labels(lk, Ck, cap_ratio)
    S = tilted_summaries(qbar, k, v, lk, Ck, s, dipole)
    dq, dqbar, G = refine_bwd(q, lq, qbar, S, s, dipole != "none", dO)
    gqbar, dk, dv = tilted_summaries_bwd(qbar, k, v, lk, Ck, s, dipole, G)
    return _centroid_bwd(dq, dqbar + gqbar, lq, Cq), dk, dv


def muse_causal_bwd(q, k, v, Cq: int, Ck: int, block: int, labels_q, labels_k, dO,
                    scale: Optional[float] = None, dipole: str = "tilted", hierarchical: bool = False,
                    cap_ratio: Optional[float] = None):
    """dq, dk, dv of muse_ref.muse_causal's output (no retrieval) with the labels fixed:
    per block, the log-sum-exp merge of the exact local part and the far part (one
    two-stage approximation over all earlier keys, or one per square of the hierarchy).
    cap_ratio: key clusters capped over the whole sequence as in the forward; a key left
    out of the summaries still takes part in its own block's exact attention."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    dO = np.asarray(dO, np.float64)
    N, D = q.shape
    s = default_scale(D) if scale is None else scale
    nb = N // block
    _, lq, qbar = _cluster(q, Cq, 1, labels_q, None, 0.0)
    _, lk, _ = _cluster(k, Ck, 1, labels_k, None, 0.0)
    lk = cap_key_labels(lk, Ck, cap_ratio)   # labels seen by the summaries
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    dqbar = np.zeros_like(qbar)
    squares = hierarchy_squares(nb) if hierarchical else [(b, b + 1, 0, b) for b in range(1, nb)]
    for b in range(nb):
        r0, r1 = b * block, (b + 1) * block
        rows = np.arange(r0, r1)
        allowed = rows[None, :] <= rows[:, None]
        parts = [_attend(q[r0:r1], k[r0:r1], v[r0:r1], s, allowed)]
        far = []  # (key range, summaries) of every far-field piece of this block
        for q0, q1, k0, k1 in squares:
            if q0 <= b < q1:
                ks = slice(k0 * block, k1 * block)
                S = tilted_summaries(qbar, k[ks], v[ks], lk[ks], Ck, s, dipole)
                parts.append(refine(q[r0:r1], lq[r0:r1], qbar, S, s, dipole != "none"))
                far.append((ks, S))
        grads = lse_merge_bwd(parts, dO[r0:r1])
        gq, gk, gv = attend_bwd(q[r0:r1], k[r0:r1], v[r0:r1], s, allowed, grads[0][0], grads[0][1])
        dq[r0:r1] += gq
        dk[r0:r1] += gk
        dv[r0:r1] += gv
        for (ks, S), (do_p, dL_p) in zip(far, grads[1:]):
            gq, gqbar, G = refine_bwd(q[r0:r1], lq[r0:r1], qbar, S, s, dipole != "none", do_p, dL_p)
            dq[r0:r1] += gq
            dqbar += gqbar
            gqbar, gk, gv = tilted_summaries_bwd(qbar, k[ks], v[ks], lk[ks], Ck, s, dipole, G)
            dqbar += gqbar
            dk[ks] += gk
            dv[ks] += gv
    return _centroid_bwd(dq, dqbar, lq, Cq), dk, dv
