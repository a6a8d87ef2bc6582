"""Plain, slow, float64 CPU oracle of the Multipole Semantic Attention (MuSe) forward pass.

TEST INFRASTRUCTURE ONLY. Imported by the tests, the smoke check and the bench's
CPU-baseline leg; never by the GPU library. It shares no code with the HIP path.

Sources. The method is known only from secondary pages about arXiv 2509.10406
(R. Mitchell, K. Kersting, "Multipole Semantic Attention: A Fast Approximation of
Softmax Attention for Pretraining"):
  [REVIEW]  pith.science review page of the paper: "What carries the argument",
            "Core claim", "Circularity Check", "Assumptions & free parameters",
            "Referee Report" (minor comment on Algorithm 3), caption of Figure 2.
  [RECORD] pith.science verdict record of the paper, field "key_machinery".
  [GIST]    gist.science technical summary (Dutch), "Methodologie",
            "Kernmechanismen" items 1 to 4.
  [ABS2]    fugumt.com listing of the v2 abstract.
The paper's own equations are not reproduced on any page; the formulas below
are the cumulant-expansion reading spelled out in each docstring. Readings of
points the pages leave open are tagged [R1]..[R15]; each is stated where it is used.

Pins (tests/test_oracle_*.py, CPU only):
  exact_attention      pinned: hand-worked closed form; torch SDPA (fp64, CPU).
  lloyd_kmeans         pinned: hand-worked 1-D example; known partition of
                       well-separated data; Lloyd monotonicity; centroid = mean.
  tilted_summaries     pinned: finite differences of the exact per-cluster
                       log-normaliser and tilted value mean; singleton and
                       degenerate clusters reduce to exact attention.
  refine               pinned: singleton / centroid-equal cases -> exact attention;
                       epsilon-order of the error (first-order exactness of the
                       tilted dipole); key-translation invariance; linearity in V.
  muse_acausal         pinned through the above.
  muse_causal          pinned: block = N and singleton clusters -> exact causal;
                       causality in V; retrieval of everything -> exact causal;
                       hierarchical: squares tile the strictly lower block triangle
                       once, two blocks = the prefix form, singleton and degenerate
                       clusters -> exact causal, causality in V.
  retrieval_selection  pinned: planted high-score atoms are selected; brute-force
                       ranking on tiny inputs.
  bucket_order         pinned: hand-worked example (ties kept in position order,
                       empty buckets, causal blocks); permutation and offset invariants.
  cap_key_labels       pinned: hand-worked cap sizes and kept members; a cap above every
                       cluster size changes nothing; capped MuSe equals MuSe on the inputs
                       with the dropped keys removed (acausal), exact in-block attention
                       keeps them (causal).
"""

from __future__ import annotations

import dataclasses
from typing import List, Optional, Sequence, Tuple

import numpy as np

NEG_INF = -np.inf


def default_scale(D: int) -> float:
    """Softmax temperature s = 1/sqrt(D) [R1]: MuSe is a drop-in replacement for standard
    attention ([ABS2]), whose logits are scaled this way."""
    return 1.0 / np.sqrt(D)


# --------------------------------------------------------------------------------------
# exact softmax attention (the quantity MuSe approximates; [GIST] "Probleemstelling")
# --------------------------------------------------------------------------------------

def _attend(qrows: np.ndarray, keys: np.ndarray, vals: np.ndarray, scale: float,
            allowed: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray]:
    """o_n = sum_m softmax_m(s q_n.k_m) v_m over allowed keys; L_n = logsumexp_m s q_n.k_m.

    A row with no allowed key gets o = 0 and L = -inf (it contributes nothing to a
    log-sum-exp merge)."""
    a = scale * (qrows @ keys.T)
    if allowed is not None:
        a = np.where(allowed, a, NEG_INF)
    mx = a.max(axis=1, keepdims=True) if a.shape[1] else np.full((a.shape[0], 1), NEG_INF)
    empty = ~np.isfinite(mx[:, 0])
    mx_safe = np.where(np.isfinite(mx), mx, 0.0)
    e = np.exp(a - mx_safe)
    z = e.sum(axis=1)
    o = np.zeros((qrows.shape[0], vals.shape[1]))
    L = np.full(qrows.shape[0], NEG_INF)
    ok = ~empty
    o[ok] = (e[ok] @ vals) / z[ok, None]
    L[ok] = mx_safe[ok, 0] + np.log(z[ok])
    return o, L


def exact_attention(q, k, v, scale: Optional[float] = None, causal: bool = False,
                    row_block: int = 512) -> Tuple[np.ndarray, np.ndarray]:
    """Exact softmax attention of one head (q [N,D], k [M,D], v [M,Dv]) in float64.

    causal: query n sees keys m <= n. Tiled over query rows only to bound memory.
    Returns (o [N,Dv], L [N]) with L the log of the softmax normaliser."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    s = default_scale(q.shape[1]) if scale is None else scale
    N = q.shape[0]
    o = np.empty((N, v.shape[1]))
    L = np.empty(N)
    cols = np.arange(k.shape[0])
    for r0 in range(0, N, row_block):
        r1 = min(N, r0 + row_block)
        allowed = (cols[None, :] <= np.arange(r0, r1)[:, None]) if causal else None
        o[r0:r1], L[r0:r1] = _attend(q[r0:r1], k, v, s, allowed)
    return o, L


def lse_merge(o1, L1, o2, L2) -> Tuple[np.ndarray, np.ndarray]:
    """Combine two softmax partial results over disjoint key sets.

    L = log(e^L1 + e^L2); o = e^(L1-L) o1 + e^(L2-L) o2. Either side may be empty
    (L = -inf); at least one side is non-empty for every row."""
    L = np.logaddexp(L1, L2)
    w1 = np.where(np.isfinite(L1), np.exp(L1 - L), 0.0)
    w2 = np.where(np.isfinite(L2), np.exp(L2 - L), 0.0)
    return w1[:, None] * o1 + w2[:, None] * o2, L


# --------------------------------------------------------------------------------------
# K-means: queries and keys are clustered separately, each in its own space
# ([GIST] Kernmechanismen 1; [REVIEW] "Core claim"; [REVIEW] free parameter
# "K-means iterations")
# --------------------------------------------------------------------------------------

@dataclasses.dataclass
class KMeansResult:
    labels: np.ndarray          # [n] int64, labels of the last assignment step
    centroids: np.ndarray       # [C, D] float64, member means after the last update
    trace: List[np.ndarray]     # per-iteration labels
    near_ties: int = 0          # follow mode: labels adopted from the compared run
    mismatches: int = 0         # follow mode: differing labels that were NOT near-ties
    mismatch_info: list = dataclasses.field(default_factory=list)


def squared_distances(x: np.ndarray, c: np.ndarray, chunk: int = 1024) -> np.ndarray:
    """d[n, j] = sum_d (x[n,d] - c[j,d])^2, written out directly (no expansion)."""
    out = np.empty((x.shape[0], c.shape[0]))
    for r0 in range(0, x.shape[0], chunk):
        diff = x[r0:r0 + chunk, None, :] - c[None, :, :]
        out[r0:r0 + chunk] = np.einsum("ncd,ncd->nc", diff, diff)
    return out


def lloyd_kmeans(x, C: int, iters: int, follow_trace: Optional[Sequence[np.ndarray]] = None,
                 tie_rel: float = 1e-5) -> KMeansResult:
    """Fixed-iteration Lloyd K-means with Euclidean distance [R2].

    init: c_j = x[floor(j*n/C)] for j = 0..C-1 (strided, deterministic).
    repeat ``iters`` times:
        assign: label_n = argmin_j ||x_n - c_j||^2, exact ties to the lowest j;
        update: c_j = mean of its members; a cluster with no member keeps c_j.
    The result pairs the last assignment's labels with the centroids updated from
    them (so every non-empty centroid is the mean of its members).

    follow_trace: optional per-iteration labels from another implementation. Where
    its label g differs from the argmin o, the point counts as a near-tie when
    d_g - d_o <= tie_rel * d_g; then g is adopted so that both runs continue from the
    same partition. Other differences are counted as mismatches (o is kept)."""
    x = np.asarray(x, np.float64)
    n = x.shape[0]
    c = x[(np.arange(C) * n) // C].copy()
    trace: List[np.ndarray] = []
    res = KMeansResult(np.zeros(n, np.int64), c, trace)
    labels = np.zeros(n, np.int64)
    for t in range(iters):
        d = squared_distances(x, c)
        labels = np.argmin(d, axis=1)  # first minimum = lowest index on exact ties
        if follow_trace is not None:
            g = np.asarray(follow_trace[t]).astype(np.int64)
            diff = np.nonzero(g != labels)[0]
            if diff.size:
                dg = d[diff, g[diff]]
                do = d[diff, labels[diff]]
                near = (dg - do) <= tie_rel * dg
                res.near_ties += int(near.sum())
                res.mismatches += int((~near).sum())
                for p in diff[~near][:8]:
                    res.mismatch_info.append((t, int(p), int(labels[p]), int(g[p]),
                                              float(d[p, labels[p]]), float(d[p, g[p]])))
                labels = labels.copy()
                labels[diff[near]] = g[diff[near]]
        trace.append(labels.copy())
        for j in range(C):
            members = labels == j
            if members.any():
                c[j] = x[members].mean(axis=0)
    res.labels = labels
    res.centroids = c
    return res


def bucket_order(labels, C: int, block: int = 0) -> Tuple[np.ndarray, np.ndarray]:
    """Positions of one head grouped by (spatial block, cluster): the stable sort of
    the positions by the key block * C + label, and the start of every bucket.

    The paper gathers each cluster's members into a ragged tensor padded per cluster
    ([REVIEW] "Assumptions & free parameters": cluster size cap, "caps the ragged-tensor
    block size"); this replaces it by the members listed bucket after bucket (block b,
    cluster j) with positions ascending inside a bucket. block = 0: one block (acausal).
    Returns perm [n] and offs [nb * C + 1] with perm[offs[b*C+j]:offs[b*C+j+1]] the
    positions of bucket (b, j) and offs[-1] = n."""
    labels = np.asarray(labels).astype(np.int64)
    n = labels.shape[0]
    blk = np.zeros(n, np.int64) if block <= 0 else np.arange(n) // block
    nb = 1 if block <= 0 else n // block
    key = blk * C + labels
    perm = np.argsort(key, kind="stable")
    counts = np.bincount(key, minlength=nb * C)
    offs = np.concatenate([[0], np.cumsum(counts)])
    return perm, offs


# --------------------------------------------------------------------------------------
# Stage 1: coarse query centroids attend to fine key clusters
# ([REVIEW] "What carries the argument", "Core claim"; [RECORD] key_machinery;
#  [GIST] Kernmechanismen 2, "Fase 1" and "Exponential Tilting")
# --------------------------------------------------------------------------------------

@dataclasses.dataclass
class Summaries:
    logZ: np.ndarray   # [Cq, Ck]  log sum_{m in S_j} exp(s qbar_i . k_m); -inf for empty j
    K: np.ndarray      # [Cq, Ck, D]  tilted key mean K_ij
    V: np.ndarray      # [Cq, Ck, Dv] tilted value mean V_ij
    Dip: np.ndarray    # [Cq, Dv, D]  aggregated dipole D_i = sum_j P_ij C_ij


def tilted_summaries(qbar, k, v, key_labels, Ck: int, scale: float,
                     dipole: str = "tilted") -> Summaries:
    """Per (query cluster i, key cluster j) monopole summaries and per-i dipole.

    Treat key cluster j (members S_j) as a distribution tilted by the query
    centroid qbar_i:  a_m = s qbar_i.k_m,  w_m = exp(a_m) / Z_ij.
        log Z_ij = logsumexp_{m in S_j} a_m           (log-normaliser)
        K_ij     = sum_m w_m k_m                       (tilted key mean: monopole [R4])
        V_ij     = sum_m w_m v_m                       (tilted value mean: monopole)
        C_ij     = sum_m w_m (v_m - V_ij)(k_m - K_ij)^T  (tilted value-key covariance,
                                                        value index first: dipole [R6])
    The dipole is aggregated per query cluster with the stage-1 cluster weights
    P_ij = softmax_j(log Z_ij):  D_i = sum_j P_ij C_ij  [R5].
    An empty key cluster has log Z = -inf and drops out [R7].

    dipole: "tilted" (the above), "none" (D_i = 0), or "untilted": C_ij replaced by
    the plain within-cluster covariance of cluster j (the paper's partially
    specialised dipole, [REVIEW] referee minor comment on Algorithm 3)."""
    qbar = np.asarray(qbar, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    key_labels = np.asarray(key_labels)
    Cq, D = qbar.shape
    Dv = v.shape[1]
    logZ = np.full((Cq, Ck), NEG_INF)
    Kt = np.zeros((Cq, Ck, D))
    Vt = np.zeros((Cq, Ck, Dv))
    members = [np.nonzero(key_labels == j)[0] for j in range(Ck)]
    weights = [None] * Ck
    for j, idx in enumerate(members):
        if idx.size == 0:
            continue
        a = scale * (qbar @ k[idx].T)            # [Cq, n_j]
        mx = a.max(axis=1, keepdims=True)
        e = np.exp(a - mx)
        z = e.sum(axis=1)
        logZ[:, j] = mx[:, 0] + np.log(z)
        w = e / z[:, None]
        weights[j] = w
        Kt[:, j] = w @ k[idx]
        Vt[:, j] = w @ v[idx]
    # stage-1 cluster weights P_ij = softmax over j of log Z_ij
    mx = logZ.max(axis=1, keepdims=True)
    P = np.where(np.isfinite(logZ), np.exp(logZ - mx), 0.0)
    P /= P.sum(axis=1, keepdims=True)
    Dip = np.zeros((Cq, Dv, D))
    if dipole == "none":
        return Summaries(logZ, Kt, Vt, Dip)
    for j, idx in enumerate(members):
        if idx.size == 0:
            continue
        if dipole == "tilted":
            vc = v[idx][None, :, :] - Vt[:, j][:, None, :]        # [Cq, n_j, Dv]
            kc = k[idx][None, :, :] - Kt[:, j][:, None, :]        # [Cq, n_j, D]
            Cij = np.matmul((vc * weights[j][:, :, None]).transpose(0, 2, 1), kc)  # [Cq, Dv, D]
        elif dipole == "untilted":
            vc = v[idx] - v[idx].mean(axis=0)
            kc = k[idx] - k[idx].mean(axis=0)
            Cij = np.broadcast_to((vc.T @ kc) / idx.size, (Cq, Dv, D))
        else:
            raise ValueError(f"unknown dipole mode {dipole!r}")
        Dip += P[:, j, None, None] * Cij
    return Summaries(logZ, Kt, Vt, Dip)


# --------------------------------------------------------------------------------------
# Stage 2: each query refines its cluster's summaries with its residual
# ([GIST] Kernmechanismen 1 "Decompositie" and 2 "Fase 2"; [REVIEW] "What carries
#  the argument": three of the four terms of exp((qbar+qt).(kbar+kt)) are kept)
# --------------------------------------------------------------------------------------

def refine(q, q_labels, qbar, S: Summaries, scale: float, dipole: bool = True,
           rows: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Per query n in cluster i with residual qt = q_n - qbar_i:
        l_j = log Z_ij + s qt.K_ij           (first cumulant: log mass of cluster j seen by q_n)
        p   = softmax_j(l)
        o_n = sum_j p_j V_ij + s D_i qt      (monopole + dipole)
        L_n = logsumexp_j l_j
    rows: optional subset of query indices (others are returned as NaN)."""
    q = np.asarray(q, np.float64)
    q_labels = np.asarray(q_labels)
    N = q.shape[0]
    Dv = S.V.shape[2]
    o = np.full((N, Dv), np.nan)
    L = np.full(N, np.nan)
    sel = np.arange(N) if rows is None else np.asarray(rows)
    for i in np.unique(q_labels[sel]):
        idx = sel[q_labels[sel] == i]
        qt = q[idx] - qbar[i]                                   # [n_i, D]
        l = S.logZ[i][None, :] + scale * (qt @ S.K[i].T)          # [n_i, Ck]
        mx = l.max(axis=1, keepdims=True)
        finite = np.isfinite(mx[:, 0])
        mx_safe = np.where(np.isfinite(mx), mx, 0.0)
        e = np.where(np.isfinite(l), np.exp(l - mx_safe), 0.0)
        z = e.sum(axis=1)
        oi = np.zeros((idx.size, Dv))
        Li = np.full(idx.size, NEG_INF)
        oi[finite] = (e[finite] @ S.V[i]) / z[finite, None]
        Li[finite] = mx_safe[finite, 0] + np.log(z[finite])
        if dipole:
            oi[finite] += scale * (qt[finite] @ S.Dip[i].T)
        o[idx] = oi
        L[idx] = Li
    return o, L


# --------------------------------------------------------------------------------------
# Whole forward passes
# --------------------------------------------------------------------------------------

@dataclasses.dataclass
class MuseResult:
    o: np.ndarray
    lse: np.ndarray
    km_q: Optional[KMeansResult]
    km_k: Optional[KMeansResult]
    labels_q: np.ndarray
    labels_k: np.ndarray
    qbar: np.ndarray
    retrieval_near_ties: int = 0
    retrieval_mismatches: int = 0


def _cluster(x, C, iters, labels_in, follow, tie_rel):
    """Labels and centroids: K-means, or caller-fixed labels with member-mean centroids."""
    x = np.asarray(x, np.float64)
    if labels_in is not None:
        labels = np.asarray(labels_in).astype(np.int64)
        c = np.zeros((C, x.shape[1]))
        for j in range(C):
            m = labels == j
            if m.any():
                c[j] = x[m].mean(axis=0)
        return None, labels, c
    km = lloyd_kmeans(x, C, iters, follow, tie_rel)
    return km, km.labels, km.centroids


def cap_key_labels(labels, Ck: int, cap_ratio: Optional[float]) -> np.ndarray:
    """Key clusters capped at U = ceil(cap_ratio * n / Ck) members [R16].

    The paper pads each cluster's members into a ragged tensor whose row length is the
    cap ([REVIEW] "Assumptions & free parameters": cluster size cap ratio 1.5, 1.25 to 4.0
    explored, "caps the ragged-tensor block size"). Reading: the members of key cluster j,
    taken in position order, fill its row; those beyond the first U do not fit and take no
    part in the stage-1 summaries of their cluster (log-normaliser, tilted means, dipole).
    Returns the labels with every dropped key set to -1 (a label no cluster has);
    cap_ratio None means no cap."""
    labels = np.asarray(labels).astype(np.int64).copy()
    if cap_ratio is None:
        return labels
    n = labels.shape[0]
    U = int(np.ceil(cap_ratio * n / Ck))
    for j in range(Ck):
        members = np.nonzero(labels == j)[0]     # ascending positions
        labels[members[U:]] = -1
    return labels


def muse_acausal(q, k, v, Cq: int, Ck: int, iters: int, scale: Optional[float] = None,
                 dipole: str = "tilted", labels_q=None, labels_k=None,
                 follow_q=None, follow_k=None, tie_rel: float = 1e-5,
                 rows: Optional[np.ndarray] = None, cap_ratio: Optional[float] = None) -> MuseResult:
    """Acausal MuSe forward of one head: K-means on Q (Cq) and on K (Ck), stage 1
    summaries, stage 2 refinement. Two-stage scheme per [REVIEW] "Core claim".
    cap_ratio: key clusters capped in stage 1 (cap_key_labels)."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    s = default_scale(q.shape[1]) if scale is None else scale
    km_q, lq, qbar = _cluster(q, Cq, iters, labels_q, follow_q, tie_rel)
    km_k, lk, _ = _cluster(k, Ck, iters, labels_k, follow_k, tie_rel)
    S = tilted_summaries(qbar, k, v, cap_key_labels(lk, Ck, cap_ratio), Ck, s, dipole)
    o, L = refine(q, lq, qbar, S, s, dipole != "none", rows)
    return MuseResult(o, L, km_q, km_k, lq, lk, qbar)


def _atom_log_masses(a_prefix, labels_prefix, blocks_prefix, Ck, nblocks):
    """sigma(j,b') = logsumexp of a over keys of cluster j in block b' (-inf if none)."""
    sig = np.full((Ck, nblocks), NEG_INF)
    for j in range(Ck):
        for bb in range(nblocks):
            m = (labels_prefix == j) & (blocks_prefix == bb)
            if m.any():
                am = a_prefix[m]
                mx = am.max()
                sig[j, bb] = mx + np.log(np.exp(am - mx).sum())
    return sig


def _lse_rows(x):
    with np.errstate(invalid="ignore", divide="ignore"):
        mx = x.max(axis=1, keepdims=True)
        mx_safe = np.where(np.isfinite(mx), mx, 0.0)
        return np.where(np.isfinite(mx[:, 0]),
                        mx_safe[:, 0] + np.log(np.where(np.isfinite(x), np.exp(x - mx_safe), 0.0).sum(axis=1)),
                        NEG_INF)


def _top(values: np.ndarray, k: int) -> list:
    """Indices of the k largest finite values, descending, ties to the lower index."""
    order = np.argsort(-values, kind="stable")
    return [int(x) for x in order[:k] if np.isfinite(values[x])]


def _valid_top(values: np.ndarray, chosen: list, k: int, tol: float) -> bool:
    """Is `chosen` a top-k of `values` once gaps up to `tol` count as ties?"""
    fin = [int(x) for x in np.nonzero(np.isfinite(values))[0]]
    if len(chosen) != min(k, len(fin)) or len(set(chosen)) != len(chosen):
        return False
    if any(not np.isfinite(values[x]) for x in chosen):
        return False
    rest = [x for x in fin if x not in chosen]
    return not rest or min(values[x] for x in chosen) >= max(values[x] for x in rest) - tol


def retrieval_selection(a_prefix: np.ndarray, labels_prefix: np.ndarray,
                        blocks_prefix: np.ndarray, Ck: int, nblocks: int,
                        k1: int, k2: int, follow=None, tol: float = 1e-4):
    """Retrieved keys for one (query cluster, block) [R9]; [GIST] Kernmechanismen 4.

    a_prefix: s qbar_i . k_m for the prefix keys; labels/blocks: their key cluster and
    spatial block. Atom log-mass sigma(j,b') = logsumexp of a over keys of cluster j in
    block b'; cluster score sigma(j) = logsumexp_b' sigma(j,b').
      1. J = the k1 clusters of largest sigma(j)   (cluster selection),
      2. for j in J, the k2 blocks of largest sigma(j,b')  (spatial block selection).
    Descending order, ties to the lower index, empty (-inf) candidates never chosen,
    fewer candidates than k -> all of them. Returns a boolean mask over prefix keys.

    follow: optional selection of another implementation, a list of (j, [b', ...]). It is
    adopted when it is a valid top-k at both levels once score gaps up to `tol` (natural
    log units) count as ties; then the return value is (mask, 1 if it differed else 0, 0),
    otherwise (own mask, 0, 1). Without follow only the mask is returned."""
    sig = _atom_log_masses(a_prefix, labels_prefix, blocks_prefix, Ck, nblocks)
    sj = _lse_rows(sig)
    J = _top(sj, k1)
    sel = [(j, _top(sig[j], k2)) for j in J]

    def mask_of(selection):
        take = np.zeros(a_prefix.shape[0], bool)
        for j, bl in selection:
            for bb in bl:
                take |= (labels_prefix == j) & (blocks_prefix == bb)
        return take

    if follow is None:
        return mask_of(sel)
    fj = [j for j, _ in follow]
    same = sorted(fj) == sorted(J) and all(sorted(bl) == sorted(dict(sel)[j]) for j, bl in follow)
    if same:
        return mask_of(sel), 0, 0
    ok = _valid_top(sj, fj, k1, tol) and all(_valid_top(sig[j], list(bl), k2, tol) for j, bl in follow)
    if ok:
        return mask_of(follow), 1, 0
    return mask_of(sel), 0, 1


def hierarchy_squares(nb: int) -> List[Tuple[int, int, int, int]]:
    """Below-diagonal squares of the hierarchical causal decomposition [R15], in block units.

    The pages draw the causal attention matrix cut into exact diagonal blocks and
    below-diagonal squares handled by MuSe, with one square per level and position so
    that the cost grows as N C D log N ([REVIEW] Figure 2 caption; "free parameters":
    causal block size of the hierarchical decomposition; "invented entities":
    hierarchical block decomposition). Reading: the grid of nb x nb blocks is padded to
    the next power of two P and split recursively; a diagonal square of side w > 1
    splits into two diagonal halves and the square below the diagonal (queries of the
    lower half, keys of the upper half), which MuSe covers. Squares are clipped to the
    nb real query blocks and dropped when empty. Returns (q0, q1, k0, k1): query blocks
    [q0, q1) attend to key blocks [k0, k1) through one two-stage approximation."""
    P = 1
    while P < nb:
        P *= 2
    out: List[Tuple[int, int, int, int]] = []

    def split(lo: int, w: int):
        if w <= 1:
            return
        h = w // 2
        q0, q1 = lo + h, min(lo + w, nb)
        if q0 < q1:
            out.append((q0, q1, lo, lo + h))
        split(lo, h)
        split(lo + h, h)

    split(0, P)
    return out


def muse_causal(q, k, v, Cq: int, Ck: int, iters: int, block: int,
                scale: Optional[float] = None, dipole: str = "tilted",
                topk_clusters: int = 0, topk_blocks: int = 0,
                labels_q=None, labels_k=None, follow_q=None, follow_k=None,
                tie_rel: float = 1e-5, blocks_to_eval: Optional[Sequence[int]] = None,
                retrieval_follow: Optional[np.ndarray] = None,
                hierarchical: bool = False, cap_ratio: Optional[float] = None) -> MuseResult:
    """Causal MuSe forward of one head [R8].

    Clusters are fitted once per head over the whole sequence. For a query n in
    spatial block b (blocks of ``block`` tokens):
      * local: exact softmax over keys m in [b*block, n]  ([REVIEW] Figure 2: exact
        attention on the diagonal blocks);
      * far (b >= 1): stage 1 and stage 2 over the keys of all preceding blocks,
        m < b*block, with the global clusters  ([GIST] Kernmechanismen 3: a block sees
        the summaries of all preceding blocks). Computed directly from those keys.
      * o_n = log-sum-exp merge of the two partial results.
    With retrieval (topk_clusters = k1 > 0, [GIST] Kernmechanismen 4): for each
    (query cluster i, block b) the keys R of the selected (cluster, block) atoms join
    the local block in the exact part, and the far summaries cover the remaining
    prefix keys only.

    blocks_to_eval: optional list of blocks whose rows are computed (others NaN).
    retrieval_follow: optional [nblocks, Cq, k1, 1 + k2] selections of another
    implementation (cluster id then block ids per chosen cluster, -1 padded), adopted
    where they are valid up to near-ties (see retrieval_selection); the counts are
    returned in MuseResult.retrieval_near_ties / retrieval_mismatches.

    hierarchical: the far field of a block is not one summary of all earlier keys but
    the log-sum-exp merge of one two-stage approximation per square of the hierarchy
    (hierarchy_squares, [R15]), each over its own key range with the global clusters.
    Retrieval is not combined with it.

    cap_ratio: key clusters capped (cap_key_labels, over the whole sequence: a cluster
    keeps its earliest U members); the dropped keys leave the far-field summaries and are
    still attended exactly inside their own block. Not combined with retrieval."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    N, D = q.shape
    s = default_scale(D) if scale is None else scale
    if N % block:
        raise ValueError("N must be a multiple of block")
    nb = N // block
    km_q, lq, qbar = _cluster(q, Cq, iters, labels_q, follow_q, tie_rel)
    km_k, lk, _ = _cluster(k, Ck, iters, labels_k, follow_k, tie_rel)
    if cap_ratio is not None and topk_clusters > 0:
        raise ValueError("the cluster cap is not combined with retrieval")
    lk_s = cap_key_labels(lk, Ck, cap_ratio)   # labels seen by the stage-1 summaries
    o = np.full((N, v.shape[1]), np.nan)
    L = np.full(N, np.nan)
    key_block = np.arange(N) // block
    near = mism = 0
    todo = range(nb) if blocks_to_eval is None else blocks_to_eval
    if hierarchical:
        if topk_clusters > 0:
            raise ValueError("retrieval is not combined with the hierarchy")
        want = set(int(b) for b in todo)
        far = {b: (np.zeros((block, v.shape[1])), np.full(block, NEG_INF)) for b in want}
        for q0, q1, k0, k1 in hierarchy_squares(nb):
            hit = [b for b in range(q0, q1) if b in want]
            if not hit:
                continue
            ks = slice(k0 * block, k1 * block)
            S = tilted_summaries(qbar, k[ks], v[ks], lk_s[ks], Ck, s, dipole)
            for b in hit:
                rs = slice(b * block, (b + 1) * block)
                o_s, L_s = refine(q[rs], lq[rs], qbar, S, s, dipole != "none")
                far[b] = lse_merge(far[b][0], far[b][1], o_s, L_s)
        for b in want:
            r0, r1 = b * block, (b + 1) * block
            rows = np.arange(r0, r1)
            o_loc, L_loc = _attend(q[r0:r1], k[r0:r1], v[r0:r1], s, rows[None, :] <= rows[:, None])
            o[r0:r1], L[r0:r1] = lse_merge(far[b][0], far[b][1], o_loc, L_loc)
        return MuseResult(o, L, km_q, km_k, lq, lk, qbar)
    for b in todo:
        r0, r1 = b * block, (b + 1) * block
        rows = np.arange(r0, r1)
        loc_allowed = (np.arange(r0, r1)[None, :] <= rows[:, None])
        if b == 0:
            o[r0:r1], L[r0:r1] = _attend(q[r0:r1], k[r0:r1], v[r0:r1], s, loc_allowed)
            continue
        pre = slice(0, r0)
        if topk_clusters <= 0:
            o_loc, L_loc = _attend(q[r0:r1], k[r0:r1], v[r0:r1], s, loc_allowed)
            S = tilted_summaries(qbar, k[pre], v[pre], lk_s[pre], Ck, s, dipole)
            o_far, L_far = refine(q[r0:r1], lq[r0:r1], qbar, S, s, dipole != "none")
            o[r0:r1], L[r0:r1] = lse_merge(o_far, L_far, o_loc, L_loc)
            continue
        for i in np.unique(lq[r0:r1]):
            qi = rows[lq[r0:r1] == i]
            a = s * (k[pre] @ qbar[i])
            if retrieval_follow is None:
                take = retrieval_selection(a, lk[pre], key_block[pre], Ck, b, topk_clusters, topk_blocks)
            else:
                fl = []
                for row in np.asarray(retrieval_follow[b, i]):
                    if row[0] >= 0:
                        fl.append((int(row[0]), [int(x) for x in row[1:] if x >= 0]))
                take, nt, mm = retrieval_selection(a, lk[pre], key_block[pre], Ck, b, topk_clusters,
                                                   topk_blocks, follow=fl)
                near += nt
                mism += mm
            R = np.nonzero(take)[0]
            F = np.nonzero(~take)[0]
            keys = np.concatenate([R, np.arange(r0, r1)])
            allowed = np.ones((qi.size, keys.size), bool)
            allowed[:, R.size:] = np.arange(r0, r1)[None, :] <= qi[:, None]
            o_ex, L_ex = _attend(q[qi], k[keys], v[keys], s, allowed)
            if F.size:
                S = tilted_summaries(qbar[i:i + 1], k[F], v[F], lk[F], Ck, s, dipole)
                o_far, L_far = refine(q[qi], np.zeros(qi.size, np.int64), qbar[i:i + 1], S, s,
                                      dipole != "none")
            else:
                o_far, L_far = np.zeros_like(o_ex), np.full(qi.size, NEG_INF)
            o[qi], L[qi] = lse_merge(o_far, L_far, o_ex, L_ex)
    res = MuseResult(o, L, km_q, km_k, lq, lk, qbar)
    res.retrieval_near_ties, res.retrieval_mismatches = near, mism
    return res
