"""Pins of the backward oracle (oracle/muse_bwd_ref.py), CPU only.

* central finite differences of the forward oracle (muse_acausal / muse_causal with the
  labels fixed), over every input element, for the tilted, untilted and no-dipole modes,
  the prefix and hierarchical causal forms, s = 1/sqrt(D) and s = 1, and capped key
  clusters;
* exact attention's backward against torch autograd of scaled dot-product attention in
  float64 (an independent implementation);
* reductions that fix the answer without finite differences: singleton clusters give
  exact attention's gradients; with keys (queries) equal to their centroids MuSe is exact
  attention for every value of the other inputs, so their gradients are exact attention's;
  with degenerate queries dq is exact attention's too under the tilted dipole (the forward
  error is second order in the query residual) and differs without it (first order).
"""

import numpy as np
import pytest
import torch

from oracle import exact_attention, muse_acausal, muse_causal
from oracle.muse_bwd_ref import exact_attention_bwd, muse_acausal_bwd, muse_causal_bwd


def _problem(seed, N=40, D=6, Dv=5, Cq=3, Ck=5, empty_k=True):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((N, D)) * 0.8
    k = rng.standard_normal((N, D)) * 0.8
    v = rng.standard_normal((N, Dv))
    lq = rng.integers(0, Cq, N)
    lk = rng.integers(0, Ck, N)
    if empty_k:
        lk[lk == 1] = 2   # one empty key cluster
    dO = rng.standard_normal((N, Dv))
    return q, k, v, lq, lk, dO


def _fd(fun, x, h=1e-6):
    """Central differences of the scalar fun() with respect to every element of x (in place)."""
    g = np.zeros_like(x)
    for idx in np.ndindex(x.shape):
        x0 = x[idx]
        x[idx] = x0 + h
        fp = fun()
        x[idx] = x0 - h
        fm = fun()
        x[idx] = x0
        g[idx] = (fp - fm) / (2 * h)
    return g


def _check(analytic, numeric, tol=2e-6):
    err = np.abs(analytic - numeric).max() / max(np.abs(numeric).max(), 1e-12)
    assert err < tol, err


@pytest.mark.parametrize("dipole", ["tilted", "untilted", "none"])
@pytest.mark.parametrize("scale", [None, 1.0])
def test_acausal_finite_differences(dipole, scale):
    q, k, v, lq, lk, dO = _problem(1)
    Cq, Ck = 3, 5

    def f():
        return float((muse_acausal(q, k, v, Cq, Ck, 1, scale=scale, dipole=dipole, labels_q=lq,
                                   labels_k=lk).o * dO).sum())

    dq, dk, dv = muse_acausal_bwd(q, k, v, Cq, Ck, lq, lk, dO, scale=scale, dipole=dipole)
    _check(dq, _fd(f, q))
    _check(dk, _fd(f, k))
    _check(dv, _fd(f, v))


@pytest.mark.parametrize("dipole,hier", [("tilted", False), ("untilted", False), ("none", False),
                                         ("tilted", True)])
def test_causal_finite_differences(dipole, hier):
    # 4 blocks of 10: the hierarchy gives block 3 two squares
    q, k, v, lq, lk, dO = _problem(2, N=40)
    Cq, Ck, block = 3, 5, 10

    def f():
        return float((muse_causal(q, k, v, Cq, Ck, 1, block, dipole=dipole, labels_q=lq, labels_k=lk,
                                  hierarchical=hier).o * dO).sum())

    dq, dk, dv = muse_causal_bwd(q, k, v, Cq, Ck, block, lq, lk, dO, dipole=dipole, hierarchical=hier)
    _check(dq, _fd(f, q))
    _check(dk, _fd(f, k))
    _check(dv, _fd(f, v))


@pytest.mark.parametrize("causal,dipole", [(False, "tilted"), (False, "untilted"), (True, "tilted"),
                                           (True, "none")])
def test_cap_finite_differences(causal, dipole):
    # a cap of 1.0: clusters of more than N / Ck members lose their later keys from the
    # summaries (40 keys, 5 clusters: at most 8 kept each)
    q, k, v, lq, lk, dO = _problem(4, N=40, empty_k=False)
    Cq, Ck, block, cap = 3, 5, 10, 1.0
    assert max(np.bincount(lk, minlength=Ck)) > 8  # some key is left out

    def f():
        if causal:
            r = muse_causal(q, k, v, Cq, Ck, 1, block, dipole=dipole, labels_q=lq, labels_k=lk, cap_ratio=cap)
        else:
            r = muse_acausal(q, k, v, Cq, Ck, 1, dipole=dipole, labels_q=lq, labels_k=lk, cap_ratio=cap)
        return float((r.o * dO).sum())

    if causal:
        dq, dk, dv = muse_causal_bwd(q, k, v, Cq, Ck, block, lq, lk, dO, dipole=dipole, cap_ratio=cap)
    else:
        dq, dk, dv = muse_acausal_bwd(q, k, v, Cq, Ck, lq, lk, dO, dipole=dipole, cap_ratio=cap)
    _check(dq, _fd(f, q))
    _check(dk, _fd(f, k))
    _check(dv, _fd(f, v))


@pytest.mark.parametrize("causal", [False, True])
def test_exact_backward_against_torch_autograd(causal):
    rng = np.random.default_rng(3)
    q, k, v, dO = (rng.standard_normal((33, 8)) for _ in range(4))
    dq, dk, dv = exact_attention_bwd(q, k, v, dO, causal=causal)
    Q, K, V = (torch.tensor(t, dtype=torch.float64, requires_grad=True) for t in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(Q[None], K[None], V[None], is_causal=causal)[0]
    o.backward(torch.tensor(dO))
    for a, t in ((dq, Q), (dk, K), (dv, V)):
        np.testing.assert_allclose(a, t.grad.numpy(), rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_singleton_clusters_give_exact_gradients(causal):
    # as many clusters as points: both residuals vanish and MuSe is exact attention
    rng = np.random.default_rng(4)
    N, D = 24, 6
    q, k, v, dO = (rng.standard_normal((N, D)) for _ in range(4))
    lab = np.arange(N)
    if causal:
        g = muse_causal_bwd(q, k, v, N, N, 8, lab, lab, dO)
    else:
        g = muse_acausal_bwd(q, k, v, N, N, lab, lab, dO)
    ref = exact_attention_bwd(q, k, v, dO, causal=causal)
    for a, b in zip(g, ref):
        np.testing.assert_allclose(a, b, rtol=1e-9, atol=1e-11)


def _degenerate(which, seed=5, N=48, D=6, C=4):
    """Queries or keys equal to their cluster centroids (C distinct rows, each repeated)."""
    rng = np.random.default_rng(seed)
    q, k, v, dO = (rng.standard_normal((N, D)) for _ in range(4))
    lab_d = np.arange(N) % C
    rows = rng.standard_normal((C, D))
    if which == "k":
        k = rows[lab_d].copy()
    else:
        q = rows[lab_d].copy()
    lab_other = rng.integers(0, 3, N)
    return q, k, v, dO, lab_d, lab_other, C


@pytest.mark.parametrize("which", ["k", "q"])
def test_centroid_equal_inputs_give_exact_gradients(which):
    q, k, v, dO, lab_d, lab_o, C = _degenerate(which)
    lq, lk, Cq, Ck = (lab_o, lab_d, 3, C) if which == "k" else (lab_d, lab_o, C, 3)
    # the forward equals exact attention here ...
    o = muse_acausal(q, k, v, Cq, Ck, 1, labels_q=lq, labels_k=lk).o
    np.testing.assert_allclose(o, exact_attention(q, k, v)[0], rtol=1e-10, atol=1e-12)
    ref = exact_attention_bwd(q, k, v, dO)
    for dipole in ("tilted", "untilted", "none"):
        g = muse_acausal_bwd(q, k, v, Cq, Ck, lq, lk, dO, dipole=dipole)
        # ... for every value of the other two inputs (the degenerate side's residual stays
        # zero), so their gradients are exact attention's in every dipole mode
        others = (0, 2) if which == "k" else (1, 2)
        for t in others:
            np.testing.assert_allclose(g[t], ref[t], rtol=1e-8, atol=1e-10)
    # degenerate queries: with the tilted dipole the forward error is second order in the
    # query residual, so dq is exact attention's too; without the dipole it is first order
    # (s Cov(v, kt) qt) and dq differs. (Degenerate keys: the dipole is aggregated with the
    # stage-1 weights P_ij rather than each query's p_nj, which leaves a first-order key
    # term of size O(qt^2): dk is not pinned there.)
    if which == "q":
        gt = muse_acausal_bwd(q, k, v, Cq, Ck, lq, lk, dO, dipole="tilted")
        np.testing.assert_allclose(gt[0], ref[0], rtol=1e-8, atol=1e-10)
        gn = muse_acausal_bwd(q, k, v, Cq, Ck, lq, lk, dO, dipole="none")
        assert np.abs(gn[0] - ref[0]).max() > 1e-3 * np.abs(ref[0]).max()


def test_causal_centroid_equal_keys_give_exact_gradients():
    q, k, v, dO, lab_d, lab_o, C = _degenerate("k", N=48)
    g = muse_causal_bwd(q, k, v, 3, C, 12, lab_o, lab_d, dO)
    ref = exact_attention_bwd(q, k, v, dO, causal=True)
    np.testing.assert_allclose(g[0], ref[0], rtol=1e-8, atol=1e-10)
    np.testing.assert_allclose(g[2], ref[2], rtol=1e-8, atol=1e-10)


def test_causal_centroid_equal_queries_give_exact_gradients():
    q, k, v, dO, lab_d, lab_o, C = _degenerate("q", N=48)
    g = muse_causal_bwd(q, k, v, C, 3, 12, lab_d, lab_o, dO)
    ref = exact_attention_bwd(q, k, v, dO, causal=True)
    for a, b in zip(g, ref):
        np.testing.assert_allclose(a, b, rtol=1e-8, atol=1e-10)
