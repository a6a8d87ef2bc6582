"""Pins of the oracle's exact attention and Lloyd K-means (CPU only)."""

import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import exact_attention, lloyd_kmeans, lse_merge, squared_distances

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- exact attention

def test_exact_attention_closed_form():
    # one query, two keys, D=1, s=1: weights 1 : e  (softmax of logits 0 and 1)
    q = np.array([[1.0]])
    k = np.array([[0.0], [1.0]])
    v = np.array([[0.0, 1.0], [2.0, 3.0]])
    o, L = exact_attention(q, k, v, scale=1.0)
    e = math.e
    assert np.allclose(o[0], [2 * e / (1 + e), (1 + 3 * e) / (1 + e)], rtol=0, atol=1e-15)
    assert abs(L[0] - math.log(1 + e)) < 1e-15


@pytest.mark.parametrize("causal", [False, True])
def test_exact_attention_matches_torch_sdpa(causal):
    rng = np.random.default_rng(0)
    N, D = 300, 32
    q, k, v = (rng.standard_normal((N, D)) for _ in range(3))
    o, L = exact_attention(q, k, v, causal=causal, row_block=64)
    t = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(k)[None], torch.from_numpy(v)[None], is_causal=causal)
    assert np.max(np.abs(o - t[0].numpy())) < 1e-12
    # L = log sum exp of the scaled logits, checked for a few rows by direct summation
    for n in (0, 7, N - 1):
        m = n + 1 if causal else N
        logits = (q[n] @ k[:m].T) / math.sqrt(D)
        assert abs(L[n] - (logits.max() + math.log(np.exp(logits - logits.max()).sum()))) < 1e-12


def test_lse_merge_equals_attention_over_union():
    rng = np.random.default_rng(1)
    q, k, v = rng.standard_normal((5, 8)), rng.standard_normal((40, 8)), rng.standard_normal((40, 3))
    o1, L1 = exact_attention(q, k[:13], v[:13])
    o2, L2 = exact_attention(q, k[13:], v[13:])
    o, L = lse_merge(o1, L1, o2, L2)
    oe, Le = exact_attention(q, k, v)
    assert np.max(np.abs(o - oe)) < 1e-13 and np.max(np.abs(L - Le)) < 1e-13
    # an empty side (L = -inf) leaves the other unchanged
    o3, L3 = lse_merge(np.zeros_like(o1), np.full(5, -np.inf), o1, L1)
    assert np.array_equal(o3, o1) and np.array_equal(L3, L1)


# ---------------------------------------------------------------- K-means

def _golden_cases():
    with open(os.path.join(GOLDEN, "kmeans_handworked.json")) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _golden_cases(), ids=lambda c: c["name"])
def test_kmeans_handworked(case):
    x = np.array(case["x"], float)[:, None]
    for t, (labels, cent) in enumerate(zip(case["trace"], case["centroids_after"])):
        r = lloyd_kmeans(x, case["C"], t + 1)
        assert r.labels.tolist() == labels
        assert [list(tr) for tr in r.trace] == case["trace"][: t + 1]
        assert np.allclose(r.centroids[:, 0], cent, rtol=0, atol=1e-15)


def test_squared_distances_direct():
    x = np.array([[1.0, 2.0], [0.0, 0.0]])
    c = np.array([[1.0, 0.0], [3.0, 4.0], [0.0, 0.0]])
    assert np.array_equal(squared_distances(x, c), [[4.0, 8.0, 5.0], [1.0, 25.0, 0.0]])


def test_kmeans_recovers_well_separated_partition():
    # 8 tight groups far apart; the sequence is laid out so that the strided init
    # x[floor(j n / C)] falls in a different group for every j -> known partition.
    rng = np.random.default_rng(2)
    C, per, D = 8, 25, 6
    centers = rng.standard_normal((C, D)) * 20
    truth = np.repeat(np.arange(C), per)
    x = centers[truth] + 0.01 * rng.standard_normal((C * per, D))
    r = lloyd_kmeans(x, C, 3)
    assert np.array_equal(r.labels, truth)
    for j in range(C):
        assert np.allclose(r.centroids[j], x[truth == j].mean(axis=0), atol=1e-13)


def test_kmeans_lloyd_invariants():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((400, 5))
    C = 12
    prev = None
    for T in range(1, 7):
        r = lloyd_kmeans(x, C, T)
        # centroids after the update are member means of the returned labels
        for j in range(C):
            m = r.labels == j
            if m.any():
                assert np.allclose(r.centroids[j], x[m].mean(axis=0), atol=1e-13)
        # each label is the argmin to the centroids of the previous iteration
        c_prev = x[(np.arange(C) * 400) // C] if T == 1 else lloyd_kmeans(x, C, T - 1).centroids
        d = squared_distances(x, c_prev)
        assert np.array_equal(r.labels, np.argmin(d, axis=1))
        # the K-means objective never increases (Lloyd's monotonicity)
        obj = np.sum((x - r.centroids[r.labels]) ** 2)
        if prev is not None:
            assert obj <= prev + 1e-9
        prev = obj


def test_kmeans_follow_mode_near_tie_adoption():
    # init picks x[0]=0 and x[2]=2; the last point sits at 1+1e-9, a near-tie between them
    x = np.array([[0.0], [5.0], [2.0], [1.0 + 1e-9]])
    r = lloyd_kmeans(x, 2, 1)
    assert r.labels.tolist() == [0, 1, 1, 1]
    # a compared run that chose 0 for the near-tie point is adopted, not flagged
    f = lloyd_kmeans(x, 2, 1, follow_trace=[np.array([0, 1, 1, 0])])
    assert f.labels.tolist() == [0, 1, 1, 0] and f.near_ties == 1 and f.mismatches == 0
    # a clear disagreement is flagged and not adopted
    g = lloyd_kmeans(x, 2, 1, follow_trace=[np.array([1, 1, 1, 1])])
    assert g.mismatches == 1 and g.near_ties == 0 and g.labels.tolist() == [0, 1, 1, 1]
