"""Pins of the oracle's capped key clusters (cap_key_labels and the cap_ratio option of
muse_acausal / muse_causal), CPU only. The reading: key cluster j keeps its first
U = ceil(ratio * n / Ck) members in position order in its stage-1 summaries."""

import numpy as np
import pytest

from oracle import cap_key_labels, exact_attention, muse_acausal, muse_causal


def test_hand_worked_cap():
    # n = 10, Ck = 4, ratio 1.5: U = ceil(3.75) = 4; cluster 2 has 6 members, the last
    # two (positions 8, 9) are dropped; cluster 0 (3 members) and 1 (1) are unchanged
    labels = [2, 0, 2, 1, 2, 0, 2, 0, 2, 2]
    out = cap_key_labels(labels, 4, 1.5)
    assert out.tolist() == [2, 0, 2, 1, 2, 0, 2, 0, -1, -1]
    # ratio 1.25: U = ceil(3.125) = 4 as well; ratio 1.0: U = 3 (cluster 0 keeps all 3)
    assert cap_key_labels(labels, 4, 1.25).tolist() == out.tolist()
    assert cap_key_labels(labels, 4, 1.0).tolist() == [2, 0, 2, 1, 2, 0, -1, 0, -1, -1]
    assert cap_key_labels(labels, 4, None).tolist() == labels


def _problem(seed, N=96, D=6, Cq=3, Ck=4):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((N, D)) * 0.7
    k = rng.standard_normal((N, D)) * 0.7
    v = rng.standard_normal((N, D))
    lq = rng.integers(0, Cq, N)
    # unbalanced key clusters: cluster 0 takes half of the keys
    lk = np.where(rng.random(N) < 0.5, 0, rng.integers(1, Ck, N))
    return q, k, v, lq, lk


def test_large_cap_changes_nothing():
    q, k, v, lq, lk = _problem(1)
    big = max(np.bincount(lk)) * 4 / len(lk) + 1.0   # U above every cluster size
    a = muse_acausal(q, k, v, 3, 4, 1, labels_q=lq, labels_k=lk)
    b = muse_acausal(q, k, v, 3, 4, 1, labels_q=lq, labels_k=lk, cap_ratio=big)
    np.testing.assert_array_equal(a.o, b.o)


@pytest.mark.parametrize("ratio", [1.0, 1.25, 1.5])
def test_acausal_cap_equals_dropping_the_keys(ratio):
    # the capped forward equals the forward on the inputs without the dropped keys (same
    # clusters for the rest), the kept set written out independently here
    q, k, v, lq, lk = _problem(2)
    N, Ck = len(lk), 4
    U = int(np.ceil(ratio * N / Ck))
    keep = np.ones(N, bool)
    seen = {}
    for m in range(N):
        seen[lk[m]] = seen.get(lk[m], 0) + 1
        keep[m] = seen[lk[m]] <= U
    assert not keep.all()
    a = muse_acausal(q, k, v, 3, Ck, 1, labels_q=lq, labels_k=lk, cap_ratio=ratio)
    b = muse_acausal(q, k[keep], v[keep], 3, Ck, 1, labels_q=lq, labels_k=lk[keep])
    np.testing.assert_allclose(a.o, b.o, rtol=1e-12, atol=1e-12)


def test_causal_cap():
    q, k, v, lq, lk = _problem(3, N=96)
    # one block: no far field, the cap changes nothing (exact causal attention)
    r = muse_causal(q, k, v, 3, 4, 1, 96, labels_q=lq, labels_k=lk, cap_ratio=1.0)
    np.testing.assert_allclose(r.o, exact_attention(q, k, v, causal=True)[0], rtol=1e-12, atol=1e-12)
    # several blocks: block 0 is exact; a later block's far field ignores the keys the cap
    # dropped, which only affects blocks after them
    a = muse_causal(q, k, v, 3, 4, 1, 24, labels_q=lq, labels_k=lk)
    b = muse_causal(q, k, v, 3, 4, 1, 24, labels_q=lq, labels_k=lk, cap_ratio=1.0)
    np.testing.assert_allclose(a.o[:24], b.o[:24], rtol=1e-12, atol=1e-12)
    dropped = cap_key_labels(lk, 4, 1.0) < 0
    first = int(np.argmax(dropped))
    blk = first // 24
    np.testing.assert_allclose(a.o[:(blk + 1) * 24], b.o[:(blk + 1) * 24], rtol=1e-12, atol=1e-12)
    assert np.abs(a.o[(blk + 1) * 24:] - b.o[(blk + 1) * 24:]).max() > 1e-6
    with pytest.raises(ValueError):
        muse_causal(q, k, v, 3, 4, 1, 24, labels_q=lq, labels_k=lk, cap_ratio=1.5, topk_clusters=1, topk_blocks=1)
