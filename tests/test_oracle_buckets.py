"""Pins of the oracle's bucket order (the stable grouping of a head's positions by
(spatial block, cluster) that replaces the paper's ragged per-cluster tensors)."""

import numpy as np

from oracle import bucket_order


def test_hand_worked_acausal():
    # labels of 7 positions, 3 clusters: cluster 1 holds positions 0, 3, 6 (in that order),
    # cluster 2 holds 1 and 4, cluster 0 holds 2 and 5
    perm, offs = bucket_order([1, 2, 0, 1, 2, 0, 1], 3)
    assert perm.tolist() == [2, 5, 0, 3, 6, 1, 4]
    assert offs.tolist() == [0, 2, 5, 7]


def test_hand_worked_causal_with_empty_buckets():
    # 8 positions in blocks of 4, 3 clusters; block 0 has no member of cluster 1,
    # block 1 none of cluster 0
    labels = [2, 0, 2, 0, 1, 2, 1, 1]
    perm, offs = bucket_order(labels, 3, block=4)
    assert perm.tolist() == [1, 3, 0, 2, 4, 6, 7, 5]
    assert offs.tolist() == [0, 2, 2, 4, 4, 7, 8]


def test_invariants_random():
    rng = np.random.default_rng(3)
    for n, C, block in [(1000, 7, 0), (1024, 16, 256), (512, 1, 64), (300, 128, 0)]:
        labels = rng.integers(0, C, size=n)
        perm, offs = bucket_order(labels, C, block)
        nb = 1 if block == 0 else n // block
        assert sorted(perm.tolist()) == list(range(n))
        assert offs[0] == 0 and offs[-1] == n and len(offs) == nb * C + 1
        assert np.all(np.diff(offs) >= 0)
        for b in range(nb):
            for j in range(C):
                seg = perm[offs[b * C + j]:offs[b * C + j + 1]]
                assert np.all(labels[seg] == j)
                assert np.all(np.diff(seg) > 0)
                if block:
                    assert np.all(seg // block == b)
