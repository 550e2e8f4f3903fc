"""Pins of the sample-selection oracle (SE-KD3X sample axis, "Rethinking
Selective Knowledge Distillation" Method section 2): samples of constant
entropy (their means are those constants), unequal lengths (the mean weighs
each position once), ties to the lower sample index, permutation of the
samples, empty samples last, and the kept count floor(num*B/den).
"""
import numpy as np
import pytest

from oracle import oracle_select_samples


def test_constant_entropy_samples():
    consts = np.array([3.0, 7.0, 5.0, 1.0, 6.0])
    lens = np.array([4, 2, 7, 1, 3])
    off = np.concatenate([[0], np.cumsum(lens)])
    e = np.repeat(consts, lens)
    mask, idx, k, means = oracle_select_samples(e, off, 40, 100)   # floor(0.4 * 5) = 2
    assert k == 2
    assert list(idx) == [1, 4]
    assert np.array_equal(means, consts)


def test_mean_weighs_each_position_once():
    # sample 0: [10, 0, 0, 0] -> 2.5; sample 1: [3] -> 3; sample 2: [2, 2] -> 2
    e = np.array([10.0, 0.0, 0.0, 0.0, 3.0, 2.0, 2.0])
    off = [0, 4, 5, 7]
    _, idx, k, means = oracle_select_samples(e, off, 1, 3)
    assert k == 1 and list(idx) == [1]
    assert np.allclose(means, [2.5, 3.0, 2.0])


def test_ties_lower_index_and_empty_last():
    e = np.array([2.0, 2.0, 2.0, 2.0])
    off = [0, 1, 1, 2, 3, 4]          # sample 1 is empty
    mask, idx, k, means = oracle_select_samples(e, off, 4, 5)      # floor(0.8 * 5) = 4
    assert list(idx) == [0, 2, 3, 4]
    assert means[1] == -np.inf
    mask, idx, k, _ = oracle_select_samples(e, off, 1, 1)
    assert k == 5 and list(idx) == [0, 1, 2, 3, 4]


def test_permutation_of_samples():
    rng = np.random.default_rng(71)
    B = 30
    lens = rng.integers(1, 9, size=B)
    off = np.concatenate([[0], np.cumsum(lens)])
    e = rng.random(off[-1]) * 10
    mask, _, k, _ = oracle_select_samples(e, off, 30, 100)
    perm = rng.permutation(B)
    e2 = np.concatenate([e[off[b]:off[b + 1]] for b in perm])
    off2 = np.concatenate([[0], np.cumsum(lens[perm])])
    mask2, _, k2, _ = oracle_select_samples(e2, off2, 30, 100)
    assert k2 == k
    assert np.array_equal(mask2, mask[perm])


def test_rejects_bad_arguments():
    with pytest.raises(ValueError):
        oracle_select_samples(np.zeros(3), [0, 2, 1], 1, 2)
    with pytest.raises(ValueError):
        oracle_select_samples(np.zeros(3), [0, 3], 3, 2)
