"""Pins of the teacher top-K cache oracle against facts that do not depend on
its own formula: brute force on tiny inputs, a closed form (identity weights),
tie order, permutation of the vocabulary, K = V, and the bf16 rounding of a
value half way between two bf16 numbers.

The cache keeps each position's K largest teacher logits ("offline top-K
logits" in "Making Knowledge Distillation Cheap Enough to Run at Scale" as
written up by aibase.it), ordered by logit descending with the lower id first
on ties (the cache validation there checks the top-K order).
"""
import numpy as np
import pytest

from oracle import oracle_teacher_topk


def test_brute_force_tiny():
    rng = np.random.default_rng(41)
    S, H, V, K = 5, 6, 40, 7
    h = rng.standard_normal((S, H)).astype(np.float32)
    W = rng.standard_normal((V, H)).astype(np.float32)
    ids, logits = oracle_teacher_topk(h, W, K)
    for t in range(S):
        entries = []
        for v in range(V):
            z = 0.0
            for i in range(H):
                z += float(h[t, i]) * float(W[v, i])
            entries.append((-z, v))
        entries.sort()
        want_ids = [v for _, v in entries[:K]]
        want_z = [-nz for nz, _ in entries[:K]]
        assert list(ids[t]) == want_ids
        assert np.allclose(logits[t], np.float32(want_z), rtol=1e-6, atol=1e-6)


def test_identity_weights_pick_largest_coordinates():
    # W = 3 I: the logits are 3 x the hidden coordinates
    rng = np.random.default_rng(42)
    S, H, K = 4, 30, 9
    h = rng.standard_normal((S, H)).astype(np.float32)
    W = 3.0 * np.eye(H, dtype=np.float32)
    ids, logits = oracle_teacher_topk(h, W, K)
    for t in range(S):
        want = np.argsort(-h[t], kind="stable")[:K]
        assert np.array_equal(ids[t], want)
        assert np.array_equal(logits[t], (3.0 * h[t, want].astype(np.float64)).astype(np.float32))


def test_equal_logits_lower_id_first():
    rng = np.random.default_rng(43)
    S, H, V, K = 3, 8, 50, 6
    h = np.abs(rng.standard_normal((S, H))).astype(np.float32) + 0.1
    W = rng.standard_normal((V, H)).astype(np.float32) * 0.01
    big = np.full(H, 2.0, dtype=np.float32)
    for v in (31, 5, 17):          # three equal rows, far above the rest
        W[v] = big
    W[40] = big * 0.5              # the next one down
    ids, logits = oracle_teacher_topk(h, W, K)
    for t in range(S):
        assert list(ids[t][:4]) == [5, 17, 31, 40]
        assert logits[t][0] == logits[t][1] == logits[t][2]
        assert np.all(np.diff(logits[t]) <= 0)


def test_vocabulary_permutation():
    rng = np.random.default_rng(44)
    S, H, V, K = 6, 10, 80, 12
    h = rng.standard_normal((S, H)).astype(np.float32)
    W = rng.standard_normal((V, H)).astype(np.float32)
    perm = rng.permutation(V)
    ids, logits = oracle_teacher_topk(h, W, K)
    ids_p, logits_p = oracle_teacher_topk(h, W[perm], K)
    # entry i of the permuted vocabulary is original entry perm[i]
    assert np.array_equal(perm[ids_p], ids)
    assert np.array_equal(logits_p, logits)


def test_K_equals_V_is_a_full_sort():
    rng = np.random.default_rng(45)
    h = rng.standard_normal((2, 5)).astype(np.float32)
    W = rng.standard_normal((17, 5)).astype(np.float32)
    ids, logits = oracle_teacher_topk(h, W, 17)
    for t in range(2):
        assert sorted(ids[t].tolist()) == list(range(17))
        assert np.all(np.diff(logits[t]) <= 0)


def test_bf16_output_ties_to_even():
    # z = 1 + 2^-8 lies half way between the bf16 values 1 and 1 + 2^-7: ties
    # to even gives 1; z = 1 + 3 * 2^-8 lies half way between 1 + 2^-7 and
    # 1 + 2^-6 and goes up to 1 + 2^-6
    h = np.array([[1.0, 1.0]], dtype=np.float32)
    W = np.array([[1.0, 2.0 ** -8], [1.0, 3 * 2.0 ** -8], [0.0, 0.0]], dtype=np.float32)
    ids, f32 = oracle_teacher_topk(h, W, 3)
    _, b16 = oracle_teacher_topk(h, W, 3, out_dtype="bf16")
    assert list(ids[0]) == [1, 0, 2]
    assert f32[0].tolist() == [1 + 3 * 2.0 ** -8, 1 + 2.0 ** -8, 0.0]
    assert b16[0].tolist() == [1 + 2.0 ** -6, 1.0, 0.0]


def test_rejects_bad_K():
    h = np.zeros((1, 2), dtype=np.float32)
    W = np.zeros((3, 2), dtype=np.float32)
    with pytest.raises(ValueError):
        oracle_teacher_topk(h, W, 4)
