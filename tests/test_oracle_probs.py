"""Pins of the oracle with teacher targets given as probabilities (sampled
sparse targets, the class axis of SE-KD3X in "Rethinking Selective Knowledge
Distillation", Method section 2): agreement with the logit path on the same
distribution, the closed form of a one-hot target (the student's
cross-entropy), invariance to scale and to splitting an id's mass over
duplicate entries, and exclusion of malformed rows.
"""
import math

import numpy as np

from oracle import oracle_from_logits, oracle_loss_grads, oracle_validate_topk


def _case(seed, S=7, H=6, V=31, K=5):
    rng = np.random.default_rng(seed)
    hidden = rng.standard_normal((S, H))
    W = rng.standard_normal((V, H)) / np.sqrt(H)
    ids = np.stack([rng.choice(V, K, replace=False) for _ in range(S)])
    tl = rng.standard_normal((S, K)) * 2.0
    return hidden, W, ids, tl


def test_softmax_targets_match_the_logit_path():
    hidden, W, ids, tl = _case(61)
    ids[2, 3] = ids[2, 1]                        # a duplicate id
    T = 1.7
    e = np.exp(tl / T - np.max(tl / T, axis=1, keepdims=True))
    p = e / e.sum(axis=1, keepdims=True)
    a = oracle_loss_grads(hidden, W, ids, tl, T=T)
    b = oracle_loss_grads(hidden, W, ids, p, T=T, probs=True)
    assert abs(a["loss"] - b["loss"]) <= 1e-12 * abs(a["loss"])
    for k in ("kl_rows", "dH", "dW"):
        assert np.allclose(a[k], b[k], rtol=1e-11, atol=1e-14)


def test_one_hot_target_is_the_student_cross_entropy():
    hidden, W, ids, _ = _case(62)
    S, K = ids.shape
    T = 1.3
    p = np.zeros((S, K))
    p[:, 0] = 1.0
    Z = hidden @ W.T
    r = oracle_from_logits(Z, ids, p, T=T, probs=True)
    for t in range(S):
        zt = Z[t] / T
        lse = zt.max() + math.log(np.sum(np.exp(zt - zt.max())))
        assert abs(r["kl_rows"][t] - (lse - zt[ids[t, 0]])) <= 1e-12
        q = np.exp(zt - lse)
        onehot = np.zeros_like(q)
        onehot[ids[t, 0]] = 1.0
        assert np.allclose(r["dZ"][t], (q - onehot) / (T * S), rtol=1e-12, atol=1e-16)


def test_scale_and_duplicate_entries_do_not_matter():
    hidden, W, ids, _ = _case(63)
    rng = np.random.default_rng(64)
    p = rng.random(ids.shape) + 0.05
    a = oracle_loss_grads(hidden, W, ids, p, probs=True)
    b = oracle_loss_grads(hidden, W, ids, 3.0 * p, probs=True)
    assert abs(a["loss"] - b["loss"]) <= 1e-12 * abs(a["loss"])
    # one id's mass split over two entries
    ids2 = np.concatenate([ids, ids[:, :1]], axis=1)
    p2 = np.concatenate([p, p[:, :1] * 0.25], axis=1)
    p2[:, 0] *= 0.75
    c = oracle_loss_grads(hidden, W, ids2, p2, probs=True)
    assert abs(a["loss"] - c["loss"]) <= 1e-12 * abs(a["loss"])
    assert np.allclose(a["dW"], c["dW"], rtol=1e-11, atol=1e-14)


def test_malformed_rows_are_missing():
    hidden, W, ids, _ = _case(65)
    p = np.full(ids.shape, 0.2)
    p[1, 2] = -0.1          # negative
    p[3, 0] = np.nan        # NaN
    p[4, :] = 0.0           # no mass
    r = oracle_loss_grads(hidden, W, ids, p, probs=True)
    assert list(np.flatnonzero(~r["valid"])) == [1, 3, 4]
    assert np.all(r["dH"][[1, 3, 4]] == 0.0)
    ok = np.ones(ids.shape[0], dtype=bool)
    ok[[1, 3, 4]] = False
    sub = oracle_loss_grads(hidden[ok], W, ids[ok], p[ok], probs=True)
    assert abs(r["loss"] - sub["loss"]) <= 1e-12 * abs(sub["loss"])


def test_validation_counts_for_probabilities_by_hand():
    # counted by hand: ids 12 and -3 are out of range for V = 10; values -0.5,
    # NaN, +inf and -inf are not finite and >= 0; rows 1 (zeros only) and 3
    # (only bad values) hold no finite positive value
    ids = np.array([[0, 5, 12], [1, 2, 3], [4, -3, 6], [7, 8, 9]])
    pv = np.array([[0.5, 0.0, 0.25],
                   [0.0, 0.0, 0.0],
                   [-0.5, 0.3, np.nan],
                   [np.inf, -np.inf, np.nan]])
    assert oracle_validate_topk(ids, pv, 10, probs=True) == (2, 2, 5)
    # the same values read as logits: only NaN and +inf are bad, no row is all -inf
    assert oracle_validate_topk(ids, pv, 10) == (2, 0, 3)


def test_validation_flags_exactly_the_rows_the_loss_leaves_out():
    hidden, W, ids, _ = _case(66, S=40)
    rng = np.random.default_rng(67)
    p = rng.random(ids.shape)
    p[rng.random(ids.shape) < 0.3] = 0.0
    p[rng.random(ids.shape) < 0.05] = -1.0
    p[rng.random(ids.shape) < 0.05] = np.nan
    p[7, :] = 0.0
    r = oracle_loss_grads(hidden, W, ids, p, probs=True)
    # a row is left out of the loss exactly when validating it alone reports it
    # empty or holding a bad value
    for t in range(ids.shape[0]):
        _, n_empty, n_bad = oracle_validate_topk(ids[t:t + 1], p[t:t + 1], W.shape[0], probs=True)
        assert (n_empty + n_bad > 0) == (not r["valid"][t])
    assert not r["valid"][7]


def test_softmax_targets_validate_clean():
    _, _, ids, tl = _case(68)
    e = np.exp(tl - tl.max(axis=1, keepdims=True))
    assert oracle_validate_topk(ids, e / e.sum(axis=1, keepdims=True), 31, probs=True) == (0, 0, 0)
