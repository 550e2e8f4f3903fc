"""Pins of the position-signal and selection-policy oracles ("Rethinking
Selective Knowledge Distillation" Method section 1: student cross-entropy,
teacher uncertainty 1 - p_t(y_t), student entropy; top-k% per sequence; a
global threshold).

- cross-entropy against torch's cross_entropy in fp64 (a textbook routine);
- teacher uncertainty against the dense teacher grid (1 - P[t, y_t]) and a
  scalar math.exp loop, with its special cases (label not among the ids,
  a one-entry row, a missing row, a label out of range);
- selection against an independent pure-Python sort per segment, with ties,
  NaN, infinities and signed zeros; the one-segment case against the global
  entropy selection; the threshold policy against a scalar loop.
"""
import math

import numpy as np
import pytest
import torch

from oracle import (oracle_entropy, oracle_position_signals, oracle_select_above,
                    oracle_select_by_signal, oracle_select_top_fraction, teacher_distribution)


def _case(S=9, H=6, V=23, K=5, seed=3, probs=False):
    rng = np.random.default_rng(seed)
    hidden = rng.standard_normal((S, H))
    W = rng.standard_normal((V, H)) / math.sqrt(H)
    ids = np.stack([rng.choice(V, size=K, replace=False) for _ in range(S)]).astype(np.int32)
    ids[1, 2] = ids[1, 0]                       # a duplicate id
    if probs:
        tl = rng.random((S, K))
        tl[2, 1] = 0.0
    else:
        tl = 8.0 - 1.5 * np.log(np.arange(K) + 1.0) + rng.standard_normal((S, K))
        tl[2, 1] = -np.inf
    labels = rng.integers(0, V, size=S)
    labels[0] = ids[0, 1]                       # a label the teacher row holds
    labels[1] = ids[1, 0]                       # ... held twice
    return hidden, W, ids, tl, labels


def test_ce_matches_torch_cross_entropy():
    hidden, W, ids, tl, labels = _case()
    r = oracle_position_signals(hidden, W, ids, tl, labels, T=2.0)
    Z = torch.tensor(hidden) @ torch.tensor(W).T
    ref = torch.nn.functional.cross_entropy(Z, torch.tensor(labels), reduction="none").numpy()
    assert np.max(np.abs(r["ce"] - ref)) <= 1e-12
    assert np.all(r["ce"] >= 0.0)


def test_entropy_signal_is_the_student_entropy():
    hidden, W, ids, tl, labels = _case(seed=5)
    r = oracle_position_signals(hidden, W, ids, tl, labels, chunk=4)
    assert np.max(np.abs(r["entropy"] - oracle_entropy(hidden, W))) <= 1e-12


@pytest.mark.parametrize("probs", [False, True])
@pytest.mark.parametrize("T", [1.0, 0.7])
def test_teacher_uncertainty_against_dense_grid(probs, T):
    hidden, W, ids, tl, labels = _case(seed=11, probs=probs)
    V = W.shape[0]
    r = oracle_position_signals(hidden, W, ids, tl, labels, T=T, probs=probs)
    P, _, present = teacher_distribution(ids, tl, V, T, probs)
    ref = np.where(present, 1.0 - P[np.arange(len(labels)), labels], np.nan)
    assert np.allclose(r["teacher_unc"], ref, atol=1e-12, rtol=0, equal_nan=True)


def test_teacher_uncertainty_scalar_loop():
    hidden, W, ids, tl, labels = _case(S=5, K=4, seed=17)
    T = 1.3
    r = oracle_position_signals(hidden, W, ids, tl, labels, T=T)
    for t in range(5):
        ws = [math.exp(tl[t, k] / T) if np.isfinite(tl[t, k]) else 0.0 for k in range(4)]
        hit = math.fsum(w for w, i in zip(ws, ids[t]) if i == labels[t])
        assert abs(r["teacher_unc"][t] - (1.0 - hit / math.fsum(ws))) <= 1e-13


def test_teacher_uncertainty_special_cases():
    hidden, W, ids, tl, labels = _case(S=4, K=3, seed=23)
    V = W.shape[0]
    labels = labels.copy()
    labels[0] = next(v for v in range(V) if v not in ids[0])     # not among the ids: p = 0
    tl = tl.copy()
    tl[1] = -np.inf                                              # missing teacher row
    labels[3] = V                                                # label out of range
    r = oracle_position_signals(hidden, W, ids, tl, labels)
    assert r["teacher_unc"][0] == 1.0
    assert np.isnan(r["teacher_unc"][1]) and np.isfinite(r["ce"][1])
    assert np.isnan(r["teacher_unc"][3]) and np.isnan(r["ce"][3])
    # a one-entry row whose id is the label: the teacher is certain
    r1 = oracle_position_signals(hidden[:1], W, ids[:1, :1], tl[:1, :1], ids[:1, 0])
    assert r1["teacher_unc"][0] == 0.0


def _python_select(x, off, num, den):
    mask = [0] * len(x)
    thr = []
    for b in range(len(off) - 1):
        a, e = off[b], off[b + 1]
        cand = [(x[i], i) for i in range(a, e) if not math.isnan(x[i])]
        cand.sort(key=lambda p: (-p[0], p[1]))
        k = min(num * (e - a) // den, len(cand))
        for _, i in cand[:k]:
            mask[i] = 1
        thr.append(min(v for v, _ in cand[:k]) if k else float("nan"))
    return mask, thr


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_select_by_signal_against_python_sort(seed):
    rng = np.random.default_rng(100 + seed)
    S = 300
    x = rng.choice([-1.5, 0.0, -0.0, 0.25, 2.0, 7.0, np.inf, -np.inf, np.nan], size=S)
    x = np.where(rng.random(S) < 0.5, rng.standard_normal(S), x)
    lens = rng.integers(0, 40, size=12)
    off = np.concatenate([[0], np.cumsum(lens)])
    off = off[off <= S]
    num, den = int(rng.integers(0, 11)), 10
    mask, idx, cnt, thr = oracle_select_by_signal(x, off, num, den)
    pm, pthr = _python_select(list(x), [int(o) for o in off], num, den)
    assert list(mask) == pm
    assert np.array_equal(idx, np.flatnonzero(mask)) and cnt == sum(pm)
    assert np.allclose(thr, pthr, equal_nan=True)
    assert not np.any(mask[off[-1]:])            # positions past the last segment


def test_select_by_signal_one_segment_is_global_selection():
    rng = np.random.default_rng(9)
    e = np.round(rng.random(257) * 5, 1)          # many ties
    for num, den in [(20, 100), (1, 3), (0, 5), (5, 5)]:
        m1, i1, c1, _ = oracle_select_by_signal(e, None, num, den)
        m2, i2, c2 = oracle_select_top_fraction(e, num, den)
        assert np.array_equal(m1, m2) and np.array_equal(i1, i2) and c1 == c2


def test_select_by_signal_edges():
    x = np.array([1.0, np.nan, 3.0, np.nan, 2.0])
    m, idx, c, thr = oracle_select_by_signal(x, [0, 5], 1, 1)       # all non-NaN
    assert list(idx) == [0, 2, 4] and thr[0] == 1.0
    m, idx, c, thr = oracle_select_by_signal(x, [0, 5], 0, 1)       # none
    assert c == 0 and np.isnan(thr[0])
    m, idx, c, thr = oracle_select_by_signal(x, [0, 2, 2, 5], 1, 2)  # floor(len/2) each
    assert list(idx) == [0, 2] and np.isnan(thr[1])
    with pytest.raises(ValueError):
        oracle_select_by_signal(x, [0, 3, 2], 1, 2)


def test_select_above():
    rng = np.random.default_rng(4)
    x = rng.standard_normal(100)
    x[::7] = np.nan
    for tau in [-np.inf, -0.5, 0.0, 1.2, np.inf]:
        m, idx, c = oracle_select_above(x, tau)
        ref = [i for i in range(100) if not math.isnan(x[i]) and x[i] >= tau]
        assert list(idx) == ref and c == len(ref) and int(m.sum()) == c
    # the threshold of a pooled top-k% selection keeps exactly that selection
    y = rng.standard_normal(200)
    _, i1, _, thr = oracle_select_by_signal(y, None, 15, 100)
    _, i2, _ = oracle_select_above(y, thr[0])
    assert np.array_equal(i1, i2)


def test_validate_order_against_scalar_loops():
    """Top-K order checks of the cache ("operations": the top-K sorting)."""
    from oracle import oracle_validate_topk_order
    rng = np.random.default_rng(8)
    S, K = 60, 7
    tl = -np.sort(-rng.standard_normal((S, K)), axis=1)
    ids = np.stack([rng.choice(50, K, replace=False) for _ in range(S)])
    tl[3, 4], tl[3, 5] = tl[3, 5], tl[3, 4] + 0.5          # an increase
    tl[9, 2] = np.nan                                       # compares with nothing
    tl[11, :] = 1.0                                         # equal values are in order
    tl[12, 6] = -np.inf                                     # -inf last is in order
    tl[13, 0] = -np.inf                                     # -inf first is not
    ids[20, 5] = ids[20, 1]
    ids[21, 6] = ids[21, 0]
    got = oracle_validate_topk_order(ids, tl)
    uns = sum(any(tl[t, k] < tl[t, k + 1] for k in range(K - 1)) for t in range(S))
    dup = sum(len(set(ids[t])) < K for t in range(S))
    assert got == (uns, dup) == (2, 2)
    assert oracle_validate_topk_order(ids[:, :1], tl[:, :1]) == (0, 0)
