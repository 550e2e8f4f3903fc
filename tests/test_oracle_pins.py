"""Pins of the fp64 oracle against facts fixed by the mathematics and the pages.

None of these tests retypes the oracle's formula: each checks it against an
independent fact (finite differences, Gibbs' inequality, a library routine for
a special case, a scalar brute force, invariances), chosen so that a dropped
term, a wrong sign or index, or a transposed operand fails at least one.
"""
import math

import numpy as np
import pytest

from oracle import (oracle_dW_rows, oracle_entropy, oracle_entropy_rows, oracle_from_logits,
                    oracle_loss_grads, oracle_rows, oracle_select_top_fraction,
                    oracle_validate_topk, oracle_entropy_select_kl)

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _case(rng, S, H, V, K, distinct=True, scale=1.0):
    hid = rng.standard_normal((S, H)) * scale
    W = rng.standard_normal((V, H)) / math.sqrt(H)
    if distinct:
        ids = np.stack([rng.choice(V, size=K, replace=False) for _ in range(S)]).astype(np.int32)
    else:
        ids = rng.integers(0, V, size=(S, K)).astype(np.int32)
    tl = 3.0 - np.arange(K)[None, :] * 0.7 + 0.5 * rng.standard_normal((S, K))
    return hid, W, ids, tl


# ---------------------------------------------------------------- gradients

@pytest.mark.parametrize("T", [1.0, 2.0])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_finite_difference_gradients(T, seed):
    rng = np.random.Generator(np.random.PCG64(100 + seed))
    S, H, V, K = 6, 5, 11, 4
    hid, W, ids, tl = _case(rng, S, H, V, K, distinct=(seed != 2))
    mask = (rng.random(S) < 0.7).astype(np.uint8)
    mask[0] = 1
    g = 1.7
    r = oracle_loss_grads(hid, W, ids, tl, T=T, mask=mask, grad_loss=g)

    def f(hh, ww):
        return g * oracle_loss_grads(hh, ww, ids, tl, T=T, mask=mask)["loss"]

    eps = 1e-5
    dH = np.zeros_like(hid)
    for i in range(S):
        for j in range(H):
            a, b = hid.copy(), hid.copy()
            a[i, j] += eps
            b[i, j] -= eps
            dH[i, j] = (f(a, W) - f(b, W)) / (2 * eps)
    dW = np.zeros_like(W)
    for i in range(V):
        for j in range(H):
            a, b = W.copy(), W.copy()
            a[i, j] += eps
            b[i, j] -= eps
            dW[i, j] = (f(hid, a) - f(hid, b)) / (2 * eps)
    assert np.max(np.abs(r["dH"] - dH)) <= 1e-6 * max(1e-3, np.max(np.abs(dH)))
    assert np.max(np.abs(r["dW"] - dW)) <= 1e-6 * max(1e-3, np.max(np.abs(dW)))


# ---------------------------------------------------------------- loss value

@pytest.mark.parametrize("seed", range(5))
def test_kl_nonnegative(seed):
    # Gibbs: sum_k p_k log(p_k/q_k) >= -log sum_k q_k >= 0.
    rng = np.random.Generator(np.random.PCG64(200 + seed))
    Z = rng.standard_normal((40, 30)) * 3
    ids = np.stack([rng.choice(30, size=6, replace=False) for _ in range(40)])
    tl = rng.standard_normal((40, 6)) * 2
    for T in (0.5, 1.0, 3.0):
        r = oracle_from_logits(Z, ids, tl, T)
        assert np.all(r["kl_rows"] >= -1e-13)
        assert r["loss"] >= 0.0


def test_kl_zero_when_student_equals_teacher():
    rng = np.random.Generator(np.random.PCG64(7))
    S, V, K = 9, 20, 5
    ids = np.stack([rng.choice(V, size=K, replace=False) for _ in range(S)])
    tl = rng.standard_normal((S, K)) * 2
    Z = np.full((S, V), -np.inf)
    shift = rng.standard_normal(S) * 10
    for t in range(S):
        Z[t, ids[t]] = tl[t] + shift[t]
    for T in (1.0, 2.5):
        r = oracle_from_logits(Z, ids, tl, T)
        assert abs(r["loss"]) <= 1e-12
        assert np.max(np.abs(r["kl_rows"])) <= 1e-12
        assert np.max(np.abs(r["dZ"])) <= 1e-12


def test_kl_positive_when_student_differs():
    # dropping a term of the KL (e.g. the teacher entropy) would make this fail
    Z = np.array([[0.0, 0.0, 0.0, 0.0]])
    ids = np.array([[0, 1]])
    tl = np.array([[0.0, 0.0]])
    r = oracle_from_logits(Z, ids, tl, 1.0)
    # p = (1/2, 1/2) on ids 0,1; q uniform 1/4: KL = log 2
    assert abs(r["loss"] - math.log(2.0)) <= 1e-15


# ---------------------------------------------------------------- chunking

@pytest.mark.parametrize("C", [1, 7, 32, 50])
def test_dense_equals_chunked(C):
    rng = np.random.Generator(np.random.PCG64(300))
    S, H, V, K = 50, 8, 40, 6
    hid, W, ids, tl = _case(rng, S, H, V, K)
    mask = (rng.random(S) < 0.6).astype(np.uint8)
    d = oracle_loss_grads(hid, W, ids, tl, T=1.5, mask=mask)
    c = oracle_loss_grads(hid, W, ids, tl, T=1.5, mask=mask, chunk=C)
    assert d["N"] == c["N"]
    assert abs(d["loss"] - c["loss"]) <= 1e-12 * abs(d["loss"])
    assert np.allclose(d["dH"], c["dH"], rtol=0, atol=1e-12 * np.max(np.abs(d["dH"])))
    assert np.allclose(d["dW"], c["dW"], rtol=0, atol=1e-12 * np.max(np.abs(d["dW"])))
    assert np.allclose(d["lse"], c["lse"], rtol=1e-13, atol=0)


def test_rows_match_full():
    rng = np.random.Generator(np.random.PCG64(301))
    S, H, V, K = 20, 6, 25, 4
    hid, W, ids, tl = _case(rng, S, H, V, K)
    full = oracle_loss_grads(hid, W, ids, tl, T=2.0)
    rows = [3, 11, 19]
    r = oracle_rows(hid[rows], W, ids[rows], tl[rows], 2.0, N=S)
    assert np.allclose(r["kl_rows"], full["kl_rows"][rows], rtol=1e-13, atol=0)
    assert np.allclose(r["lse"], full["lse"][rows], rtol=1e-13, atol=0)
    assert np.allclose(r["dH"], full["dH"][rows], rtol=1e-12, atol=1e-18)


# ---------------------------------------------------------------- reductions to textbook routines

@pytest.mark.parametrize("T", [1.0, 2.0])
def test_k1_is_cross_entropy(T):
    torch = pytest.importorskip("torch")
    rng = np.random.Generator(np.random.PCG64(400))
    S, V = 30, 17
    Z = rng.standard_normal((S, V)) * 2
    ids = rng.integers(0, V, size=(S, 1))
    tl = rng.standard_normal((S, 1))
    r = oracle_from_logits(Z, ids, tl, T)
    ce = torch.nn.functional.cross_entropy(torch.from_numpy(Z / T), torch.from_numpy(ids[:, 0]).long())
    assert abs(r["loss"] - float(ce)) <= 1e-12 * abs(float(ce))


@pytest.mark.parametrize("T", [1.0, 0.7])
def test_k_equals_v_is_full_kl(T):
    torch = pytest.importorskip("torch")
    rng = np.random.Generator(np.random.PCG64(401))
    S, V = 12, 9
    Z = rng.standard_normal((S, V)) * 2
    ids = np.stack([rng.permutation(V) for _ in range(S)])
    tl = rng.standard_normal((S, V)) * 2
    r = oracle_from_logits(Z, ids, tl, T)
    # teacher logits in vocabulary order
    Lv = np.zeros((S, V))
    for t in range(S):
        Lv[t, ids[t]] = tl[t]
    inp = torch.log_softmax(torch.from_numpy(Z / T), dim=1)
    tgt = torch.log_softmax(torch.from_numpy(Lv / T), dim=1)
    ref = torch.nn.functional.kl_div(inp, tgt, reduction="batchmean", log_target=True)
    assert abs(r["loss"] - float(ref)) <= 1e-12 * abs(float(ref))


def test_w_zero_closed_form():
    rng = np.random.Generator(np.random.PCG64(402))
    S, H, V, K, T = 10, 4, 13, 3, 1.5
    hid = rng.standard_normal((S, H))
    W = np.zeros((V, H))
    ids = np.stack([rng.choice(V, size=K, replace=False) for _ in range(S)])
    tl = rng.standard_normal((S, K))
    r = oracle_loss_grads(hid, W, ids, tl, T=T)
    # uniform student: KL_t = log V - H(p_t)
    exp_loss = 0.0
    Gx = np.zeros((S, V))
    for t in range(S):
        e = [math.exp(x / T) for x in tl[t]]
        z = math.fsum(e)
        p = [x / z for x in e]
        exp_loss += math.log(V) + math.fsum(pi * math.log(pi) for pi in p)
        for k in range(K):
            Gx[t, ids[t, k]] -= p[k]
    exp_loss /= S
    Gx = (Gx + 1.0 / V) / (T * S)
    assert abs(r["loss"] - exp_loss) <= 1e-12
    assert np.all(r["dH"] == 0.0)
    assert np.max(np.abs(r["dW"] - Gx.T @ hid)) <= 1e-12


# ---------------------------------------------------------------- identities

def test_shift_temperature_permutation_identities():
    rng = np.random.Generator(np.random.PCG64(500))
    S, V, K = 15, 21, 5
    Z = rng.standard_normal((S, V)) * 2
    ids = np.stack([rng.choice(V, size=K, replace=False) for _ in range(S)])
    tl = rng.standard_normal((S, K)) * 2
    base = oracle_from_logits(Z, ids, tl, 1.7)["loss"]
    c = rng.standard_normal(S)[:, None] * 5
    d = rng.standard_normal(S)[:, None] * 5
    assert abs(oracle_from_logits(Z + c, ids, tl, 1.7)["loss"] - base) <= 1e-12 * base
    assert abs(oracle_from_logits(Z, ids, tl + d, 1.7)["loss"] - base) <= 1e-12 * base
    assert abs(oracle_from_logits(Z / 1.7, ids, tl / 1.7, 1.0)["loss"] - base) <= 1e-12 * base
    perm = np.stack([rng.permutation(K) for _ in range(S)])
    ids_p = np.take_along_axis(ids, perm, axis=1)
    tl_p = np.take_along_axis(tl, perm, axis=1)
    assert abs(oracle_from_logits(Z, ids_p, tl_p, 1.7)["loss"] - base) <= 1e-12 * base


def test_gradient_invariants():
    rng = np.random.Generator(np.random.PCG64(501))
    S, H, V, K = 16, 7, 23, 4
    hid, W, ids, tl = _case(rng, S, H, V, K)
    mask = np.zeros(S, dtype=np.uint8)
    mask[::3] = 1
    r = oracle_loss_grads(hid, W, ids, tl, T=1.3, mask=mask)
    scale = np.max(np.abs(r["dW"]))
    assert np.max(np.abs(r["dW"].sum(axis=0))) <= 1e-12 * max(scale, 1e-30) * V
    assert np.all(r["dH"][mask == 0] == 0.0)
    assert np.any(r["dH"][mask == 1] != 0.0)


def test_duplicates_add_probabilities():
    rng = np.random.Generator(np.random.PCG64(502))
    V, T = 8, 2.0
    Z = rng.standard_normal((1, V))
    a, b = 1.3, -0.4
    dup = oracle_from_logits(Z, np.array([[3, 3, 5]]), np.array([[a, b, 0.2]]), T)
    merged_logit = T * math.log(math.exp(a / T) + math.exp(b / T))
    one = oracle_from_logits(Z, np.array([[3, 5]]), np.array([[merged_logit, 0.2]]), T)
    assert abs(dup["loss"] - one["loss"]) <= 1e-13
    assert np.max(np.abs(dup["dZ"] - one["dZ"])) <= 1e-14


def test_neg_inf_teacher_entries_and_missing_rows():
    rng = np.random.Generator(np.random.PCG64(503))
    V = 10
    Z = rng.standard_normal((3, V))
    ids = np.array([[1, 2, 3], [4, 5, 6], [7, 8, 9]])
    tl = np.array([[0.5, -np.inf, 0.1], [-np.inf, -np.inf, -np.inf], [1.0, 2.0, 3.0]])
    r = oracle_from_logits(Z, ids, tl, 1.0)
    assert r["N"] == 2 and not r["valid"][1]
    # padding entry behaves as if absent
    r0 = oracle_from_logits(Z[:1], np.array([[1, 3]]), np.array([[0.5, 0.1]]), 1.0)
    assert abs(r["kl_rows"][0] - r0["kl_rows"][0]) <= 1e-14
    # missing row excluded like a masked row
    rm = oracle_from_logits(Z[[0, 2]], ids[[0, 2]], tl[[0, 2]], 1.0)
    assert abs(r["loss"] - rm["loss"]) <= 1e-14
    assert np.all(r["dZ"][1] == 0.0)


def test_empty_mask_gives_zero():
    rng = np.random.Generator(np.random.PCG64(504))
    hid, W, ids, tl = _case(rng, 5, 3, 9, 2)
    r = oracle_loss_grads(hid, W, ids, tl, mask=np.zeros(5, dtype=np.uint8), chunk=2)
    assert r["loss"] == 0.0 and r["N"] == 0
    assert np.all(r["dH"] == 0.0) and np.all(r["dW"] == 0.0)


# ---------------------------------------------------------------- brute force

def _brute(hid, W, ids, tl, T, mask, g):
    """Scalar loops with math.fsum; independent of the vectorised oracle."""
    S, H = len(hid), len(hid[0])
    V = len(W)
    z = [[math.fsum(hid[t][h] * W[v][h] for h in range(H)) for v in range(V)] for t in range(S)]
    kl, G = [], []
    valid = [bool(mask[t]) for t in range(S)]
    N = sum(valid)
    for t in range(S):
        mx = max(x / T for x in z[t])
        den = math.fsum(math.exp(x / T - mx) for x in z[t])
        q = [math.exp(x / T - mx) / den for x in z[t]]
        tm = max(x / T for x in tl[t])
        tden = math.fsum(math.exp(x / T - tm) for x in tl[t])
        p = [0.0] * V
        for k in range(len(ids[t])):
            p[ids[t][k]] += math.exp(tl[t][k] / T - tm) / tden
        kl.append(math.fsum(p[v] * math.log(p[v] / q[v]) for v in range(V) if p[v] > 0))
        G.append([(g * (q[v] - p[v]) / (T * N)) if valid[t] else 0.0 for v in range(V)])
    loss = math.fsum(kl[t] for t in range(S) if valid[t]) / N
    dH = [[math.fsum(G[t][v] * W[v][h] for v in range(V)) for h in range(H)] for t in range(S)]
    dW = [[math.fsum(G[t][v] * hid[t][h] for t in range(S)) for h in range(H)] for v in range(V)]
    return loss, np.array(dH), np.array(dW)


@pytest.mark.parametrize("seed", [0, 1])
def test_brute_force_scalar_loops(seed):
    rng = np.random.Generator(np.random.PCG64(600 + seed))
    S, H, V, K = 4, 3, 7, 3
    hid, W, ids, tl = _case(rng, S, H, V, K, distinct=(seed == 0))
    mask = np.array([1, 0, 1, 1], dtype=np.uint8)
    T, g = 1.3, 0.8
    loss, dH, dW = _brute(hid.tolist(), W.tolist(), ids.tolist(), tl.tolist(), T, mask, g)
    r = oracle_loss_grads(hid, W, ids, tl, T=T, mask=mask, grad_loss=g)
    assert abs(r["loss"] - loss) <= 1e-13 * abs(loss)
    assert np.max(np.abs(r["dH"] - dH)) <= 1e-13 * np.max(np.abs(dH))
    assert np.max(np.abs(r["dW"] - dW)) <= 1e-13 * np.max(np.abs(dW))


# ---------------------------------------------------------------- entropy and selection

def test_entropy_special_cases():
    scipy_stats = pytest.importorskip("scipy.stats")
    V = 50
    assert abs(oracle_entropy_rows(np.zeros((1, V)))[0] - math.log(V)) <= 1e-13
    onehot = np.full((1, V), -200.0)
    onehot[0, 3] = 200.0
    assert abs(oracle_entropy_rows(onehot)[0]) <= 1e-12
    rng = np.random.Generator(np.random.PCG64(700))
    Z = rng.standard_normal((6, V)) * 2
    q = np.exp(Z - Z.max(axis=1, keepdims=True))
    q /= q.sum(axis=1, keepdims=True)
    ref = scipy_stats.entropy(q, axis=1)
    assert np.max(np.abs(oracle_entropy_rows(Z) - ref)) <= 1e-12


def test_entropy_chunk_invariance():
    rng = np.random.Generator(np.random.PCG64(701))
    hid = rng.standard_normal((20, 6))
    W = rng.standard_normal((30, 6))
    a = oracle_entropy(hid, W)
    b = oracle_entropy(hid, W, chunk=3)
    assert np.max(np.abs(a - b)) <= 1e-13


@pytest.mark.parametrize("S,num,den", [(100, 20, 100), (37, 1, 3), (5, 0, 1), (8, 1, 1), (33, 20, 100)])
def test_selection_against_python_sort(S, num, den):
    rng = np.random.Generator(np.random.PCG64(702 + S))
    e = np.round(rng.random(S) * 4, 1)  # many exact ties
    mask, idx, k = oracle_select_top_fraction(e, num, den)
    kk = num * S // den
    ref = sorted(sorted(range(S), key=lambda t: (-float(e[t]), t))[:kk])
    assert k == kk
    assert idx.tolist() == ref
    assert mask.sum() == kk and all(mask[t] == 1 for t in ref)


def test_entropy_select_kl_uses_selected_rows():
    rng = np.random.Generator(np.random.PCG64(703))
    hid, W, ids, tl = _case(rng, 25, 5, 30, 3, scale=2.0)
    r = oracle_entropy_select_kl(hid, W, ids, tl, num=20, den=100)
    assert r["count"] == 5 and r["N"] == 5
    assert np.all(r["dH"][r["mask"] == 0] == 0.0)
    ent = oracle_entropy(hid, W)
    assert set(r["idx"].tolist()) == set(np.argsort(-ent, kind="stable")[:5].tolist())


def test_validate_counts():
    ids = np.array([[0, 5, 9], [10, -1, 3], [2, 2, 2]])
    tl = np.array([[1.0, 2.0, 3.0], [-np.inf, -np.inf, -np.inf], [np.nan, np.inf, 0.0]])
    assert oracle_validate_topk(ids, tl, 10) == (2, 1, 2)


@pytest.mark.parametrize("T", [1.0, 2.0])
def test_dW_rows_match_dense_definition(T):
    # dW at sampled vocabulary rows, from every row's lse, equals the rows of
    # the dense oracle's dW; with a mask, duplicate ids, -inf teacher entries
    # and an all -inf (missing) row
    rng = np.random.default_rng(31)
    S, H, V, K = 9, 5, 13, 4
    hidden = rng.standard_normal((S, H))
    W = rng.standard_normal((V, H)) / np.sqrt(H)
    ids = np.stack([rng.choice(V, K, replace=False) for _ in range(S)])
    ids[2, 1] = ids[2, 0]                       # duplicate id
    tl = np.sort(rng.standard_normal((S, K)), axis=1)[:, ::-1].copy()
    tl[4, 3] = -np.inf                          # one -inf entry
    tl[6, :] = -np.inf                          # a missing row
    mask = np.ones(S, dtype=bool)
    mask[1] = False
    ref = oracle_loss_grads(hidden, W, ids, tl, T=T, mask=mask, grad_loss=0.7)
    vocab_rows = np.array([0, 3, int(ids[2, 0]), 12])
    got = oracle_dW_rows(hidden, W, ids, tl, T, ref["lse"], ref["valid"], vocab_rows, grad_loss=0.7)
    assert np.allclose(got, ref["dW"][vocab_rows], rtol=1e-12, atol=1e-14)


def test_rows_forward_only_matches():
    rng = np.random.default_rng(32)
    S, H, V, K = 6, 4, 11, 3
    hidden = rng.standard_normal((S, H))
    W = rng.standard_normal((V, H))
    ids = np.stack([rng.choice(V, K, replace=False) for _ in range(S)])
    tl = rng.standard_normal((S, K))
    ref = oracle_loss_grads(hidden, W, ids, tl, T=1.5)
    got = oracle_rows(hidden, W, ids, tl, 1.5, S, grads=False)
    assert "dH" not in got
    assert np.allclose(got["kl_rows"], ref["kl_rows"], rtol=1e-12, atol=1e-14)
    assert np.allclose(got["lse"], ref["lse"], rtol=1e-12, atol=1e-14)
