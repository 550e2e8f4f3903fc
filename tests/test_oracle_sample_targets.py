"""Pins of the sampled sparse-target oracle (RS-KD, the class axis of SE-KD3X in
"Rethinking Selective Knowledge Distillation", Method section 2): a scalar
inverse-transform loop, a distribution with exact probabilities and uniforms
placed on and around its cumulative steps, monotonicity in u, the clamp at the
top, and the frequencies of many draws against the probabilities."""
import math

import numpy as np

from oracle import oracle_teacher_sample


def test_scalar_inverse_transform():
    rng = np.random.default_rng(5)
    S, H, V, N = 4, 6, 9, 7
    h = rng.standard_normal((S, H))
    W = rng.standard_normal((V, H))
    T = 1.7
    u = rng.random((S, N))
    ids = oracle_teacher_sample(h, W, T, u)
    for t in range(S):
        z = [sum(h[t, k] * W[v, k] for k in range(H)) / T for v in range(V)]
        m = max(z)
        e = [math.exp(x - m) for x in z]
        tot = math.fsum(e)
        for n in range(N):
            acc, pick = 0.0, None
            for v in range(V):
                acc += e[v] / tot
                if acc > u[t, n]:
                    pick = v
                    break
            assert ids[t, n] == (pick if pick is not None else V - 1)


def test_exact_probabilities_and_steps():
    # logits ln(1), ln(2), ln(5) (H = 1, hidden = 1, T = 1): p = 1/8, 2/8, 5/8,
    # so F steps at 0.125 and 0.375 (to within the rounding of exp and log);
    # uniforms 1e-9 either side of each step
    W = np.log(np.array([[1.0], [2.0], [5.0]]))
    h = np.ones((1, 1))
    d = 1e-9
    u = np.array([[0.0, 0.125 - d, 0.125 + d, 0.375 - d, 0.375 + d, 1.0 - d]])
    ids = oracle_teacher_sample(h, W, 1.0, u)
    assert list(ids[0]) == [0, 0, 1, 1, 2, 2]


def test_monotone_and_clamped():
    rng = np.random.default_rng(6)
    h = rng.standard_normal((3, 5))
    W = rng.standard_normal((40, 5))
    u = np.sort(rng.random((3, 50)), axis=1)
    ids = oracle_teacher_sample(h, W, 1.0, u)
    assert np.all(np.diff(ids, axis=1) >= 0)
    top = oracle_teacher_sample(h, W, 1.0, np.full((3, 1), np.nextafter(1.0, 0.0)))
    assert np.all(top <= 39)


def test_frequencies_follow_probabilities():
    rng = np.random.default_rng(7)
    H, V, N = 4, 12, 200000
    h = rng.standard_normal((1, H))
    W = rng.standard_normal((V, H))
    T = 0.9
    ids = oracle_teacher_sample(h, W, T, rng.random((1, N)))
    z = (h @ W.T)[0] / T
    p = np.exp(z - z.max())
    p /= p.sum()
    freq = np.bincount(ids[0], minlength=V) / N
    # binomial standard error; 5 sigma
    assert np.all(np.abs(freq - p) <= 5 * np.sqrt(p * (1 - p) / N) + 1e-12)


def test_cdf_matches_scalar_softmax():
    from oracle import oracle_teacher_cdf
    rng = np.random.default_rng(12)
    h = rng.standard_normal((3, 4))
    W = rng.standard_normal((11, 4))
    T = 0.6
    P, F = oracle_teacher_cdf(h, W, T)
    for t in range(3):
        z = [sum(h[t, k] * W[v, k] for k in range(4)) / T for v in range(11)]
        e = [math.exp(x - max(z)) for x in z]
        tot = math.fsum(e)
        run = 0.0
        for v in range(11):
            run += e[v] / tot
            assert abs(P[t, v] - e[v] / tot) <= 1e-15
            assert abs(F[t, v] - run) <= 1e-14
