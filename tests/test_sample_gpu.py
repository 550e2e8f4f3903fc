"""GPU parity of the sampled teacher targets (kd_teacher_sample, through the C
ABI; RS-KD, the class axis of SE-KD3X in "Rethinking Selective Knowledge
Distillation", Method section 2) against the fp64 oracle.

The kernel forms the teacher probabilities in fp32 from fp32-accumulated
logits, so its cumulative distribution F differs from the fp64 one by a few
1e-6 (the relative error of exp of an fp32 logit, about |dz| / T with |dz| the
accumulation error of the logit). A uniform that close to a step of F may
land on the neighbouring id, so the checks are:
  - exact ids for uniforms at the middle of steps of the fp64 F whose
    probability is at least 1e-3 (the nearest step boundary is then at least
    5e-4 away, five times the bound below);
  - for random uniforms, every id v brackets its uniform u within DELTA:
    F(v-1) - DELTA <= u < F(v) + DELTA, and the ids of a row never decrease;
  - edges: u = 0 and u just below 1, one draw per row, rows spread over
    several chunks with a ragged last one, a vocabulary that is not a
    multiple of the 128-entry units, fp32 inputs, invalid uniforms rejected;
  - many rows drawing in one vocabulary tile (several slices of the draw
    pass), and the same ids whatever the chunking;
  - positions whose hidden state holds inf or NaN get -1 on every draw, the
    others are unaffected.
Inputs are synthetic teachers with hidden states of standard deviation 4 and
weights of 1/sqrt(H), which gives peaked distributions (top probability of a
few percent to tens of percent).
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

from kd_synth import bf16_bits_from_f32, f32_from_bf16_bits  # noqa: E402
from oracle import oracle_teacher_cdf, oracle_teacher_sample  # noqa: E402
from tests.kd_gpu_helpers import np_bf16_to_torch  # noqa: E402

DELTA = 1e-4        # bound on |F_kernel - F_fp64| used by the bracket checks
P_MID = 1e-3        # steps at least this tall get exact ids at their middle


@pytest.fixture(scope="module")
def kd():
    import chunked_top_kl_amd as m
    return m


def teacher(S, H, V, seed, dtype="bf16", hidden_std=4.0):
    rng = np.random.Generator(np.random.PCG64(seed))
    h = rng.standard_normal((S, H), dtype=np.float32) * np.float32(hidden_std)
    W = rng.standard_normal((V, H), dtype=np.float32) * np.float32(1.0 / np.sqrt(H))
    if dtype == "bf16":
        hb, wb = bf16_bits_from_f32(h), bf16_bits_from_f32(W)
        return f32_from_bf16_bits(hb), f32_from_bf16_bits(wb), np_bf16_to_torch(hb), np_bf16_to_torch(wb)
    return h, W, torch.from_numpy(h).cuda(), torch.from_numpy(W).cuda()


def midpoint_uniforms(P, F, N, rng):
    """N uniforms per row at the middle of steps of height >= P_MID (sorted), and
    the ids they must give."""
    S = P.shape[0]
    u = np.zeros((S, N))
    want = np.zeros((S, N), dtype=np.int32)
    for t in range(S):
        tall = np.flatnonzero(P[t] >= P_MID)
        v = np.sort(rng.choice(tall, size=N, replace=len(tall) < N))
        lo = np.where(v > 0, F[t, np.maximum(v - 1, 0)], 0.0)
        u[t] = 0.5 * (lo + F[t, v])
        want[t] = v
    return u, want


def run(kd, th, tW, u, T, chunk):
    ids = kd.kd_teacher_sample(th, tW, torch.from_numpy(np.ascontiguousarray(u)).cuda(), T=T,
                               chunk=chunk)
    torch.cuda.synchronize()
    return ids.cpu().numpy()


def check_brackets(ids, u, F):
    S, N = ids.shape
    V = F.shape[1]
    assert ids.min() >= 0 and ids.max() < V
    rows = np.arange(S)[:, None]
    hi = F[rows, ids]
    lo = np.where(ids > 0, F[rows, np.maximum(ids - 1, 0)], 0.0)
    assert np.all(lo - DELTA <= u), float(np.max(lo - u))
    assert np.all(u < hi + DELTA), float(np.max(u - hi))
    assert np.all(np.diff(ids, axis=1) >= 0)


@pytest.mark.parametrize("dtype,S,H,V,T,chunk,N", [
    ("bf16", 300, 256, 5000, 0.75, 128, 16),     # 3 chunks, ragged rows and vocabulary
    ("f32", 130, 72, 1000, 1.0, 64, 8),
    ("bf16", 77, 64, 257, 1.5, 1024, 5),          # one chunk, a one-entry last unit
    ("bf16", 50, 64, 100, 1.0, 16, 4),            # V below one 128-entry unit
])
def test_midpoints_exact(kd, dtype, S, H, V, T, chunk, N):
    h, W, th, tW = teacher(S, H, V, seed=S + V, dtype=dtype)
    P, F = oracle_teacher_cdf(h, W, T)
    u, want = midpoint_uniforms(P, F, N, np.random.default_rng(V))
    assert np.array_equal(oracle_teacher_sample(h, W, T, u), want)
    got = run(kd, th, tW, u, T, chunk)
    assert np.array_equal(got, want)


def test_random_uniforms(kd):
    S, H, V, N, T = 257, 128, 3001, 64, 1.0
    h, W, th, tW = teacher(S, H, V, seed=41)
    rng = np.random.default_rng(42)
    u = np.sort(rng.random((S, N)), axis=1)
    got = run(kd, th, tW, u, T, chunk=100)
    _, F = oracle_teacher_cdf(h, W, T)
    check_brackets(got, u, F)
    ref = oracle_teacher_sample(h, W, T, u)
    assert np.mean(got == ref) >= 0.9


def test_many_rows_drawing_in_one_tile(kd):
    # every position's distribution peaks on the same few ids, so one
    # vocabulary tile holds far more than 256 drawing rows (several slices of
    # the draw pass); the ids must not depend on the chunking (each row is
    # sampled on its own), and must match the oracle at step middles
    S, H, V, N, T = 1500, 128, 3000, 32, 1.0
    h, W, th, tW = teacher(S, H, V, seed=77)
    # a shared direction in every hidden state, and ids 1300..1303 aligned with it
    rng = np.random.Generator(np.random.PCG64(78))
    d = rng.standard_normal(H).astype(np.float32)
    d /= np.linalg.norm(d)
    h = h + np.float32(8.0) * d[None, :]
    W[1300:1304] += np.float32(1.5) * d[None, :]
    hb, wb = bf16_bits_from_f32(h), bf16_bits_from_f32(W)
    h, W = f32_from_bf16_bits(hb), f32_from_bf16_bits(wb)
    th, tW = np_bf16_to_torch(hb), np_bf16_to_torch(wb)
    P, F = oracle_teacher_cdf(h, W, T)
    assert np.median(P[:, 1300:1304].sum(axis=1)) > 0.5
    u, want = midpoint_uniforms(P, F, N, np.random.default_rng(79))
    whole = run(kd, th, tW, u, T, chunk=S)
    small = run(kd, th, tW, u, T, chunk=100)
    assert np.array_equal(whole, small)
    assert np.array_equal(whole, want)
    assert np.sum((want >= 1280) & (want < 1536)) > 4 * 256


def test_edges(kd):
    S, H, V, T = 40, 64, 700, 1.0
    h, W, th, tW = teacher(S, H, V, seed=5)
    P, F = oracle_teacher_cdf(h, W, T)
    # u = 0: the first id of positive probability. Just below 1 the fp64 answer
    # is the last id, but a last id whose probability is below the fp32
    # resolution of its 128-entry unit (about 1e-7 of the unit's mass) sits
    # inside the stated tolerance of u, so an earlier id is also correct there
    u = np.tile(np.array([0.0, 0.5, np.nextafter(1.0, 0.0)]), (S, 1))
    got = run(kd, th, tW, u, T, chunk=16)
    ref = oracle_teacher_sample(h, W, T, u)
    assert np.all(ref[:, 0] == 0) and np.all(ref[:, 2] == V - 1)
    assert np.array_equal(got[:, 0], ref[:, 0])
    check_brackets(got, u, F)
    for t in np.flatnonzero(got[:, 2] != V - 1):
        assert P[t, got[t, 2] + 1:].sum() <= DELTA
    assert np.mean(got[:, 2] == V - 1) >= 0.9
    # one draw per row
    u1 = np.random.default_rng(6).random((S, 1))
    got1 = run(kd, th, tW, u1, T, chunk=1024)
    check_brackets(got1, u1, F)


def test_rows_with_non_finite_logits(kd):
    # a position whose hidden state holds inf or NaN has no distribution: every
    # draw gives -1, and the other positions are sampled as usual
    S, H, V, N, T = 200, 64, 900, 12, 1.0
    h, W, th, tW = teacher(S, H, V, seed=31)
    bad = [3, 77, 199]
    hb = bf16_bits_from_f32(h)
    hb[3, 5] = 0x7F80          # +inf
    hb[77, 0] = 0x7FC0         # NaN
    hb[199, 63] = 0xFF80       # -inf
    th = np_bf16_to_torch(hb)
    good = np.setdiff1d(np.arange(S), bad)
    P, F = oracle_teacher_cdf(h[good], W, T)
    u = np.sort(np.random.default_rng(32).random((S, N)), axis=1)
    um, want = midpoint_uniforms(P, F, N, np.random.default_rng(33))
    u[good] = um
    got = run(kd, th, tW, u, T, chunk=64)
    assert np.all(got[bad] == -1)
    assert np.array_equal(got[good], want)


@pytest.mark.parametrize("bad", ["one", "negative", "nan", "decreasing"])
def test_invalid_uniforms_rejected(kd, bad):
    S, H, V = 8, 64, 300
    _, _, th, tW = teacher(S, H, V, seed=9)
    u = np.sort(np.random.default_rng(1).random((S, 4)), axis=1)
    if bad == "one":
        u[3, 3] = 1.0
    elif bad == "negative":
        u[0, 0] = -1e-12
    elif bad == "nan":
        u[5, 1] = np.nan
    else:
        u[6, 1], u[6, 2] = u[6, 2], u[6, 1] - 1e-3
    with pytest.raises(kd.KdError) as e:
        run(kd, th, tW, u, 1.0, 1024)
    assert e.value.code == 10


def test_full_vocabulary_sampled_rows(kd):
    """The 32K-context teacher shapes (H = 2880, V = 201088, 100 draws per
    position) over 1100 positions: two chunks of 1024, the second ragged.
    Exact ids at step middles on sampled rows (the oracle evaluates those rows
    only); elsewhere ids in range and non-decreasing."""
    S, H, V, N, T = 1100, 2880, 201088, 100, 1.0
    h, W, th, tW = teacher(S, H, V, seed=77)
    rows = np.array([0, 1, 511, 1023, 1024, 1099])
    P, F = oracle_teacher_cdf(h[rows], W, T)
    rng = np.random.default_rng(78)
    u = np.sort(rng.random((S, N)), axis=1)
    um, want = midpoint_uniforms(P, F, N, rng)
    u[rows] = um
    got = run(kd, th, tW, u, T, chunk=1024)
    assert np.array_equal(got[rows], want)
    assert got.min() >= 0 and got.max() < V
    assert np.all(np.diff(got, axis=1) >= 0)
