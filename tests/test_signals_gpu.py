"""GPU parity of the position signals and selection policies
("Rethinking Selective Knowledge Distillation", Method section 1) against the
fp64 oracle, through the C ABI.

Signals (kd_position_signals): entropy and cross-entropy at T = 1 share the
entropy sweep's fp32 tile sums, so both are held to the entropy bound (2e-5
nats, plus the fp64 dot product's rounding for ce: 5e-5 in all); the teacher
uncertainty is computed in fp64 from the same stored values as the oracle
(1e-12). Cases: ragged bf16 shapes with labels out of range, labels among the
teacher ids (held twice), a missing teacher row; probabilities; fp32 inputs.

Selection (kd_select_by_signal, kd_select_above): bit for bit on the same
seeded signals (ties, NaN, infinities, signed zeros), random segments with
empty ones and positions outside every segment, one long segment, the pooled
threshold reproducing its selection, malformed offsets rejected.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

from kd_synth import make_problem  # noqa: E402
from oracle import (oracle_position_signals, oracle_select_above,  # noqa: E402
                    oracle_select_by_signal)
from tests.kd_gpu_helpers import to_device  # noqa: E402

ENT_TOL = 2e-5
CE_TOL = 5e-5
TU_TOL = 1e-12


@pytest.fixture(scope="module")
def kd():
    import chunked_top_kl_amd as m
    return m


def _labels(p, seed):
    rng = np.random.default_rng(seed)
    y = rng.integers(0, p.V, size=p.S).astype(np.int32)
    y[::17] = -100                           # no label
    y[5::23] = p.V                           # out of range
    y[1::11] = p.ids[1::11, 3]               # a label the teacher row holds
    return y


def _check_signals(kd, p, labels, probs=False):
    hidden, W, ids, tl = to_device(p)
    lab = torch.from_numpy(labels).cuda()
    got = kd.kd_position_signals(hidden, W, ids, tl, lab, T=p.T, teacher_probs=probs)
    torch.cuda.synchronize()
    ref = oracle_position_signals(p.hidden, p.W, p.ids, p.tlogits, labels, T=p.T, probs=probs,
                                  chunk=256)
    e = got["entropy"].cpu().numpy()
    assert np.max(np.abs(e - ref["entropy"])) <= ENT_TOL
    for name, tol in (("ce", CE_TOL), ("teacher_unc", TU_TOL)):
        g, r = got[name].cpu().numpy(), ref[name]
        assert np.array_equal(np.isnan(g), np.isnan(r)), name
        ok = ~np.isnan(r)
        err = float(np.max(np.abs(g[ok] - r[ok]))) if ok.any() else 0.0
        print(f"{name} max abs err {err:.3e}")
        assert err <= tol, name
    return got, ref


def test_signals_ragged_bf16(kd):
    p = make_problem(700, 264, 3001, 16, T=0.75, seed=301)   # T exact in the ABI's float
    p.tlogits[7] = -np.inf                   # a missing teacher row (fp32 copy) ...
    p.tl_bits[7] = 0xFF80                    # ... and its bf16 storage
    p.ids[2, 5] = p.ids[2, 1]                # a duplicate id ...
    labels = _labels(p, 302)
    labels[2] = p.ids[2, 1]                  # ... that is the label
    got, ref = _check_signals(kd, p, labels)
    assert np.isnan(got["teacher_unc"][7].item()) and np.isfinite(got["ce"][7].item())
    assert np.isnan(got["ce"][0].item())     # label -100


def test_signals_probabilities(kd):
    p = make_problem(300, 128, 2048, 8, T=1.5, seed=303, tl_dtype="f32")
    rng = np.random.default_rng(304)
    p.tlogits[:] = rng.random(p.tlogits.shape).astype(np.float32)
    p.tlogits[3, 2] = 0.0
    p.tlogits[9, 0] = -0.25                   # malformed row: takes no part
    _check_signals(kd, p, _labels(p, 305), probs=True)


def test_signals_fp32_tiny(kd):
    p = make_problem(128, 64, 1000, 10, T=1.0, hw_dtype="f32", tl_dtype="f32", seed=306)
    _check_signals(kd, p, _labels(p, 307))


def test_signals_subsets(kd):
    # only the teacher uncertainty: no projection sweep; only the entropy
    p = make_problem(200, 64, 777, 6, seed=308)
    hidden, W, ids, tl = to_device(p)
    labels = _labels(p, 309)
    lab = torch.from_numpy(labels).cuda()
    ref = oracle_position_signals(p.hidden, p.W, p.ids, p.tlogits, labels, T=p.T)
    kd.kd_profile_reset()
    kd.kd_profile_enable(True)
    got = kd.kd_position_signals(hidden, W, ids, tl, lab, entropy=False)
    torch.cuda.synchronize()
    kd.kd_profile_enable(False)
    steps = kd.kd_profile_read()
    kd.kd_profile_reset()
    assert got["entropy"] is None
    g = got["teacher_unc"].cpu().numpy()
    assert np.allclose(g, ref["teacher_unc"], atol=TU_TOL, rtol=0, equal_nan=True)
    got = kd.kd_position_signals(hidden, W)
    assert got["ce"] is None and got["teacher_unc"] is None
    assert np.max(np.abs(got["entropy"].cpu().numpy() - ref["entropy"])) <= ENT_TOL
    assert "position_signals" in steps


def _signal(S, seed):
    rng = np.random.default_rng(seed)
    x = rng.choice([-1.5, 0.0, -0.0, 0.25, 2.0, 7.0, np.inf, -np.inf, np.nan], size=S)
    return np.where(rng.random(S) < 0.6, np.round(rng.standard_normal(S), 2), x)


def _select(kd, x, off, num, den):
    tx = torch.from_numpy(x).cuda()
    toff = None if off is None else torch.from_numpy(np.asarray(off, dtype=np.int64)).cuda()
    mask, idx, cnt, thr = kd.kd_select_by_signal(tx, toff, num, den)
    torch.cuda.synchronize()
    rmask, ridx, rc, rthr = oracle_select_by_signal(x, off, num, den)
    assert cnt == rc
    assert np.array_equal(mask.cpu().numpy(), rmask)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    t = thr.cpu().numpy()
    assert np.array_equal(np.isnan(t), np.isnan(rthr)) and np.all(t[~np.isnan(t)] == rthr[~np.isnan(rthr)])
    return rmask, rthr


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_select_segments_match_oracle(kd, seed):
    rng = np.random.default_rng(400 + seed)
    S = 5000
    x = _signal(S, 410 + seed)
    lens = rng.integers(0, 700, size=14)
    lens[3] = 0
    off = np.concatenate([[0], np.cumsum(lens)])
    off = off[off <= S - 37]                  # positions past the last segment
    for num, den in [(20, 100), (1, 3), (0, 7), (7, 7), (99, 100)]:
        _select(kd, x, off, num, den)


def test_select_one_long_segment(kd):
    x = _signal(70001, 420)
    x[1000:3000] = 4.0                        # a long run of ties
    for num, den in [(20, 100), (1, 70001), (70000, 70001)]:
        _select(kd, x, None, num, den)


def test_select_all_nan_and_tiny_segments(kd):
    x = np.full(64, np.nan)
    x[10] = 1.0
    _select(kd, x, [0, 10, 11, 12, 64], 1, 1)
    _select(kd, np.arange(40, dtype=np.float64)[::-1].copy(), np.arange(41), 1, 1)


def test_threshold_policy(kd):
    x = _signal(3000, 430)
    tx = torch.from_numpy(x).cuda()
    for tau in [-np.inf, -0.5, 0.0, 1.25, np.inf]:
        mask, idx, cnt = kd.kd_select_above(tx, tau)
        rmask, ridx, rc = oracle_select_above(x, tau)
        assert cnt == rc and np.array_equal(mask.cpu().numpy(), rmask)
        assert np.array_equal(idx.cpu().numpy(), ridx)
    # the threshold of a pooled selection, applied globally, keeps the same
    # positions (no ties at the threshold in this signal)
    y = np.random.default_rng(431).standard_normal(4000)
    ty = torch.from_numpy(y).cuda()
    _, i1, _, thr = kd.kd_select_by_signal(ty, None, 15, 100)
    _, i2, _ = kd.kd_select_above(ty, float(thr[0].item()))
    assert torch.equal(i1, i2)


def test_select_rejects_bad_offsets(kd):
    x = torch.zeros(10, dtype=torch.float64, device="cuda")
    for off in ([0, 5, 3], [0, 11], [-1, 4]):
        with pytest.raises(kd.KdError):
            kd.kd_select_by_signal(x, torch.tensor(off, dtype=torch.int64, device="cuda"), 1, 2)


def test_signals_and_selection_full_size(kd):
    """The entropy-selective workload's shapes (S=32768 H=2048 V=151936 K=100,
    T=1): signals of every position on the GPU, the oracle at sampled rows;
    per-sequence selection over 32 sequences of random lengths covering all
    positions, bit for bit on a seeded signal."""
    S, H, V, K = 32768, 2048, 151936, 100
    p = make_problem(S, H, V, K, T=1.0, chunk=1024, seed=1005)
    hidden, W, ids, tl = to_device(p)
    labels = _labels(p, 440)
    got = kd.kd_position_signals(hidden, W, ids, tl, torch.from_numpy(labels).cuda(), T=p.T)
    torch.cuda.synchronize()
    rng = np.random.default_rng(441)
    rows = np.unique(np.concatenate([[0, S - 1], rng.choice(S, 94, replace=False)]))
    ref = oracle_position_signals(p.hidden[rows], p.W, p.ids[rows], p.tlogits[rows], labels[rows],
                                  T=p.T, chunk=32)
    assert np.max(np.abs(got["entropy"].cpu().numpy()[rows] - ref["entropy"])) <= ENT_TOL
    for name, tol in (("ce", CE_TOL), ("teacher_unc", TU_TOL)):
        g, r = got[name].cpu().numpy()[rows], ref[name]
        assert np.array_equal(np.isnan(g), np.isnan(r)), name
        ok = ~np.isnan(r)
        assert float(np.max(np.abs(g[ok] - r[ok]))) <= tol, name
    x = np.round(rng.standard_normal(S), 3)              # ties at 1e-3 resolution
    cuts = np.sort(rng.choice(np.arange(1, S), 31, replace=False))
    off = np.concatenate([[0], cuts, [S]])
    _select(kd, x, off, 20, 100)


@pytest.mark.parametrize("case", ["spread", "crowded"])
def test_per_sequence_entropy_selection(kd, case):
    """SE-KD within each sequence (kd_select_top_fraction_segments): the kept set
    equals the one fp64 entropies give, bit for bit. Crowded entropies (closer
    than the sweep's error bound) make the fp64 band refinement decide; the
    test asserts that it ran."""
    from oracle import oracle_entropy
    rng = np.random.default_rng(450)
    lens = rng.integers(1, 200, size=24)
    lens[5] = 0
    off = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    S = int(off[-1]) + 13                               # positions past the last segment
    p = make_problem(S, 128, 4001, 4, seed=451, hidden_std=(0.05 if case == "crowded" else 1.5))
    hidden, W, _, _ = to_device(p)
    ent = kd.kd_student_entropy(hidden, W)
    toff = torch.from_numpy(off).cuda()
    kd.kd_profile_reset()
    kd.kd_profile_enable(True)
    mask, idx, cnt = kd.kd_select_top_fraction_segments(ent, toff, hidden, W, 30, 100)
    torch.cuda.synchronize()
    kd.kd_profile_enable(False)
    steps = kd.kd_profile_read()
    kd.kd_profile_reset()
    ref_e = oracle_entropy(p.hidden, p.W, chunk=500)
    rmask, ridx, rc, _ = oracle_select_by_signal(ref_e, off, 30, 100)
    assert cnt == rc
    assert np.array_equal(mask.cpu().numpy(), rmask)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    if case == "crowded":
        assert "select_refine_fp64" in steps


def test_per_sequence_selection_with_less_accurate_entropies(kd):
    """Per-sequence SE-KD on entropies given with errors of up to 1e-4 nats,
    five times the band's least bound: the error measured on the probe
    positions widens every segment's band, so the kept set is still the fp64
    oracle's (a band of +-4e-5 would leave positions on the wrong side)."""
    from oracle import oracle_entropy
    S = 3000
    off = (np.arange(7, dtype=np.int64) * S) // 6
    p = make_problem(S, 128, 4001, 4, seed=21, hidden_std=0.2)
    hidden, W, _, _ = to_device(p)
    ent = kd.kd_student_entropy(hidden, W)
    noise = np.random.default_rng(22).uniform(-1e-4, 1e-4, size=S)
    noisy = ent + torch.from_numpy(noise).cuda()
    mask, idx, cnt = kd.kd_select_top_fraction_segments(noisy, torch.from_numpy(off).cuda(), hidden,
                                                        W, 20, 100)
    torch.cuda.synchronize()
    ref_e = oracle_entropy(p.hidden, p.W, chunk=500)
    rmask, ridx, rc, _ = oracle_select_by_signal(ref_e, off, 20, 100)
    assert cnt == rc
    assert np.array_equal(mask.cpu().numpy(), rmask)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    _, nidx, _, _ = oracle_select_by_signal(ref_e + noise, off, 20, 100)
    assert not np.array_equal(nidx, ridx)


def test_per_sequence_selection_band_above_65536_positions(kd):
    """Per-sequence SE-KD where the straddling bands of all segments hold more
    than 65536 positions in all: every one is refined in fp64 (in pieces) and
    the kept set equals the fp64 oracle's bit for bit."""
    from oracle import oracle_entropy
    S = 80000
    off = (np.arange(41, dtype=np.int64) * S) // 40
    p = make_problem(S, 64, 2000, 4, seed=452, hidden_std=0.01)
    hidden, W, _, _ = to_device(p)
    ent = kd.kd_student_entropy(hidden, W)
    kd.kd_profile_reset()
    kd.kd_profile_enable(True)
    mask, idx, cnt = kd.kd_select_top_fraction_segments(ent, torch.from_numpy(off).cuda(), hidden, W,
                                                        20, 100)
    torch.cuda.synchronize()
    kd.kd_profile_enable(False)
    steps = kd.kd_profile_read()
    kd.kd_profile_reset()
    # a refinement launch and an entropy launch per piece of 4096 positions
    # (bf16 rows): more than 65536 positions were refined
    assert steps["select_refine_fp64"][0] > 2 * (65536 // 4096)
    ref_e = oracle_entropy(p.hidden, p.W, chunk=4000)
    rmask, ridx, rc, _ = oracle_select_by_signal(ref_e, off, 20, 100)
    assert cnt == rc
    assert np.array_equal(mask.cpu().numpy(), rmask)
    assert np.array_equal(idx.cpu().numpy(), ridx)


@pytest.mark.parametrize("K", [1, 100, 700])
def test_validate_order(kd, K):
    """Cache top-K order checks (kd_validate_topk_order) against the oracle:
    planted increases, NaN, -inf first, and duplicate ids; bf16 and fp32."""
    from oracle import oracle_validate_topk_order
    p = make_problem(500, 8, 50000, K, seed=460)
    rng = np.random.default_rng(461)
    ids = p.ids.copy()
    tl = p.tlogits.copy()
    if K > 1:
        for t in rng.choice(500, 40, replace=False):
            k = int(rng.integers(0, K - 1))
            tl[t, k], tl[t, k + 1] = tl[t, k + 1], tl[t, k] + np.float32(1.0)
        tl[7, K // 2] = np.nan
        tl[8, 0] = -np.inf
        for t in rng.choice(500, 25, replace=False):
            a, b = rng.choice(K, 2, replace=False)
            ids[t, a] = ids[t, b]
    for f32 in (False, True):
        if f32:
            tlt = torch.from_numpy(np.ascontiguousarray(tl, dtype=np.float32)).cuda()
            ref_tl = tl
        else:
            from kd_synth import bf16_bits_from_f32, f32_from_bf16_bits
            bits = bf16_bits_from_f32(tl.astype(np.float32))
            ref_tl = f32_from_bf16_bits(bits)
            tlt = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()
        got = kd.kd_validate_topk_order(torch.from_numpy(ids).cuda(), tlt, p.V)
        assert got == oracle_validate_topk_order(ids, ref_tl)
