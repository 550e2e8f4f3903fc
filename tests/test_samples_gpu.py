"""GPU parity of sample selection by mean student entropy (kd_select_samples,
the sample axis of SE-KD3X in "Rethinking Selective Knowledge Distillation",
Method section 2) against the fp64 oracle: the kept samples bit for bit.

Cases: samples of random lengths; crowded entropies (sample means closer than
the fp32-path error, so the fp64 refinement of the band decides); entropies
given with errors beyond the band's least bound (the measured error widens
it); duplicate
samples (exact ties, lower index first); empty samples and the kept-count
edges; malformed offsets rejected.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

from kd_synth import bf16_bits_from_f32, f32_from_bf16_bits, make_problem  # noqa: E402
from oracle import oracle_entropy, oracle_select_samples  # noqa: E402
from tests.kd_gpu_helpers import np_bf16_to_torch, to_device  # noqa: E402


@pytest.fixture(scope="module")
def kd():
    import chunked_top_kl_amd as m
    return m


def offsets_of(lengths):
    return np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)


def run(kd, hidden_np, W_np, hidden, W, off, num, den):
    ent = kd.kd_student_entropy(hidden, W)
    toff = torch.from_numpy(off).cuda()
    mask, idx, cnt = kd.kd_select_samples(ent, toff, hidden, W, num, den)
    torch.cuda.synchronize()
    ref_e = oracle_entropy(hidden_np, W_np, chunk=500)
    rmask, ridx, rk, _ = oracle_select_samples(ref_e, off, num, den)
    assert cnt == rk
    assert np.array_equal(mask.cpu().numpy(), rmask)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    return rmask


@pytest.mark.parametrize("case", ["spread", "crowded"])
def test_samples_match_oracle(kd, case):
    rng = np.random.default_rng(72)
    lengths = rng.integers(1, 120, size=48)
    S = int(lengths.sum())
    p = make_problem(S, 128, 4001, 4, seed=73, hidden_std=(0.05 if case == "crowded" else 1.5))
    hidden, W, _, _ = to_device(p)
    kd.kd_profile_reset()
    kd.kd_profile_enable(True)
    run(kd, p.hidden, p.W, hidden, W, offsets_of(lengths), 30, 100)
    kd.kd_profile_enable(False)
    steps = kd.kd_profile_read()
    kd.kd_profile_reset()
    if case == "crowded":
        # the sample means are closer than the fp32-path error: the band is refined
        assert "select_refine_fp64" in steps


def test_band_of_many_samples_and_positions(kd):
    # more than 4096 band samples holding more than 65536 positions, means
    # crowded inside the fp32-path error: every position of the band samples is
    # recomputed in fp64 (in pieces) and the band ranked on fp64 means
    rng = np.random.default_rng(78)
    lengths = rng.integers(1, 32, size=6000)
    S = int(lengths.sum())
    assert S > 65536
    p = make_problem(S, 64, 2000, 4, seed=79, hidden_std=0.01)
    hidden, W, _, _ = to_device(p)
    kd.kd_profile_reset()
    kd.kd_profile_enable(True)
    run(kd, p.hidden, p.W, hidden, W, offsets_of(lengths), 20, 100)
    kd.kd_profile_enable(False)
    steps = kd.kd_profile_read()
    kd.kd_profile_reset()
    # a refinement launch and an entropy launch per piece of 4096 positions
    # (bf16 rows): more than 65536 positions were refined
    assert steps["select_refine_fp64"][0] > 2 * (65536 // 4096)


def test_samples_with_less_accurate_entropies(kd):
    # entropies given with errors of up to 1e-4 nats (beyond the band's least
    # bound of 2e-5), samples of 5 positions: the measured error widens the
    # band over the means and the kept samples are still the fp64 ones
    S = 600 * 5
    off = (np.arange(601, dtype=np.int64) * S) // 600
    p = make_problem(S, 128, 4001, 4, seed=23, hidden_std=0.2)
    hidden, W, _, _ = to_device(p)
    ent = kd.kd_student_entropy(hidden, W)
    noise = np.random.default_rng(24).uniform(-1e-4, 1e-4, size=S)
    noisy = ent + torch.from_numpy(noise).cuda()
    mask, idx, cnt = kd.kd_select_samples(noisy, torch.from_numpy(off).cuda(), hidden, W, 20, 100)
    torch.cuda.synchronize()
    ref_e = oracle_entropy(p.hidden, p.W, chunk=500)
    rmask, ridx, rk, _ = oracle_select_samples(ref_e, off, 20, 100)
    assert cnt == rk
    assert np.array_equal(mask.cpu().numpy(), rmask)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    _, nidx, _, _ = oracle_select_samples(ref_e + noise, off, 20, 100)
    assert not np.array_equal(nidx, ridx)


def test_duplicate_samples_tie_to_lower_index(kd):
    rng = np.random.default_rng(74)
    lengths = np.array([20, 35, 20, 20, 35, 10])
    S = int(lengths.sum())
    p = make_problem(S, 64, 3000, 4, seed=75, hidden_std=1.0)
    off = offsets_of(lengths)
    hb = p.hidden_bits.copy()
    hb[off[2]:off[3]] = hb[off[0]:off[1]]       # sample 2 = sample 0
    hb[off[3]:off[4]] = hb[off[0]:off[1]]       # sample 3 = sample 0
    hidden_np = f32_from_bf16_bits(hb)
    hidden = np_bf16_to_torch(hb)
    _, W, _, _ = to_device(p)
    for num in (1, 2, 3, 4, 5):
        run(kd, hidden_np, p.W, hidden, W, off, num, 6)


def test_empty_samples_and_count_edges(kd):
    lengths = np.array([5, 0, 7, 0, 3, 9])
    S = int(lengths.sum())
    p = make_problem(S, 64, 2000, 4, seed=76)
    hidden, W, _, _ = to_device(p)
    off = offsets_of(lengths)
    for num, den in ((0, 1), (1, 1), (2, 3), (5, 6)):
        run(kd, p.hidden, p.W, hidden, W, off, num, den)


def test_malformed_offsets_rejected(kd):
    p = make_problem(50, 64, 1000, 4, seed=77)
    hidden, W, _, _ = to_device(p)
    ent = kd.kd_student_entropy(hidden, W)
    for off in ([0, 30, 20, 50], [0, 10, 60], [-1, 10, 50]):
        with pytest.raises(kd.KdError) as ei:
            kd.kd_select_samples(ent, torch.tensor(off, dtype=torch.int64, device="cuda"), hidden, W,
                                 1, 2)
        assert ei.value.code == 10
