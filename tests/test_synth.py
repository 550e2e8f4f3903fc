"""Checks of the seeded input generator (shared by the oracle and the GPU tests)."""
import numpy as np
import pytest

from kd_synth import bf16_bits_from_f32, draw_distinct_ids, f32_from_bf16_bits, make_problem


def test_bf16_rounding_matches_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.Generator(np.random.PCG64(1))
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 3,
                        np.array([0.0, -0.0, 1e-40, -1e-40, 3.4e38, -3.4e38, np.inf, -np.inf],
                                 dtype=np.float32)])
    ours = bf16_bits_from_f32(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(f32_from_bf16_bits(ours),
                          torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_problem_is_deterministic_and_well_formed():
    a = make_problem(64, 32, 500, 10, seed=7)
    b = make_problem(64, 32, 500, 10, seed=7)
    c = make_problem(64, 32, 500, 10, seed=8)
    assert np.array_equal(a.hidden_bits, b.hidden_bits) and np.array_equal(a.ids, b.ids)
    assert not np.array_equal(a.hidden_bits, c.hidden_bits)
    assert a.ids.dtype == np.int32 and a.ids.min() >= 0 and a.ids.max() < 500
    srt = np.sort(a.ids, axis=1)
    assert not np.any(srt[:, 1:] == srt[:, :-1])
    assert np.all(np.diff(a.tlogits, axis=1) <= 0)
    assert np.array_equal(f32_from_bf16_bits(a.hidden_bits), a.hidden)
    assert np.array_equal(f32_from_bf16_bits(a.tl_bits), a.tlogits)


def test_fp32_problem_and_moments():
    p = make_problem(256, 64, 1000, 10, hw_dtype="f32", tl_dtype="f32", seed=3)
    assert p.hidden_bits is None and p.hidden.dtype == np.float32
    assert abs(p.hidden.std() - 1.0) < 0.02
    assert abs(p.W.std() * np.sqrt(64) - 1.0) < 0.02
    # logits: 8 - 1.5 ln(k+1) plus noise of variance 0.5, then sorted; sorting keeps
    # each row's sum, so the grand mean is that of the base curve
    base = 8.0 - 1.5 * np.log(np.arange(10) + 1.0)
    assert abs(p.tlogits.mean() - base.mean()) < 0.02
    # a row's sum is the base sum plus K independent noise draws: its variance is K * 0.5
    assert 0.3 < np.var(p.tlogits.sum(axis=1) - base.sum()) / 10 < 0.7


def test_distinct_ids_dense_case():
    rng = np.random.Generator(np.random.PCG64(4))
    ids = draw_distinct_ids(rng, 20, 9, 10)
    for row in ids:
        assert len(set(row.tolist())) == 9
