"""GPU parity of the teacher top-K cache writer (kd_teacher_topk, through the C
ABI) against the fp64 oracle: ids bit for bit, logits within one unit in the
last place of the stored dtype (both are the fp64 logit rounded once; the two
fp64 sums differ only in summation order).

Cases: the pilot alone (V <= 16384) and pilot + emit (V > 16384); bf16 and
fp32 inputs and caches; a ragged last chunk; K = V; equal logits (lower id
first); all-zero weights (every logit ties, so every row takes the large-band
path); hidden widths that are not a multiple of 64; sampled rows at the 32K
context shapes; and the round trip through the cache validation.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

from kd_synth import bf16_bits_from_f32, f32_from_bf16_bits  # noqa: E402
from oracle import oracle_teacher_topk  # noqa: E402
from tests.kd_gpu_helpers import np_bf16_to_torch  # noqa: E402


@pytest.fixture(scope="module")
def kd():
    import chunked_top_kl_amd as m
    return m


def teacher_inputs(S, H, V, seed, dtype="bf16", w_std=None):
    rng = np.random.Generator(np.random.PCG64(seed))
    h = rng.standard_normal((S, H), dtype=np.float32)
    W = rng.standard_normal((V, H), dtype=np.float32) * np.float32(w_std or 1.0 / np.sqrt(H))
    if dtype == "bf16":
        hb, wb = bf16_bits_from_f32(h), bf16_bits_from_f32(W)
        return f32_from_bf16_bits(hb), f32_from_bf16_bits(wb), np_bf16_to_torch(hb), np_bf16_to_torch(wb)
    return h, W, torch.from_numpy(h).cuda(), torch.from_numpy(W).cuda()


def ulp(x, dtype):
    x = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(x, 1e-30)))
    return np.exp2(e - (7 if dtype == "bf16" else 23))


def check(kd, h, W, th, tW, K, chunk, out="bf16", rows=None):
    ids, logits = kd.kd_teacher_topk(th, tW, K, chunk=chunk,
                                     out_dtype=torch.bfloat16 if out == "bf16" else torch.float32)
    torch.cuda.synchronize()
    got_ids = ids.cpu().numpy()
    got = logits.float().cpu().numpy()
    if rows is not None:
        got_ids, got = got_ids[rows], got[rows]
        h = h[rows]
    ref_ids, ref = oracle_teacher_topk(h, W, K, out_dtype=out)
    assert np.array_equal(got_ids, ref_ids)
    assert np.all(np.abs(got.astype(np.float64) - ref) <= ulp(ref, out))
    return got_ids, got


@pytest.mark.parametrize("V", [5000, 20000])
def test_bf16_pilot_and_emit(kd, V):
    h, W, th, tW = teacher_inputs(300, 64, V, seed=50 + V)
    check(kd, h, W, th, tW, K=20, chunk=128)


def test_f32_inputs_and_cache_ragged_chunks(kd):
    h, W, th, tW = teacher_inputs(333, 200, 17000, seed=51, dtype="f32")
    check(kd, h, W, th, tW, K=100, chunk=128, out="f32")


def test_K_equals_V(kd):
    h, W, th, tW = teacher_inputs(70, 64, 300, seed=52)
    ids, got = check(kd, h, W, th, tW, K=300, chunk=64)
    assert np.all(np.sort(ids, axis=1) == np.arange(300)[None, :])


def test_equal_logits_lower_id_first(kd):
    h, W, th, tW = teacher_inputs(50, 64, 3000, seed=53)
    hp = np.abs(h) + np.float32(0.1)
    Wt = W.copy()
    for v in (2047, 3, 1000):
        Wt[v] = np.float32(0.5)
    Wt[2999] = np.float32(0.25)
    hb = bf16_bits_from_f32(hp)
    wb = bf16_bits_from_f32(Wt)
    hp, Wt = f32_from_bf16_bits(hb), f32_from_bf16_bits(wb)
    ids, _ = check(kd, hp, Wt, np_bf16_to_torch(hb), np_bf16_to_torch(wb), K=8, chunk=32)
    assert np.all(ids[:, :4] == np.array([3, 1000, 2047, 2999])[None, :])


def test_all_logits_equal_large_band(kd):
    # W = 0: every logit is 0, each row's band is the whole vocabulary (more
    # than the LDS list holds), and the lowest ids win
    S, H, V, K = 40, 64, 5000, 10
    h, _, th, _ = teacher_inputs(S, H, V, seed=54)
    W = np.zeros((V, H), dtype=np.float32)
    tW = torch.zeros(V, H, dtype=torch.bfloat16, device="cuda")
    ids, got = check(kd, h, W, th, tW, K=K, chunk=16)
    assert np.all(ids == np.arange(K)[None, :])
    assert np.all(got == 0.0)


def test_roundtrip_through_validation(kd):
    S, H, V, K = 256, 64, 4000, 50
    h, W, th, tW = teacher_inputs(S, H, V, seed=55)
    ids, logits = kd.kd_teacher_topk(th, tW, K, chunk=100)
    bad_id, empty, bad_logit = kd.kd_validate_topk(ids, logits, V)
    assert (bad_id, empty, bad_logit) == (0, 0, 0)
    lg = logits.float().cpu().numpy()
    assert np.all(np.diff(lg, axis=1) <= 0)


def test_full_size_sampled_rows(kd):
    # 32K context shapes: S=32768 H=2880 V=201088 K=100, chunk 2048; 32 rows
    S, H, V, K = 32768, 2880, 201088, 100
    h, W, th, tW = teacher_inputs(S, H, V, seed=1003)
    rng = np.random.default_rng(84)
    rows = np.sort(rng.choice(S, 32, replace=False))
    rows[-1] = S - 1
    rows = np.unique(rows)
    check(kd, h, W, th, tW, K=K, chunk=2048, rows=rows)
