"""GPU parity of the loss with teacher targets given as probabilities
(KD_TEACHER_PROBS: sampled sparse targets, the class axis of SE-KD3X in
"Rethinking Selective Knowledge Distillation", Method section 2) against the
fp64 oracle, through the C ABI. Tolerances are those of the logit path.

Cases: fp32 and bf16 probabilities with duplicate ids, zero entries, a
negative value, a NaN and an all-zero row (both excluded), with a mask and
several chunks; softmax targets against the logit path on the GPU; and the
validation counts for probabilities.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

from kd_synth import bf16_bits_from_f32, f32_from_bf16_bits, make_problem  # noqa: E402
from oracle import oracle_loss_grads, oracle_validate_topk  # noqa: E402
from tests.kd_gpu_helpers import (BF16_GRAD_FRAC, BF16_LOSS_RTOL, max_abs_frac, np_bf16_to_torch,  # noqa: E402
                                  rel, to_device)


@pytest.fixture(scope="module")
def kd():
    import chunked_top_kl_amd as m
    return m


def sampled_targets(p, seed, dtype):
    """Probabilities at the problem's ids: uniform draws, some zeros, not normalised."""
    rng = np.random.default_rng(seed)
    pr = rng.random(p.ids.shape).astype(np.float32)
    pr[rng.random(p.ids.shape) < 0.2] = 0.0
    pr[3, :] = 0.0                     # no mass: missing
    pr[5, 2] = -0.25                   # negative: missing
    pr[8, 1] = np.nan                  # NaN: missing
    p.ids[11, 4] = p.ids[11, 0]        # a duplicate id: the two add
    if dtype == "bf16":
        bits = bf16_bits_from_f32(pr)
        return f32_from_bf16_bits(bits), np_bf16_to_torch(bits)
    return pr, torch.from_numpy(pr).cuda()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_probability_targets_match_oracle(kd, dtype):
    p = make_problem(700, 192, 5000, 50, T=1.5, chunk=256, seed=66)
    pr, tpr = sampled_targets(p, 67, dtype)
    mask = np.ones(p.S, dtype=bool)
    mask[100:140] = False
    hidden, W, ids, _ = to_device(p)
    mk = torch.from_numpy(mask.astype(np.uint8)).cuda()
    out = kd.kd_topk_kl_fwd(hidden, W, ids, tpr, p.T, p.chunk, mk, want_kl_rows=True,
                            teacher_probs=True)
    g = torch.tensor([0.8], dtype=torch.float32, device="cuda")
    dh, dW = kd.kd_topk_kl_bwd(hidden, W, ids, tpr, out["lse"], g, p.T, p.chunk, mk,
                               teacher_probs=True)
    torch.cuda.synchronize()
    ref = oracle_loss_grads(p.hidden, p.W, p.ids, pr, T=p.T, mask=mask, grad_loss=0.8, probs=True)
    v = ref["valid"]
    assert not v[3] and not v[5] and not v[8]
    assert rel(float(out["loss"][0]), ref["loss"]) <= BF16_LOSS_RTOL
    kl = out["kl_rows"].cpu().numpy()
    assert np.max(np.abs(kl[v] - ref["kl_rows"][v])) <= 1e-3 * max(1.0, float(np.max(ref["kl_rows"][v])))
    dh, dW = dh.cpu().numpy(), dW.cpu().numpy()
    assert max_abs_frac(dh, ref["dH"]) <= BF16_GRAD_FRAC
    assert max_abs_frac(dW, ref["dW"]) <= BF16_GRAD_FRAC
    assert np.all(dh[~v] == 0.0)


def test_softmax_targets_agree_with_logit_path(kd):
    p = make_problem(400, 128, 3000, 20, T=2.0, chunk=128, tl_dtype="f32", seed=68)
    l = p.tlogits.astype(np.float64) / p.T
    e = np.exp(l - l.max(axis=1, keepdims=True))
    pr = (e / e.sum(axis=1, keepdims=True)).astype(np.float32)
    hidden, W, ids, tl = to_device(p)
    a = kd.kd_topk_kl_fwd(hidden, W, ids, tl, p.T, p.chunk, want_kl_rows=True)
    b = kd.kd_topk_kl_fwd(hidden, W, ids, torch.from_numpy(pr).cuda(), p.T, p.chunk,
                          want_kl_rows=True, teacher_probs=True)
    torch.cuda.synchronize()
    assert rel(float(b["loss"][0]), float(a["loss"][0])) <= 1e-5
    assert np.max(np.abs(a["kl_rows"].cpu().numpy() - b["kl_rows"].cpu().numpy())) <= 1e-4


def test_validation_counts_for_probabilities(kd):
    p = make_problem(64, 64, 500, 8, T=1.0, chunk=32, seed=69)
    pr, tpr = sampled_targets(p, 70, "f32")
    ids = torch.from_numpy(np.ascontiguousarray(p.ids, dtype=np.int32)).cuda()
    got = kd.kd_validate_topk(ids, tpr, p.V, teacher_probs=True)
    assert got == oracle_validate_topk(p.ids, pr, p.V, probs=True)
