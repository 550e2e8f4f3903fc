"""GPU parity of the comparator loss forms (dense, forward-chunked) against the
fp64 oracle, through the C ABI. "Making Knowledge Distillation Cheap Enough to
Run at Scale" (section "what chunked KL loss does") measures these forms
beside the fused chunked loss: the same loss from a dense teacher grid and
dense student log-probabilities, or from a sparse teacher and chunked
positions with the student logits kept for the backward.

Both forms keep the student logits as bf16, so they are held to the same
tolerances as the fused path (loss relative 1e-3, gradients 2e-2 max|oracle|).
Cases: ragged shapes over several chunks and a ragged tail, with a mask,
duplicate ids, -inf teacher entries and a missing row; T = 2; accumulate_dW;
the three forms' losses agree; fp32 inputs and unknown forms are refused.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

from kd_synth import bf16_bits_from_f32, f32_from_bf16_bits, make_problem  # noqa: E402
from oracle import oracle_loss_grads  # noqa: E402
from tests.kd_gpu_helpers import (BF16_GRAD_FRAC, BF16_LOSS_RTOL, max_abs_frac,  # noqa: E402
                                  np_bf16_to_torch, rel, to_device)


@pytest.fixture(scope="module")
def kd():
    import chunked_top_kl_amd as m
    return m


def awkward_problem(seed):
    p = make_problem(700, 136, 3001, 9, T=2.0, chunk=256, seed=seed)
    p.ids[5, 3] = p.ids[5, 1]                       # duplicate id: probabilities add
    tl = p.tlogits.copy()
    tl[9, 6:] = -np.inf                             # -inf entries: probability 0
    tl[13, :] = -np.inf                             # a missing row
    p.tl_bits = bf16_bits_from_f32(tl)
    p.tlogits = f32_from_bf16_bits(p.tl_bits)
    return p


@pytest.mark.parametrize("form", ["dense", "forward_chunked"])
def test_comparator_matches_oracle(kd, form):
    code = kd.KD_FORM_DENSE if form == "dense" else kd.KD_FORM_FORWARD_CHUNKED
    p = awkward_problem(301)
    mask = np.random.default_rng(302).random(p.S) < 0.8
    hidden, W, ids, tl = to_device(p)
    mk = torch.from_numpy(mask.astype(np.uint8)).cuda()
    out = kd.kd_kl_comparator_fwd(hidden, W, ids, tl, code, p.T, p.chunk, mk, want_kl_rows=True)
    g = torch.full((1,), 0.75, dtype=torch.float32, device="cuda")
    dh, dW = kd.kd_kl_comparator_bwd(hidden, W, ids, tl, out["lse"], g, code, out["workspace"],
                                     p.T, p.chunk, mk)
    torch.cuda.synchronize()
    ref = oracle_loss_grads(p.hidden, p.W, p.ids, p.tlogits, T=p.T, mask=mask, grad_loss=0.75,
                            chunk=128)
    v = ref["valid"]
    assert not v[13]
    assert rel(float(out["loss"][0]), ref["loss"]) <= BF16_LOSS_RTOL
    kl = out["kl_rows"].cpu().numpy()
    assert np.max(np.abs(kl[v] - ref["kl_rows"][v])) <= 1e-3 * max(1.0, float(np.max(ref["kl_rows"])))
    lse = out["lse"].cpu().numpy()
    assert np.max(np.abs(lse[v] - ref["lse"][v])) <= 1e-3 * max(1.0, float(np.max(np.abs(ref["lse"]))))
    assert np.all(lse[~v] == 0.0)
    dh, dW = dh.cpu().numpy(), dW.cpu().numpy()
    assert max_abs_frac(dh, ref["dH"]) <= BF16_GRAD_FRAC
    assert max_abs_frac(dW, ref["dW"]) <= BF16_GRAD_FRAC
    assert np.all(dh[~v] == 0.0)


@pytest.mark.parametrize("form", ["dense", "forward_chunked"])
def test_comparator_accumulates_dW_and_agrees_with_fused(kd, form):
    code = kd.KD_FORM_DENSE if form == "dense" else kd.KD_FORM_FORWARD_CHUNKED
    p = make_problem(1100, 256, 5003, 20, T=1.0, chunk=512, seed=303)
    hidden, W, ids, tl = to_device(p)
    fused = kd.kd_topk_kl_fwd(hidden, W, ids, tl, p.T, p.chunk, want_kl_rows=True)
    out = kd.kd_kl_comparator_fwd(hidden, W, ids, tl, code, p.T, p.chunk, want_kl_rows=True)
    g = torch.ones(1, dtype=torch.float32, device="cuda")
    dW0 = torch.randn(p.V, p.H, dtype=torch.float32, device="cuda") * 1e-4
    dh, dW = kd.kd_kl_comparator_bwd(hidden, W, ids, tl, out["lse"], g, code, out["workspace"],
                                     p.T, p.chunk, dW=dW0.clone(), accumulate_dW=True)
    _, dWf = kd.kd_topk_kl_bwd(hidden, W, ids, tl, fused["lse"], g, p.T, p.chunk)
    torch.cuda.synchronize()
    assert rel(float(out["loss"][0]), float(fused["loss"][0])) <= 1e-4
    ref = oracle_loss_grads(p.hidden, p.W, p.ids, p.tlogits, T=p.T, chunk=256)
    assert rel(float(out["loss"][0]), ref["loss"]) <= BF16_LOSS_RTOL
    assert max_abs_frac((dW - dW0).cpu().numpy(), ref["dW"]) <= BF16_GRAD_FRAC
    assert max_abs_frac(dWf.cpu().numpy(), ref["dW"]) <= BF16_GRAD_FRAC


def test_comparator_refusals(kd):
    p = make_problem(64, 64, 500, 4, T=1.0, chunk=32, hw_dtype="f32", tl_dtype="f32", seed=304)
    hidden, W, ids, tl = to_device(p)
    with pytest.raises(kd.KdError):
        kd.kd_kl_comparator_fwd(hidden, W, ids, tl, kd.KD_FORM_DENSE, 1.0, 32)
    q = make_problem(64, 64, 500, 4, T=1.0, chunk=32, seed=305)
    hidden, W, ids, tl = to_device(q)
    with pytest.raises(kd.KdError):
        kd.kd_kl_comparator_fwd(hidden, W, ids, tl, 7, 1.0, 32)
    with pytest.raises(kd.KdError):
        kd.kd_kl_comparator_fwd(hidden, W, ids, tl, kd.KD_FORM_FUSED, 1.0, 32)
