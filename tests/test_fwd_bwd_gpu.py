"""GPU parity of the forward and backward in one call (kd_topk_kl_fwd_bwd),
through the C ABI, against the fp64 oracle and against the two calls
(kd_topk_kl_fwd, then kd_topk_kl_bwd) on the same inputs.

The one call keeps each chunk's fp32 logits and forms the chunk's gradient
tile from them instead of projecting the chunk again. What it must agree on:
  * with the oracle: the tolerances of the other parity tests (loss relative
    error <= 1e-3, gradients max-abs error <= 2e-2 * max |oracle gradient|);
  * with the two calls: z_topk bit for bit (the same products in the same
    order), lse and KL within fp32 rounding (the log-normaliser is merged
    over other vocabulary ranges), dHidden and dW within 1e-3 of their
    largest magnitude (the gradient tile differs only through lse).
Shapes span several 256-row tiles, ragged tails in S, V, H and the chunk,
masks, missing rows, duplicate ids, several dW groups, probability targets
and empty problems.
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

TWO_CALL_GRAD_FRAC = 1e-3   # one call against two calls: dHidden, dW


@pytest.fixture(scope="module")
def kd():
    import chunked_top_kl_amd as m
    return m


def _np(out):
    return {k: (v.cpu().numpy() if isinstance(v, torch.Tensor) else v) for k, v in out.items()}


def one_call(kd, p, mask=None, grad=1.0, dW=None, accumulate=False, workspace=None):
    hidden, W, ids, tl = to_device(p)
    mk = None if mask is None else torch.from_numpy(mask.astype(np.uint8)).cuda()
    g = torch.tensor([grad], dtype=torch.float32, device="cuda")
    out = kd.kd_topk_kl_fwd_bwd(hidden, W, ids, tl, g, p.T, p.chunk, mk, want_kl_rows=True,
                                want_z_topk=True, dW=dW, accumulate_dW=accumulate,
                                workspace=workspace)
    torch.cuda.synchronize()
    return _np(out)


def two_calls(kd, p, mask=None, grad=1.0):
    hidden, W, ids, tl = to_device(p)
    mk = None if mask is None else torch.from_numpy(mask.astype(np.uint8)).cuda()
    out = kd.kd_topk_kl_fwd(hidden, W, ids, tl, p.T, p.chunk, mk, want_kl_rows=True,
                            want_z_topk=True)
    g = torch.tensor([grad], dtype=torch.float32, device="cuda")
    dh, dW = kd.kd_topk_kl_bwd(hidden, W, ids, tl, out["lse"], g, p.T, p.chunk, mk)
    torch.cuda.synchronize()
    res = _np(out)
    res["dhidden"] = dh.cpu().numpy()
    res["dW"] = dW.cpu().numpy()
    return res


def check_oracle(p, got, mask=None, grad=1.0, chunk=None):
    ref = oracle_loss_grads(p.hidden, p.W, p.ids, p.tlogits, T=p.T, mask=mask, grad_loss=grad,
                            chunk=chunk)
    print(f"loss one call={float(got['loss'][0]):.7f} oracle={ref['loss']:.7f} N={ref['N']}")
    assert rel(float(got["loss"][0]), ref["loss"]) <= BF16_LOSS_RTOL
    v = ref["valid"]
    assert np.max(np.abs(got["lse"][v] - ref["lse"][v])) <= 1e-4 * max(1.0, np.max(np.abs(ref["lse"][v])))
    assert np.all(got["lse"][~v] == 0.0) and np.all(got["kl_rows"][~v] == 0.0)
    assert np.max(np.abs(got["kl_rows"][v] - ref["kl_rows"][v])) <= 1e-3 * max(1.0, np.max(ref["kl_rows"][v]))
    eh, ew = max_abs_frac(got["dhidden"], ref["dH"]), max_abs_frac(got["dW"], ref["dW"])
    print(f"dH err frac={eh:.3e} dW err frac={ew:.3e}")
    assert eh <= BF16_GRAD_FRAC and ew <= BF16_GRAD_FRAC
    assert np.all(got["dhidden"][~v] == 0.0)
    return ref


def check_two_calls(got, two):
    assert rel(float(got["loss"][0]), float(two["loss"][0])) <= 1e-5
    assert np.max(np.abs(got["lse"] - two["lse"])) <= 1e-5 * max(1.0, float(np.max(np.abs(two["lse"]))))
    assert np.max(np.abs(got["kl_rows"] - two["kl_rows"])) <= 1e-4 * max(1.0, float(np.max(two["kl_rows"])))
    # the logits at the teacher ids come from the same products: bit for bit
    assert np.array_equal(got["z_topk"].view(np.uint32), two["z_topk"].view(np.uint32))
    assert max_abs_frac(got["dhidden"], two["dhidden"]) <= TWO_CALL_GRAD_FRAC
    assert max_abs_frac(got["dW"], two["dW"]) <= TWO_CALL_GRAD_FRAC


@pytest.mark.parametrize("S,H,V,K,chunk,T,grad", [
    (1000, 136, 1537, 17, 96, 2.0, 1.3),     # ragged S/V/H/chunk, V % 8 != 0
    (300, 64, 4099, 100, 300, 1.0, 1.0),     # one chunk, V % 256 tail
    (513, 256, 777, 33, 512, 0.7, -0.6),     # S just past two tiles, negative upstream gradient
    (640, 224, 2003, 9, 320, 1.0, 0.25),     # H tail of 224 columns
    (700, 64, 300, 5, 700, 1.0, 1.0),        # V below two vocabulary tiles
    (260, 8, 100, 3, 64, 1.0, 1.0),          # H of one 16-byte granule, V below half a tile
])
def test_one_call_ragged(kd, S, H, V, K, chunk, T, grad):
    p = make_problem(S, H, V, K, T=T, chunk=chunk, seed=3 * S + V)
    got = one_call(kd, p, grad=grad)
    check_oracle(p, got, grad=grad)
    check_two_calls(got, two_calls(kd, p, grad=grad))


def test_one_call_mask_missing_rows_duplicates(kd):
    S, H, V, K = 777, 128, 3001, 12
    p = make_problem(S, H, V, K, T=1.5, chunk=200, seed=78)
    p.ids[5, 3] = p.ids[5, 4]
    p.ids[9, :] = p.ids[9, 0]
    tl = p.tlogits.copy()
    tl[11, 2:6] = -np.inf
    tl[20, :] = -np.inf
    tl[21, :] = -np.inf
    p.tl_bits = bf16_bits_from_f32(tl)
    p.tlogits = f32_from_bf16_bits(p.tl_bits)
    rng = np.random.Generator(np.random.PCG64(6))
    mask = (rng.random(S) < 0.3).astype(np.uint8)
    mask[[5, 9, 11, 20]] = 1
    got = one_call(kd, p, mask=mask)
    ref = check_oracle(p, got, mask=mask)
    assert ref["N"] == int(mask.sum()) - int(mask[20]) - int(mask[21])
    # outside the loss: z_topk NaN, as the two calls give
    off = ~ref["valid"]
    assert np.all(np.isnan(got["z_topk"][off]))
    check_two_calls(got, two_calls(kd, p, mask=mask))
    # without a mask the missing rows are still left out
    got2 = one_call(kd, p)
    check_oracle(p, got2)
    check_two_calls(got2, two_calls(kd, p))


def test_one_call_dw_groups_mask_and_accumulate(kd):
    # chunks of 2000 rows, dW groups of 4 chunks; the mask compacts 9000 rows
    # to 5500, so the second group holds a partial chunk. dW accumulates into
    # a buffer of 0.5.
    p = make_problem(9000, 64, 1000, 10, T=2.0, chunk=2000, seed=23)
    rng = np.random.default_rng(7)
    keep = np.sort(rng.choice(9000, size=5500, replace=False))
    mask = np.zeros(9000, dtype=bool)
    mask[keep] = True
    base = torch.full((p.V, p.H), 0.5, dtype=torch.float32, device="cuda")
    got = one_call(kd, p, mask=mask, dW=base, accumulate=True)
    got["dW"] = got["dW"] - 0.5
    check_oracle(p, got, mask=mask, chunk=1000)
    check_two_calls(got, two_calls(kd, p, mask=mask))


def test_one_call_reuses_its_workspace(kd):
    # two calls on one workspace, the second on a smaller problem with other
    # values: nothing of the first call leaks into the second
    p1 = make_problem(1200, 128, 2500, 20, T=1.0, chunk=512, seed=31)
    p2 = make_problem(700, 128, 2500, 20, T=1.0, chunk=512, seed=32)
    hidden, W, ids, tl = to_device(p1)
    need = kd.kd_topk_kl_fwd_bwd_workspace_bytes(hidden, W, ids, tl, p1.T, p1.chunk)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    check_oracle(p1, one_call(kd, p1, workspace=ws))
    got = one_call(kd, p2, workspace=ws)
    check_oracle(p2, got)
    check_two_calls(got, two_calls(kd, p2))


def test_one_call_zero_gradient_and_empty(kd):
    p = make_problem(600, 64, 1500, 8, T=1.0, chunk=256, seed=41)
    got = one_call(kd, p, grad=0.0)
    assert np.all(got["dhidden"] == 0.0) and np.all(got["dW"] == 0.0)
    check_two_calls(got, two_calls(kd, p, grad=0.0))
    # all positions masked out: N = 0
    got = one_call(kd, p, mask=np.zeros(600, dtype=np.uint8))
    assert got["loss"][0] == 0.0 and np.all(got["dhidden"] == 0) and np.all(got["dW"] == 0)
    assert np.all(got["lse"] == 0) and np.all(np.isnan(got["z_topk"]))
    # S = 0: loss 0, dW written as zeros
    W = torch.randn(300, 64, device="cuda").to(torch.bfloat16)
    hidden = torch.empty(0, 64, device="cuda", dtype=torch.bfloat16)
    ids = torch.empty(0, 5, device="cuda", dtype=torch.int32)
    tl = torch.empty(0, 5, device="cuda", dtype=torch.bfloat16)
    g = torch.ones(1, dtype=torch.float32, device="cuda")
    out = kd.kd_topk_kl_fwd_bwd(hidden, W, ids, tl, g, 1.0, 16,
                                dW=torch.full((300, 64), 7.0, device="cuda"))
    torch.cuda.synchronize()
    assert float(out["loss"][0]) == 0.0 and out["dhidden"].numel() == 0
    assert torch.all(out["dW"] == 0)


@pytest.mark.parametrize("S,H,V,K,chunk,T", [
    (128, 64, 1000, 10, 32, 1.0),       # the tiny fp32 configuration
    (700, 200, 1537, 13, 256, 2.0),     # ragged fp32: H tail of 200, V % 8 != 0
])
def test_one_call_fp32(kd, S, H, V, K, chunk, T):
    p = make_problem(S, H, V, K, T=T, chunk=chunk, hw_dtype="f32", tl_dtype="f32", seed=S + H)
    got = one_call(kd, p, grad=0.9)
    ref = oracle_loss_grads(p.hidden, p.W, p.ids, p.tlogits, T=p.T, grad_loss=0.9)
    assert rel(float(got["loss"][0]), ref["loss"]) <= 1e-5
    assert max_abs_frac(got["dhidden"], ref["dH"]) <= 1e-4
    assert max_abs_frac(got["dW"], ref["dW"]) <= 1e-4
    check_two_calls(got, two_calls(kd, p, grad=0.9))


def test_one_call_probability_targets(kd):
    # teacher probabilities at the ids (KD_TEACHER_PROBS), with zeros, a
    # negative value, a NaN and an all-zero row (the last three rows excluded)
    p = make_problem(700, 192, 5000, 50, T=1.5, chunk=256, seed=68)
    rng = np.random.default_rng(69)
    pr = rng.random(p.ids.shape).astype(np.float32)
    pr[rng.random(p.ids.shape) < 0.2] = 0.0
    pr[3, :] = 0.0
    pr[5, 2] = -0.25
    pr[8, 1] = np.nan
    bits = bf16_bits_from_f32(pr)
    pr = f32_from_bf16_bits(bits)
    tpr = np_bf16_to_torch(bits)
    mask = np.ones(p.S, dtype=bool)
    mask[100:140] = False
    hidden, W, ids, _ = to_device(p)
    mk = torch.from_numpy(mask.astype(np.uint8)).cuda()
    g = torch.tensor([0.8], dtype=torch.float32, device="cuda")
    out = _np(kd.kd_topk_kl_fwd_bwd(hidden, W, ids, tpr, g, p.T, p.chunk, mk, want_kl_rows=True,
                                    want_z_topk=True, teacher_probs=True))
    torch.cuda.synchronize()
    ref = oracle_loss_grads(p.hidden, p.W, p.ids, pr, T=p.T, mask=mask, grad_loss=0.8, probs=True)
    assert rel(float(out["loss"][0]), ref["loss"]) <= BF16_LOSS_RTOL
    assert max_abs_frac(out["dhidden"], ref["dH"]) <= BF16_GRAD_FRAC
    assert max_abs_frac(out["dW"], ref["dW"]) <= BF16_GRAD_FRAC
    assert np.all(out["dhidden"][~ref["valid"]] == 0.0)
    two = kd.kd_topk_kl_fwd(hidden, W, ids, tpr, p.T, p.chunk, mk, want_kl_rows=True,
                            want_z_topk=True, teacher_probs=True)
    dh, dW = kd.kd_topk_kl_bwd(hidden, W, ids, tpr, two["lse"], g, p.T, p.chunk, mk,
                               teacher_probs=True)
    torch.cuda.synchronize()
    res = _np(two)
    res["dhidden"] = dh.cpu().numpy()
    res["dW"] = dW.cpu().numpy()
    check_two_calls(out, res)


def test_one_call_autograd(kd):
    # the autograd wrapper with the gradients formed in the forward: the same
    # loss and gradients as the two-call wrapper, for an upstream gradient of 2
    p = make_problem(500, 128, 2100, 12, T=1.3, chunk=192, seed=17)
    hidden, W, ids, tl = to_device(p)
    grads = []
    for one_call in (True, False):
        h = hidden.clone().requires_grad_(True)
        w = W.clone().requires_grad_(True)
        loss = kd.kd_topk_kl(h, w, ids, tl, p.T, p.chunk, one_call=one_call) * 2.0
        loss.backward()
        grads.append((float(loss.detach()), h.grad.float().cpu().numpy(),
                      w.grad.float().cpu().numpy()))
    ref = oracle_loss_grads(p.hidden, p.W, p.ids, p.tlogits, T=p.T, grad_loss=2.0)
    (l1, dh1, dw1), (l2, dh2, dw2) = grads
    assert rel(l1 / 2.0, ref["loss"]) <= BF16_LOSS_RTOL and rel(l1, l2) <= 1e-5
    assert max_abs_frac(dh1, ref["dH"]) <= BF16_GRAD_FRAC
    assert max_abs_frac(dw1, ref["dW"]) <= BF16_GRAD_FRAC
    # the bf16 gradients of the two wrappers round the same fp32 values up to
    # the gradient tile's lse difference
    assert max_abs_frac(dh1, dh2) <= 1e-2 and max_abs_frac(dw1, dw2) <= 1e-2


def test_scale_f32(kd):
    # x *= g over aligned and unaligned ranges with a ragged tail
    base = torch.arange(1, 1 + 4099, dtype=torch.float32, device="cuda")
    g = torch.tensor([-0.75], dtype=torch.float32, device="cuda")
    for lo in (0, 1):
        x = base.clone()
        kd.kd_scale_f32(x[lo:], g)
        torch.cuda.synchronize()
        want = base.clone()
        want[lo:] *= -0.75
        assert torch.equal(x, want)
