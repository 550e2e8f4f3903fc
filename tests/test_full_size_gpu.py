"""GPU parity at the full sizes of the workload configurations, in the launch
configuration the benchmark times (the configuration's chunk, bf16, default
workspace), through the C ABI.

The fp64 oracle cannot compute every output at these sizes on the host, so
each test states what it compares:
  * 8K context: loss, lse and KL of every row (the oracle's forward over all
    rows), dHidden at 256 sampled rows and dW at 256 sampled vocabulary rows
    (from the oracle's own lse of every row).
  * 32K context, large vocabulary, and 256K context: lse, KL and dHidden at
    sampled rows; the loss equals the mean of the per-row KL; the rows of dW
    sum to zero over the vocabulary (the gradient of each row's softmax sums
    to zero, at any size).
  * entropy-selective: the entropy of every position (oracle, fp64), the kept
    index set bit for bit, and the selective KL at sampled kept rows.
Tolerances are those of the other parity tests.
"""
import math

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

from kd_synth import make_problem  # noqa: E402
from oracle import (oracle_dW_rows, oracle_entropy, oracle_rows,  # noqa: E402
                    oracle_select_top_fraction)
from tests.kd_gpu_helpers import BF16_GRAD_FRAC, BF16_LOSS_RTOL, rel, to_device  # noqa: E402


@pytest.fixture(scope="module")
def kd():
    import chunked_top_kl_amd as m
    return m


def gpu_fwd_bwd(kd, p, mask=None):
    hidden, W, ids, tl = to_device(p)
    mk = None if mask is None else torch.from_numpy(mask.astype(np.uint8)).cuda()
    out = kd.kd_topk_kl_fwd(hidden, W, ids, tl, p.T, p.chunk, mk, want_kl_rows=True)
    g = torch.ones(1, dtype=torch.float32, device="cuda")
    dh, dW = kd.kd_topk_kl_bwd(hidden, W, ids, tl, out["lse"], g, p.T, p.chunk, mk)
    torch.cuda.synchronize()
    return out, dh, dW


def check_rows(p, out, dh, rows, N):
    """lse, KL and dHidden of sampled rows against the oracle's definition."""
    ref = oracle_rows(p.hidden[rows], p.W, p.ids[rows], p.tlogits[rows], p.T, N)
    lse = out["lse"].cpu().numpy()[rows]
    kl = out["kl_rows"].cpu().numpy()[rows]
    assert np.max(np.abs(lse - ref["lse"])) <= 1e-4 * max(1.0, float(np.max(np.abs(ref["lse"]))))
    assert np.max(np.abs(kl - ref["kl_rows"])) <= 1e-3 * max(1.0, float(np.max(ref["kl_rows"])))
    got_dh = dh.cpu().numpy()[rows]
    err = float(np.max(np.abs(got_dh - ref["dH"])))
    assert err <= BF16_GRAD_FRAC * float(np.max(np.abs(ref["dH"])))
    return ref


def check_loss_is_mean_kl(out, N):
    kl = out["kl_rows"].cpu().numpy().astype(np.float64)
    assert rel(float(out["loss"][0]), math.fsum(kl) / N) <= 1e-5


def check_dW_rows_sum_to_zero(dW):
    # sum over the vocabulary of each column of dW, against the sum of magnitudes
    colsum = torch.sum(dW, dim=0, dtype=torch.float64)
    absum = torch.sum(dW.abs(), dim=0, dtype=torch.float64)
    assert float(torch.max(colsum.abs() / absum.clamp_min(1e-30))) <= 1e-2


def test_full_8k_context(kd):
    # S=8192 H=3072 V=128256 K=100 T=1 chunk=1024
    p = make_problem(8192, 3072, 128256, 100, T=1.0, chunk=1024, seed=1002)
    out, dh, dW = gpu_fwd_bwd(kd, p)
    S = p.S
    # oracle forward over every row, in row blocks
    kl = np.empty(S)
    lse = np.empty(S)
    for r0 in range(0, S, 512):
        rr = oracle_rows(p.hidden[r0:r0 + 512], p.W, p.ids[r0:r0 + 512], p.tlogits[r0:r0 + 512],
                         p.T, S, grads=False)
        kl[r0:r0 + 512] = rr["kl_rows"]
        lse[r0:r0 + 512] = rr["lse"]
    loss = math.fsum(kl) / S
    assert rel(float(out["loss"][0]), loss) <= BF16_LOSS_RTOL
    got_lse = out["lse"].cpu().numpy()
    assert np.max(np.abs(got_lse - lse)) <= 1e-4 * max(1.0, float(np.max(np.abs(lse))))
    got_kl = out["kl_rows"].cpu().numpy()
    assert np.max(np.abs(got_kl - kl)) <= 1e-3 * max(1.0, float(np.max(kl)))
    rng = np.random.default_rng(81)
    rows = np.sort(rng.choice(S, 256, replace=False))
    check_rows(p, out, dh, rows, S)
    vrows = np.sort(rng.choice(p.V, 256, replace=False))
    vrows[0] = int(p.ids[0, 0])                          # at least one teacher id
    vrows = np.unique(vrows)
    ref_dw = oracle_dW_rows(p.hidden, p.W, p.ids, p.tlogits, p.T, lse, np.ones(S, bool), vrows)
    got_dw = dW.cpu().numpy()[vrows]
    err = float(np.max(np.abs(got_dw - ref_dw)))
    assert err <= BF16_GRAD_FRAC * float(np.max(np.abs(ref_dw)))


@pytest.mark.parametrize("cfg", ["32k_context", "256k_context"])
def test_full_size_sampled_rows(kd, cfg):
    if cfg == "32k_context":
        p = make_problem(32768, 2880, 201088, 100, T=1.0, chunk=2048, seed=1003)
        nrows = 128
    else:
        p = make_problem(262144, 3072, 128256, 100, T=2.0, chunk=2048, seed=1004)
        nrows = 64
    out, dh, dW = gpu_fwd_bwd(kd, p)
    S = p.S
    rng = np.random.default_rng(82)
    rows = np.sort(rng.choice(S, nrows, replace=False))
    rows[-1] = S - 1                                     # the ragged end of the last chunk
    rows = np.unique(rows)
    check_rows(p, out, dh, rows, S)
    check_loss_is_mean_kl(out, S)
    check_dW_rows_sum_to_zero(dW)


def test_full_entropy_selective(kd):
    # S=32768 H=2048 V=151936 K=100, top 20% by entropy, chunk 1024, T=1
    S, H, V, K = 32768, 2048, 151936, 100
    p = make_problem(S, H, V, K, T=1.0, chunk=1024, seed=1005)
    hidden, W, ids, tl = to_device(p)
    ent = kd.kd_student_entropy(hidden, W)
    mask, idx, cnt = kd.kd_select_top_fraction(ent, hidden, W, 20, 100)
    torch.cuda.synchronize()
    ref_e = oracle_entropy(p.hidden, p.W, chunk=512)
    got_e = ent.cpu().numpy()
    assert np.max(np.abs(got_e - ref_e)) <= 2e-5
    rmask, ridx, rk = oracle_select_top_fraction(ref_e, 20, 100)
    assert cnt == rk == (20 * S) // 100
    assert np.array_equal(idx.cpu().numpy(), ridx)
    m = mask.cpu().numpy().astype(bool)
    out, dh, dW = gpu_fwd_bwd(kd, p, mask=m)
    rng = np.random.default_rng(83)
    rows = np.sort(rng.choice(ridx, 128, replace=False))
    check_rows(p, out, dh, rows, int(rk))
    # unselected rows take no part: zero dHidden, zero lse
    off = np.flatnonzero(~m)[:512]
    assert np.all(dh.cpu().numpy()[off] == 0.0)
    assert np.all(out["lse"].cpu().numpy()[off] == 0.0)
    kl = out["kl_rows"].cpu().numpy().astype(np.float64)
    assert rel(float(out["loss"][0]), math.fsum(kl[m]) / int(rk)) <= 1e-5
    check_dW_rows_sum_to_zero(dW)
