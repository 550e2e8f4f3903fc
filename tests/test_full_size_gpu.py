"""GPU parity at the full sizes of the workload configurations, in the launch
configuration the benchmark times (the configuration's chunk, bf16, default
workspace), through the C ABI, against the fp64 oracle.

What is compared with the oracle at each size:
  * 8K context: loss, lse and KL of every row (the oracle's forward over all
    rows, computed here), dHidden at 1024 sampled rows and dW at 512 sampled
    vocabulary rows.
  * 32K context (large vocabulary) and 256K context: the loss, and the lse
    and KL of every row, against the oracle's values stored in tests/golden
    (written by tests/golden/make_full_size.py, which calls only the oracle;
    the test first checks that the seeded generator reproduced the inputs
    those values were computed on); dHidden at 1024 sampled rows (the first
    and last row of every chunk, the ragged end, random rows) and dW at 512
    sampled vocabulary rows (teacher ids, the last vocabulary tile, random
    rows; every row of dW sums over all dW groups of chunks), both from the
    oracle computed here.
  * entropy-selective: the entropy of every position against the stored
    oracle values, the kept index set bit for bit, and the selective KL's
    loss, the lse and KL of every kept row, dHidden at 1024 kept rows and dW
    at 512 vocabulary rows against the oracle over the kept rows.
  * the forward and backward in one call (kd_topk_kl_fwd_bwd) at the
    32K-context and 256K-context sizes: the loss and every row's lse and KL
    against the stored oracle values, dHidden at 1024 rows and dW at 512
    vocabulary rows.
  * the comparator forms (dense, forward-chunked) at the 32K-context size:
    the loss and every row's lse and KL against the stored oracle values,
    dHidden at 256 rows and dW at 128 vocabulary rows.
The rows of dW also sum to zero over the vocabulary (an extra check).
Tolerances are those of the other parity tests.
"""
import math

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

from kd_synth import make_problem  # noqa: E402
from oracle import (oracle_dW_rows, oracle_rows, oracle_select_top_fraction)  # noqa: E402
from tests.golden.make_full_size import input_digest, load, load_problem  # noqa: E402
from tests.kd_gpu_helpers import BF16_GRAD_FRAC, BF16_LOSS_RTOL, rel, to_device  # noqa: E402

N_DH_ROWS = 1024
N_DW_ROWS = 512


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
    res = dict(loss=float(out["loss"][0]), lse=out["lse"].cpu().numpy(),
               kl=out["kl_rows"].cpu().numpy(), dh=dh.cpu().numpy(), dW=dW)
    del hidden, W, ids, tl, out, dh
    return res


def stored(name):
    """The oracle's stored per-row values for a workload, after checking that
    the generator reproduced the inputs they were computed on."""
    meta, ref = load(name)
    p = load_problem(name)
    assert input_digest(p) == meta["inputs_sha256"], \
        "the seeded inputs differ from those of the stored oracle values"
    return p, meta, ref


def check_row_values(lse, kl, ref_lse, ref_kl):
    assert np.max(np.abs(lse - ref_lse)) <= 1e-4 * max(1.0, float(np.max(np.abs(ref_lse))))
    assert np.max(np.abs(kl - ref_kl)) <= 1e-3 * max(1.0, float(np.max(ref_kl)))


def sampled_rows(rows_in_loss, chunk, n, rng):
    """n of the loss's rows (given in compacted order): the first and last of
    every chunk, the last row, and random rows."""
    N = len(rows_in_loss)
    pick = set()
    for c0 in range(0, N, chunk):
        pick.add(c0)
        pick.add(min(N, c0 + chunk) - 1)
    rest = np.setdiff1d(np.arange(N), np.fromiter(pick, dtype=np.int64))
    extra = rng.choice(rest, max(0, n - len(pick)), replace=False)
    sel = np.sort(np.concatenate([np.fromiter(pick, dtype=np.int64), extra]))
    return rows_in_loss[sel]


def sampled_vocab(p, rows, n, rng):
    """n vocabulary rows: teacher ids of a few loss rows, the last vocabulary
    tile (256 rows) and the very last row, row 0, random rows."""
    v = {0, p.V - 1}
    v.update(int(x) for x in p.ids[rows[0], :16])
    v.update(int(x) for x in p.ids[rows[-1], :16])
    v.update(range(max(0, p.V - 256), p.V, 17))
    rest = np.setdiff1d(np.arange(p.V), np.fromiter(v, dtype=np.int64))
    extra = rng.choice(rest, max(0, n - len(v)), replace=False)
    return np.sort(np.concatenate([np.fromiter(v, dtype=np.int64), extra]))


def check_dh_rows(p, W64, dh, rows, N):
    ref = np.empty((len(rows), p.H))
    for b0 in range(0, len(rows), 256):
        r = rows[b0:b0 + 256]
        ref[b0:b0 + 256] = oracle_rows(p.hidden[r], W64, p.ids[r], p.tlogits[r], p.T, N)["dH"]
    err = float(np.max(np.abs(dh[rows] - ref)))
    assert err <= BF16_GRAD_FRAC * float(np.max(np.abs(ref))), err


def check_dw_rows(p, W64, dW, lse, valid, vrows):
    ref = oracle_dW_rows(p.hidden, W64, p.ids, p.tlogits, p.T, lse, valid, vrows)
    got = dW[torch.from_numpy(vrows).cuda()].cpu().numpy()
    err = float(np.max(np.abs(got - ref)))
    assert err <= BF16_GRAD_FRAC * float(np.max(np.abs(ref))), err


def check_dW_rows_sum_to_zero(dW):
    # sum over the vocabulary of each column of dW, against the sum of magnitudes
    colsum = torch.sum(dW, dim=0, dtype=torch.float64)
    absum = torch.sum(dW.abs(), dim=0, dtype=torch.float64)
    assert float(torch.max(colsum.abs() / absum.clamp_min(1e-30))) <= 1e-2


def test_full_8k_context(kd):
    # S=8192 H=3072 V=128256 K=100 T=1 chunk=1024
    p = make_problem(8192, 3072, 128256, 100, T=1.0, chunk=1024, seed=1002)
    r = gpu_fwd_bwd(kd, p)
    S = p.S
    W64 = p.W.astype(np.float64)
    # oracle forward over every row, in row blocks
    kl = np.empty(S)
    lse = np.empty(S)
    for r0 in range(0, S, 512):
        rr = oracle_rows(p.hidden[r0:r0 + 512], W64, p.ids[r0:r0 + 512], p.tlogits[r0:r0 + 512],
                         p.T, S, grads=False)
        kl[r0:r0 + 512] = rr["kl_rows"]
        lse[r0:r0 + 512] = rr["lse"]
    assert rel(r["loss"], math.fsum(kl) / S) <= BF16_LOSS_RTOL
    check_row_values(r["lse"], r["kl"], lse, kl)
    rng = np.random.default_rng(81)
    rows = sampled_rows(np.arange(S), p.chunk, N_DH_ROWS, rng)
    check_dh_rows(p, W64, r["dh"], rows, S)
    check_dw_rows(p, W64, r["dW"], lse, np.ones(S, bool), sampled_vocab(p, rows, N_DW_ROWS, rng))
    check_dW_rows_sum_to_zero(r["dW"])


@pytest.mark.parametrize("cfg", ["32k_context", "256k_context"])
def test_full_size_against_oracle(kd, cfg):
    p, meta, ref = stored(cfg)
    r = gpu_fwd_bwd(kd, p)
    S = p.S
    assert rel(r["loss"], meta["loss"]) <= BF16_LOSS_RTOL
    check_row_values(r["lse"], r["kl"], ref["lse"], ref["kl"])
    W64 = p.W.astype(np.float64)
    rng = np.random.default_rng(82)
    rows = sampled_rows(np.arange(S), p.chunk, N_DH_ROWS, rng)
    check_dh_rows(p, W64, r["dh"], rows, S)
    check_dw_rows(p, W64, r["dW"], ref["lse"], np.ones(S, bool),
                  sampled_vocab(p, rows, N_DW_ROWS, rng))
    check_dW_rows_sum_to_zero(r["dW"])


def test_full_entropy_selective(kd):
    # S=32768 H=2048 V=151936 K=100, top 20% by entropy, chunk 1024, T=1
    p, meta, ref = stored("entropy_selective")
    S = p.S
    hidden, W, ids, tl = to_device(p)
    ent = kd.kd_student_entropy(hidden, W)
    mask, idx, cnt = kd.kd_select_top_fraction(ent, hidden, W, 20, 100)
    torch.cuda.synchronize()
    got_e = ent.cpu().numpy()
    assert np.max(np.abs(got_e - ref["entropy"])) <= 2e-5
    rmask, ridx, rk = oracle_select_top_fraction(ref["entropy"], 20, 100)
    assert np.array_equal(ridx, ref["idx"])
    assert cnt == rk == (20 * S) // 100
    assert np.array_equal(idx.cpu().numpy(), ridx)
    del hidden, W, ids, tl, ent, idx
    m = mask.cpu().numpy().astype(bool)
    r = gpu_fwd_bwd(kd, p, mask=m)
    assert rel(r["loss"], meta["loss"]) <= BF16_LOSS_RTOL
    check_row_values(r["lse"][ridx], r["kl"][ridx], ref["lse"], ref["kl"])
    # unselected rows take no part: zero dHidden, zero lse
    off = np.flatnonzero(~m)
    assert np.all(r["dh"][off] == 0.0)
    assert np.all(r["lse"][off] == 0.0)
    W64 = p.W.astype(np.float64)
    rng = np.random.default_rng(83)
    rows = sampled_rows(ridx, p.chunk, N_DH_ROWS, rng)
    check_dh_rows(p, W64, r["dh"], rows, int(rk))
    lse_all = np.zeros(S)
    lse_all[ridx] = ref["lse"]
    check_dw_rows(p, W64, r["dW"], lse_all, m, sampled_vocab(p, rows, N_DW_ROWS, rng))
    check_dW_rows_sum_to_zero(r["dW"])


@pytest.mark.parametrize("form", ["forward_chunked", "dense"])
def test_full_32k_context_comparator_forms(kd, form):
    # the comparator forms at the 32K-context size (the dense form's grids take
    # about 66 GB of workspace): loss, every row's lse and KL against the stored
    # oracle values; dHidden at 256 rows and dW at 128 vocabulary rows
    p, meta, ref = stored("32k_context")
    code = kd.KD_FORM_DENSE if form == "dense" else kd.KD_FORM_FORWARD_CHUNKED
    hidden, W, ids, tl = to_device(p)
    out = kd.kd_kl_comparator_fwd(hidden, W, ids, tl, code, p.T, p.chunk, want_kl_rows=True)
    g = torch.ones(1, dtype=torch.float32, device="cuda")
    dh, dW = kd.kd_kl_comparator_bwd(hidden, W, ids, tl, out["lse"], g, code, out["workspace"],
                                     p.T, p.chunk)
    torch.cuda.synchronize()
    del out["workspace"]
    assert rel(float(out["loss"][0]), meta["loss"]) <= BF16_LOSS_RTOL
    check_row_values(out["lse"].cpu().numpy(), out["kl_rows"].cpu().numpy(), ref["lse"], ref["kl"])
    W64 = p.W.astype(np.float64)
    rng = np.random.default_rng(84)
    rows = sampled_rows(np.arange(p.S), p.chunk, 256, rng)
    check_dh_rows(p, W64, dh.cpu().numpy(), rows, p.S)
    check_dw_rows(p, W64, dW, ref["lse"], np.ones(p.S, bool), sampled_vocab(p, rows, 128, rng))


@pytest.mark.parametrize("cfg", ["32k_context", "256k_context"])
def test_full_size_one_call(kd, cfg):
    # the forward and backward in one call, with the configuration's chunk
    p, meta, ref = stored(cfg)
    hidden, W, ids, tl = to_device(p)
    g = torch.ones(1, dtype=torch.float32, device="cuda")
    out = kd.kd_topk_kl_fwd_bwd(hidden, W, ids, tl, g, p.T, p.chunk, want_kl_rows=True)
    torch.cuda.synchronize()
    del hidden, W, ids, tl
    assert rel(float(out["loss"][0]), meta["loss"]) <= BF16_LOSS_RTOL
    check_row_values(out["lse"].cpu().numpy(), out["kl_rows"].cpu().numpy(), ref["lse"], ref["kl"])
    W64 = p.W.astype(np.float64)
    rng = np.random.default_rng(85)
    rows = sampled_rows(np.arange(p.S), p.chunk, N_DH_ROWS, rng)
    check_dh_rows(p, W64, out["dhidden"].cpu().numpy(), rows, p.S)
    check_dw_rows(p, W64, out["dW"], ref["lse"], np.ones(p.S, bool),
                  sampled_vocab(p, rows, N_DW_ROWS, rng))
    check_dW_rows_sum_to_zero(out["dW"])
