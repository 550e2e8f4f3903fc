"""GPU parity of the HIP library against the fp64 oracle (through the C ABI).

Sizes here are ones the oracle finishes in seconds while still spanning several
256-row tiles, ragged tails in S, V, H and the chunk, masks, duplicate ids,
-inf teacher entries and temperature 2. Tolerances (bf16 inputs, fp32
accumulation): loss relative error <= 1e-3, gradients max-abs error <=
2e-2 * max |oracle gradient|; indexing outputs are compared bit for bit.
"""
import math

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

from kd_synth import make_problem, bf16_bits_from_f32, f32_from_bf16_bits  # noqa: E402
from oracle import (oracle_loss_grads, oracle_entropy, oracle_select_top_fraction,  # noqa: E402
                    oracle_validate_topk)
from tests.kd_gpu_helpers import (BF16_GRAD_FRAC, BF16_LOSS_RTOL, max_abs_frac, rel,  # noqa: E402
                                  to_device, np_bf16_to_torch)


@pytest.fixture(scope="module")
def kd():
    import chunked_top_kl_amd as m
    return m


def run_fwd_bwd(kd, p, mask=None, grad=1.0, want=True):
    hidden, W, ids, tl = to_device(p)
    mk = None if mask is None else torch.from_numpy(mask.astype(np.uint8)).cuda()
    out = kd.kd_topk_kl_fwd(hidden, W, ids, tl, p.T, p.chunk, mk, want_kl_rows=want,
                            want_z_topk=want)
    g = torch.tensor([grad], dtype=torch.float32, device="cuda")
    dh, dW = kd.kd_topk_kl_bwd(hidden, W, ids, tl, out["lse"], g, p.T, p.chunk, mk)
    torch.cuda.synchronize()
    res = {k: (v.cpu().numpy() if v is not None else None) for k, v in out.items()}
    res["dH"] = dh.cpu().numpy()
    res["dW"] = dW.cpu().numpy()
    return res


def check_against_oracle(p, got, mask=None, grad=1.0, loss_rtol=BF16_LOSS_RTOL,
                         grad_frac=BF16_GRAD_FRAC, chunk=None):
    ref = oracle_loss_grads(p.hidden, p.W, p.ids, p.tlogits, T=p.T, mask=mask, grad_loss=grad,
                            chunk=chunk)
    print(f"loss gpu={float(got['loss'][0]):.7f} oracle={ref['loss']:.7f} N={ref['N']}")
    assert rel(float(got["loss"][0]), ref["loss"]) <= loss_rtol
    v = ref["valid"]
    assert np.max(np.abs(got["lse"][v] - ref["lse"][v])) <= 1e-4 * max(1.0, np.max(np.abs(ref["lse"][v])))
    assert np.all(got["lse"][~v] == 0.0)
    if got.get("kl_rows") is not None:
        assert np.max(np.abs(got["kl_rows"][v] - ref["kl_rows"][v])) <= 1e-3 * max(1.0, np.max(ref["kl_rows"][v]))
    eh, ew = max_abs_frac(got["dH"], ref["dH"]), max_abs_frac(got["dW"], ref["dW"])
    print(f"dH err frac={eh:.3e} dW err frac={ew:.3e}")
    assert eh <= grad_frac and ew <= grad_frac
    assert np.all(got["dH"][~v] == 0.0)
    return ref


def test_c1_tiny_fp32(kd):
    # S=128, H=64, V=1000, K=10, T=1, fp32 throughout, chunk 32
    p = make_problem(128, 64, 1000, 10, T=1.0, chunk=32, hw_dtype="f32", tl_dtype="f32", seed=1001)
    got = run_fwd_bwd(kd, p)
    check_against_oracle(p, got, loss_rtol=1e-5, grad_frac=1e-4)


@pytest.mark.parametrize("S,H,V,K,chunk,T", [
    (1000, 136, 1537, 17, 96, 2.0),     # ragged S/V/H/chunk, V % 8 != 0, H % 64 != 0
    (300, 64, 4099, 100, 300, 1.0),     # one chunk, V % 256 tail
    (513, 256, 777, 33, 512, 0.7),      # S just past two tiles
    (640, 224, 2003, 9, 320, 1.0),      # H tail of 224 columns: 4 and 3 column blocks
])
def test_bf16_ragged(kd, S, H, V, K, chunk, T):
    p = make_problem(S, H, V, K, T=T, chunk=chunk, seed=S + V)
    got = run_fwd_bwd(kd, p, grad=1.3)
    check_against_oracle(p, got, grad=1.3)


def test_mask_missing_rows_duplicates_neg_inf(kd):
    S, H, V, K = 777, 128, 3001, 12
    p = make_problem(S, H, V, K, T=1.5, chunk=200, seed=77)
    rng = np.random.Generator(np.random.PCG64(5))
    # duplicate ids in some rows, -inf entries in others, two rows entirely -inf
    p.ids[5, 3] = p.ids[5, 4]
    p.ids[9, :] = p.ids[9, 0]
    tl = p.tlogits.copy()
    tl[11, 2:6] = -np.inf
    tl[20, :] = -np.inf
    tl[21, :] = -np.inf
    p.tl_bits = bf16_bits_from_f32(tl)
    p.tlogits = f32_from_bf16_bits(p.tl_bits)
    mask = (rng.random(S) < 0.1).astype(np.uint8)
    mask[[5, 9, 11, 20]] = 1
    got = run_fwd_bwd(kd, p, mask=mask)
    ref = check_against_oracle(p, got, mask=mask)
    assert ref["N"] == int(mask.sum()) - int(mask[20]) - int(mask[21])
    # also without mask: missing rows are excluded
    got2 = run_fwd_bwd(kd, p)
    check_against_oracle(p, got2)


@pytest.mark.parametrize("K", [65, 128, 129, 300])
def test_prepass_sort_paths_long_duplicate_runs(kd, K):
    """Both teacher-prepass sorts (rows of up to 128 entries in registers, longer
    rows in LDS) with runs of equal ids long enough to cross lanes and the two
    entries a lane holds, and -inf entries; the probabilities of equal ids
    add."""
    # V < 4K: the input recipe then draws each row as a random K-subset (its
    # redraw of colliding rows would take very long at K = 300 of 3001)
    S, H, V = 300, 64, 4 * K - 1
    p = make_problem(S, H, V, K, T=1.3, chunk=128, seed=500 + K)
    rng = np.random.Generator(np.random.PCG64(K))
    rows = np.arange(0, S, 2)
    p.ids[rows] = rng.integers(0, 20, size=(len(rows), K)).astype(np.int32)
    p.ids[7, : K // 2] = 3                      # one run over half the row
    tl = p.tlogits.copy()
    tl[11, 1:K:3] = -np.inf
    p.tl_bits = bf16_bits_from_f32(tl)
    p.tlogits = f32_from_bf16_bits(p.tl_bits)
    got = run_fwd_bwd(kd, p, grad=0.7)
    check_against_oracle(p, got, grad=0.7)


def test_z_topk_gathers_the_cached_ids_exactly(kd):
    # W[v,0] = floor(v/256), W[v,1] = v mod 256 (exact in bf16); even rows e0, odd rows e1,
    # each pair shares its teacher ids: z at the gathered ids decodes back to the id.
    S, H, V, K = 512, 64, 60001, 37
    p = make_problem(S, H, V, K, T=1.0, chunk=128, seed=9)
    W = np.zeros((V, H), dtype=np.float32)
    W[:, 0] = np.arange(V) // 256
    W[:, 1] = np.arange(V) % 256
    hid = np.zeros((S, H), dtype=np.float32)
    hid[0::2, 0] = 1.0
    hid[1::2, 1] = 1.0
    p.ids[1::2] = p.ids[0::2]
    p.W_bits, p.hidden_bits = bf16_bits_from_f32(W), bf16_bits_from_f32(hid)
    p.W, p.hidden = f32_from_bf16_bits(p.W_bits), f32_from_bf16_bits(p.hidden_bits)
    got = run_fwd_bwd(kd, p)
    z = got["z_topk"]
    assert not np.any(np.isnan(z))
    dec = 256 * z[0::2].astype(np.int64) + z[1::2].astype(np.int64)
    assert np.array_equal(z, np.round(z))
    assert np.array_equal(dec, p.ids[0::2].astype(np.int64))
    check_against_oracle(p, got)


def test_determinism_bitwise(kd):
    p = make_problem(700, 192, 5000, 50, T=1.0, chunk=256, seed=3)
    a = run_fwd_bwd(kd, p)
    b = run_fwd_bwd(kd, p)
    for k in ("loss", "lse", "kl_rows", "z_topk", "dH", "dW"):
        assert np.array_equal(a[k].view(np.uint32), b[k].view(np.uint32)), k


def test_chunk_size_only_changes_rounding(kd):
    p = make_problem(900, 128, 3000, 20, T=1.0, chunk=64, seed=4)
    a = run_fwd_bwd(kd, p)
    p.chunk = 900
    b = run_fwd_bwd(kd, p)
    assert a["loss"][0] == b["loss"][0]          # the forward does not depend on the chunk
    assert max_abs_frac(a["dH"], b["dH"]) < 1e-6
    assert max_abs_frac(a["dW"], b["dW"]) < 1e-5


def test_accumulate_dW(kd):
    p = make_problem(400, 64, 2000, 8, T=1.0, chunk=128, seed=6)
    hidden, W, ids, tl = to_device(p)
    out = kd.kd_topk_kl_fwd(hidden, W, ids, tl, p.T, p.chunk)
    g = torch.ones(1, dtype=torch.float32, device="cuda")
    _, dW1 = kd.kd_topk_kl_bwd(hidden, W, ids, tl, out["lse"], g, p.T, p.chunk)
    base = torch.full_like(dW1, 0.25)
    _, dW2 = kd.kd_topk_kl_bwd(hidden, W, ids, tl, out["lse"], g, p.T, p.chunk, dW=base.clone(),
                               accumulate_dW=True)
    assert torch.allclose(dW2 - 0.25, dW1, rtol=0, atol=1e-6)


def test_dw_groups_of_chunks(kd):
    # dW contracts up to 8192 tokens of consecutive chunks per launch: with a
    # chunk of 2000 rows a group holds 4 chunks, so S = 9000 gives one full
    # group and a second group of one partial chunk (1000 rows)
    p = make_problem(9000, 64, 1000, 10, T=1.0, chunk=2000, seed=21)
    got = run_fwd_bwd(kd, p, want=False)
    check_against_oracle(p, got, chunk=1000)


def test_dw_groups_with_mask_ending_inside_a_group(kd):
    # the masked rows compact to N = 4500: chunks 0 and 1 are full, chunk 2
    # holds 500 rows, chunk 3 and the second group hold none; dW accumulates
    # into a non-zero buffer
    p = make_problem(9000, 64, 1000, 10, T=2.0, chunk=2000, seed=22)
    rng = np.random.default_rng(5)
    keep = np.sort(rng.choice(9000, size=4500, replace=False))
    mask = np.zeros(9000, dtype=bool)
    mask[keep] = True
    got = run_fwd_bwd(kd, p, mask=mask, want=False)
    ref = check_against_oracle(p, got, mask=mask, chunk=1000)
    hidden, W, ids, tl = to_device(p)
    mk = torch.from_numpy(mask.astype(np.uint8)).cuda()
    out = kd.kd_topk_kl_fwd(hidden, W, ids, tl, p.T, p.chunk, mk)
    g = torch.ones(1, dtype=torch.float32, device="cuda")
    base = torch.full((p.V, p.H), 0.5, dtype=torch.float32, device="cuda")
    _, dW2 = kd.kd_topk_kl_bwd(hidden, W, ids, tl, out["lse"], g, p.T, p.chunk, mk,
                               dW=base, accumulate_dW=True)
    err = float(np.max(np.abs(dW2.cpu().numpy() - 0.5 - ref["dW"])))
    assert err <= BF16_GRAD_FRAC * float(np.max(np.abs(ref["dW"])))


def test_empty_problems(kd):
    # S = 0: loss 0, dW written as zeros
    W = torch.randn(300, 64, device="cuda").to(torch.bfloat16)
    hidden = torch.empty(0, 64, device="cuda", dtype=torch.bfloat16)
    ids = torch.empty(0, 5, device="cuda", dtype=torch.int32)
    tl = torch.empty(0, 5, device="cuda", dtype=torch.bfloat16)
    out = kd.kd_topk_kl_fwd(hidden, W, ids, tl, 1.0, 16)
    g = torch.ones(1, dtype=torch.float32, device="cuda")
    dh, dW = kd.kd_topk_kl_bwd(hidden, W, ids, tl, out["lse"], g, 1.0, 16,
                               dW=torch.full((300, 64), 7.0, device="cuda"))
    torch.cuda.synchronize()
    assert float(out["loss"][0]) == 0.0 and dh.numel() == 0
    assert torch.all(dW == 0)
    # all positions masked out: N = 0
    p = make_problem(260, 64, 1000, 10, seed=8)
    got = run_fwd_bwd(kd, p, mask=np.zeros(260, dtype=np.uint8))
    assert got["loss"][0] == 0.0 and np.all(got["dH"] == 0) and np.all(got["dW"] == 0)
    assert np.all(got["lse"] == 0) and np.all(np.isnan(got["z_topk"]))


def test_fp32_h_tail(kd):
    # fp32 contractions with H = 200: the waves of the h tile compute 4 and
    # 3 of their column blocks
    p = make_problem(300, 200, 1500, 8, T=1.0, chunk=128, hw_dtype="f32", tl_dtype="f32",
                     seed=12)
    check_against_oracle(p, run_fwd_bwd(kd, p), loss_rtol=1e-5, grad_frac=1e-4)


def test_k1_and_k_equals_v(kd):
    p = make_problem(300, 64, 500, 1, T=1.0, chunk=100, seed=10)
    check_against_oracle(p, run_fwd_bwd(kd, p))
    p = make_problem(200, 64, 64, 64, T=2.0, chunk=64, seed=11)
    check_against_oracle(p, run_fwd_bwd(kd, p))


@pytest.mark.parametrize("S,H,V,K,chunk,T", [
    (512, 3072, 128256, 100, 1024, 1.0),    # 8K-context config shapes (S reduced)
    (384, 2880, 201088, 100, 256, 1.0),     # 32K-context config shapes, two chunks
    (300, 3072, 128256, 100, 2048, 2.0),    # 256K-context config shapes, T = 2
])
def test_config_shapes_reduced_S(kd, S, H, V, K, chunk, T):
    p = make_problem(S, H, V, K, T=T, chunk=chunk, seed=1000 + S)
    got = run_fwd_bwd(kd, p, want=False)
    check_against_oracle(p, got, chunk=128)


def test_validate_counts(kd):
    p = make_problem(50, 64, 1000, 6, seed=12)
    ids = p.ids.copy()
    ids[3, 1] = -4
    ids[7, 0] = 1000
    ids[7, 5] = 5000
    tl = p.tlogits.copy()
    tl[10, :] = -np.inf
    tl[11, 2] = np.nan
    tl[12, 0] = np.inf
    ref = oracle_validate_topk(ids, tl, 1000)
    got = kd.kd_validate_topk(torch.from_numpy(ids).cuda(),
                              np_bf16_to_torch(bf16_bits_from_f32(tl.astype(np.float32))), 1000)
    assert got == ref == (3, 1, 2)
    # out-of-range ids are skipped by the loss kernels (no fault), rows stay finite
    hidden, W, _, tlt = to_device(p)
    out = kd.kd_topk_kl_fwd(hidden, W, torch.from_numpy(ids).cuda(), tlt, 1.0, 16)
    torch.cuda.synchronize()
    assert math.isfinite(float(out["loss"][0]))


def test_workspace_error_surfaces(kd):
    p = make_problem(64, 64, 500, 4, seed=13)
    hidden, W, ids, tl = to_device(p)
    small = torch.empty(1024, dtype=torch.uint8, device="cuda")
    with pytest.raises(kd.KdError):
        prob = kd.make_problem(64, 64, 500, 4, 16, 1.0, kd.KD_BF16, kd.KD_BF16)
        import ctypes
        z = torch.empty(64, device="cuda")
        rc = kd.lib.kd_topk_kl_fwd(ctypes.byref(prob), kd._ptr(hidden), kd._ptr(W), kd._ptr(ids),
                                   kd._ptr(tl), None, kd._ptr(z), kd._ptr(z), None, None,
                                   kd._ptr(small), small.numel(), None)
        kd._check(rc, "fwd")


# ---------------------------------------------------------------- entropy and selection

def test_entropy_matches_oracle(kd):
    p = make_problem(600, 256, 5003, 4, seed=14, hidden_std=2.0)
    hidden, W, _, _ = to_device(p)
    ent = kd.kd_student_entropy(hidden, W).cpu().numpy()
    ref = oracle_entropy(p.hidden, p.W, chunk=200)
    err = np.max(np.abs(ent - ref))
    print(f"entropy max abs err {err:.3e}")
    assert err <= 2e-5


def test_entropy_and_selection_with_large_logits(kd):
    # logits of standard deviation 4 (hidden ~ N(0, 16), W ~ N(0, 1/H)) at a
    # hidden size of 2048: the fp32-path entropies stay within the 2e-5 nats
    # that the selection's band assumes, and the kept set is the fp64 one
    S, H, V = 2000, 2048, 6007
    p = make_problem(S, H, V, 4, seed=16, hidden_std=4.0)
    hidden, W, _, _ = to_device(p)
    ent = kd.kd_student_entropy(hidden, W)
    mask, idx, cnt = kd.kd_select_top_fraction(ent, hidden, W, 20, 100)
    ref = oracle_entropy(p.hidden, p.W, chunk=500)
    err = float(np.max(np.abs(ent.cpu().numpy() - ref)))
    print(f"entropy max abs err at logit std 4: {err:.3e}")
    assert err <= 2e-5
    rmask, ridx, rk = oracle_select_top_fraction(ref, 20, 100)
    assert cnt == rk
    assert np.array_equal(idx.cpu().numpy(), ridx)


def test_selection_widens_the_band_for_less_accurate_entropies(kd):
    # entropies given with errors of up to 1e-4 nats, five times the band's
    # least bound: a band of +-4e-5 would leave positions on the wrong side
    # of the cut, but the error measured on the probe positions widens it, so
    # the kept set is still the fp64 oracle's
    S, H, V = 3000, 128, 4001
    p = make_problem(S, H, V, 4, seed=19, hidden_std=0.2)
    hidden, W, _, _ = to_device(p)
    ent = kd.kd_student_entropy(hidden, W)
    noise = np.random.default_rng(20).uniform(-1e-4, 1e-4, size=S)
    noisy = ent + torch.from_numpy(noise).cuda()
    mask, idx, cnt = kd.kd_select_top_fraction(noisy, hidden, W, 20, 100)
    ref_e = oracle_entropy(p.hidden, p.W, chunk=500)
    rmask, ridx, rk = oracle_select_top_fraction(ref_e, 20, 100)
    assert cnt == rk
    assert np.array_equal(idx.cpu().numpy(), ridx)
    assert np.array_equal(mask.cpu().numpy(), rmask)
    # the noisy values alone decide differently
    _, nidx, _ = oracle_select_top_fraction(ref_e + noise, 20, 100)
    assert not np.array_equal(nidx, ridx)


@pytest.mark.parametrize("case", ["spread", "crowded", "ties"])
def test_selection_index_set_bit_exact(kd, case):
    S, H, V = 3000, 128, 4001
    p = make_problem(S, H, V, 4, seed=15, hidden_std=(0.05 if case == "crowded" else 1.5))
    if case == "ties":
        p.hidden_bits[1::3] = p.hidden_bits[0::3][: len(p.hidden_bits[1::3])]
        p.hidden = f32_from_bf16_bits(p.hidden_bits)
    hidden, W, _, _ = to_device(p)
    ent = kd.kd_student_entropy(hidden, W)
    mask, idx, cnt = kd.kd_select_top_fraction(ent, hidden, W, 20, 100)
    ref_e = oracle_entropy(p.hidden, p.W, chunk=500)
    rmask, ridx, rk = oracle_select_top_fraction(ref_e, 20, 100)
    assert cnt == rk
    assert np.array_equal(idx.cpu().numpy(), ridx)
    assert np.array_equal(mask.cpu().numpy(), rmask)


@pytest.mark.parametrize("H,hw", [(200, "bf16"), (1096, "bf16"), (200, "f32")])
def test_selection_ragged_hidden(kd, H, hw):
    # hidden widths that leave a partial step (not a multiple of 64) and a
    # second, ragged piece of the band rows (above 1024), and fp32 inputs;
    # a crowded entropy distribution so that the fp64 refinement decides
    S, V = 1200, 2999
    p = make_problem(S, H, V, 4, seed=17, hidden_std=0.05, hw_dtype=hw, tl_dtype="f32")
    hidden, W, _, _ = to_device(p)
    ent = kd.kd_student_entropy(hidden, W)
    mask, idx, cnt = kd.kd_select_top_fraction(ent, hidden, W, 20, 100)
    ref_e = oracle_entropy(p.hidden, p.W, chunk=400)
    rmask, ridx, rk = oracle_select_top_fraction(ref_e, 20, 100)
    assert cnt == rk
    assert np.array_equal(idx.cpu().numpy(), ridx)
    assert np.array_equal(mask.cpu().numpy(), rmask)


def test_selection_band_larger_than_a_refinement_piece(kd):
    # entropies crowded well inside the fp32-path error bound: the whole band
    # (about S positions, several pieces of 4096) is recomputed in fp64 and
    # ranked there; the kept set equals the fp64 oracle's bit for bit
    S, H, V = 20000, 128, 4001
    p = make_problem(S, H, V, 4, seed=18, hidden_std=0.01)
    hidden, W, _, _ = to_device(p)
    ent = kd.kd_student_entropy(hidden, W)
    kd.kd_profile_reset()
    kd.kd_profile_enable(True)
    mask, idx, cnt = kd.kd_select_top_fraction(ent, hidden, W, 20, 100)
    torch.cuda.synchronize()
    kd.kd_profile_enable(False)
    steps = kd.kd_profile_read()
    kd.kd_profile_reset()
    # a refinement launch and an entropy launch per piece of 4096 band rows
    # (bf16 rows are refined one piece per launch): more than one piece ran
    assert steps["select_refine_fp64"][0] >= 4
    ref_e = oracle_entropy(p.hidden, p.W, chunk=2000)
    rmask, ridx, rk = oracle_select_top_fraction(ref_e, 20, 100)
    assert cnt == rk
    assert np.array_equal(idx.cpu().numpy(), ridx)
    assert np.array_equal(mask.cpu().numpy(), rmask)


def test_entropy_selective_variant_reduced(kd):
    # entropy-selective config shapes (H=2048, V=151936) at S=2048: entropy over all
    # positions, top 20% kept, then the KL forward and backward on the kept rows only
    S, H, V, K = 2048, 2048, 151936, 100
    p = make_problem(S, H, V, K, T=1.0, chunk=1024, seed=1005)
    hidden, W, ids, tl = to_device(p)
    ent = kd.kd_student_entropy(hidden, W)
    mask, idx, cnt = kd.kd_select_top_fraction(ent, hidden, W, 20, 100)
    ref_e = oracle_entropy(p.hidden, p.W, chunk=256)
    rmask, ridx, rk = oracle_select_top_fraction(ref_e, 20, 100)
    assert cnt == rk == (20 * S) // 100
    assert np.array_equal(idx.cpu().numpy(), ridx)
    got = run_fwd_bwd(kd, p, mask=mask.cpu().numpy())
    check_against_oracle(p, got, mask=rmask, chunk=256)


def test_autograd_function(kd):
    p = make_problem(300, 64, 1000, 10, T=1.0, chunk=100, seed=16)
    hidden, W, ids, tl = to_device(p)
    h = hidden.clone().requires_grad_(True)
    w = W.clone().requires_grad_(True)
    loss = kd.kd_topk_kl(h, w, ids, tl, 1.0, 100) * 2.0
    loss.backward()
    ref = oracle_loss_grads(p.hidden, p.W, p.ids, p.tlogits, T=1.0, grad_loss=2.0)
    assert rel(float(loss) / 2.0, ref["loss"]) <= BF16_LOSS_RTOL
    assert max_abs_frac(h.grad.float().cpu().numpy(), ref["dH"]) <= BF16_GRAD_FRAC
    assert max_abs_frac(w.grad.float().cpu().numpy(), ref["dW"]) <= BF16_GRAD_FRAC
