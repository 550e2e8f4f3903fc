"""The forward entry point that allocates nothing (kd_topk_kl_fwd_noalloc,
for callers that cannot allocate device memory) against kd_topk_kl_fwd,
through the C ABI: the same kernels on the same inputs give the same bits.
Two calls in a row on the library's one scratch array, the second on a
smaller problem (with a mask), and a problem beyond the scratch rejected
before any launch."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

from kd_synth import make_problem  # noqa: E402
from oracle import oracle_loss_grads  # noqa: E402
from tests.kd_gpu_helpers import BF16_LOSS_RTOL, rel, to_device  # noqa: E402


@pytest.fixture(scope="module")
def kd():
    import chunked_top_kl_amd as m
    return m


def same_bits(a, b):
    return torch.equal(a.view(torch.int32), b.view(torch.int32))


@pytest.mark.parametrize("case", [0, 1])
def test_noalloc_forward_equals_workspace_forward(kd, case):
    # case 0: the larger problem first, then the smaller one with a mask;
    # case 1: the other order (the second call reuses what the first left)
    shapes = [dict(S=3000, H=256, V=5003, K=20, T=2.0, chunk=512, seed=91, masked=False),
              dict(S=700, H=128, V=3001, K=7, T=1.0, chunk=256, seed=92, masked=True)]
    if case == 1:
        shapes = shapes[::-1]
    for sh in shapes:
        p = make_problem(sh["S"], sh["H"], sh["V"], sh["K"], T=sh["T"], chunk=sh["chunk"],
                         seed=sh["seed"])
        hidden, W, ids, tl = to_device(p)
        mask = None
        if sh["masked"]:
            m = np.random.default_rng(sh["seed"]).random(p.S) < 0.7
            mask = torch.from_numpy(m.astype(np.uint8)).cuda()
        ref = kd.kd_topk_kl_fwd(hidden, W, ids, tl, p.T, p.chunk, mask, want_kl_rows=True,
                                want_z_topk=True)
        got = kd.kd_topk_kl_fwd_noalloc(hidden, W, ids, tl, p.T, p.chunk, mask, want_kl_rows=True,
                                        want_z_topk=True)
        torch.cuda.synchronize()
        for key in ("loss", "lse", "kl_rows", "z_topk"):
            assert same_bits(got[key], ref[key]), key
        want = oracle_loss_grads(p.hidden, p.W, p.ids, p.tlogits, T=p.T,
                                 mask=None if mask is None else mask.cpu().numpy(), chunk=256)
        assert rel(float(got["loss"][0]), want["loss"]) <= BF16_LOSS_RTOL


def test_noalloc_rejects_a_problem_beyond_its_scratch(kd):
    # about S * (16 K + 13) bytes: 60000 rows of 100 entries need ~97 MB > 64 MiB
    S, H, V, K = 60000, 64, 1000, 100
    hidden = torch.zeros(S, H, dtype=torch.bfloat16, device="cuda")
    W = torch.zeros(V, H, dtype=torch.bfloat16, device="cuda")
    ids = torch.zeros(S, K, dtype=torch.int32, device="cuda")
    tl = torch.zeros(S, K, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(kd.KdError) as ei:
        kd.kd_topk_kl_fwd_noalloc(hidden, W, ids, tl, 1.0, 1024)
    assert ei.value.code == 6
