"""Host-side checks of the C ABI that need no GPU: the library loads, exports every
symbol the header declares, and rejects invalid arguments before touching the device."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kd_topk_kl.h")

kd = pytest.importorskip("chunked_top_kl_amd", reason="HIP library not built")

KD_OK, KD_ERR_NULL, KD_ERR_SHAPE, KD_ERR_DTYPE, KD_ERR_TEMPERATURE = 0, 1, 2, 3, 4
KD_ERR_CHUNK, KD_ERR_WORKSPACE, KD_ERR_ARG = 5, 6, 10


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b(kd_\w+)\s*\(", src, flags=re.M)
    return sorted(set(names))


def test_header_symbols_exported():
    names = declared_functions()
    assert "kd_topk_kl_fwd" in names and "kd_topk_kl_bwd" in names
    assert len(names) >= 11
    for n in names:
        assert hasattr(kd.lib, n), f"{n} not exported by {kd.LIB_PATH}"


def test_version_and_status_strings():
    assert kd.kd_abi_version() == 7
    for c in range(11):
        assert kd.kd_status_str(c).startswith("KD_")
    assert "unknown" in kd.kd_status_str(99)


def prob(**kw):
    d = dict(S=128, H=64, V=1000, K=10, chunk=32, T=1.0, hw=kd.KD_BF16, tl=kd.KD_BF16, kind=0)
    d.update(kw)
    return kd.make_problem(d["S"], d["H"], d["V"], d["K"], d["chunk"], d["T"], d["hw"], d["tl"],
                           d["kind"])


@pytest.mark.parametrize("kw,code", [
    (dict(S=-1), KD_ERR_SHAPE), (dict(H=0), KD_ERR_SHAPE), (dict(H=60), KD_ERR_SHAPE),
    (dict(V=0), KD_ERR_SHAPE), (dict(K=0), KD_ERR_SHAPE), (dict(K=1001), KD_ERR_SHAPE),
    (dict(K=5000, V=10000), KD_ERR_SHAPE), (dict(hw=7), KD_ERR_DTYPE), (dict(tl=-1), KD_ERR_DTYPE),
    (dict(T=0.0), KD_ERR_TEMPERATURE), (dict(T=-1.0), KD_ERR_TEMPERATURE),
    (dict(T=float("nan")), KD_ERR_TEMPERATURE), (dict(T=float("inf")), KD_ERR_TEMPERATURE),
    (dict(chunk=0), KD_ERR_CHUNK), (dict(kind=2), 10), (dict(kind=-1), 10),
])
def test_invalid_problems_rejected(kw, code):
    p = prob(**kw)
    assert kd.kd_topk_kl_workspace_bytes(p) == 0
    fake = ctypes.c_void_p(0x1000)
    rc = kd.lib.kd_topk_kl_fwd(ctypes.byref(p), fake, fake, fake, fake, None, fake, fake, None,
                               None, fake, 1 << 40, None)
    assert rc == code


def test_null_and_workspace_errors():
    p = prob()
    fake = ctypes.c_void_p(0x1000)
    assert kd.lib.kd_topk_kl_fwd(None, fake, fake, fake, fake, None, fake, fake, None, None, fake,
                                 1 << 40, None) == KD_ERR_NULL
    assert kd.lib.kd_topk_kl_fwd(ctypes.byref(p), None, fake, fake, fake, None, fake, fake, None,
                                 None, fake, 1 << 40, None) == KD_ERR_NULL
    need = kd.kd_topk_kl_workspace_bytes(p)
    assert need > 0
    # too small, misaligned, NULL workspace
    assert kd.lib.kd_topk_kl_fwd(ctypes.byref(p), fake, fake, fake, fake, None, fake, fake, None,
                                 None, ctypes.c_void_p(0x10000), need - 1, None) == KD_ERR_WORKSPACE
    assert kd.lib.kd_topk_kl_fwd(ctypes.byref(p), fake, fake, fake, fake, None, fake, fake, None,
                                 None, ctypes.c_void_p(0x10010), need, None) == KD_ERR_WORKSPACE
    assert kd.lib.kd_topk_kl_bwd(ctypes.byref(p), fake, fake, fake, fake, None, fake, fake, fake,
                                 fake, 2, ctypes.c_void_p(0x10000), need, None) == KD_ERR_ARG
    cnt = ctypes.c_int64(0)
    assert kd.lib.kd_select_top_fraction(ctypes.byref(p), fake, fake, fake, 3, 2, fake, None,
                                         ctypes.byref(cnt), ctypes.c_void_p(0x10000), need,
                                         None) == KD_ERR_ARG


def test_workspace_linear_in_S_and_bounded_in_V():
    sizes = [kd.kd_topk_kl_workspace_bytes(prob(S=S, H=3072, V=128256, K=100, chunk=2048))
             for S in (16384, 32768, 65536, 131072, 262144)]
    d = [b - a for a, b in zip(sizes, sizes[1:])]
    per_token = [x / dS for x, dS in zip(d, (16384, 32768, 65536, 131072))]
    # per-token slope (teacher tables + split partials) stays a few KB per token; the
    # split count of the sweep varies a little with the number of token tiles
    assert max(per_token) < 1.3 * min(per_token)
    assert 1000 < min(per_token) and max(per_token) < 6000
    # the one V-sized buffer (bf16) is the gradient tiles of a dW group of chunks,
    # about 8192 token rows whatever the chunk: it does not grow with S or chunk
    a = kd.kd_topk_kl_workspace_bytes(prob(S=32768, H=2880, V=201088, K=100, chunk=1024))
    b = kd.kd_topk_kl_workspace_bytes(prob(S=32768, H=2880, V=201088, K=100, chunk=2048))
    c = kd.kd_topk_kl_workspace_bytes(prob(S=262144, H=2880, V=201088, K=100, chunk=2048))
    assert min(a, b) >= 8192 * 201088 * 2
    assert abs(b - a) < 1024 * 201088 * 2
    assert c - b < (262144 - 32768) * 6000


def test_signal_and_selection_argument_errors():
    """Host-side rejections of the position-signal and selection entry points."""
    p = prob()
    fake = ctypes.c_void_p(0x1000)
    ws = ctypes.c_void_p(0x10000)
    need = kd.kd_topk_kl_workspace_bytes(p)
    cnt = ctypes.c_int64(0)
    sel = kd.lib.kd_select_by_signal
    for num, den in [(1, 0), (3, 2), (-1, 4), (1, 1 << 31)]:
        assert sel(ctypes.byref(p), fake, None, 1, num, den, fake, None, None, ctypes.byref(cnt), ws,
                   need, None) == KD_ERR_ARG
    assert sel(ctypes.byref(p), fake, fake, -1, 1, 2, fake, None, None, ctypes.byref(cnt), ws,
               need, None) == KD_ERR_ARG
    assert sel(ctypes.byref(p), fake, fake, 129, 1, 2, fake, None, None, ctypes.byref(cnt), ws,
               need, None) == KD_ERR_ARG                      # B > S
    assert sel(ctypes.byref(p), fake, None, 1, 1, 2, fake, None, None, None, ws, need,
               None) == KD_ERR_NULL
    assert sel(ctypes.byref(p), None, None, 1, 1, 2, fake, None, None, ctypes.byref(cnt), ws, need,
               None) == KD_ERR_NULL
    assert sel(ctypes.byref(p), fake, None, 1, 1, 2, fake, None, None, ctypes.byref(cnt), ws,
               need - 1, None) == KD_ERR_WORKSPACE
    above = kd.lib.kd_select_above
    assert above(ctypes.byref(p), fake, float("nan"), fake, None, ctypes.byref(cnt), ws, need,
                 None) == KD_ERR_ARG
    assert above(ctypes.byref(p), None, 0.0, fake, None, ctypes.byref(cnt), ws, need,
                 None) == KD_ERR_NULL
    sig = kd.lib.kd_position_signals
    # ce or teacher uncertainty without labels, teacher uncertainty without the cache
    assert sig(ctypes.byref(p), fake, fake, fake, fake, None, None, fake, None, ws, need,
               None) == KD_ERR_NULL
    assert sig(ctypes.byref(p), fake, fake, None, fake, fake, None, None, fake, ws, need,
               None) == KD_ERR_NULL
    assert sig(ctypes.byref(p), None, fake, fake, fake, fake, fake, None, None, ws, need,
               None) == KD_ERR_NULL
    bad = prob(T=0.0)
    assert sig(ctypes.byref(bad), fake, fake, fake, fake, fake, fake, None, None, ws, need,
               None) == KD_ERR_TEMPERATURE


def test_per_sequence_selection_argument_errors():
    p = prob()
    fake = ctypes.c_void_p(0x1000)
    ws = ctypes.c_void_p(0x10000)
    need = kd.kd_topk_kl_workspace_bytes(p)
    cnt = ctypes.c_int64(0)
    f = kd.lib.kd_select_top_fraction_segments
    assert f(ctypes.byref(p), fake, fake, fake, fake, 4, 3, 2, fake, None, ctypes.byref(cnt), ws,
             need, None) == KD_ERR_ARG
    assert f(ctypes.byref(p), fake, fake, fake, fake, 129, 1, 2, fake, None, ctypes.byref(cnt), ws,
             need, None) == KD_ERR_ARG
    assert f(ctypes.byref(p), fake, fake, fake, None, 4, 1, 2, fake, None, ctypes.byref(cnt), ws,
             need, None) == KD_ERR_NULL
    assert f(ctypes.byref(p), None, fake, fake, fake, 4, 1, 2, fake, None, ctypes.byref(cnt), ws,
             need, None) == KD_ERR_NULL
    assert f(ctypes.byref(p), fake, fake, fake, fake, 4, 1, 2, fake, None, ctypes.byref(cnt), ws,
             need - 1, None) == KD_ERR_WORKSPACE


def test_teacher_sample_argument_errors():
    fake = ctypes.c_void_p(0x1000)
    ws = ctypes.c_void_p(0x10000)
    f = kd.lib.kd_teacher_sample
    p = prob(K=100)
    need = kd.kd_teacher_sample_workspace_bytes(p)
    assert need > 0
    assert kd.kd_teacher_sample_workspace_bytes(prob(K=1001)) == 0       # N > V
    assert f(ctypes.byref(prob(K=1001)), fake, fake, fake, fake, ws, need, None) == KD_ERR_SHAPE
    assert f(ctypes.byref(prob(T=0.0)), fake, fake, fake, fake, ws, need, None) == KD_ERR_TEMPERATURE
    assert f(ctypes.byref(p), fake, fake, None, fake, ws, need, None) == KD_ERR_NULL
    assert f(ctypes.byref(p), fake, fake, fake, None, ws, need, None) == KD_ERR_NULL
    assert f(ctypes.byref(p), fake, None, fake, fake, ws, need, None) == KD_ERR_NULL
    assert f(ctypes.byref(p), fake, fake, fake, fake, ws, need - 1, None) == KD_ERR_WORKSPACE
    assert f(ctypes.byref(p), fake, fake, fake, fake, ctypes.c_void_p(0x10010), need,
             None) == KD_ERR_WORKSPACE
    # the workspace holds per-chunk unit masses and draws, not [S, V]
    big = kd.kd_teacher_sample_workspace_bytes(prob(S=32768, H=2880, V=201088, K=100, chunk=1024))
    assert big < 64 << 20


@pytest.mark.parametrize("kw", [dict(V=4_300_000, K=10), dict(V=2_200_000, K=10, hw=1),
                                dict(chunk=5_000_000, S=10_000_000)])
def test_operand_ranges_beyond_2gib_rejected(kw):
    # a 256-row operand tile of the gradient tile / W^T (about V elements per
    # row) or of the transposed chunk (about chunk elements per row) must fit
    # one buffer range of less than 2^31 bytes
    p = prob(**kw)
    assert kd.kd_topk_kl_workspace_bytes(p) == 0
    fake = ctypes.c_void_p(0x1000)
    rc = kd.lib.kd_topk_kl_fwd(ctypes.byref(p), fake, fake, fake, fake, None, fake, fake, None,
                               None, fake, 1 << 40, None)
    assert rc == KD_ERR_SHAPE


def test_largest_accepted_vocabulary():
    assert kd.kd_topk_kl_workspace_bytes(prob(V=4_000_000, K=10)) > 0
    assert kd.kd_topk_kl_workspace_bytes(prob(V=2_000_000, K=10, hw=1)) > 0


def test_one_call_workspace_and_argument_errors():
    # the one call needs the two-call workspace plus one chunk of fp32 logits
    # (4 * chunk * V, in whole 256 x 256 tiles) and one float per row
    p = prob(S=32768, H=2880, V=201088, K=100, chunk=2048)
    lib = kd.lib
    two = kd.kd_topk_kl_workspace_bytes(p)
    one = lib.kd_topk_kl_fwd_bwd_workspace_bytes(ctypes.byref(p))
    tiles = ((2048 + 255) // 256) * ((201088 + 255) // 256)
    assert one - two >= tiles * 65536 * 4 + 32768 * 4
    assert one - two < tiles * 65536 * 4 + 32768 * 4 + 2 * 256
    # the extra part does not grow with S
    p2 = prob(S=262144, H=2880, V=201088, K=100, chunk=2048)
    extra2 = lib.kd_topk_kl_fwd_bwd_workspace_bytes(ctypes.byref(p2)) - kd.kd_topk_kl_workspace_bytes(p2)
    assert extra2 - (one - two) < (262144 - 32768) * 4 + 256
    fake = ctypes.c_void_p(0x1000)
    ws = ctypes.c_void_p(0x10000)
    f = lib.kd_topk_kl_fwd_bwd
    # argument order: problem, hidden, W, ids, logits, mask, grad_loss, loss,
    # lse, kl_rows, z_topk, dhidden, dW, accumulate_dW, ws, ws_bytes, stream
    assert f(ctypes.byref(p), fake, fake, fake, fake, None, None, fake, fake, None, None, fake, fake,
             0, ws, one, None) == KD_ERR_NULL
    assert f(ctypes.byref(p), fake, fake, fake, fake, None, fake, fake, fake, None, None, None, fake,
             0, ws, one, None) == KD_ERR_NULL
    assert f(ctypes.byref(p), fake, fake, fake, fake, None, fake, fake, fake, None, None, fake, fake,
             2, ws, one, None) == 10
    assert f(ctypes.byref(p), fake, fake, fake, fake, None, fake, fake, fake, None, None, fake, fake,
             0, ws, one - 1, None) == 6
    assert f(ctypes.byref(p), fake, fake, fake, fake, None, fake, fake, fake, None, None, fake, fake,
             0, ctypes.c_void_p(0x10010), one, None) == 6
    bad = prob(S=32768, H=2880, V=201088, K=100, chunk=0)
    assert lib.kd_topk_kl_fwd_bwd_workspace_bytes(ctypes.byref(bad)) == 0
    assert lib.kd_scale_f32(None, 4, fake, None) == KD_ERR_NULL
    assert lib.kd_scale_f32(fake, -1, fake, None) == KD_ERR_SHAPE
    assert lib.kd_scale_f32(None, 0, None, None) == KD_OK
