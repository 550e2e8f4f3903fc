"""Python binding of the fused chunked top-K KL distillation loss (HIP, gfx950).

Argument marshalling only: every step of the computation runs in the HIP
library ``libkdtopk.so`` built from ``csrc/`` (see ``build.py``); PyTorch
supplies device memory and the stream. The entry points carry the C names of
``include/kd_topk_kl.h``. There is no CPU fallback: importing this package
without the built library raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "KD_BF16", "KD_F32", "KD_TEACHER_LOGITS", "KD_TEACHER_PROBS", "KdError", "kd_problem", "lib",
    "kd_abi_version", "kd_status_str", "kd_topk_kl_workspace_bytes",
    "kd_topk_kl_fwd", "kd_topk_kl_fwd_noalloc", "kd_topk_kl_bwd", "kd_student_entropy",
    "kd_topk_kl_fwd_bwd_workspace_bytes", "kd_topk_kl_fwd_bwd", "kd_scale_f32",
    "KD_FORM_FUSED", "KD_FORM_DENSE", "KD_FORM_FORWARD_CHUNKED", "kd_kl_comparator_fwd",
    "kd_kl_comparator_bwd",
    "kd_select_top_fraction", "kd_select_samples", "kd_validate_topk",
    "kd_position_signals", "kd_select_by_signal", "kd_select_above",
    "kd_select_top_fraction_segments", "kd_validate_topk_order",
    "kd_teacher_topk_workspace_bytes", "kd_teacher_topk",
    "kd_teacher_sample_workspace_bytes", "kd_teacher_sample",
    "kd_profile_enable", "kd_profile_read", "kd_profile_reset",
    "KDTopKKL", "KDTopKKLOneCall", "kd_topk_kl", "LIB_PATH",
]

KD_BF16, KD_F32 = 0, 1
KD_TEACHER_LOGITS, KD_TEACHER_PROBS = 0, 1
LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkdtopk.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python chunked_top_kl_amd/build.py` (or `__graft_entry__.build()`) "
        "(hipcc for gfx950). There is no fallback implementation.")

lib = ctypes.CDLL(LIB_PATH)


class kd_problem(ctypes.Structure):
    _fields_ = [("S", ctypes.c_int64), ("H", ctypes.c_int64), ("V", ctypes.c_int64),
                ("K", ctypes.c_int64), ("chunk", ctypes.c_int64),
                ("temperature", ctypes.c_float), ("hw_dtype", ctypes.c_int32),
                ("tl_dtype", ctypes.c_int32), ("tl_kind", ctypes.c_int32)]


class kd_kernel_stat(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 48), ("launches", ctypes.c_int64),
                ("total_ms", ctypes.c_double)]


_P = ctypes.c_void_p
_PP = ctypes.POINTER(kd_problem)
_I64P = ctypes.POINTER(ctypes.c_int64)
lib.kd_abi_version.restype = ctypes.c_int
lib.kd_status_str.restype = ctypes.c_char_p
lib.kd_status_str.argtypes = [ctypes.c_int]
lib.kd_topk_kl_workspace_bytes.restype = ctypes.c_size_t
lib.kd_topk_kl_workspace_bytes.argtypes = [_PP]
lib.kd_topk_kl_fwd.restype = ctypes.c_int
lib.kd_topk_kl_fwd.argtypes = [_PP, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
lib.kd_topk_kl_fwd_noalloc.restype = ctypes.c_int
lib.kd_topk_kl_fwd_noalloc.argtypes = [_PP, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P]
KD_NOALLOC_SCRATCH_BYTES = 64 << 20
KD_FORM_FUSED, KD_FORM_DENSE, KD_FORM_FORWARD_CHUNKED = 0, 1, 2
lib.kd_kl_comparator_workspace_bytes.restype = ctypes.c_size_t
lib.kd_kl_comparator_workspace_bytes.argtypes = [_PP, ctypes.c_int]
lib.kd_kl_comparator_fwd.restype = ctypes.c_int
lib.kd_kl_comparator_fwd.argtypes = [_PP, ctypes.c_int, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                     ctypes.c_size_t, _P]
lib.kd_kl_comparator_bwd.restype = ctypes.c_int
lib.kd_kl_comparator_bwd.argtypes = [_PP, ctypes.c_int, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                     ctypes.c_int, _P, ctypes.c_size_t, _P]
lib.kd_topk_kl_bwd.restype = ctypes.c_int
lib.kd_topk_kl_bwd.argtypes = [_PP, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_int, _P,
                               ctypes.c_size_t, _P]
lib.kd_topk_kl_fwd_bwd_workspace_bytes.restype = ctypes.c_size_t
lib.kd_topk_kl_fwd_bwd_workspace_bytes.argtypes = [_PP]
lib.kd_topk_kl_fwd_bwd.restype = ctypes.c_int
lib.kd_topk_kl_fwd_bwd.argtypes = [_PP, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                   ctypes.c_int, _P, ctypes.c_size_t, _P]
lib.kd_scale_f32.restype = ctypes.c_int
lib.kd_scale_f32.argtypes = [_P, ctypes.c_int64, _P, _P]
lib.kd_student_entropy.restype = ctypes.c_int
lib.kd_student_entropy.argtypes = [_PP, _P, _P, _P, _P, ctypes.c_size_t, _P]
lib.kd_select_top_fraction.restype = ctypes.c_int
lib.kd_select_top_fraction.argtypes = [_PP, _P, _P, _P, ctypes.c_int64, ctypes.c_int64, _P, _P,
                                       _I64P, _P, ctypes.c_size_t, _P]
lib.kd_select_samples.restype = ctypes.c_int
lib.kd_select_samples.argtypes = [_PP, _P, _P, _P, _P, ctypes.c_int64, ctypes.c_int64,
                                  ctypes.c_int64, _P, _P, _I64P, _P, ctypes.c_size_t, _P]
lib.kd_position_signals.restype = ctypes.c_int
lib.kd_position_signals.argtypes = [_PP, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
lib.kd_select_by_signal.restype = ctypes.c_int
lib.kd_select_by_signal.argtypes = [_PP, _P, _P, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                    _P, _P, _P, _I64P, _P, ctypes.c_size_t, _P]
lib.kd_select_top_fraction_segments.restype = ctypes.c_int
lib.kd_select_top_fraction_segments.argtypes = [_PP, _P, _P, _P, _P, ctypes.c_int64, ctypes.c_int64,
                                                ctypes.c_int64, _P, _P, _I64P, _P, ctypes.c_size_t,
                                                _P]
lib.kd_select_above.restype = ctypes.c_int
lib.kd_select_above.argtypes = [_PP, _P, ctypes.c_double, _P, _P, _I64P, _P, ctypes.c_size_t, _P]
lib.kd_validate_topk_order.restype = ctypes.c_int
lib.kd_validate_topk_order.argtypes = [_PP, _P, _P, _I64P, _I64P, _P, ctypes.c_size_t, _P]
lib.kd_validate_topk.restype = ctypes.c_int
lib.kd_validate_topk.argtypes = [_PP, _P, _P, _I64P, _I64P, _I64P, _P, ctypes.c_size_t, _P]
lib.kd_teacher_topk_workspace_bytes.restype = ctypes.c_size_t
lib.kd_teacher_topk_workspace_bytes.argtypes = [_PP]
lib.kd_teacher_topk.restype = ctypes.c_int
lib.kd_teacher_topk.argtypes = [_PP, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
lib.kd_teacher_sample_workspace_bytes.restype = ctypes.c_size_t
lib.kd_teacher_sample_workspace_bytes.argtypes = [_PP]
lib.kd_teacher_sample.restype = ctypes.c_int
lib.kd_teacher_sample.argtypes = [_PP, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
lib.kd_profile_enable.restype = ctypes.c_int
lib.kd_profile_enable.argtypes = [ctypes.c_int]
lib.kd_profile_read.restype = ctypes.c_int
lib.kd_profile_read.argtypes = [ctypes.POINTER(kd_kernel_stat), ctypes.c_int]
lib.kd_profile_reset.restype = ctypes.c_int


class KdError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {kd_status_str(code)}")


def _check(code: int, where: str):
    if code != 0:
        raise KdError(code, where)


def kd_abi_version() -> int:
    return lib.kd_abi_version()


def kd_status_str(code: int) -> str:
    return lib.kd_status_str(int(code)).decode()


def _dtype_code(t: torch.dtype) -> int:
    if t == torch.bfloat16:
        return KD_BF16
    if t == torch.float32:
        return KD_F32
    raise TypeError(f"unsupported dtype {t}: bfloat16 or float32 expected")


def make_problem(S, H, V, K, chunk, T, hw_dtype, tl_dtype, tl_kind=0) -> kd_problem:
    return kd_problem(int(S), int(H), int(V), int(K), int(chunk), float(T), int(hw_dtype),
                      int(tl_dtype), int(tl_kind))


def kd_topk_kl_workspace_bytes(problem: kd_problem) -> int:
    return int(lib.kd_topk_kl_workspace_bytes(ctypes.byref(problem)))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _problem_of(hidden, W, topk_ids, topk_logits, T, chunk, teacher_probs=False):
    if hidden.dim() != 2 or W.dim() != 2 or topk_ids.dim() != 2 or topk_logits.dim() != 2:
        raise ValueError("hidden [S,H], W [V,H], topk_ids [S,K], topk_logits [S,K] expected")
    S, H = hidden.shape
    V = W.shape[0]
    K = topk_ids.shape[1]
    if W.shape[1] != H or topk_ids.shape[0] != S or tuple(topk_logits.shape) != (S, K):
        raise ValueError("inconsistent shapes")
    if hidden.dtype != W.dtype:
        raise TypeError("hidden and W must share a dtype")
    if topk_ids.dtype != torch.int32:
        raise TypeError("topk_ids must be int32")
    for t in (hidden, W, topk_ids, topk_logits):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("tensors must be contiguous device tensors")
    return make_problem(S, H, V, K, chunk, T, _dtype_code(hidden.dtype),
                        _dtype_code(topk_logits.dtype),
                        KD_TEACHER_PROBS if teacher_probs else KD_TEACHER_LOGITS)


def _mask_arg(mask, S):
    if mask is None:
        return None
    if mask.dtype not in (torch.uint8, torch.bool) or mask.numel() != S or not mask.is_contiguous():
        raise ValueError("mask must be a contiguous uint8/bool tensor of S elements")
    return mask


def _workspace(problem, device, workspace):
    need = kd_topk_kl_workspace_bytes(problem)
    if need == 0:
        _check(2, "kd_topk_kl_workspace_bytes")
    if workspace is not None and workspace.numel() >= need and workspace.data_ptr() % 256 == 0:
        return workspace
    return torch.empty(need, dtype=torch.uint8, device=device)


def kd_topk_kl_fwd(hidden, W, topk_ids, topk_logits, T=1.0, chunk=1024, mask=None,
                   want_kl_rows=False, want_z_topk=False, workspace=None, teacher_probs=False):
    """Forward pass. Returns dict(loss [1] f32, lse [S] f32, kl_rows, z_topk).
    teacher_probs: topk_logits hold probabilities (sampled targets), not logits."""
    p = _problem_of(hidden, W, topk_ids, topk_logits, T, chunk, teacher_probs)
    mask = _mask_arg(mask, p.S)
    dev = hidden.device
    ws = _workspace(p, dev, workspace)
    loss = torch.empty(1, dtype=torch.float32, device=dev)
    lse = torch.empty(p.S, dtype=torch.float32, device=dev)
    kl = torch.empty(p.S, dtype=torch.float32, device=dev) if want_kl_rows else None
    zt = torch.empty(p.S, p.K, dtype=torch.float32, device=dev) if want_z_topk else None
    _check(lib.kd_topk_kl_fwd(ctypes.byref(p), _ptr(hidden), _ptr(W), _ptr(topk_ids),
                              _ptr(topk_logits), _ptr(mask), _ptr(loss), _ptr(lse), _ptr(kl),
                              _ptr(zt), _ptr(ws), ws.numel(), _stream(dev)), "kd_topk_kl_fwd")
    return dict(loss=loss, lse=lse, kl_rows=kl, z_topk=zt)


def kd_topk_kl_fwd_noalloc(hidden, W, topk_ids, topk_logits, T=1.0, chunk=1024, mask=None,
                           want_kl_rows=False, want_z_topk=False, teacher_probs=False):
    """kd_topk_kl_fwd through the entry point that allocates nothing on the
    device: the library's fixed per-GPU scratch stands in for the workspace.
    The outputs are allocated here, by the caller. Calls that overlap in time
    on one GPU race."""
    p = _problem_of(hidden, W, topk_ids, topk_logits, T, chunk, teacher_probs)
    mask = _mask_arg(mask, p.S)
    dev = hidden.device
    loss = torch.empty(1, dtype=torch.float32, device=dev)
    lse = torch.empty(p.S, dtype=torch.float32, device=dev)
    kl = torch.empty(p.S, dtype=torch.float32, device=dev) if want_kl_rows else None
    zt = torch.empty(p.S, p.K, dtype=torch.float32, device=dev) if want_z_topk else None
    _check(lib.kd_topk_kl_fwd_noalloc(ctypes.byref(p), _ptr(hidden), _ptr(W), _ptr(topk_ids),
                                      _ptr(topk_logits), _ptr(mask), _ptr(loss), _ptr(lse),
                                      _ptr(kl), _ptr(zt), _stream(dev)), "kd_topk_kl_fwd_noalloc")
    return dict(loss=loss, lse=lse, kl_rows=kl, z_topk=zt)


def kd_topk_kl_bwd(hidden, W, topk_ids, topk_logits, lse, grad_loss, T=1.0, chunk=1024,
                   mask=None, dW=None, accumulate_dW=False, workspace=None, teacher_probs=False):
    """Backward pass. Returns (dhidden [S,H] f32, dW [V,H] f32)."""
    p = _problem_of(hidden, W, topk_ids, topk_logits, T, chunk, teacher_probs)
    mask = _mask_arg(mask, p.S)
    dev = hidden.device
    ws = _workspace(p, dev, workspace)
    if grad_loss.dtype != torch.float32 or grad_loss.numel() != 1:
        raise ValueError("grad_loss must be a float32 tensor of one element")
    grad_loss = grad_loss.contiguous()
    dh = torch.empty(p.S, p.H, dtype=torch.float32, device=dev)
    if dW is None:
        dW = torch.empty(p.V, p.H, dtype=torch.float32, device=dev)
        accumulate_dW = False
    elif dW.dtype != torch.float32 or tuple(dW.shape) != (p.V, p.H) or not dW.is_contiguous():
        raise ValueError("dW must be a contiguous float32 [V,H] tensor")
    _check(lib.kd_topk_kl_bwd(ctypes.byref(p), _ptr(hidden), _ptr(W), _ptr(topk_ids),
                              _ptr(topk_logits), _ptr(mask), _ptr(lse), _ptr(grad_loss),
                              _ptr(dh), _ptr(dW), 1 if accumulate_dW else 0, _ptr(ws),
                              ws.numel(), _stream(dev)), "kd_topk_kl_bwd")
    return dh, dW


def kd_topk_kl_fwd_bwd_workspace_bytes(hidden, W, topk_ids, topk_logits, T=1.0, chunk=1024,
                                       teacher_probs=False) -> int:
    p = _problem_of(hidden, W, topk_ids, topk_logits, T, chunk, teacher_probs)
    return int(lib.kd_topk_kl_fwd_bwd_workspace_bytes(ctypes.byref(p)))


def kd_topk_kl_fwd_bwd(hidden, W, topk_ids, topk_logits, grad_loss, T=1.0, chunk=1024,
                       mask=None, want_kl_rows=False, want_z_topk=False, dW=None,
                       accumulate_dW=False, workspace=None, teacher_probs=False):
    """Forward and backward in one call, with the upstream gradient grad_loss
    ([1] float32) known up front. Returns dict(loss, lse, kl_rows, z_topk,
    dhidden, dW): those of kd_topk_kl_fwd followed by kd_topk_kl_bwd."""
    p = _problem_of(hidden, W, topk_ids, topk_logits, T, chunk, teacher_probs)
    mask = _mask_arg(mask, p.S)
    dev = hidden.device
    need = lib.kd_topk_kl_fwd_bwd_workspace_bytes(ctypes.byref(p))
    if need == 0:
        raise KdError(2, "kd_topk_kl_fwd_bwd_workspace_bytes")
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    elif workspace.numel() < need:
        raise ValueError(f"workspace too small: {workspace.numel()} < {need} bytes")
    if grad_loss.dtype != torch.float32 or grad_loss.numel() != 1:
        raise ValueError("grad_loss must be a float32 tensor of one element")
    grad_loss = grad_loss.contiguous()
    loss = torch.empty(1, dtype=torch.float32, device=dev)
    lse = torch.empty(p.S, dtype=torch.float32, device=dev)
    kl = torch.empty(p.S, dtype=torch.float32, device=dev) if want_kl_rows else None
    zt = torch.empty(p.S, p.K, dtype=torch.float32, device=dev) if want_z_topk else None
    dh = torch.empty(p.S, p.H, dtype=torch.float32, device=dev)
    if dW is None:
        dW = torch.empty(p.V, p.H, dtype=torch.float32, device=dev)
        accumulate_dW = False
    elif dW.dtype != torch.float32 or tuple(dW.shape) != (p.V, p.H) or not dW.is_contiguous():
        raise ValueError("dW must be a contiguous float32 [V,H] tensor")
    _check(lib.kd_topk_kl_fwd_bwd(ctypes.byref(p), _ptr(hidden), _ptr(W), _ptr(topk_ids),
                                  _ptr(topk_logits), _ptr(mask), _ptr(grad_loss), _ptr(loss),
                                  _ptr(lse), _ptr(kl), _ptr(zt), _ptr(dh), _ptr(dW),
                                  1 if accumulate_dW else 0, _ptr(workspace), workspace.numel(),
                                  _stream(dev)), "kd_topk_kl_fwd_bwd")
    return dict(loss=loss, lse=lse, kl_rows=kl, z_topk=zt, dhidden=dh, dW=dW)


def kd_scale_f32(x, g):
    """x *= g[0] in place (x: contiguous float32 device tensor, g: [1] float32)."""
    if x.dtype != torch.float32 or not x.is_contiguous():
        raise ValueError("x must be a contiguous float32 tensor")
    if g.dtype != torch.float32 or g.numel() != 1:
        raise ValueError("g must be a float32 tensor of one element")
    g = g.contiguous()
    _check(lib.kd_scale_f32(_ptr(x), x.numel(), _ptr(g), _stream(x.device)), "kd_scale_f32")
    return x


def kd_kl_comparator_fwd(hidden, W, topk_ids, topk_logits, form, T=1.0, chunk=1024, mask=None,
                         want_kl_rows=False, workspace=None, teacher_probs=False):
    """Forward of a comparator loss form (KD_FORM_DENSE or KD_FORM_FORWARD_CHUNKED).
    Returns dict(loss, lse, kl_rows, workspace): pass the same workspace to
    kd_kl_comparator_bwd, which reads the grids the forward stored there."""
    p = _problem_of(hidden, W, topk_ids, topk_logits, T, chunk, teacher_probs)
    mask = _mask_arg(mask, p.S)
    dev = hidden.device
    need = lib.kd_kl_comparator_workspace_bytes(ctypes.byref(p), int(form))
    if need == 0:
        raise KdError(10, "kd_kl_comparator_workspace_bytes")
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    elif workspace.numel() < need:
        raise ValueError(f"workspace too small: {workspace.numel()} < {need} bytes")
    loss = torch.empty(1, dtype=torch.float32, device=dev)
    lse = torch.empty(p.S, dtype=torch.float32, device=dev)
    kl = torch.empty(p.S, dtype=torch.float32, device=dev) if want_kl_rows else None
    _check(lib.kd_kl_comparator_fwd(ctypes.byref(p), int(form), _ptr(hidden), _ptr(W),
                                    _ptr(topk_ids), _ptr(topk_logits), _ptr(mask), _ptr(loss),
                                    _ptr(lse), _ptr(kl), _ptr(workspace), workspace.numel(),
                                    _stream(dev)), "kd_kl_comparator_fwd")
    return dict(loss=loss, lse=lse, kl_rows=kl, workspace=workspace)


def kd_kl_comparator_bwd(hidden, W, topk_ids, topk_logits, lse, grad_loss, form, workspace,
                         T=1.0, chunk=1024, mask=None, dW=None, accumulate_dW=False,
                         teacher_probs=False):
    """Backward of a comparator loss form, from the grids its forward left in
    `workspace`. Returns (dhidden [S,H] f32, dW [V,H] f32)."""
    p = _problem_of(hidden, W, topk_ids, topk_logits, T, chunk, teacher_probs)
    mask = _mask_arg(mask, p.S)
    dev = hidden.device
    if grad_loss.dtype != torch.float32 or grad_loss.numel() != 1:
        raise ValueError("grad_loss must be a float32 tensor of one element")
    grad_loss = grad_loss.contiguous()
    dh = torch.empty(p.S, p.H, dtype=torch.float32, device=dev)
    if dW is None:
        dW = torch.empty(p.V, p.H, dtype=torch.float32, device=dev)
        accumulate_dW = False
    elif dW.dtype != torch.float32 or tuple(dW.shape) != (p.V, p.H) or not dW.is_contiguous():
        raise ValueError("dW must be a contiguous float32 [V,H] tensor")
    _check(lib.kd_kl_comparator_bwd(ctypes.byref(p), int(form), _ptr(hidden), _ptr(W),
                                    _ptr(topk_ids), _ptr(topk_logits), _ptr(mask), _ptr(lse),
                                    _ptr(grad_loss), _ptr(dh), _ptr(dW),
                                    1 if accumulate_dW else 0, _ptr(workspace), workspace.numel(),
                                    _stream(dev)), "kd_kl_comparator_bwd")
    return dh, dW


def kd_student_entropy(hidden, W, chunk=1024, workspace=None):
    """Per-position entropy (nats) of softmax(hidden W^T), float64 [S]."""
    S, H = hidden.shape
    p = make_problem(S, H, W.shape[0], 1, chunk, 1.0, _dtype_code(hidden.dtype), KD_BF16)
    dev = hidden.device
    ws = _workspace(p, dev, workspace)
    ent = torch.empty(S, dtype=torch.float64, device=dev)
    _check(lib.kd_student_entropy(ctypes.byref(p), _ptr(hidden), _ptr(W), _ptr(ent), _ptr(ws),
                                  ws.numel(), _stream(dev)), "kd_student_entropy")
    return ent


def kd_select_top_fraction(entropy, hidden, W, num=20, den=100, chunk=1024, workspace=None):
    """Keep floor(num*S/den) highest-entropy positions. Returns (mask u8 [S], idx i32 [count], count)."""
    S, H = hidden.shape
    p = make_problem(S, H, W.shape[0], 1, chunk, 1.0, _dtype_code(hidden.dtype), KD_BF16)
    dev = hidden.device
    ws = _workspace(p, dev, workspace)
    mask = torch.empty(S, dtype=torch.uint8, device=dev)
    idx = torch.empty(max(S, 1), dtype=torch.int32, device=dev)
    cnt = ctypes.c_int64(0)
    _check(lib.kd_select_top_fraction(ctypes.byref(p), _ptr(hidden), _ptr(W), _ptr(entropy),
                                      int(num), int(den), _ptr(mask), _ptr(idx), ctypes.byref(cnt),
                                      _ptr(ws), ws.numel(), _stream(dev)),
           "kd_select_top_fraction")
    return mask, idx[: cnt.value], cnt.value


def kd_select_samples(entropy, offsets, hidden, W, num=20, den=100, chunk=1024, workspace=None):
    """Keep floor(num*B/den) of the B samples (positions [offsets[b], offsets[b+1])) by mean
    entropy. Returns (mask u8 [B], idx i32 [count], count)."""
    S, H = hidden.shape
    B = offsets.numel() - 1
    if offsets.dtype != torch.int64 or not offsets.is_contiguous() or B < 0:
        raise ValueError("offsets must be a contiguous int64 tensor of B+1 entries")
    p = make_problem(S, H, W.shape[0], 1, chunk, 1.0, _dtype_code(hidden.dtype), KD_BF16)
    dev = hidden.device
    ws = _workspace(p, dev, workspace)
    mask = torch.empty(max(B, 1), dtype=torch.uint8, device=dev)
    idx = torch.empty(max(B, 1), dtype=torch.int32, device=dev)
    cnt = ctypes.c_int64(0)
    _check(lib.kd_select_samples(ctypes.byref(p), _ptr(hidden), _ptr(W), _ptr(entropy),
                                 _ptr(offsets), int(B), int(num), int(den), _ptr(mask), _ptr(idx),
                                 ctypes.byref(cnt), _ptr(ws), ws.numel(), _stream(dev)),
           "kd_select_samples")
    return mask[:B], idx[: cnt.value], cnt.value


def kd_position_signals(hidden, W, topk_ids=None, topk_logits=None, labels=None, T=1.0,
                        teacher_probs=False, entropy=True, chunk=1024, workspace=None):
    """Per-position signals, float64 [S] each (None when not computed): entropy at
    T = 1 (when entropy=True), the student's cross-entropy on the label at T = 1
    (when labels are given) and the teacher uncertainty 1 - p_t(y_t) (when labels
    and the teacher rows are given). Returns dict(entropy, ce, teacher_unc)."""
    if hidden.dim() != 2 or W.dim() != 2 or hidden.shape[1] != W.shape[1]:
        raise ValueError("hidden [S,H] and W [V,H] expected")
    S, H = hidden.shape
    V = W.shape[0]
    teacher = topk_ids is not None and topk_logits is not None and labels is not None
    K = topk_ids.shape[1] if teacher else 1
    tl_dtype = _dtype_code(topk_logits.dtype) if teacher else KD_BF16
    if labels is not None and (labels.dtype != torch.int32 or labels.numel() != S
                               or not labels.is_contiguous()):
        raise ValueError("labels must be a contiguous int32 tensor of S entries")
    p = make_problem(S, H, V, K, chunk, T, _dtype_code(hidden.dtype), tl_dtype,
                     KD_TEACHER_PROBS if teacher_probs else KD_TEACHER_LOGITS)
    dev = hidden.device
    ws = _workspace(p, dev, workspace)
    f64 = dict(dtype=torch.float64, device=dev)
    ent = torch.empty(S, **f64) if entropy else None
    ce = torch.empty(S, **f64) if labels is not None else None
    tu = torch.empty(S, **f64) if teacher else None
    _check(lib.kd_position_signals(ctypes.byref(p), _ptr(hidden), _ptr(W),
                                   _ptr(topk_ids if teacher else None),
                                   _ptr(topk_logits if teacher else None), _ptr(labels), _ptr(ent),
                                   _ptr(ce), _ptr(tu), _ptr(ws), ws.numel(), _stream(dev)),
           "kd_position_signals")
    return dict(entropy=ent, ce=ce, teacher_unc=tu)


def _signal_problem(signal):
    if signal.dtype != torch.float64 or signal.dim() != 1 or not signal.is_contiguous():
        raise ValueError("signal must be a contiguous float64 vector")
    # only S matters to the selection entry points
    return make_problem(signal.numel(), 8, 1, 1, 1, 1.0, KD_BF16, KD_BF16)


def kd_select_by_signal(signal, offsets=None, num=20, den=100, workspace=None):
    """Top num/den of each segment [offsets[b], offsets[b+1]) by signal (one segment
    [0, S) without offsets), highest first, lower index on ties, NaN never kept.
    Returns (mask u8 [S], idx i32 [count], count, thresholds f64 [B])."""
    p = _signal_problem(signal)
    S = signal.numel()
    if offsets is not None and (offsets.dtype != torch.int64 or not offsets.is_contiguous()
                                or offsets.numel() < 1):
        raise ValueError("offsets must be a contiguous int64 tensor of B+1 entries")
    B = 1 if offsets is None else offsets.numel() - 1
    dev = signal.device
    ws = _workspace(p, dev, workspace)
    mask = torch.empty(max(S, 1), dtype=torch.uint8, device=dev)
    idx = torch.empty(max(S, 1), dtype=torch.int32, device=dev)
    thr = torch.empty(max(B, 1), dtype=torch.float64, device=dev)
    cnt = ctypes.c_int64(0)
    _check(lib.kd_select_by_signal(ctypes.byref(p), _ptr(signal), _ptr(offsets), int(B), int(num),
                                   int(den), _ptr(mask), _ptr(idx), _ptr(thr), ctypes.byref(cnt),
                                   _ptr(ws), ws.numel(), _stream(dev)), "kd_select_by_signal")
    return mask[:S], idx[: cnt.value], cnt.value, thr[:B]


def kd_select_top_fraction_segments(entropy, offsets, hidden, W, num=20, den=100, chunk=1024,
                                    workspace=None):
    """Per-sequence top num/den by entropy (segments [offsets[b], offsets[b+1])), decided
    as fp64 entropies decide. Returns (mask u8 [S], idx i32 [count], count)."""
    S, H = hidden.shape
    if offsets.dtype != torch.int64 or not offsets.is_contiguous() or offsets.numel() < 1:
        raise ValueError("offsets must be a contiguous int64 tensor of B+1 entries")
    B = offsets.numel() - 1
    p = make_problem(S, H, W.shape[0], 1, chunk, 1.0, _dtype_code(hidden.dtype), KD_BF16)
    dev = hidden.device
    ws = _workspace(p, dev, workspace)
    mask = torch.empty(max(S, 1), dtype=torch.uint8, device=dev)
    idx = torch.empty(max(S, 1), dtype=torch.int32, device=dev)
    cnt = ctypes.c_int64(0)
    _check(lib.kd_select_top_fraction_segments(ctypes.byref(p), _ptr(hidden), _ptr(W),
                                               _ptr(entropy), _ptr(offsets), int(B), int(num),
                                               int(den), _ptr(mask), _ptr(idx), ctypes.byref(cnt),
                                               _ptr(ws), ws.numel(), _stream(dev)),
           "kd_select_top_fraction_segments")
    return mask[:S], idx[: cnt.value], cnt.value


def kd_select_above(signal, tau, workspace=None):
    """Global threshold: keep signal >= tau (NaN never). Returns (mask u8 [S], idx i32
    [count], count)."""
    p = _signal_problem(signal)
    S = signal.numel()
    dev = signal.device
    ws = _workspace(p, dev, workspace)
    mask = torch.empty(max(S, 1), dtype=torch.uint8, device=dev)
    idx = torch.empty(max(S, 1), dtype=torch.int32, device=dev)
    cnt = ctypes.c_int64(0)
    _check(lib.kd_select_above(ctypes.byref(p), _ptr(signal), float(tau), _ptr(mask), _ptr(idx),
                               ctypes.byref(cnt), _ptr(ws), ws.numel(), _stream(dev)),
           "kd_select_above")
    return mask[:S], idx[: cnt.value], cnt.value


def kd_teacher_topk_workspace_bytes(problem: kd_problem) -> int:
    return int(lib.kd_teacher_topk_workspace_bytes(ctypes.byref(problem)))


def kd_teacher_topk(hidden, W, K, chunk=2048, out_dtype=torch.bfloat16, workspace=None):
    """Teacher top-K cache of every position: (ids int32 [S,K], logits [S,K] out_dtype),
    the K largest teacher logits of each row of hidden W^T, largest first, lower id first
    on ties (chosen in fp64; logits are the fp64 values rounded)."""
    if hidden.dim() != 2 or W.dim() != 2 or hidden.shape[1] != W.shape[1]:
        raise ValueError("hidden [S,H] and W [V,H] expected")
    if hidden.dtype != W.dtype or not hidden.is_contiguous() or not W.is_contiguous():
        raise ValueError("hidden and W must be contiguous and of one dtype")
    S, H = hidden.shape
    p = make_problem(S, H, W.shape[0], K, chunk, 1.0, _dtype_code(hidden.dtype),
                     _dtype_code(out_dtype))
    dev = hidden.device
    need = kd_teacher_topk_workspace_bytes(p)
    if need == 0:
        raise KdError(2, "kd_teacher_topk")
    if workspace is None or workspace.numel() < need or workspace.data_ptr() % 256 != 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ids = torch.empty(S, K, dtype=torch.int32, device=dev)
    logits = torch.empty(S, K, dtype=out_dtype, device=dev)
    _check(lib.kd_teacher_topk(ctypes.byref(p), _ptr(hidden), _ptr(W), _ptr(ids), _ptr(logits),
                               _ptr(workspace), workspace.numel(), _stream(dev)),
           "kd_teacher_topk")
    return ids, logits


def kd_teacher_sample_workspace_bytes(problem: kd_problem) -> int:
    return int(lib.kd_teacher_sample_workspace_bytes(ctypes.byref(problem)))


def kd_teacher_sample(hidden, W, uniforms, T=1.0, chunk=1024, workspace=None):
    """Sampled teacher targets: ids int32 [S,N], entry (t, n) the smallest id v whose
    cumulative probability under softmax(hidden_t W^T / T) exceeds uniforms[t, n]
    (uniforms: float64 [S,N] in [0, 1), each row non-decreasing)."""
    if hidden.dim() != 2 or W.dim() != 2 or hidden.shape[1] != W.shape[1]:
        raise ValueError("hidden [S,H] and W [V,H] expected")
    if hidden.dtype != W.dtype or not hidden.is_contiguous() or not W.is_contiguous():
        raise ValueError("hidden and W must be contiguous and of one dtype")
    if (uniforms.dtype != torch.float64 or uniforms.dim() != 2 or not uniforms.is_contiguous()
            or uniforms.shape[0] != hidden.shape[0]):
        raise ValueError("uniforms: contiguous float64 [S,N] expected")
    S, H = hidden.shape
    N = uniforms.shape[1]
    p = make_problem(S, H, W.shape[0], N, chunk, T, _dtype_code(hidden.dtype), KD_F32)
    dev = hidden.device
    need = kd_teacher_sample_workspace_bytes(p)
    if need == 0:
        raise KdError(2, "kd_teacher_sample")
    if workspace is None or workspace.numel() < need or workspace.data_ptr() % 256 != 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ids = torch.empty(S, N, dtype=torch.int32, device=dev)
    _check(lib.kd_teacher_sample(ctypes.byref(p), _ptr(hidden), _ptr(W), _ptr(uniforms),
                                 _ptr(ids), _ptr(workspace), workspace.numel(), _stream(dev)),
           "kd_teacher_sample")
    return ids


def kd_validate_topk_order(topk_ids, topk_logits, V, workspace=None):
    """(rows whose K values are not non-increasing, rows holding an id twice)."""
    S, K = topk_ids.shape
    p = make_problem(S, 8, V, K, 1, 1.0, KD_BF16, _dtype_code(topk_logits.dtype))
    dev = topk_ids.device
    ws = _workspace(p, dev, workspace)
    a, b = ctypes.c_int64(0), ctypes.c_int64(0)
    _check(lib.kd_validate_topk_order(ctypes.byref(p), _ptr(topk_ids), _ptr(topk_logits),
                                      ctypes.byref(a), ctypes.byref(b), _ptr(ws), ws.numel(),
                                      _stream(dev)), "kd_validate_topk_order")
    return a.value, b.value


def kd_validate_topk(topk_ids, topk_logits, V, workspace=None, teacher_probs=False):
    """Counts of (ids outside [0,V), all -inf rows, NaN/+inf logits); for probabilities,
    (ids outside [0,V), rows without a positive value, negative or non-finite values)."""
    S, K = topk_ids.shape
    p = make_problem(S, 8, V, K, 1, 1.0, KD_BF16, _dtype_code(topk_logits.dtype),
                     KD_TEACHER_PROBS if teacher_probs else KD_TEACHER_LOGITS)
    dev = topk_ids.device
    ws = _workspace(p, dev, workspace)
    a, b, c = ctypes.c_int64(0), ctypes.c_int64(0), ctypes.c_int64(0)
    _check(lib.kd_validate_topk(ctypes.byref(p), _ptr(topk_ids), _ptr(topk_logits),
                                ctypes.byref(a), ctypes.byref(b), ctypes.byref(c), _ptr(ws),
                                ws.numel(), _stream(dev)), "kd_validate_topk")
    return a.value, b.value, c.value


def kd_profile_enable(on=True):
    _check(lib.kd_profile_enable(1 if on else 0), "kd_profile_enable")


def kd_profile_reset():
    _check(lib.kd_profile_reset(), "kd_profile_reset")


def kd_profile_read(max_entries=64):
    """Per-kernel {name: (launches, total_ms)} recorded while profiling was on."""
    arr = (kd_kernel_stat * max_entries)()
    n = lib.kd_profile_read(arr, max_entries)
    if n < 0:
        _check(-n, "kd_profile_read")
    return {arr[i].name.decode(): (arr[i].launches, arr[i].total_ms) for i in range(n)}


class KDTopKKL(torch.autograd.Function):
    """loss = mean over valid positions of KL(p_teacher || softmax(hidden W^T / T))."""

    @staticmethod
    def forward(ctx, hidden, W, topk_ids, topk_logits, T, chunk, mask, teacher_probs=False):
        out = kd_topk_kl_fwd(hidden, W, topk_ids, topk_logits, T, chunk, mask,
                             teacher_probs=teacher_probs)
        ctx.save_for_backward(hidden, W, topk_ids, topk_logits, out["lse"], mask)
        ctx.T, ctx.chunk, ctx.has_mask = T, chunk, mask is not None
        ctx.teacher_probs = teacher_probs
        return out["loss"][0]

    @staticmethod
    def backward(ctx, grad):
        hidden, W, topk_ids, topk_logits, lse, mask = ctx.saved_tensors
        g = grad.detach().reshape(1).to(torch.float32).contiguous()
        dh, dW = kd_topk_kl_bwd(hidden, W, topk_ids, topk_logits, lse, g, ctx.T, ctx.chunk,
                                mask if ctx.has_mask else None, teacher_probs=ctx.teacher_probs)
        dh = dh.to(hidden.dtype) if ctx.needs_input_grad[0] else None
        dW = dW.to(W.dtype) if ctx.needs_input_grad[1] else None
        return dh, dW, None, None, None, None, None, None


class KDTopKKLOneCall(torch.autograd.Function):
    """The same loss, with its gradients formed during the forward by
    kd_topk_kl_fwd_bwd at an upstream gradient of 1 (each chunk projected once);
    the backward scales them by the upstream gradient it receives."""

    @staticmethod
    def forward(ctx, hidden, W, topk_ids, topk_logits, T, chunk, mask, teacher_probs=False):
        one = torch.ones(1, dtype=torch.float32, device=hidden.device)
        out = kd_topk_kl_fwd_bwd(hidden, W, topk_ids, topk_logits, one, T, chunk, mask,
                                 teacher_probs=teacher_probs)
        ctx.save_for_backward(out["dhidden"], out["dW"])
        ctx.dtypes = (hidden.dtype, W.dtype)
        return out["loss"][0]

    @staticmethod
    def backward(ctx, grad):
        dh, dW = ctx.saved_tensors
        g = grad.detach().reshape(1).to(torch.float32).contiguous()
        dh_out = dW_out = None
        if ctx.needs_input_grad[0]:
            dh_out = kd_scale_f32(dh, g).to(ctx.dtypes[0])
        if ctx.needs_input_grad[1]:
            dW_out = kd_scale_f32(dW, g).to(ctx.dtypes[1])
        return dh_out, dW_out, None, None, None, None, None, None


def kd_topk_kl(hidden, W, topk_ids, topk_logits, T=1.0, chunk=1024, mask=None,
               teacher_probs=False, one_call=False):
    """Differentiable fused chunked top-K KL loss (scalar). teacher_probs: topk_logits
    hold teacher probabilities (sampled sparse targets) instead of logits.
    one_call: form the gradients in the forward (kd_topk_kl_fwd_bwd: one chunk
    of fp32 logits more memory, no second projection), for training steps that
    always run the backward."""
    fn = KDTopKKLOneCall if one_call else KDTopKKL
    return fn.apply(hidden, W, topk_ids, topk_logits, float(T), int(chunk), mask,
                    bool(teacher_probs))
