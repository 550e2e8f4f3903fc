"""Helpers shared by the GPU tests: move a synthetic problem to the device and
compare library outputs with the fp64 oracle."""
import numpy as np
import torch

from kd_synth import Problem

BF16_LOSS_RTOL = 1e-3     # loss: relative error bound for bf16 inputs, fp32 accumulation
BF16_GRAD_FRAC = 2e-2     # gradients: max-abs error <= this * max |oracle gradient|


def np_bf16_to_torch(bits: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def to_device(p: Problem, device="cuda"):
    if p.hw_dtype == "bf16":
        hidden = np_bf16_to_torch(p.hidden_bits, device)
        W = np_bf16_to_torch(p.W_bits, device)
    else:
        hidden = torch.from_numpy(p.hidden).to(device)
        W = torch.from_numpy(p.W).to(device)
    ids = torch.from_numpy(np.ascontiguousarray(p.ids, dtype=np.int32)).to(device)
    if p.tl_dtype == "bf16":
        tl = np_bf16_to_torch(p.tl_bits, device)
    else:
        tl = torch.from_numpy(np.ascontiguousarray(p.tlogits, dtype=np.float32)).to(device)
    return hidden, W, ids, tl


def max_abs_frac(got: np.ndarray, ref: np.ndarray) -> float:
    scale = float(np.max(np.abs(ref))) if ref.size else 0.0
    if scale == 0.0:
        return float(np.max(np.abs(got))) if got.size else 0.0
    return float(np.max(np.abs(got - ref))) / scale


def rel(a: float, b: float) -> float:
    return abs(a - b) / max(abs(b), 1e-30)
