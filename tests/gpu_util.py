"""Helpers shared by the GPU tests: conversions between synth storage arrays and torch."""
import numpy as np
import pytest
import torch


def have_gpu():
    return torch.cuda.is_available()


def require_gpu():
    if not have_gpu():
        pytest.skip("needs a GPU")


def dev_bf16(bits: np.ndarray):
    """uint16 bf16 bit patterns -> torch.bfloat16 device tensor."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16).copy()).view(torch.bfloat16).cuda()


def dev_f32(a: np.ndarray):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def to_bits(t: torch.Tensor) -> np.ndarray:
    """torch.bfloat16 -> uint16 bits (host)."""
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def bf16_to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def storage(a: np.ndarray, dtype: str):
    if dtype == "bf16":
        return dev_bf16(a)
    return dev_f32(a)
