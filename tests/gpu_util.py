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


def moe_device_weights(w):
    """Router (bf16) and natural-layout MXFP4 expert stacks of every layer of a MoE synth model:
    x_w13 [E+S, 2F, d/2] (gate rows then up rows), x_w2 [E+S, d, F/2], and their e8m0 scales."""
    s = w.shape
    out = {}
    for i in range(s.n_layers):
        out[f"l{i}.router"] = dev_bf16(w[f"l{i}.router"])
        gp, gs = w.expert_stack(i, "wg")
        up, us = w.expert_stack(i, "wu")
        dp, ds = w.expert_stack(i, "wd")
        for name, arr in ((f"l{i}.x_w13", np.concatenate([gp, up], axis=1)),
                          (f"l{i}.x_w13_scale", np.concatenate([gs, us], axis=1)),
                          (f"l{i}.x_w2", dp), (f"l{i}.x_w2_scale", ds)):
            out[name] = torch.from_numpy(np.ascontiguousarray(arr)).cuda()
    return out
