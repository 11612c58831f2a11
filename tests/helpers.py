"""Shared test utilities: host <-> device moves and error metrics."""
import numpy as np
import torch

import synth


def dev():
    return torch.device("cuda:0")


def to_dev(a: np.ndarray) -> torch.Tensor:
    """numpy host array -> device tensor. uint16 arrays are bf16 bit patterns."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(dev()).view(torch.bfloat16)
    return torch.from_numpy(a).to(dev())


def to_host(t: torch.Tensor) -> np.ndarray:
    """device tensor -> numpy; bf16 comes back as uint16 bit patterns."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).numpy()
    return t.numpy()


def as_f64(a: np.ndarray) -> np.ndarray:
    if a.dtype == np.uint16:
        return synth.bf16_to_f32(a).astype(np.float64)
    return np.asarray(a, np.float64)


def normwise_err(got: np.ndarray, ref: np.ndarray) -> float:
    """max_i |got_i - ref_i| / max_i |ref_i| (0 when both are all zero)."""
    got = as_f64(got)
    ref = np.asarray(ref, np.float64)
    den = np.abs(ref).max() if ref.size else 0.0
    num = np.abs(got - ref).max() if ref.size else 0.0
    if den == 0.0:
        return float(num)
    return float(num / den)


TOL = {"f32": 1e-5, "bf16": 2e-2, "fp8": 6e-2}
GAP = 1e-3
