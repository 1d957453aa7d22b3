"""Helpers shared by the GPU tests: moving generator outputs to the device and
comparing against the oracle with the stated tolerances."""
import numpy as np
import torch

import kd_synth

# Tolerances of the parity bar: loss relative error, gradient error relative to
# the tensor's largest magnitude, per-row log-sum-exp relative error.
LOSS_RTOL = 1e-3
GRAD_TOL = 2e-2
LSE_RTOL = 1e-3


def device():
    return torch.device("cuda:0")


def to_dev(x: np.ndarray, dtype: str) -> torch.Tensor:
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(device())
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(device())


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def val_to_f64(val: np.ndarray, dtype: str) -> np.ndarray:
    return kd_synth.to_float64(val, dtype)


def rel_max_err(got: np.ndarray, ref: np.ndarray) -> float:
    scale = float(np.abs(ref).max())
    return float(np.abs(got - ref).max()) / (scale if scale > 0 else 1.0)


def bf16_bits_of(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)
