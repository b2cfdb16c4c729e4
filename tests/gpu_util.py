"""Helpers for GPU tests: move seeded host inputs to the device and back."""
import numpy as np
import torch

from io_aware_tiled_fwd_amd import inputs

DEV = "cuda"

# Parity bars (max-abs) for the operations' outputs.
TOL_F32_O = 1e-4
TOL_F32_L = 1e-4
TOL_BF16_O = 2e-2
TOL_BF16_L = 1e-3
TOL_BF16_GRAD = 2e-2


def to_dev(bits, dtype):
    """uint16 bf16 patterns, uint8 e4m3 bytes or float32 values -> device
    tensor (bf16, uint8 or float32)."""
    if dtype == "fp8":
        return torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint8)).to(DEV)
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)
    return torch.from_numpy(np.ascontiguousarray(bits, dtype=np.float32)).to(DEV)


def f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def upload(ts: "inputs.Tensors"):
    return {n: to_dev(ts.bits[n], ts.dtype) for n in ts.names}


def maxabs(a, b):
    a, b = np.asarray(a), np.asarray(b)
    if a.size == 0:
        return 0.0
    assert np.all(np.isfinite(a)), "non-finite output"
    return float(np.max(np.abs(a - b)))


def bf16_from_f64(x):
    """Host values rounded to bf16 and widened back (exact representatives)."""
    return inputs.bf16_to_f64(inputs.bf16_bits(np.asarray(x, dtype=np.float32)))
