"""Shared helpers for the GPU parity tests: device copies of the seeded
inputs and the parity metric."""
from __future__ import annotations

import numpy as np
import torch

DEV = torch.device("cuda:0") if torch.cuda.is_available() else None

# Tolerances on max |gpu - oracle| / RMS(oracle), per output tensor.
TOL_BF16 = 2e-2
TOL_F32 = 1e-4


def to_dev(x, dtype):
    if x is None:
        return None
    t = torch.from_numpy(np.ascontiguousarray(x))
    return t.to(device=DEV, dtype=dtype).contiguous()


def qkv_torch_dtype(name: str):
    return torch.bfloat16 if name == "bf16" else torch.float32


def device_inputs(inp: dict) -> dict:
    dt = qkv_torch_dtype(inp["dtype"])
    return dict(q=to_dev(inp["q"], dt), k=to_dev(inp["k"], dt), v=to_dev(inp["v"], dt),
                g=to_dev(inp["g"], torch.float32), g_gamma=to_dev(inp["g_gamma"], torch.float32),
                initial_state=to_dev(inp["initial_state"], torch.float32))


def err_ratio(x, ref) -> float:
    """max |x - ref| / RMS(ref), in float64."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if ref.size == 0:
        return 0.0
    rms = float(np.sqrt(np.mean(ref * ref)))
    if rms == 0.0:
        return float(np.max(np.abs(x - ref))) if x.size else 0.0
    return float(np.max(np.abs(x - ref))) / rms
