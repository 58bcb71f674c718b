"""Shared helpers for the GPU parity tests: device copies of the seeded
inputs, the parity metric, and sampled oracle evaluation of single
(sequence, head) units."""
from __future__ import annotations

import numpy as np
import torch

import oracle

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


def oracle_units(inp: dict, units, nthreads=None):
    """Oracle outputs for selected (sequence n, head h) units of a chunked
    forward.  Returns list of (n, h, token_slice, o [L, V], final [K, V])."""
    out = []
    cu = inp["cu_seqlens"]
    for n, h in units:
        if cu is not None:
            s, e = int(cu[n]), int(cu[n + 1])
            b = 0
        else:
            s, e = 0, inp["T"]
            b = n
        hk = h // (inp["H"] // inp["k"].shape[2])    # kv head of query head h
        q = inp["q"][b:b + 1, s:e, h:h + 1]
        k = inp["k"][b:b + 1, s:e, hk:hk + 1]
        v = inp["v"][b:b + 1, s:e, hk:hk + 1]
        g = None if inp["g"] is None else inp["g"][b:b + 1, s:e, h:h + 1]
        gg = None if inp["g_gamma"] is None else inp["g_gamma"][h:h + 1]
        h0 = None if inp["initial_state"] is None else inp["initial_state"][n:n + 1, h:h + 1]
        o, ht = oracle.fwd(q, k, v, g=g, g_gamma=gg, scale=inp["scale"], initial_state=h0,
                           nthreads=nthreads)
        out.append((n, h, (b, s, e), o[0, :, 0], ht[0, 0]))
    return out


def gpu_unit_slices(o_gpu: np.ndarray, ht_gpu, ref_units):
    """Gather the GPU outputs matching oracle_units' selection."""
    xs_o, xs_h, rs_o, rs_h = [], [], [], []
    for n, h, (b, s, e), o_ref, ht_ref in ref_units:
        xs_o.append(o_gpu[b, s:e, h])
        rs_o.append(o_ref)
        if ht_gpu is not None:
            xs_h.append(ht_gpu[n, h])
            rs_h.append(ht_ref)
    cat = lambda xs: np.concatenate([np.asarray(x, dtype=np.float64).ravel() for x in xs]) if xs else np.zeros(0)
    return cat(xs_o), cat(rs_o), cat(xs_h), cat(rs_h)
