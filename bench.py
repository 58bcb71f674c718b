#!/usr/bin/env python3
"""Benchmark of the Simple GLA hot path on one MI355X.

A step is one pass of the whole chunked forward (chunk-local gate cumsum,
inter-chunk state pass and output pass: one sgla_chunk_fwd call) over one
batch of the long hybrid-layer prefill workload: B=8, T=8192, H=16,
K=V=128, bf16 q/k/v ~ N(0,1) with k L2-normalised per head, the per-head
RetNet decay g_gamma[h] = log(1 - 2^(-5-5h/16)), scale 1/sqrt(K), chunk 64,
fp32 o, final state written.  ``value`` is tokens/s over the K timed steps
with all inputs already resident in HBM (input/output copies are rotated so
the 256 MB last-level cache cannot hold a step's working set).  Before the
counted warmup steps the device runs untimed steps for --warm-seconds
(default 1 s) so the timed steps see steady-state clocks.

The JSON line also carries:
  roofline      -- the chunked forward against its bound (HBM for this
                   workload): algorithmic bytes per call divided by the call's
                   average duration, measured with HIP events on the stream
                   the kernels run on (the events bracket every launch of the
                   call; ``kernel`` names them); ``traffic`` comes from a
                   committed rocprofv3 FETCH_SIZE/WRITE_SIZE summary when it
                   matches the current kernel sources, else null;
  mfma          -- the same call's algorithmic FLOPs against the bf16 dense
                   MFMA peak;
  configs       -- the same record for every named chunked workload (tiny
                   fp32, dense bf16 K=V=512, packed varlen K=V=128 and the
                   headline), each with tokens/s, TFLOP/s, the HBM and MFMA
                   fractions, the attainable-roofline fraction, traffic and
                   (from the cpu_baseline leg) its parity against the oracle;
  decode        -- the in-place decode step on 256 sequences x 32 heads x
                   128 x 128 fp32 state, 64 consecutive steps, HBM GB/s;
  backward      -- sgla_chunk_bwd on the packed K = V = 128 workload (dq, dk,
                   dv, dg, dh0);
  backward_wide -- sgla_chunk_bwd on the dense K = V = 512 workload;
  normalizer    -- sgla_chunk_normalizer on the same workload, HBM GB/s;
  gla           -- sgla_gla_chunk_fwd (per-key gates) on the same workload;
  parallel      -- sgla_parallel_fwd with the decayed attention matrix;
  parallel_f32  -- the same for float32 inputs (B=1, T=4096, H=16,
                   K=V=128), priced against the fp32 matrix-core peak;
  cpu_baseline  -- the fp64 CPU oracle timed on the host cores on whole
                   batches of the headline workload (a reported baseline
                   only), with the host CPU model; the same leg runs the
                   oracle once per timed workload and reports the GPU
                   outputs' error against it (max |err| / RMS and RMS err /
                   RMS over the whole o and final state) in each record.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, TFLOP/s
F32_MFMA_PEAK_TFLOPS = 157.3    # MI355X dense fp32 MFMA, TFLOP/s
F64_MFMA_PEAK_TFLOPS = 78.6     # MI355X dense fp64 MFMA, TFLOP/s
MALL_BYTES = 256 << 20
METRIC = "chunked Simple-GLA fwd tokens/s + % bf16 MFMA peak; decode HBM GB/s"


# The device sources each traffic record's kernels are built from (the dense
# K = 512 forward: preparation + state/output kernels; the decode step): a
# committed traffic record is used only while these files are unchanged.
KERNEL_SOURCES = {
    "chunk_fwd": ("chunk_prep_bf16.hip", "chunk_fwd_bf16_wide.hip", "mfma_common.h", "gate_scan.h",
                  "unit_map.h"),
    # with packed or segmented inputs the call also runs the table and
    # segment-state kernels, whose traffic the record includes
    "chunk_fwd_bf16_kernel": ("chunk_fwd_bf16.hip", "segment_state.hip", "table_put.hip", "mfma_common.h",
                              "gate_scan.h", "unit_map.h"),
    "chunk_fwd_f32_kernel": ("chunk_fwd_f32.hip", "gate_scan.h", "unit_map.h"),
    "recurrent_step_kernel": ("recurrent_step.hip",),
    "recurrent_step_vk_kernel": ("recurrent_step.hip",),
    "parallel_fwd_kernel": ("parallel_fwd.hip", "mfma_common.h", "gate_scan.h", "unit_map.h"),
    "parallel_fwd_f32_kernel": ("parallel_fwd_f32.hip", "mfma_common.h", "gate_scan.h", "unit_map.h"),
}


def kernel_source_hash(name: str = "chunk_fwd") -> str:
    d = os.path.join(ROOT, "gated_linear_attention_amd", "csrc")
    h = hashlib.sha256()
    for f in sorted(KERNEL_SOURCES[name]):
        with open(os.path.join(d, f), "rb") as fh:
            h.update(f.encode())
            h.update(fh.read())
    return h.hexdigest()[:16]


def chunk_algorithmic(inp) -> tuple[float, float]:
    """(bytes, flops) one launch must move / perform at minimum.

    bytes: q read once, k and v read once per kv head, g read once (if
    given), initial state read once (if given), o written once, final state
    written once.  flops per chunk of L tokens and query head: L(L+1)(K+V)
    for the causal q k^T and A v products plus 4 L K V for q h and the state
    update."""
    B, T, H, K, V = inp["B"], inp["T"], inp["H"], inp["K"], inp["V"]
    Hkv = inp.get("Hkv", H)
    esz = 2 if inp["dtype"] == "bf16" else 4
    N = inp["N"]
    tokens = B * T
    nbytes = tokens * (H * K + Hkv * (K + V)) * esz + tokens * H * 4 * V
    if inp["g"] is not None:
        nbytes += tokens * H * 4
    if inp["initial_state"] is not None:
        nbytes += N * H * K * V * 4
    if inp["output_final_state"]:
        nbytes += N * H * K * V * 4
    if inp["cu_seqlens"] is not None:
        lens = [int(x) for x in (inp["cu_seqlens"][1:] - inp["cu_seqlens"][:-1])]
    else:
        lens = [T] * B
    flops = 0
    for L in lens:
        for s in range(0, L, 64):
            c = min(64, L - s)
            flops += c * (c + 1) * (K + V) + 4 * c * K * V
    flops *= H
    return float(nbytes), float(flops)


def chunk_kernels(inp) -> list:
    """The kernels one sgla_chunk_fwd call dispatches for these inputs, in
    launch order (K >= 256 bf16: a per-chunk preparation kernel, then the
    state/output kernel)."""
    if inp["dtype"] != "bf16":
        return ["chunk_fwd_f32_kernel"]
    if inp["K"] >= 256:
        return ["chunk_prep_bf16_kernel", "chunk_fwd_bf16_wide_kernel"]
    return ["chunk_fwd_bf16_kernel"]


def load_traffic(workload: str, kernel: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if
    it was taken on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_hash") != kernel_source_hash(kernel):
        return None
    return rec.get("hbm_bytes_per_launch")


def warm_device(fn, seconds: float):
    """Run untimed work for ``seconds`` so clocks reach their steady state
    before the counted warmup and timed steps."""
    import torch
    if seconds <= 0:
        return
    t0 = time.perf_counter()
    i = 0
    while time.perf_counter() - t0 < seconds:
        fn(i)
        i += 1
        if i % 16 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()


def bench_chunk(workload: str, steps: int, warmup: int, warm_seconds: float,
                expand_kv: bool = False):
    import ctypes

    import numpy as np
    import torch

    import gated_linear_attention_amd as sgla
    from gla_workloads import CHUNK_CONFIGS, make_chunk_inputs

    w = CHUNK_CONFIGS[workload]
    inp = make_chunk_inputs(w)
    if expand_kv and inp["Hkv"] != inp["H"]:
        # the multi-head equivalent of grouped kv heads: every kv head repeated
        # for the query heads that read it
        rep_ = inp["H"] // inp["Hkv"]
        inp = dict(inp, k=np.repeat(inp["k"], rep_, axis=2), v=np.repeat(inp["v"], rep_, axis=2),
                   Hkv=inp["H"])
    dev = torch.device("cuda:0")
    qdt = torch.bfloat16 if inp["dtype"] == "bf16" else torch.float32
    B, T, H, K, V, N = inp["B"], inp["T"], inp["H"], inp["K"], inp["V"], inp["N"]
    alg_bytes, alg_flops = chunk_algorithmic(inp)
    ncopies = max(1, min(4, math.ceil(2 * MALL_BYTES / alg_bytes) + 1))
    qkv_code = 1 if inp["dtype"] == "bf16" else 2
    args = sgla._chunk_args(B, T, H, K, V, N, inp["chunk_size"], qkv_code, 2, inp["scale"],
                            inp["output_final_state"], inp["Hkv"])
    cu = None
    cu_ptr = None
    if inp["cu_seqlens"] is not None:
        cu = torch.as_tensor(inp["cu_seqlens"], dtype=torch.int64).contiguous()
        cu_ptr = ctypes.c_void_p(cu.data_ptr())
    ws_bytes = sgla._workspace_size(args, cu_ptr)
    t = lambda a, dt: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(dev, dt)
    copies = []
    for _ in range(ncopies):
        c = dict(q=t(inp["q"], qdt), k=t(inp["k"], qdt), v=t(inp["v"], qdt),
                 g=t(inp["g"], torch.float32), gg=t(inp["g_gamma"], torch.float32),
                 h0=t(inp["initial_state"], torch.float32),
                 o=torch.empty((B, T, H, V), device=dev, dtype=torch.float32),
                 ht=torch.empty((N, H, K, V), device=dev, dtype=torch.float32)
                 if inp["output_final_state"] else None,
                 ws=torch.empty(max(ws_bytes, 1), device=dev, dtype=torch.uint8))
        p = lambda x: None if x is None else ctypes.c_void_p(x.data_ptr())
        c["call"] = (ctypes.byref(args), p(c["q"]), p(c["k"]), p(c["v"]), p(c["g"]), p(c["gg"]),
                     p(c["h0"]), cu_ptr, p(c["o"]), p(c["ht"]), p(c["ws"]), ws_bytes)
        copies.append(c)
    stream = torch.cuda.current_stream(dev)
    sp = ctypes.c_void_p(stream.cuda_stream)
    fn = sgla.lib.sgla_chunk_fwd

    def step(i):
        st = fn(*copies[i % ncopies]["call"], sp)
        if st != 0:
            raise RuntimeError(f"sgla_chunk_fwd failed: {sgla.lib.sgla_last_error().decode()}")

    warm_device(step, warm_seconds)
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    # per-launch HIP events on the launch stream (kernel duration) ...
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    # ... and the whole timed region
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record(stream)
    for i in range(steps):
        ev[i][0].record(stream)
        step(i)
        ev[i][1].record(stream)
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = t_start.elapsed_time(t_end)
    per = sorted(a.elapsed_time(b) for a, b in ev)
    kern_ms = sum(per) / len(per)
    last = copies[(steps - 1) % ncopies]
    o_host = last["o"].cpu().numpy()
    ht_host = None if last["ht"] is None else last["ht"].cpu().numpy()
    del copies
    return dict(inp=inp, total_ms=total_ms, wall_s=wall, kernel_ms_mean=kern_ms,
                kernel_ms_median=per[len(per) // 2], alg_bytes=alg_bytes, alg_flops=alg_flops,
                ncopies=ncopies, o=o_host, ht=ht_host)


def traffic_key(inp) -> str:
    """Name of the traffic record (and of its kernel-source set) for a call."""
    if inp["dtype"] != "bf16":
        return "chunk_fwd_f32_kernel"
    return "chunk_fwd" if inp["K"] >= 256 else "chunk_fwd_bf16_kernel"


def chunk_record(workload: str, r: dict, steps: int) -> dict:
    """The per-workload record: throughput, roofline fractions, traffic."""
    inp = r["inp"]
    tokens = inp["B"] * inp["T"]
    kern_s = r["kernel_ms_mean"] * 1e-3
    t_mem = r["alg_bytes"] / (HBM_PEAK_GBS * 1e9)
    t_mfma = r["alg_flops"] / (BF16_MFMA_PEAK_TFLOPS * 1e12)
    gbs = r["alg_bytes"] / kern_s / 1e9
    tflops = r["alg_flops"] / kern_s / 1e12
    if t_mem >= t_mfma:
        roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(gbs / HBM_PEAK_GBS, 4)}
    else:
        roof = {"bound": "mfma", "achieved": round(tflops, 2), "peak": BF16_MFMA_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(tflops / BF16_MFMA_PEAK_TFLOPS, 4)}
    roof["traffic"] = load_traffic(workload, traffic_key(inp))
    kernels = chunk_kernels(inp)
    roof.update({"kernel": "+".join(kernels), "launches_per_call": len(kernels),
                 "kernel_ms_mean": round(r["kernel_ms_mean"], 5),
                 "kernel_ms_median": round(r["kernel_ms_median"], 5),
                 "algorithmic_bytes_per_launch": int(r["alg_bytes"]),
                 "algorithmic_flops_per_launch": int(r["alg_flops"]),
                 "attainable_frac": round(max(t_mem, t_mfma) / kern_s, 4)})
    ms_step = r["total_ms"] / steps
    return {
        "workload": workload,
        "config": {"B": inp["B"], "T": inp["T"], "H": inp["H"], "num_kv_heads": inp["Hkv"], "K": inp["K"],
                   "V": inp["V"], "num_seqs": inp["N"], "tokens": tokens, "chunk_size": inp["chunk_size"],
                   "qkv_dtype": inp["dtype"], "o_dtype": "f32",
                   "gate": "g" if inp["g"] is not None else ("g_gamma" if inp["g_gamma"] is not None else "none"),
                   "initial_state": inp["initial_state"] is not None,
                   "output_final_state": bool(inp["output_final_state"]),
                   "rotated_input_copies": r["ncopies"], "seed": _seed_of(workload)},
        "steps": steps, "ms_per_step": round(ms_step, 5),
        "tokens_per_s": round(tokens / (ms_step * 1e-3), 1),
        "tflops": round(tflops, 2),
        "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
        "mfma_frac": round(tflops / BF16_MFMA_PEAK_TFLOPS, 4),
        "attainable_frac": round(max(t_mem, t_mfma) / kern_s, 4),
        "roofline": roof,
    }


def bench_decode(steps_timed: int, warmup: int, warm_seconds: float, state_v_first: bool = False):
    import numpy as np
    import torch

    import gated_linear_attention_amd as sgla
    from gla_workloads import DECODE_CONFIGS, make_decode_inputs

    w = DECODE_CONFIGS["decode_n256_h32_k128"]
    inp = make_decode_inputs(w)
    dev = torch.device("cuda:0")
    N, H, K, V, S, Hkv = inp["N"], inp["H"], inp["K"], inp["V"], inp["steps"], inp["Hkv"]
    t = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a)).to(dev, dt)
    state = t(np.swapaxes(inp["state"], -1, -2) if state_v_first else inp["state"], torch.float32)
    q, k, v, g = (t(inp["q"], torch.bfloat16), t(inp["k"], torch.bfloat16),
                  t(inp["v"], torch.bfloat16), t(inp["g"], torch.float32))
    o = torch.empty((N, H, V), device=dev, dtype=torch.float32)
    step = lambda i: sgla.recurrent_step(q[i % S], k[i % S], v[i % S], g[i % S], state,
                                         scale=inp["scale"], out=o, state_v_first=state_v_first)
    warm_device(step, warm_seconds)
    for i in range(warmup):
        step(i)
    stream = torch.cuda.current_stream(dev)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(S)]
    torch.cuda.synchronize()
    for i in range(S):
        ev[i][0].record(stream)
        step(i)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    per = sorted(a.elapsed_time(b) for a, b in ev)
    mean_ms = sum(per) / len(per)
    nbytes = 2 * N * H * K * V * 4 + N * (H * K + Hkv * (K + V)) * 2 + N * H * 4 + N * H * V * 4
    gbs = nbytes / (mean_ms * 1e-3) / 1e9
    return {"workload": w.name, "state_layout": "[V, K]" if state_v_first else "[K, V]",
            "N": N, "H": H, "K": K, "V": V, "steps": S,
            "ms_per_step_mean": round(mean_ms, 5), "ms_per_step_median": round(per[S // 2], 5),
            "bytes_per_step": nbytes, "achieved_GBs": round(gbs, 1),
            "peak_GBs": HBM_PEAK_GBS, "frac": round(gbs / HBM_PEAK_GBS, 4),
            "tokens_per_s": round(N / (mean_ms * 1e-3), 1),
            "traffic": load_traffic(w.name, "recurrent_step_vk_kernel" if state_v_first else "recurrent_step_kernel")}


def decode_fresh_run(steps: int = 4):
    """A fresh run of the first ``steps`` decode steps of the named decode
    workload from its initial state: the outputs of every step and the state
    after the last, for the parity check of the cpu_baseline leg."""
    import numpy as np
    import torch

    import gated_linear_attention_amd as sgla
    from gla_workloads import DECODE_CONFIGS, make_decode_inputs

    inp = make_decode_inputs(DECODE_CONFIGS["decode_n256_h32_k128"], steps=steps)
    dev = torch.device("cuda:0")
    t = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a)).to(dev, dt)
    state = t(inp["state"], torch.float32)
    outs = []
    for s in range(steps):
        o = sgla.recurrent_step(t(inp["q"][s], torch.bfloat16), t(inp["k"][s], torch.bfloat16),
                                t(inp["v"][s], torch.bfloat16), t(inp["g"][s], torch.float32), state,
                                scale=inp["scale"])
        outs.append(o.cpu().numpy())
    torch.cuda.synchronize()
    return {"inp": inp, "o": outs, "state": state.cpu().numpy()}


def bwd_algorithmic(inp) -> tuple[float, float]:
    """(bytes, flops) of one backward call at minimum.

    bytes: q, k, v, do read once, g, h0 and dht read once if given; dq, dk,
    dv (fp32), dg and dh0 written once.  flops per chunk of L tokens and head:
    L(L+1)(3K + 2V) for the causal products (A, dA, the intra parts of dq, dk
    and dv) plus 10 L K V for the dense ones (q.h and state parts of dq, dk,
    dv, the state-gradient update and the state recomputation)."""
    B, T, H, K, V, N = inp["B"], inp["T"], inp["H"], inp["K"], inp["V"], inp["N"]
    esz = 2 if inp["dtype"] == "bf16" else 4
    tokens = B * T
    nbytes = tokens * H * (2 * K + 2 * V) * esz + tokens * H * (2 * K + V) * 4
    if inp["g"] is not None:
        nbytes += 2 * tokens * H * 4
    if inp["initial_state"] is not None:
        nbytes += N * H * K * V * 4
    nbytes += 2 * N * H * K * V * 4          # dht in, dh0 out
    if inp["cu_seqlens"] is not None:
        lens = [int(x) for x in (inp["cu_seqlens"][1:] - inp["cu_seqlens"][:-1])]
    else:
        lens = [T] * B
    flops = 0
    for L in lens:
        for s in range(0, L, 64):
            c = min(64, L - s)
            flops += c * (c + 1) * (3 * K + 2 * V) + 10 * c * K * V
    return float(nbytes), float(flops * H)


def bench_backward(workload: str, steps: int, warmup: int, warm_seconds: float):
    """sgla_chunk_bwd (dq, dk, dv, dg or dg_gamma, dh0) on a chunked workload.
    bf16 inputs with K in {64, 128, 256, 512} run both passes on the bf16
    matrix cores (K > 128: key-tiled state pass and dq/dk kernel, then the
    dv kernel over all keys and the gate kernel);
    at their algorithmic intensity (about 78 flop/B at K = V = 128), far
    below the bf16 ridge, the call is priced against HBM with its
    algorithmic bytes (the per-chunk state records the state pass writes and
    the gradient pass reads are design traffic on top, not counted).  Other
    inputs run on the fp32 matrix cores and are priced against their peak."""
    import ctypes

    import numpy as np
    import torch

    import gated_linear_attention_amd as sgla
    from gla_workloads import CHUNK_CONFIGS, make_backward_inputs, make_chunk_inputs

    w = CHUNK_CONFIGS[workload]
    inp = make_chunk_inputs(w)
    bi = make_backward_inputs(inp, seed=w.seed + 100)
    dev = torch.device("cuda:0")
    qdt = torch.bfloat16 if inp["dtype"] == "bf16" else torch.float32
    B, T, H, K, V, N = inp["B"], inp["T"], inp["H"], inp["K"], inp["V"], inp["N"]
    t = lambda a, dt: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(dev, dt)
    q, k, v, do = t(inp["q"], qdt), t(inp["k"], qdt), t(inp["v"], qdt), t(bi["do"], qdt)
    g, gg = t(inp["g"], torch.float32), t(inp["g_gamma"], torch.float32)
    h0, dht = t(inp["initial_state"], torch.float32), t(bi["dht"], torch.float32)
    args = sgla._chunk_args(B, T, H, K, V, N, 64, 1 if inp["dtype"] == "bf16" else 2, 2,
                            inp["scale"], 0, H)
    cu = None if inp["cu_seqlens"] is None else torch.as_tensor(inp["cu_seqlens"], dtype=torch.int64)
    cu_ptr = None if cu is None else ctypes.c_void_p(cu.data_ptr())
    ws_bytes = sgla.lib.sgla_chunk_bwd_workspace_size(ctypes.byref(args), cu_ptr)
    f32 = dict(device=dev, dtype=torch.float32)
    outs = dict(dq=torch.empty((B, T, H, K), **f32), dk=torch.empty((B, T, H, K), **f32),
                dv=torch.empty((B, T, H, V), **f32),
                dg=torch.empty((B, T, H), **f32) if g is not None else None,
                dgg=torch.empty((H,), **f32) if gg is not None else None,
                dh0=torch.empty((N, H, K, V), **f32))
    ws = torch.empty(max(ws_bytes, 1), device=dev, dtype=torch.uint8)
    p = lambda x: None if x is None else ctypes.c_void_p(x.data_ptr())
    call = (ctypes.byref(args), p(q), p(k), p(v), p(g), p(gg), p(h0), cu_ptr, p(do), p(dht),
            p(outs["dq"]), p(outs["dk"]), p(outs["dv"]), p(outs["dg"]), p(outs["dgg"]),
            p(outs["dh0"]), p(ws), ws_bytes)
    stream = torch.cuda.current_stream(dev)
    sp = ctypes.c_void_p(stream.cuda_stream)

    def step(_i):
        st = sgla.lib.sgla_chunk_bwd(*call, sp)
        if st != 0:
            raise RuntimeError(f"sgla_chunk_bwd failed: {sgla.lib.sgla_last_error().decode()}")

    warm_device(step, warm_seconds)
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for i in range(steps):
        ev[i][0].record(stream)
        step(i)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    per = sorted(a.elapsed_time(b) for a, b in ev)
    ms = sum(per) / len(per)
    nbytes, flops = bwd_algorithmic(inp)
    tf = flops / (ms * 1e-3) / 1e12
    gbs = nbytes / (ms * 1e-3) / 1e9
    bf16_path = inp["dtype"] == "bf16" and K in (64, 128, 256, 512)
    wide = bf16_path and K > 128
    if bf16_path:
        roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(gbs / HBM_PEAK_GBS, 4)}
    else:
        roof = {"bound": "mfma", "achieved": round(tf, 2), "peak": F32_MFMA_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(tf / F32_MFMA_PEAK_TFLOPS, 4), "dtype": "f32"}
    kern = ("chunk_bwd_state_bf16_kernel+chunk_bwd_grad_bf16_kernel" if bf16_path
            else "chunk_bwd_state_kernel+chunk_bwd_grad_kernel")
    if wide:
        kern += "+chunk_bwd_dv_wide_kernel" + ("+chunk_bwd_gate_wide_kernel" if g is not None or gg is not None
                                               else "")
    n_chunks = sum(-(-int(L) // 64) for L in (np.diff(inp["cu_seqlens"]) if inp["cu_seqlens"] is not None
                                                 else [T] * B))
    return {"workload": workload, "B": B, "T": T, "H": H, "K": K, "V": V, "num_seqs": N,
            "kernel": kern,
            "launches_per_call": len(kern.split("+")) + (1 if gg is not None else 0),
            "ms_per_call_mean": round(ms, 5), "ms_per_call_median": round(per[len(per) // 2], 5),
            "tokens_per_s": round(B * T / (ms * 1e-3), 1),
            "algorithmic_flops_per_call": int(flops), "algorithmic_bytes_per_call": int(nbytes),
            # written once each, read by the gradient kernel, dH once more by
            # the wide dv kernel
            "state_record_bytes_per_call": int((5 if wide else 4) * n_chunks * H * K * V * 4),
            "roofline": roof,
            "mfma": {"achieved_tflops": round(tf, 2),
                     "peak_tflops": BF16_MFMA_PEAK_TFLOPS if bf16_path else F32_MFMA_PEAK_TFLOPS,
                     "dtype": "bf16" if bf16_path else "f32"}}


def bench_normalizer(workload: str, steps: int, warmup: int, warm_seconds: float):
    """sgla_chunk_normalizer on a chunked workload: q and k read once, g read
    once, den written once (fp32), final z written -- an HBM stream.  One
    call is three launches (per-chunk key sums, the scan over chunks, the
    per-chunk outputs) plus the packed-table upload; the roofline divides the
    algorithmic bytes by the whole call's time."""
    import numpy as np
    import torch

    import gated_linear_attention_amd as sgla
    from gla_workloads import CHUNK_CONFIGS, make_chunk_inputs

    w = CHUNK_CONFIGS[workload]
    inp = make_chunk_inputs(w)
    dev = torch.device("cuda:0")
    qdt = torch.bfloat16 if inp["dtype"] == "bf16" else torch.float32
    t = lambda a, dt: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(dev, dt)
    q, k = t(inp["q"], qdt), t(inp["k"], qdt)
    g, gg = t(inp["g"], torch.float32), t(inp["g_gamma"], torch.float32)
    step = lambda _i: sgla.chunk_normalizer(q, k, g=g, g_gamma=gg, scale=inp["scale"],
                                            output_final_state=True, cu_seqlens=inp["cu_seqlens"])
    warm_device(step, warm_seconds)
    for i in range(warmup):
        step(i)
    stream = torch.cuda.current_stream(dev)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        ev[i][0].record(stream)
        step(i)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    per = sorted(a.elapsed_time(b) for a, b in ev)
    ms = sum(per) / len(per)
    B, T, H, K, N, Hkv = inp["B"], inp["T"], inp["H"], inp["K"], inp["N"], inp["Hkv"]
    esz = 2 if inp["dtype"] == "bf16" else 4
    nbytes = B * T * ((H + Hkv) * K * esz + H * 4 + (H * 4 if g is not None else 0)) + N * H * K * 4
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"workload": workload, "kernel": "norm_chunk_sum_kernel+norm_scan_kernel+norm_chunk_out_kernel",
            "launches_per_call": 3, "ms_per_call_mean": round(ms, 5),
            "ms_per_call_median": round(per[len(per) // 2], 5), "algorithmic_bytes_per_call": int(nbytes),
            "tokens_per_s": round(B * T / (ms * 1e-3), 1),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs / HBM_PEAK_GBS, 4)}}


def bench_gla(workload: str, steps: int, warmup: int, warm_seconds: float):
    """sgla_gla_chunk_fwd (elementwise per-key gates) on a chunked workload
    with gk = logsigmoid(N(0,1)) per key.  Algorithmic FLOPs as the head-wise
    forward's (the per-key decays are elementwise work on top).  bf16 inputs
    with K in {64, 128} and V a multiple of 64 run the chain on the bf16
    matrix cores: there the algorithmic intensity (about 44 flop/B at K = V =
    128) is far below the bf16 ridge, so the call is priced against HBM;
    otherwise everything runs on the fp32 matrix cores and is priced
    against their peak."""
    import numpy as np
    import torch

    import gated_linear_attention_amd as sgla
    from gla_workloads import CHUNK_CONFIGS, make_chunk_inputs, make_key_gates

    w = CHUNK_CONFIGS[workload]
    inp = make_chunk_inputs(w)
    gk_np = make_key_gates(inp, seed=w.seed + 200)
    dev = torch.device("cuda:0")
    qdt = torch.bfloat16 if inp["dtype"] == "bf16" else torch.float32
    t = lambda a, dt: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(dev, dt)
    q, k, v, gk = t(inp["q"], qdt), t(inp["k"], qdt), t(inp["v"], qdt), t(gk_np, torch.float32)
    h0 = t(inp["initial_state"], torch.float32)
    step = lambda _i: sgla.gla_chunk_fwd(q, k, v, gk, scale=inp["scale"], initial_state=h0,
                                         output_final_state=True, cu_seqlens=inp["cu_seqlens"])
    warm_device(step, warm_seconds)
    for i in range(warmup):
        step(i)
    stream = torch.cuda.current_stream(dev)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        ev[i][0].record(stream)
        step(i)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    per = sorted(a.elapsed_time(b) for a, b in ev)
    ms = sum(per) / len(per)
    nbytes, flops = chunk_algorithmic(inp)
    B, T, H, K = inp["B"], inp["T"], inp["H"], inp["K"]
    if inp["g"] is not None:
        nbytes -= B * T * H * 4
    nbytes += B * T * H * K * 4            # the per-key gates
    tf = flops / (ms * 1e-3) / 1e12
    gbs = nbytes / (ms * 1e-3) / 1e9
    bf16_chain = inp["dtype"] == "bf16" and K in (64, 128) and inp["V"] % 64 == 0
    if bf16_chain:
        roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(gbs / HBM_PEAK_GBS, 4)}
    else:
        roof = {"bound": "mfma", "achieved": round(tf, 2), "peak": F32_MFMA_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(tf / F32_MFMA_PEAK_TFLOPS, 4), "dtype": "f32"}
    return {"workload": workload, "gate": "per-key gk",
            "kernel": "gla_prep_kernel+" + ("gla_chain_bf16_kernel" if bf16_chain else "gla_chunk_fwd_kernel"),
            "launches_per_call": 2,
            "ms_per_call_mean": round(ms, 5), "ms_per_call_median": round(per[len(per) // 2], 5),
            "tokens_per_s": round(B * T / (ms * 1e-3), 1),
            "algorithmic_flops_per_call": int(flops), "algorithmic_bytes_per_call": int(nbytes),
            "roofline": roof,
            "mfma": {"achieved_tflops": round(tf, 2),
                     "peak_tflops": BF16_MFMA_PEAK_TFLOPS if bf16_chain else F32_MFMA_PEAK_TFLOPS,
                     "dtype": "bf16" if bf16_chain else "f32"}}


def bench_parallel(workload: str, steps: int, warmup: int, warm_seconds: float):
    """sgla_parallel_fwd on a dense workload: the decayed attention matrix A
    [B, H, T, T] float32 (zeros above the diagonal) and o = A v.  With bf16
    inputs writing A dominates (B H T^2 4 bytes against a few tens of MB of
    q, k, v, g and o), so the call is priced against HBM, with a plain fill
    of a buffer of A's size timed beside it as the practical write ceiling.
    With float32 inputs the products run on the fp32 matrix cores, whose
    157.3 TFLOP/s put the call's floor above the HBM one: it is priced
    against that peak (the HBM figure is reported beside it)."""
    import numpy as np
    import torch

    import gated_linear_attention_amd as sgla
    from gla_workloads import CHUNK_CONFIGS, make_chunk_inputs

    w = CHUNK_CONFIGS[workload]
    inp = make_chunk_inputs(w)
    dev = torch.device("cuda:0")
    t = lambda a, dt: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(dev, dt)
    f32 = inp["dtype"] == "f32"
    dt = torch.float32 if f32 else torch.bfloat16
    q, k, v = t(inp["q"], dt), t(inp["k"], dt), t(inp["v"], dt)
    g, gg = t(inp["g"], torch.float32), t(inp["g_gamma"], torch.float32)
    step = lambda _i: sgla.parallel_fwd(q, k, v, g=g, g_gamma=gg, scale=inp["scale"], output_attn=True,
                                        out_dtype=torch.float32)
    warm_device(step, warm_seconds)
    for i in range(warmup):
        step(i)
    stream = torch.cuda.current_stream(dev)

    def timed(fn, n):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        torch.cuda.synchronize()
        for i in range(n):
            ev[i][0].record(stream)
            fn(i)
            ev[i][1].record(stream)
        torch.cuda.synchronize()
        return sorted(a.elapsed_time(b) for a, b in ev)

    per = timed(step, steps)
    ms = sum(per) / len(per)
    B, T, H, K, V, Hkv = inp["B"], inp["T"], inp["H"], inp["K"], inp["V"], inp["Hkv"]
    abytes = B * H * T * T * 4
    nbytes = (B * T * (H * K + Hkv * (K + V)) * (4 if f32 else 2) + (B * T * H * 4 if g is not None else 0)
              + B * T * H * V * 4 + abytes)
    flops = B * H * (T * (T + 1) // 2) * (2 * K + 2 * V)   # causal q.k and A v, as in the definition
    fill_buf = torch.empty(B * H * T * T, device=dev, dtype=torch.float32)
    fill_buf.fill_(0.0)  # first touch of the allocation outside the timing
    fper = timed(lambda _i: fill_buf.fill_(0.0), max(3, steps // 2))
    fill_gbs = abytes / (fper[len(fper) // 2] * 1e-3) / 1e9
    del fill_buf
    gbs = nbytes / (ms * 1e-3) / 1e9
    tflops = flops / (ms * 1e-3) / 1e12
    qk_flops = B * H * (T * (T + 1) // 2) * 2 * K
    floor_ms = (qk_flops / (F64_MFMA_PEAK_TFLOPS * 1e12) + (flops - qk_flops) / (F32_MFMA_PEAK_TFLOPS * 1e12)) * 1e3
    if f32:
        return {"workload": workload, "kernel": "parallel_fwd_f32_kernel", "launches_per_call": 1,
                "config": {"B": B, "T": T, "H": H, "num_kv_heads": Hkv, "K": K, "V": V, "qkv_dtype": "f32",
                           "gate": "g" if g is not None else ("g_gamma" if gg is not None else "none"),
                           "attn": "float32 [B, H, T, T]", "o_dtype": "f32"},
                "ms_per_call_mean": round(ms, 5), "ms_per_call_median": round(per[len(per) // 2], 5),
                "tokens_per_s": round(B * T / (ms * 1e-3), 1),
                "algorithmic_bytes_per_call": int(nbytes), "algorithmic_flops_per_call": int(flops),
                "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": F32_MFMA_PEAK_TFLOPS,
                             "unit": "TFLOP/s", "frac": round(tflops / F32_MFMA_PEAK_TFLOPS, 4),
                             "dtype": "f32", "traffic": load_traffic(workload, "parallel_fwd_f32_kernel"),
                             # the q.k half of the flops runs on the fp64 matrix cores (exact
                             # products of float32 inputs), the A v half on the fp32 ones
                             "design_floor_ms": round(floor_ms, 4),
                             "attainable_frac": round(floor_ms / ms, 4)},
                "hbm": {"achieved_gbs": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4)},
                "write_ceiling": {"kernel": "torch fill_ of an A-sized float32 buffer",
                                  "achieved_gbs": round(fill_gbs, 1)}}
    return {"workload": workload, "kernel": "parallel_fwd_kernel", "launches_per_call": 1,
            "config": {"B": B, "T": T, "H": H, "num_kv_heads": Hkv, "K": K, "V": V,
                       "gate": "g" if g is not None else ("g_gamma" if gg is not None else "none"),
                       "attn": "float32 [B, H, T, T]", "o_dtype": "f32"},
            "ms_per_call_mean": round(ms, 5), "ms_per_call_median": round(per[len(per) // 2], 5),
            "tokens_per_s": round(B * T / (ms * 1e-3), 1),
            "algorithmic_bytes_per_call": int(nbytes), "algorithmic_flops_per_call": int(flops),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs / HBM_PEAK_GBS, 4),
                         "traffic": load_traffic(workload, "parallel_fwd_kernel")},
            "write_ceiling": {"kernel": "torch fill_ of an A-sized float32 buffer",
                              "achieved_gbs": round(fill_gbs, 1),
                              "frac_of_ceiling": round((abytes / (ms * 1e-3) / 1e9) / fill_gbs, 4)},
            "mfma": {"achieved_tflops": round(flops / (ms * 1e-3) / 1e12, 2),
                     "peak_tflops": BF16_MFMA_PEAK_TFLOPS, "dtype": "bf16"}}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _errs(x, ref) -> dict:
    import numpy as np
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    d = np.abs(x - ref)
    if rms == 0.0:
        return {"max_err_over_rms": float(d.max()) if d.size else 0.0, "rms_err_over_rms": 0.0}
    return {"max_err_over_rms": float(f"{float(d.max()) / rms:.3e}"),
            "rms_err_over_rms": float(f"{float(np.sqrt(np.mean(d * d))) / rms:.3e}")}


def cpu_baseline(inp, chunk_results: dict, decode_check, min_seconds: float = 10.0):
    """The fp64 CPU oracle on whole batches of the headline workload,
    repeated until at least ``min_seconds`` of wall time (a bounded sample),
    then run once on every other timed workload; its outputs give each
    record's parity (whole o and final state, against the GPU outputs of the
    timed calls; decode: every step of a fresh 4-step run and the state
    after it)."""
    import oracle
    threads = oracle.default_threads()
    units = inp["N"] * inp["H"]
    reps = 0
    t0 = time.perf_counter()
    ref = None
    while True:
        ref = oracle.fwd(inp["q"], inp["k"], inp["v"], g=inp["g"], g_gamma=inp["g_gamma"],
                         scale=inp["scale"], initial_state=inp["initial_state"],
                         cu_seqlens=inp["cu_seqlens"], output_final_state=inp["output_final_state"],
                         nthreads=threads)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            break
    tokens = inp["B"] * inp["T"] * reps
    parity = {}
    for name, r in chunk_results.items():
        ri = r["inp"]
        if ri is inp:
            o_ref, ht_ref = ref
        else:
            o_ref, ht_ref = oracle.fwd(ri["q"], ri["k"], ri["v"], g=ri["g"], g_gamma=ri["g_gamma"],
                                       scale=ri["scale"], initial_state=ri["initial_state"],
                                       cu_seqlens=ri["cu_seqlens"], nthreads=threads)
        p = {"o": _errs(r["o"], o_ref), "scope": "whole tensors"}
        if r["ht"] is not None:
            p["final_state"] = _errs(r["ht"], ht_ref)
        p["tolerance"] = 2e-2 if ri["dtype"] == "bf16" else 1e-4
        p["pass"] = all(v["max_err_over_rms"] <= p["tolerance"] for k, v in p.items()
                        if k in ("o", "final_state"))
        parity[name] = p
    if decode_check is not None:
        d = decode_check
        S = d["inp"]["state"].astype("float64")
        worst = 0.0
        for s, o_gpu in enumerate(d["o"]):
            o_ref, S = oracle.step(d["inp"]["q"][s], d["inp"]["k"][s], d["inp"]["v"][s], d["inp"]["g"][s], S,
                                   scale=d["inp"]["scale"], nthreads=threads)
            worst = max(worst, _errs(o_gpu, o_ref)["max_err_over_rms"])
        es = _errs(d["state"], S)
        parity["decode"] = {"o_worst_step": {"max_err_over_rms": worst}, "state": es,
                            "scope": f"whole tensors, {len(d['o'])} steps from the initial state",
                            "tolerance": 2e-2, "pass": worst <= 2e-2 and es["max_err_over_rms"] <= 2e-2}
    return {"value": round(tokens / dt, 2), "unit": "tokens/s", "cores": min(threads, units),
            "kind": "oracle", "seconds": round(dt, 3), "cpu_model": cpu_model(),
            "host_threads_available": threads,
            "sample": f"{reps} repetitions of one full batch of the timed workload "
                      f"(B={inp['B']}, T={inp['T']}, H={inp['H']}, K={inp['K']}, V={inp['V']}: "
                      f"{units} sequence-head units, one per thread), fp64 token-by-token"}, parity


COPY_BYTES = 512 << 20


def calibrate_copy(reps: int = 3):
    """A plain copy of COPY_BYTES: reads and writes exactly that many bytes of
    HBM per launch (twice the 256 MB last-level cache, so neither side can be
    absorbed by it)."""
    import torch
    dev = torch.device("cuda:0")
    src = torch.ones(COPY_BYTES // 4, device=dev, dtype=torch.float32)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        # an elementwise kernel (not a DMA memcpy) so the counters see it
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "copy", "bytes_read_per_launch": COPY_BYTES,
                      "bytes_written_per_launch": COPY_BYTES, "launches": reps}), flush=True)


CHUNK_LEGS = ("long_gamma_k128", "varlen_bf16_k128", "dense_bf16_k512", "tiny_f32")


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="long_gamma_k128",
                    help="chunked workload of the headline (default: the long hybrid-layer prefill, "
                         "B=8 T=8192 H=16 K=V=128 with g_gamma)")
    ap.add_argument("--only-headline", action="store_true",
                    help="time the headline workload only (no other configs, no decode, backward, "
                         "normalizer, GLA or parallel legs)")
    ap.add_argument("--warm-seconds", type=float, default=1.0,
                    help="untimed device warm-up before the counted warmup steps")
    ap.add_argument("--expand-kv", action="store_true",
                    help="time grouped-kv-head workloads as plain multi-head input (k and v "
                         "repeated per query head), for comparison")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--backward-workload", default="varlen_bf16_k128",
                    help="workload of the backward timing (K <= 128)")
    ap.add_argument("--backward-wide-workload", default="dense_bf16_k512",
                    help="workload of the wide-key backward timing (K = 256 or 512)")
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the oracle leg (CPU timing and the parity of every record)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain device-to-device copy of known size (the reference "
                         "kernel that scales rocprofv3 FETCH_SIZE / WRITE_SIZE readings)")
    ap.add_argument("--parallel-only", action="store_true",
                    help="only time the parallel form (sgla_parallel_fwd) and print its record")
    a = ap.parse_args()
    if a.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {a.gpus} is not supported (every "
              "(sequence, head) unit is independent, so more GPUs would each run their own "
              "share with no communication; run with --gpus 1).", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU (torch.cuda.is_available() is False)", file=sys.stderr)
        sys.exit(2)

    if a.calibrate_copy:
        calibrate_copy()
        return
    if a.parallel_only:
        print(json.dumps({"parallel": bench_parallel("parallel_bf16_k128", a.steps, a.warmup,
                                                     a.warm_seconds),
                          "parallel_f32": bench_parallel("parallel_f32_k128", a.steps, a.warmup,
                                                         a.warm_seconds)}), flush=True)
        return
    legs = [a.workload] + ([] if a.only_headline else [w for w in CHUNK_LEGS if w != a.workload])
    results, records = {}, {}
    for wl in legs:
        steps = a.steps if wl == a.workload else 20
        print(f"[bench] {wl}", file=sys.stderr, flush=True)
        results[wl] = bench_chunk(wl, steps, a.warmup, a.warm_seconds, a.expand_kv and wl == a.workload)
        records[wl] = chunk_record(wl, results[wl], steps)
    head = records[a.workload]
    inp = results[a.workload]["inp"]
    out = {
        "metric": METRIC,
        "value": head["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": inp["dtype"],
        "data": "synthetic",
        "config": dict({"workload": a.workload}, **head["config"]),
        "roofline": head["roofline"],
        "mfma": {"achieved_tflops": head["tflops"], "peak_tflops": BF16_MFMA_PEAK_TFLOPS,
                 "frac": head["mfma_frac"]},
        "configs": records,
    }
    decode_check = None
    if not a.no_decode and not a.only_headline:
        print("[bench] decode", file=sys.stderr, flush=True)
        out["decode"] = bench_decode(64, a.warmup, a.warm_seconds)
        out["decode_state_v_first"] = bench_decode(64, a.warmup, a.warm_seconds, state_v_first=True)
        if not a.no_cpu_baseline:
            decode_check = decode_fresh_run(4)
    if not a.no_backward and not a.only_headline:
        print("[bench] backward, normalizer, GLA, parallel form", file=sys.stderr, flush=True)
        out["backward"] = bench_backward(a.backward_workload, 20, a.warmup, a.warm_seconds)
        out["backward_wide"] = bench_backward(a.backward_wide_workload, 10, a.warmup, a.warm_seconds)
        out["normalizer"] = bench_normalizer(a.backward_workload, 20, a.warmup, a.warm_seconds)
        out["gla"] = bench_gla(a.backward_workload, 20, a.warmup, a.warm_seconds)
        out["parallel"] = bench_parallel("parallel_bf16_k128", 10, a.warmup, a.warm_seconds)
        out["parallel_f32"] = bench_parallel("parallel_f32_k128", 5, a.warmup, a.warm_seconds)
    if not a.no_cpu_baseline:
        print("[bench] cpu baseline and parity", file=sys.stderr, flush=True)
        out["cpu_baseline"], parity = cpu_baseline(inp, results, decode_check)
        for wl, p in parity.items():
            if wl in records:
                records[wl]["parity"] = p
            elif wl == "decode" and "decode" in out:
                out["decode"]["parity"] = p
        out["parity_pass"] = all(p["pass"] for p in parity.values())
    print(json.dumps(out), flush=True)


def _seed_of(workload):
    from gla_workloads import CHUNK_CONFIGS
    return CHUNK_CONFIGS[workload].seed


if __name__ == "__main__":
    main()
