"""Seeded synthetic inputs for Simple GLA, shared by the tests, the benchmark
and the smoke check.

This module only draws random numbers and shapes them.  It holds none of the
operator's arithmetic (no decays, no cumulative sums, no products of q, k and
v), so the GPU path and the CPU oracle can both consume its output without
sharing any of the method.

Recipes follow the workloads the pages use for the operator (page
"flash-linear-attention 中的 Simple GLA", section 二: q, k, v drawn from a
standard normal, log gates g = logsigmoid(N(0, 1)), [B, T, H, ...] layout,
packed sequences with cu_seqlens; section 五: gate normalisers and unequal
sequence lengths), plus the five named workload shapes below.  Random draws
happen in a fixed order -- sequence lengths, q, k, v, g, initial state -- from
``numpy.random.default_rng(seed)``.

All arrays are numpy.  ``q``/``k``/``v`` are float32 arrays whose values are
exactly representable in the requested input dtype (bf16 values are produced
by round-to-nearest-even of the float32 draw), so a device copy in that dtype
is lossless and the oracle reads the very same numbers.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

__all__ = ["ChunkWorkload", "DecodeWorkload", "CHUNK_CONFIGS", "DECODE_CONFIGS",
           "round_to_bf16", "logsigmoid", "make_chunk_inputs", "make_decode_inputs",
           "make_backward_inputs", "make_key_gates",
           "retnet_gamma"]


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even), returned as
    float32.  Inputs are finite."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32).astype(np.uint64)
    lsb = (bits >> np.uint64(16)) & np.uint64(1)
    bits = (bits + np.uint64(0x7FFF) + lsb) & np.uint64(0xFFFF0000)
    return bits.astype(np.uint32).view(np.float32)


def logsigmoid(x: np.ndarray) -> np.ndarray:
    """log(sigmoid(x)) = -log(1 + exp(-x)), evaluated stably in float64."""
    x = np.asarray(x, dtype=np.float64)
    return -np.logaddexp(0.0, -x)


def retnet_gamma(H: int) -> np.ndarray:
    """Per-head RetNet-style log decay log(1 - 2^(-5 - 5h/H)), h = 0..H-1,
    evaluated in float64 and stored as float32."""
    h = np.arange(H, dtype=np.float64)
    return np.log1p(-np.exp2(-5.0 - 5.0 * h / H)).astype(np.float32)


@dataclasses.dataclass(frozen=True)
class ChunkWorkload:
    name: str
    B: int
    T: int                       # dense: tokens per row; packed: ignored (from lengths)
    H: int
    K: int
    V: int
    dtype: str                   # "bf16" or "f32" for q, k, v
    gate: str = "g"              # "g" (per token), "gamma" (per head) or "none"
    gate_normalizer: float = 1.0  # g = logsigmoid(N(0,1)) / normalizer
    num_seqs: int = 0            # > 0: packed input with this many sequences
    len_range: tuple = (64, 4096)
    fixed_lengths: Optional[tuple] = None
    initial_state: bool = False
    h0_std: float = 0.1
    normalize_k: bool = False
    chunk_size: int = 64
    scale: Optional[float] = None   # None -> 1/sqrt(K)
    output_final_state: bool = True
    seed: int = 0
    Hkv: int = 0                 # kv heads of k and v (0: H); divides H

    @property
    def packed(self) -> bool:
        return self.num_seqs > 0 or self.fixed_lengths is not None

    def with_(self, **kw) -> "ChunkWorkload":
        return dataclasses.replace(self, **kw)


@dataclasses.dataclass(frozen=True)
class DecodeWorkload:
    name: str
    N: int
    H: int
    K: int
    V: int
    steps: int
    dtype: str = "bf16"
    state_std: float = 0.1
    scale: Optional[float] = None
    seed: int = 0
    Hkv: int = 0                 # kv heads of k and v (0: H); divides H
    gate: str = "g"              # "g" (per token and head), "gamma" (per head) or "none"

    def with_(self, **kw) -> "DecodeWorkload":
        return dataclasses.replace(self, **kw)


# The five named workloads (seed = 1000 + position in this list).
CHUNK_CONFIGS = {
    "tiny_f32": ChunkWorkload("tiny_f32", B=1, T=256, H=2, K=64, V=64, dtype="f32",
                              gate="g", output_final_state=True, seed=1000),
    "dense_bf16_k512": ChunkWorkload("dense_bf16_k512", B=4, T=2048, H=4, K=512, V=512,
                                     dtype="bf16", gate="g", output_final_state=True, seed=1001),
    "varlen_bf16_k128": ChunkWorkload("varlen_bf16_k128", B=1, T=0, H=16, K=128, V=128,
                                      dtype="bf16", gate="g", num_seqs=8, len_range=(64, 4096),
                                      initial_state=True, output_final_state=True, seed=1002),
    "long_gamma_k128": ChunkWorkload("long_gamma_k128", B=8, T=8192, H=16, K=128, V=128,
                                     dtype="bf16", gate="gamma", normalize_k=True,
                                     output_final_state=True, seed=1003),
}
# Grouped kv heads (page "relinear", its GQA target: 9 query heads over 3 kv
# heads, head dimension 64); measured beside the named workloads above.
CHUNK_CONFIGS["gqa_bf16_k64_h9kv3"] = ChunkWorkload(
    "gqa_bf16_k64_h9kv3", B=32, T=2048, H=9, K=64, V=64, dtype="bf16", gate="g", Hkv=3,
    output_final_state=True, seed=1005)
# Parallel form (explicit T x T attention matrix per head): dense rows of the
# packed workload's head shape, 4096 tokens each.
CHUNK_CONFIGS["parallel_bf16_k128"] = ChunkWorkload(
    "parallel_bf16_k128", B=2, T=4096, H=16, K=128, V=128, dtype="bf16", gate="g",
    output_final_state=False, seed=1006)
# The parallel form for float32 inputs (fp32 matrix cores): one such row.
CHUNK_CONFIGS["parallel_f32_k128"] = ChunkWorkload(
    "parallel_f32_k128", B=1, T=4096, H=16, K=128, V=128, dtype="f32", gate="g",
    output_final_state=False, seed=1007)
DECODE_CONFIGS = {
    "decode_n256_h32_k128": DecodeWorkload("decode_n256_h32_k128", N=256, H=32, K=128, V=128,
                                           steps=64, dtype="bf16", seed=1004),
}


def _as_input_dtype(x: np.ndarray, dtype: str) -> np.ndarray:
    x = np.asarray(x, dtype=np.float32)
    if dtype == "bf16":
        return round_to_bf16(x)
    if dtype == "f32":
        return np.ascontiguousarray(x)
    raise ValueError(f"unknown input dtype {dtype!r}")


def make_chunk_inputs(w: ChunkWorkload) -> dict:
    """Draw one batch for a chunked forward.  Returns a dict with numpy arrays
    q [B,T,H,K], k [B,T,Hkv,K], v [B,T,Hkv,V], g [B,T,H] or None, g_gamma [H]
    or None, initial_state [N,H,K,V] or None, cu_seqlens int64 [N+1] or None,
    plus scale, chunk_size, dtype and output_final_state."""
    rng = np.random.default_rng(w.seed)
    cu = None
    if w.packed:
        if w.fixed_lengths is not None:
            lengths = np.asarray(w.fixed_lengths, dtype=np.int64)
        else:
            lo, hi = w.len_range
            lengths = rng.integers(lo, hi + 1, size=w.num_seqs).astype(np.int64)
        cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
        B, T = 1, int(cu[-1])
        N = len(lengths)
    else:
        B, T = w.B, w.T
        N = B
    H, K, V = w.H, w.K, w.V
    Hkv = w.Hkv or H
    if H % Hkv:
        raise ValueError(f"Hkv={Hkv} must divide H={H}")
    q = rng.standard_normal((B, T, H, K), dtype=np.float32)
    k = rng.standard_normal((B, T, Hkv, K), dtype=np.float32)
    v = rng.standard_normal((B, T, Hkv, V), dtype=np.float32)
    if w.normalize_k:
        nrm = np.sqrt(np.sum(k.astype(np.float64) ** 2, axis=-1, keepdims=True))
        k = (k / np.maximum(nrm, 1e-30)).astype(np.float32)
    q = _as_input_dtype(q, w.dtype)
    k = _as_input_dtype(k, w.dtype)
    v = _as_input_dtype(v, w.dtype)
    g = g_gamma = None
    if w.gate == "g":
        g = (logsigmoid(rng.standard_normal((B, T, H))) / w.gate_normalizer).astype(np.float32)
    elif w.gate == "gamma":
        g_gamma = retnet_gamma(H)
    elif w.gate != "none":
        raise ValueError(f"unknown gate kind {w.gate!r}")
    h0 = None
    if w.initial_state:
        h0 = (rng.standard_normal((N, H, K, V), dtype=np.float32) * np.float32(w.h0_std))
    scale = w.scale if w.scale is not None else K ** -0.5
    return dict(q=q, k=k, v=v, g=g, g_gamma=g_gamma, initial_state=h0, cu_seqlens=cu,
                scale=float(scale), chunk_size=w.chunk_size, dtype=w.dtype,
                output_final_state=w.output_final_state, B=B, T=T, H=H, K=K, V=V, N=N, Hkv=Hkv)


def make_backward_inputs(inp: dict, seed: int, final_state_grad: bool = True) -> dict:
    """Draw the output gradient do [B,T,H,V] (N(0,1), rounded to the input
    dtype) and, if ``final_state_grad``, the final-state gradient dht
    [N,H,K,V] (0.1 N(0,1) float32) for a batch from make_chunk_inputs."""
    rng = np.random.default_rng(seed)
    B, T, H, K, V, N = inp["B"], inp["T"], inp["H"], inp["K"], inp["V"], inp["N"]
    do = _as_input_dtype(rng.standard_normal((B, T, H, V), dtype=np.float32), inp["dtype"])
    dht = None
    if final_state_grad:
        dht = rng.standard_normal((N, H, K, V), dtype=np.float32) * np.float32(0.1)
    return dict(do=do, dht=dht)


def make_key_gates(inp: dict, seed: int, normalizer: float = 1.0) -> np.ndarray:
    """Per-key log gates gk [B, T, H, K] = logsigmoid(N(0, 1)) / normalizer,
    float32, for elementwise-gate GLA on a batch from make_chunk_inputs (the
    same recipe as the head-wise gate, one draw per key)."""
    rng = np.random.default_rng(seed)
    B, T, H, K = inp["B"], inp["T"], inp["H"], inp["K"]
    return (logsigmoid(rng.standard_normal((B, T, H, K))) / normalizer).astype(np.float32)


def make_decode_inputs(w: DecodeWorkload, steps: Optional[int] = None) -> dict:
    """Draw the initial state [N,H,K,V] float32 and ``steps`` single-token
    inputs: q [steps,N,H,K], k [steps,N,Hkv,K], v [steps,N,Hkv,V], and
    g [steps,N,H] (gate "g") or g_gamma [H] (gate "gamma"); the other is None."""
    steps = w.steps if steps is None else steps
    rng = np.random.default_rng(w.seed)
    N, H, K, V = w.N, w.H, w.K, w.V
    Hkv = w.Hkv or H
    if H % Hkv:
        raise ValueError(f"Hkv={Hkv} must divide H={H}")
    if w.gate not in ("g", "gamma", "none"):
        raise ValueError(f"unknown gate kind {w.gate!r}")
    state = rng.standard_normal((N, H, K, V), dtype=np.float32) * np.float32(w.state_std)
    qs, ks, vs, gs = [], [], [], []
    for _ in range(steps):
        qs.append(_as_input_dtype(rng.standard_normal((N, H, K), dtype=np.float32), w.dtype))
        ks.append(_as_input_dtype(rng.standard_normal((N, Hkv, K), dtype=np.float32), w.dtype))
        vs.append(_as_input_dtype(rng.standard_normal((N, Hkv, V), dtype=np.float32), w.dtype))
        if w.gate == "g":
            gs.append(logsigmoid(rng.standard_normal((N, H))).astype(np.float32))
    scale = w.scale if w.scale is not None else K ** -0.5
    return dict(state=state, q=np.stack(qs), k=np.stack(ks), v=np.stack(vs),
                g=np.stack(gs) if w.gate == "g" else None,
                g_gamma=retnet_gamma(H) if w.gate == "gamma" else None,
                scale=float(scale), dtype=w.dtype, N=N, H=H, K=K, V=V, steps=steps, Hkv=Hkv)
