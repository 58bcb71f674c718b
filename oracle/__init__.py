"""CPU fp64 oracle for Simple GLA -- test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  It wraps ``sgla_oracle.c`` (plain C,
fp64, one thread per (sequence, head) unit) through ctypes and shares nothing
with the GPU library: no code, header, constant or helper.

Semantics (page "flash-linear-attention 中的 Simple GLA", section 一 for the
recurrence, section 二 for shapes and conventions):

    S_t = exp(g_t) S_{t-1} + k_t v_t^T,   o_t = scale * S_t^T q_t.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sgla_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(out_path: str = _LIB_PATH, mutant: int = 0) -> str:
    """Compile the oracle with gcc (-O2, no fast-math).  ``mutant`` != 0 builds
    a deliberately wrong copy for the plant-a-mistake tests."""
    cmd = ["gcc", "-O2", "-fPIC", "-shared", "-std=c11", "-Wall", "-o", out_path, _SRC,
           "-lpthread", "-lm"]
    if mutant:
        cmd.insert(1, f"-DSGLA_ORACLE_MUTANT={int(mutant)}")
    subprocess.run(cmd, check=True)
    return out_path


def _bind(lib):
    dp = ctypes.POINTER(ctypes.c_double)
    lp = ctypes.POINTER(ctypes.c_int64)
    lib.sgla_oracle_fwd.restype = ctypes.c_int
    lib.sgla_oracle_fwd.argtypes = [ctypes.c_int] * 6 + [dp] * 5 + [ctypes.c_double, dp, lp,
                                                                     ctypes.c_int, dp, dp,
                                                                     ctypes.c_int]
    lib.sgla_oracle_chunk_local_cumsum.restype = ctypes.c_int
    lib.sgla_oracle_chunk_local_cumsum.argtypes = [ctypes.c_int] * 3 + [dp, lp, ctypes.c_int,
                                                                        ctypes.c_int, dp]
    lib.sgla_oracle_bwd.restype = ctypes.c_int
    lib.sgla_oracle_bwd.argtypes = ([ctypes.c_int] * 5 + [dp] * 5 + [ctypes.c_double, dp, lp, ctypes.c_int]
                                    + [dp] * 8 + [ctypes.c_int])
    lib.sgla_oracle_gla_fwd.restype = ctypes.c_int
    lib.sgla_oracle_gla_fwd.argtypes = ([ctypes.c_int] * 6 + [dp] * 4 + [ctypes.c_double, dp, lp, ctypes.c_int]
                                        + [dp] * 2 + [ctypes.c_int])
    lib.sgla_oracle_parallel.restype = ctypes.c_int
    lib.sgla_oracle_parallel.argtypes = [ctypes.c_int] * 6 + [dp] * 5 + [ctypes.c_double, dp, dp,
                                                                         ctypes.c_int]
    lib.sgla_oracle_step.restype = ctypes.c_int
    lib.sgla_oracle_step.argtypes = [ctypes.c_int] * 5 + [dp] * 5 + [ctypes.c_double, dp, dp,
                                                                     ctypes.c_int]
    return lib


def load(path: str | None = None):
    """Load (building first if absent) the oracle library."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build()
        _lib = _bind(ctypes.CDLL(_LIB_PATH))
    return _lib


def default_threads() -> int:
    """Worker threads: OMP_NUM_THREADS when set (the host's share of cores),
    else the CPUs this process may run on."""
    env = os.environ.get("OMP_NUM_THREADS", "")
    if env.isdigit() and int(env) > 0:
        return int(env)
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def _f64(x):
    if x is None:
        return None
    a = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    return a


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _vk(x, state_v_first):
    """States given or returned in the [V, K] layout (section 二, state_v_first)
    are the transposes of the [K, V] states the C oracle works on."""
    if x is None or not state_v_first:
        return x
    return np.ascontiguousarray(np.swapaxes(np.asarray(x, dtype=np.float64), -1, -2))


def fwd(q, k, v, g=None, g_gamma=None, scale=None, initial_state=None, cu_seqlens=None,
        output_final_state=True, nthreads=None, lib=None, state_v_first=False):
    """Token-by-token forward.

    q: [B, T, H, K]; k: [B, T, Hkv, K]; v: [B, T, Hkv, V] (Hkv divides H: query
    head h reads kv head h // (H // Hkv)); g: [B, T, H] or None; g_gamma: [H]
    or None; initial_state: [N, H, K, V] or None; cu_seqlens: int [N+1] or
    None (then N = B).  state_v_first: initial_state and final_state are
    [N, H, V, K] (the transposed state) instead of [N, H, K, V].
    Returns (o [B, T, H, V], final_state [N, H, K, V] or None), both float64.
    """
    initial_state = _vk(initial_state, state_v_first)
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, T, H, K = q.shape
    Hkv = k.shape[2]
    V = v.shape[-1]
    if scale is None:
        scale = K ** -0.5
    g = _f64(g)
    g_gamma = _f64(g_gamma)
    h0 = _f64(initial_state)
    cu = None
    N = B
    if cu_seqlens is not None:
        cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
        N = cu.shape[0] - 1
    o = np.zeros((B, T, H, V), dtype=np.float64)
    ht = np.zeros((N, H, K, V), dtype=np.float64) if output_final_state else None
    lib = lib or load()
    rc = lib.sgla_oracle_fwd(B, T, H, Hkv, K, V, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(g_gamma),
                             float(scale), _ptr(h0),
                             None if cu is None else cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                             N, _ptr(o), _ptr(ht), int(nthreads or default_threads()))
    if rc != 0:
        raise ValueError(f"sgla_oracle_fwd rejected its arguments (code {rc})")
    return o, _vk(ht, state_v_first)


def bwd(q, k, v, do, g=None, g_gamma=None, scale=None, initial_state=None, dht=None,
        cu_seqlens=None, nthreads=None, lib=None, state_v_first=False):
    """Token-by-token backward: gradients of sum <do, o> + sum <dht, final_state>.

    q: [B, T, H, K]; k: [B, T, Hkv, K]; v: [B, T, Hkv, V]; do: [B, T, H, V];
    g: [B, T, H] or None; g_gamma: [H] or None; initial_state, dht: [N, H, K,
    V] or None; cu_seqlens as for fwd.  Returns a dict of float64 arrays dq
    [B, T, H, K], dk [B, T, Hkv, K], dv [B, T, Hkv, V], dg [B, T, H] (None
    without g), dg_gamma [H] (None without g_gamma), dh0 [N, H, K, V].
    state_v_first: initial_state, dht and dh0 are [N, H, V, K].

    Grouped kv heads (Hkv < H): query head h reads kv head h // (H // Hkv),
    i.e. the forward sees k and v repeated n_rep = H // Hkv times along the
    head axis; by the chain rule through that repeat, dk and dv of a kv head
    are the sums of the per-query-head gradients of its n_rep copies."""
    initial_state, dht = _vk(initial_state, state_v_first), _vk(dht, state_v_first)
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    B, T, H, K = q.shape
    V = v.shape[-1]
    Hkv = k.shape[2]
    if H % Hkv != 0:
        raise ValueError("the kv head count must divide the query head count")
    if Hkv != H:
        rep = H // Hkv
        gr = bwd(q, np.repeat(k, rep, axis=2), np.repeat(v, rep, axis=2), do, g=g, g_gamma=g_gamma,
                 scale=scale, initial_state=initial_state, dht=dht, cu_seqlens=cu_seqlens,
                 nthreads=nthreads, lib=lib)
        gr["dk"] = gr["dk"].reshape(B, T, Hkv, rep, K).sum(axis=3)
        gr["dv"] = gr["dv"].reshape(B, T, Hkv, rep, V).sum(axis=3)
        gr["dh0"] = _vk(gr["dh0"], state_v_first)
        return gr
    if scale is None:
        scale = K ** -0.5
    g, g_gamma, h0, dht = _f64(g), _f64(g_gamma), _f64(initial_state), _f64(dht)
    cu = None
    N = B
    if cu_seqlens is not None:
        cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
        N = cu.shape[0] - 1
    dq = np.zeros((B, T, H, K))
    dk = np.zeros((B, T, H, K))
    dv = np.zeros((B, T, H, V))
    dg = np.zeros((B, T, H)) if g is not None else None
    dgg = np.zeros(H) if g_gamma is not None else None
    dh0 = np.zeros((N, H, K, V))
    lib = lib or load()
    rc = lib.sgla_oracle_bwd(B, T, H, K, V, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(g_gamma),
                             float(scale), _ptr(h0),
                             None if cu is None else cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                             N, _ptr(do), _ptr(dht), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg), _ptr(dgg),
                             _ptr(dh0), int(nthreads or default_threads()))
    if rc != 0:
        raise ValueError(f"sgla_oracle_bwd rejected its arguments (code {rc})")
    return dict(dq=dq, dk=dk, dv=dv, dg=dg, dg_gamma=dgg, dh0=_vk(dh0, state_v_first))


def gla_fwd(q, k, v, gk, scale=None, initial_state=None, cu_seqlens=None, output_final_state=True,
            nthreads=None, lib=None):
    """Elementwise-gate GLA, token by token: S_t = diag(exp(gk_t)) S_{t-1} +
    k_t v_t^T, o_t = scale S_t^T q_t.  q, gk: [B, T, H, K]; k: [B, T, Hkv, K];
    v: [B, T, Hkv, V]; initial_state [N, H, K, V] or None; cu_seqlens as for
    fwd.  Returns (o [B, T, H, V], final_state [N, H, K, V] or None)."""
    q, k, v, gk = _f64(q), _f64(k), _f64(v), _f64(gk)
    B, T, H, K = q.shape
    Hkv = k.shape[2]
    V = v.shape[-1]
    if scale is None:
        scale = K ** -0.5
    h0 = _f64(initial_state)
    cu = None
    N = B
    if cu_seqlens is not None:
        cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
        N = cu.shape[0] - 1
    o = np.zeros((B, T, H, V))
    ht = np.zeros((N, H, K, V)) if output_final_state else None
    lib = lib or load()
    rc = lib.sgla_oracle_gla_fwd(B, T, H, Hkv, K, V, _ptr(q), _ptr(k), _ptr(v), _ptr(gk), float(scale),
                                 _ptr(h0),
                                 None if cu is None else cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                 N, _ptr(o), _ptr(ht), int(nthreads or default_threads()))
    if rc != 0:
        raise ValueError(f"sgla_oracle_gla_fwd rejected its arguments (code {rc})")
    return o, ht


def normalizer(q, k, g=None, g_gamma=None, scale=None, initial_z=None, cu_seqlens=None,
               nthreads=None, lib=None):
    """The running normalizer of the relinear pages (their "augmented value":
    a column of ones appended to v): its state column is z_t = exp(g_t)
    z_{t-1} + k_t and its output is scale * q_t . z_t.  Computed as exactly
    that -- the forward with a single all-ones value column.

    q: [B, T, H, K]; k: [B, T, Hkv, K]; initial_z: [N, H, K] or None.
    Returns (den [B, T, H], final_z [N, H, K]), float64."""
    k = _f64(k)
    B, T, Hkv = k.shape[:3]
    ones = np.ones((B, T, Hkv, 1))
    h0 = None if initial_z is None else _f64(initial_z)[..., None]
    o, ht = fwd(q, k, ones, g=g, g_gamma=g_gamma, scale=scale, initial_state=h0,
                cu_seqlens=cu_seqlens, nthreads=nthreads, lib=lib)
    return o[..., 0], ht[..., 0]


def parallel(q, k, v, g=None, g_gamma=None, scale=None, output_attn=True, nthreads=None, lib=None):
    """Parallel form (page "flash-linear-attention 中的 Simple GLA", section 二:
    the parallel entry builds the decayed attention matrix explicitly).  Per
    batch row and query head, with G_t the running sum of the log gates,
    A[i, j] = scale (q_i . k_j) exp(G_i - G_j) for j <= i and 0 above the
    diagonal; o = A v.  Dense input from a zero state.

    q: [B, T, H, K]; k: [B, T, Hkv, K]; v: [B, T, Hkv, V]; g: [B, T, H] or
    None; g_gamma: [H] or None.  Returns (o [B, T, H, V], A [B, H, T, T] or
    None), float64."""
    q, k, v, g, g_gamma = _f64(q), _f64(k), _f64(v), _f64(g), _f64(g_gamma)
    B, T, H, K = q.shape
    Hkv = k.shape[2]
    V = v.shape[-1]
    if scale is None:
        scale = K ** -0.5
    o = np.zeros((B, T, H, V))
    attn = np.zeros((B, H, T, T)) if output_attn else None
    lib = lib or load()
    rc = lib.sgla_oracle_parallel(B, T, H, Hkv, K, V, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(g_gamma),
                                  float(scale), _ptr(o), _ptr(attn), int(nthreads or default_threads()))
    if rc != 0:
        raise ValueError(f"sgla_oracle_parallel rejected its arguments (code {rc})")
    return o, attn


def step(q, k, v, g, state, scale=None, g_gamma=None, nthreads=None, lib=None,
         state_v_first=False):
    """One decode step.  q: [N, H, K]; k: [N, Hkv, K]; v: [N, Hkv, V];
    g: [N, H] or None; g_gamma: [H] or None (at most one);
    state: [N, H, K, V], or [N, H, V, K] with state_v_first (not modified; the
    updated copy is returned in the same layout).
    Returns (o [N, H, V], new_state), float64."""
    state = _vk(state, state_v_first)
    q, k, v, g, g_gamma = _f64(q), _f64(k), _f64(v), _f64(g), _f64(g_gamma)
    S = np.array(state, dtype=np.float64, order="C", copy=True)
    N, H, K = q.shape
    Hkv = k.shape[1]
    V = v.shape[-1]
    if scale is None:
        scale = K ** -0.5
    o = np.zeros((N, H, V), dtype=np.float64)
    lib = lib or load()
    rc = lib.sgla_oracle_step(N, H, Hkv, K, V, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(g_gamma),
                              float(scale), _ptr(S), _ptr(o), int(nthreads or default_threads()))
    if rc != 0:
        raise ValueError(f"sgla_oracle_step rejected its arguments (code {rc})")
    return o, _vk(S, state_v_first)


def chunk_local_cumsum(g, chunk_size=64, cu_seqlens=None, lib=None):
    """Chunk-local inclusive cumulative sum of g [B, T, H], divided by ln 2,
    restarting at every chunk of every sequence.  Returns float64 [B, T, H]."""
    g = _f64(g)
    B, T, H = g.shape
    cu = None
    N = B
    if cu_seqlens is not None:
        cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
        N = cu.shape[0] - 1
    gc = np.zeros_like(g)
    lib = lib or load()
    rc = lib.sgla_oracle_chunk_local_cumsum(
        B, T, H, _ptr(g), None if cu is None else cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
        N, int(chunk_size), _ptr(gc))
    if rc != 0:
        raise ValueError(f"sgla_oracle_chunk_local_cumsum rejected its arguments (code {rc})")
    return gc
