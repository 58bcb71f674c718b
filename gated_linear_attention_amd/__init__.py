"""Python binding of libsgla -- Simple GLA (head-wise gated linear attention)
on MI355X (gfx950).

This module only marshals arguments: it allocates outputs and workspace with
torch on the inputs' device, passes raw device pointers and torch's current
HIP stream through the C ABI declared in ``include/sgla.h``, and turns error
statuses into exceptions.  Every step of the computation runs in the HIP
kernels of ``libsgla.so``; there is no CPU or PyTorch fallback.  If the
library has not been built, importing this package raises ImportError.

Operator (page "flash-linear-attention 中的 Simple GLA", section 一):
    S_t = exp(g_t) S_{t-1} + k_t v_t^T,    o_t = scale * S_t^T q_t
API conventions follow section 二 of that page: q [B, T, H, K], k [B, T, Hkv,
K], v [B, T, Hkv, V], g [B, T, H] log gates or g_gamma [H] per-head log decay
(not both), scale defaulting to 1/sqrt(K), states [N, H, K, V], cu_seqlens
[N + 1] with B == 1 for packed input, chunk_size 16, 32 or 64 (default 64;
the decode and parallel entries take none).  The kv
head count Hkv is read from k's shape and must divide H: query head h reads kv
head h // (H // Hkv) (grouped-query attention, page "relinear", its GQA
target); Hkv == H is plain multi-head attention.  ``state_v_first=True``
keeps every state in the [N, H, V, K] layout instead (section 二).
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = ["chunk_fwd", "chunk_fwd_noalloc", "chunk_bwd", "gla_chunk_fwd", "chunk_normalizer", "recurrent_step_normalizer",
           "parallel_fwd",
           "recurrent_step", "chunk_local_cumsum", "library_path", "lib",
           "SglaError", "ABI_VERSION"]

ABI_VERSION = 5
_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libsgla.so")

_OK, _INVALID, _SHAPE, _DTYPE, _UNSUPPORTED, _WORKSPACE, _HIP = range(7)
_BF16, _F32 = 1, 2


class SglaError(RuntimeError):
    """A HIP runtime failure reported by libsgla."""


class _ChunkArgs(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("T", ctypes.c_int32), ("H", ctypes.c_int32),
                ("K", ctypes.c_int32), ("V", ctypes.c_int32), ("num_seqs", ctypes.c_int32),
                ("chunk_size", ctypes.c_int32), ("qkv_dtype", ctypes.c_int32),
                ("o_dtype", ctypes.c_int32), ("scale", ctypes.c_float),
                ("output_final_state", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("state_v_first", ctypes.c_int32)]


def library_path() -> str:
    return _LIB_PATH


def _load():
    if not os.path.exists(_LIB_PATH):
        raise ImportError(
            f"libsgla.so is not built ({_LIB_PATH} missing); run "
            "`python gated_linear_attention_amd/build.py` (hipcc, gfx950). There is no fallback.")
    lib = ctypes.CDLL(_LIB_PATH)
    vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
    pargs = ctypes.POINTER(_ChunkArgs)
    lib.sgla_abi_version.restype = ctypes.c_int
    lib.sgla_abi_version.argtypes = []
    lib.sgla_last_error.restype = ctypes.c_char_p
    lib.sgla_last_error.argtypes = []
    lib.sgla_chunk_fwd_workspace_size.restype = sz
    lib.sgla_chunk_fwd_workspace_size.argtypes = [pargs, vp]
    lib.sgla_chunk_fwd.restype = ctypes.c_int
    lib.sgla_chunk_fwd.argtypes = [pargs, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.sgla_chunk_fwd_noalloc_max_bytes.restype = sz
    lib.sgla_chunk_fwd_noalloc_max_bytes.argtypes = []
    lib.sgla_chunk_fwd_noalloc.restype = ctypes.c_int
    lib.sgla_chunk_fwd_noalloc.argtypes = [pargs, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.sgla_chunk_bwd_workspace_size.restype = sz
    lib.sgla_chunk_bwd_workspace_size.argtypes = [pargs, vp]
    lib.sgla_chunk_bwd.restype = ctypes.c_int
    lib.sgla_chunk_bwd.argtypes = [pargs] + [vp] * 15 + [vp, sz, vp]
    lib.sgla_gla_chunk_fwd.restype = ctypes.c_int
    lib.sgla_gla_chunk_fwd.argtypes = [pargs] + [vp] * 9 + [sz, vp]
    lib.sgla_chunk_normalizer_workspace_size.restype = sz
    lib.sgla_chunk_normalizer_workspace_size.argtypes = [pargs, vp]
    lib.sgla_gla_chunk_fwd_workspace_size.restype = sz
    lib.sgla_gla_chunk_fwd_workspace_size.argtypes = [pargs, vp]
    lib.sgla_chunk_normalizer.restype = ctypes.c_int
    lib.sgla_chunk_normalizer.argtypes = [pargs] + [vp] * 9 + [sz, vp]
    lib.sgla_recurrent_step_normalizer.restype = ctypes.c_int
    lib.sgla_recurrent_step_normalizer.argtypes = [i32, i32, i32, i32, f32, i32] + [vp] * 7
    lib.sgla_chunk_local_cumsum.restype = ctypes.c_int
    lib.sgla_chunk_local_cumsum.argtypes = [pargs, vp, vp, vp, vp, sz, vp]
    lib.sgla_recurrent_step.restype = ctypes.c_int
    lib.sgla_recurrent_step.argtypes = [i32, i32, i32, i32, i32, f32, i32, i32, i32, vp, vp, vp,
                                        vp, vp, vp, vp, vp]
    lib.sgla_parallel_fwd.restype = ctypes.c_int
    lib.sgla_parallel_fwd.argtypes = [pargs] + [vp] * 8
    if lib.sgla_abi_version() != ABI_VERSION:
        raise ImportError(f"libsgla ABI {lib.sgla_abi_version()} != binding ABI {ABI_VERSION}")
    return lib


lib = _load()


def _raise(status: int, what: str):
    msg = lib.sgla_last_error().decode(errors="replace")
    if status in (_INVALID, _SHAPE, _DTYPE, _UNSUPPORTED, _WORKSPACE):
        raise ValueError(f"{what}: {msg}")
    raise SglaError(f"{what} failed (status {status}): {msg}")


def _dtype_code(t: torch.dtype, what: str) -> int:
    if t == torch.bfloat16:
        return _BF16
    if t == torch.float32:
        return _F32
    raise ValueError(f"{what} must be bfloat16 or float32, got {t}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check_dev(name, t, dev, dtype=None, shape=None):
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device != dev:
        raise ValueError(f"{name} is on {t.device}, expected {dev}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _stream(dev) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _host_cu(cu_seqlens):
    if cu_seqlens is None:
        return None
    if isinstance(cu_seqlens, torch.Tensor):
        cu = cu_seqlens.detach().to("cpu", torch.int64).contiguous()
    else:
        cu = torch.as_tensor(list(cu_seqlens), dtype=torch.int64)
    if cu.dim() != 1 or cu.numel() < 2:
        raise ValueError("cu_seqlens must be a 1-D sequence of N + 1 offsets")
    return cu


def _chunk_args(B, T, H, K, V, N, chunk_size, qkv, o_dtype, scale, out_final, Hkv=0,
                state_v_first=False):
    return _ChunkArgs(B, T, H, K, V, N, chunk_size, qkv, o_dtype, float(scale), int(out_final),
                      int(Hkv), int(bool(state_v_first)))


def _state_shape(N, H, K, V, state_v_first):
    return (N, H, V, K) if state_v_first else (N, H, K, V)


def _kv_heads(k, H, axis):
    if not isinstance(k, torch.Tensor) or k.dim() <= axis:
        raise ValueError("k must be a tensor with a kv-head axis")
    Hkv = k.shape[axis]
    if Hkv < 1 or H % Hkv != 0:
        raise ValueError(f"the kv head count of k ({Hkv}) must divide the query head count ({H})")
    return Hkv


def _workspace_size(args, cu_ptr) -> int:
    n = lib.sgla_chunk_fwd_workspace_size(ctypes.byref(args), cu_ptr)
    if n == 0:
        msg = lib.sgla_last_error()
        if msg:
            raise ValueError(f"sgla_chunk_fwd_workspace_size: {msg.decode(errors='replace')}")
    return n


def chunk_fwd(q, k, v, g=None, g_gamma=None, scale=None, initial_state=None,
              output_final_state=False, cu_seqlens=None, chunk_size=64,
              o_dtype=torch.float32, out=None, state_v_first=False):
    """Chunked Simple GLA forward on the GPU.

    Returns ``(o, final_state)``; ``final_state`` is None unless
    ``output_final_state``.  ``out`` optionally supplies a preallocated o."""
    return _chunk_fwd(q, k, v, g, g_gamma, scale, initial_state, output_final_state, cu_seqlens,
                      chunk_size, o_dtype, out, state_v_first, None, False)


def chunk_fwd_noalloc(q, k, v, g=None, g_gamma=None, scale=None, initial_state=None,
                      output_final_state=False, cu_seqlens=None, chunk_size=64,
                      o_dtype=torch.float32, out=None, final_state=None, state_v_first=False):
    """chunk_fwd through sgla_chunk_fwd_noalloc: the library's fixed scratch
    array replaces the workspace.  With ``out`` (and ``final_state`` when
    ``output_final_state``) supplied, the call allocates nothing."""
    return _chunk_fwd(q, k, v, g, g_gamma, scale, initial_state, output_final_state, cu_seqlens,
                      chunk_size, o_dtype, out, state_v_first, final_state, True)


def _chunk_fwd(q, k, v, g, g_gamma, scale, initial_state, output_final_state, cu_seqlens,
               chunk_size, o_dtype, out, state_v_first, final_state, noalloc):
    if not isinstance(q, torch.Tensor) or q.dim() != 4:
        raise ValueError("q must be a 4-D tensor [B, T, H, K]")
    dev = q.device
    B, T, H, K = q.shape
    if v.dim() != 4:
        raise ValueError("v must be a 4-D tensor [B, T, H, V]")
    V = v.shape[-1]
    Hkv = _kv_heads(k, H, 2)
    qkv = _dtype_code(q.dtype, "q")
    _check_dev("q", q, dev)
    _check_dev("k", k, dev, q.dtype, (B, T, Hkv, K))
    _check_dev("v", v, dev, q.dtype, (B, T, Hkv, V))
    if g is not None and g_gamma is not None:
        raise ValueError("g and g_gamma are mutually exclusive; pass at most one")
    _check_dev("g", g, dev, torch.float32, (B, T, H))
    _check_dev("g_gamma", g_gamma, dev, torch.float32, (H,))
    cu = _host_cu(cu_seqlens)
    N = B if cu is None else cu.numel() - 1
    if cu is not None and B != 1:
        raise ValueError(f"packed input (cu_seqlens) requires B == 1, got B={B}")
    if initial_state is not None and initial_state.shape[0] != N:
        raise ValueError(f"initial_state must have {N} rows (one per sequence), got "
                         f"{initial_state.shape[0]}")
    sshape = _state_shape(N, H, K, V, state_v_first)
    _check_dev("initial_state", initial_state, dev, torch.float32, sshape)
    if scale is None:
        scale = K ** -0.5
    od = _dtype_code(o_dtype, "o_dtype")
    args = _chunk_args(B, T, H, K, V, N, chunk_size, qkv, od, scale, output_final_state, Hkv,
                       state_v_first)
    cu_ptr = None if cu is None else ctypes.c_void_p(cu.data_ptr())
    if out is None:
        o = torch.empty((B, T, H, V), device=dev, dtype=o_dtype)
    else:
        _check_dev("out", out, dev, o_dtype, (B, T, H, V))
        o = out
    ht = None
    if output_final_state:
        if final_state is None:
            ht = torch.empty(sshape, device=dev, dtype=torch.float32)
        else:
            _check_dev("final_state", final_state, dev, torch.float32, sshape)
            ht = final_state
    if noalloc:
        st = lib.sgla_chunk_fwd_noalloc(ctypes.byref(args), _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                        _ptr(g_gamma), _ptr(initial_state), cu_ptr, _ptr(o), _ptr(ht),
                                        _stream(dev))
        if st != _OK:
            _raise(st, "sgla_chunk_fwd_noalloc")
        return o, ht
    ws_bytes = _workspace_size(args, cu_ptr)
    ws = torch.empty(max(ws_bytes, 1), device=dev, dtype=torch.uint8)
    st = lib.sgla_chunk_fwd(ctypes.byref(args), _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                            _ptr(g_gamma), _ptr(initial_state), cu_ptr, _ptr(o), _ptr(ht),
                            _ptr(ws), ws_bytes, _stream(dev))
    if st != _OK:
        _raise(st, "sgla_chunk_fwd")
    return o, ht


def chunk_bwd(q, k, v, do, g=None, g_gamma=None, scale=None, initial_state=None, dht=None,
              cu_seqlens=None, chunk_size=64, state_v_first=False):
    """Backward of chunk_fwd on the GPU: gradients of sum <do, o> + sum <dht,
    final_state> (dht None: no loss on the final state).

    q [B, T, H, K], k [B, T, Hkv, K], v [B, T, Hkv, V], do [B, T, H, V] (all
    bf16 or all float32; Hkv divides H), g, g_gamma, initial_state and
    cu_seqlens as for chunk_fwd.  Returns a dict of float32 tensors: dq [B, T,
    H, K], dk [B, T, Hkv, K], dv [B, T, Hkv, V] (a kv head's gradient sums
    the query heads that read it), dg [B, T, H] (None without g), dg_gamma [H]
    (None without g_gamma), dh0 [N, H, K, V]."""
    if not isinstance(q, torch.Tensor) or q.dim() != 4:
        raise ValueError("q must be a 4-D tensor [B, T, H, K]")
    dev = q.device
    B, T, H, K = q.shape
    if not isinstance(v, torch.Tensor) or v.dim() != 4:
        raise ValueError("v must be a 4-D tensor [B, T, Hkv, V]")
    V = v.shape[-1]
    Hkv = _kv_heads(k, H, 2)
    qkv = _dtype_code(q.dtype, "q")
    _check_dev("q", q, dev)
    _check_dev("k", k, dev, q.dtype, (B, T, Hkv, K))
    _check_dev("v", v, dev, q.dtype, (B, T, Hkv, V))
    _check_dev("do", do, dev, q.dtype, (B, T, H, V))
    if g is not None and g_gamma is not None:
        raise ValueError("g and g_gamma are mutually exclusive; pass at most one")
    _check_dev("g", g, dev, torch.float32, (B, T, H))
    _check_dev("g_gamma", g_gamma, dev, torch.float32, (H,))
    cu = _host_cu(cu_seqlens)
    N = B if cu is None else cu.numel() - 1
    if cu is not None and B != 1:
        raise ValueError(f"packed input (cu_seqlens) requires B == 1, got B={B}")
    sshape = _state_shape(N, H, K, V, state_v_first)
    _check_dev("initial_state", initial_state, dev, torch.float32, sshape)
    _check_dev("dht", dht, dev, torch.float32, sshape)
    if scale is None:
        scale = K ** -0.5
    args = _chunk_args(B, T, H, K, V, N, chunk_size, qkv, _F32, scale, 0, Hkv, state_v_first)
    cu_ptr = None if cu is None else ctypes.c_void_p(cu.data_ptr())
    n = lib.sgla_chunk_bwd_workspace_size(ctypes.byref(args), cu_ptr)
    if n == 0 and lib.sgla_last_error():
        raise ValueError(f"sgla_chunk_bwd_workspace_size: {lib.sgla_last_error().decode(errors='replace')}")
    f32 = dict(device=dev, dtype=torch.float32)
    dq = torch.empty((B, T, H, K), **f32)
    dk = torch.empty((B, T, Hkv, K), **f32)
    dv = torch.empty((B, T, Hkv, V), **f32)
    dg = torch.empty((B, T, H), **f32) if g is not None else None
    dgg = torch.empty((H,), **f32) if g_gamma is not None else None
    dh0 = torch.empty(sshape, **f32)
    ws = torch.empty(max(n, 1), device=dev, dtype=torch.uint8)
    st = lib.sgla_chunk_bwd(ctypes.byref(args), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(g_gamma),
                            _ptr(initial_state), cu_ptr, _ptr(do), _ptr(dht), _ptr(dq), _ptr(dk),
                            _ptr(dv), _ptr(dg), _ptr(dgg), _ptr(dh0), _ptr(ws), n, _stream(dev))
    if st != _OK:
        _raise(st, "sgla_chunk_bwd")
    return dict(dq=dq, dk=dk, dv=dv, dg=dg, dg_gamma=dgg, dh0=dh0)


def gla_chunk_fwd(q, k, v, gk, scale=None, initial_state=None, output_final_state=False,
                  cu_seqlens=None, chunk_size=64, o_dtype=torch.float32, state_v_first=False):
    """Chunked forward of elementwise-gate GLA: S_t = diag(exp(gk_t)) S_{t-1} +
    k_t v_t^T, o_t = scale S_t^T q_t.  q [B, T, H, K], k [B, T, Hkv, K], v [B,
    T, Hkv, V] (bf16 or float32), gk [B, T, H, K] float32 log gates (one per
    key).  Returns (o, final_state or None)."""
    if not isinstance(q, torch.Tensor) or q.dim() != 4:
        raise ValueError("q must be a 4-D tensor [B, T, H, K]")
    dev = q.device
    B, T, H, K = q.shape
    if not isinstance(v, torch.Tensor) or v.dim() != 4:
        raise ValueError("v must be a 4-D tensor [B, T, Hkv, V]")
    V = v.shape[-1]
    Hkv = _kv_heads(k, H, 2)
    qkv = _dtype_code(q.dtype, "q")
    _check_dev("q", q, dev)
    _check_dev("k", k, dev, q.dtype, (B, T, Hkv, K))
    _check_dev("v", v, dev, q.dtype, (B, T, Hkv, V))
    _check_dev("gk", gk, dev, torch.float32, (B, T, H, K))
    cu = _host_cu(cu_seqlens)
    N = B if cu is None else cu.numel() - 1
    if cu is not None and B != 1:
        raise ValueError(f"packed input (cu_seqlens) requires B == 1, got B={B}")
    sshape = _state_shape(N, H, K, V, state_v_first)
    _check_dev("initial_state", initial_state, dev, torch.float32, sshape)
    if scale is None:
        scale = K ** -0.5
    od = _dtype_code(o_dtype, "o_dtype")
    args = _chunk_args(B, T, H, K, V, N, chunk_size, qkv, od, scale, output_final_state, Hkv,
                       state_v_first)
    cu_ptr = None if cu is None else ctypes.c_void_p(cu.data_ptr())
    n = lib.sgla_gla_chunk_fwd_workspace_size(ctypes.byref(args), cu_ptr)
    if n == 0 and lib.sgla_last_error():
        raise ValueError(lib.sgla_last_error().decode(errors="replace"))
    o = torch.empty((B, T, H, V), device=dev, dtype=o_dtype)
    ht = torch.empty(sshape, device=dev, dtype=torch.float32) if output_final_state else None
    ws = torch.empty(max(n, 1), device=dev, dtype=torch.uint8)
    st = lib.sgla_gla_chunk_fwd(ctypes.byref(args), _ptr(q), _ptr(k), _ptr(v), _ptr(gk),
                                _ptr(initial_state), cu_ptr, _ptr(o), _ptr(ht), _ptr(ws), n,
                                _stream(dev))
    if st != _OK:
        _raise(st, "sgla_gla_chunk_fwd")
    return o, ht


def chunk_normalizer(q, k, g=None, g_gamma=None, scale=None, initial_z=None,
                     output_final_state=False, cu_seqlens=None, chunk_size=64):
    """Running normalizer den_t = scale * q_t . z_t, z_t = exp(g_t) z_{t-1} +
    k_t (the ones column of the relinear pages' augmented value).  q [B, T,
    H, K], k [B, T, Hkv, K]; initial_z [N, H, K] float32 or None.  Returns
    (den [B, T, H] float32, final_z [N, H, K] float32 or None)."""
    if not isinstance(q, torch.Tensor) or q.dim() != 4:
        raise ValueError("q must be a 4-D tensor [B, T, H, K]")
    dev = q.device
    B, T, H, K = q.shape
    Hkv = _kv_heads(k, H, 2)
    qkv = _dtype_code(q.dtype, "q")
    _check_dev("q", q, dev)
    _check_dev("k", k, dev, q.dtype, (B, T, Hkv, K))
    if g is not None and g_gamma is not None:
        raise ValueError("g and g_gamma are mutually exclusive; pass at most one")
    _check_dev("g", g, dev, torch.float32, (B, T, H))
    _check_dev("g_gamma", g_gamma, dev, torch.float32, (H,))
    cu = _host_cu(cu_seqlens)
    N = B if cu is None else cu.numel() - 1
    if cu is not None and B != 1:
        raise ValueError(f"packed input (cu_seqlens) requires B == 1, got B={B}")
    _check_dev("initial_z", initial_z, dev, torch.float32, (N, H, K))
    if scale is None:
        scale = K ** -0.5
    args = _chunk_args(B, T, H, K, 0, N, chunk_size, qkv, _F32, scale, output_final_state, Hkv)
    cu_ptr = None if cu is None else ctypes.c_void_p(cu.data_ptr())
    n = lib.sgla_chunk_normalizer_workspace_size(ctypes.byref(args), cu_ptr)
    if n == 0 and lib.sgla_last_error():
        raise ValueError(f"sgla_chunk_normalizer_workspace_size: "
                         f"{lib.sgla_last_error().decode(errors='replace')}")
    den = torch.empty((B, T, H), device=dev, dtype=torch.float32)
    zt = torch.empty((N, H, K), device=dev, dtype=torch.float32) if output_final_state else None
    ws = torch.empty(max(n, 1), device=dev, dtype=torch.uint8)
    st = lib.sgla_chunk_normalizer(ctypes.byref(args), _ptr(q), _ptr(k), _ptr(g), _ptr(g_gamma),
                                   _ptr(initial_z), cu_ptr, _ptr(den), _ptr(zt), _ptr(ws), n,
                                   _stream(dev))
    if st != _OK:
        _raise(st, "sgla_chunk_normalizer")
    return den, zt


def parallel_fwd(q, k, v, g=None, g_gamma=None, scale=None, output_attn=True, out_dtype=None):
    """Parallel form (page "flash-linear-attention 中的 Simple GLA", section 二:
    the parallel entry writes out the decayed attention matrix).  Per batch
    row and query head, A[i, j] = scale (q_i . k_j) exp(G_i - G_j) for j <= i
    (G the running sum of the log gates) and 0 above the diagonal; o = A v.
    Dense q [B, T, H, K], k [B, T, Hkv, K], v [B, T, Hkv, V], all bf16 or all
    float32 (float32 inputs run on the fp32 matrix cores); g [B, T, H]
    or g_gamma [H] (at most one).  Returns (o [B, T, H, V] in out_dtype
    (default: q's dtype), A [B, H, T, T] float32 or None)."""
    if not isinstance(q, torch.Tensor) or q.dim() != 4:
        raise ValueError("q must be a 4-D tensor [B, T, H, K]")
    dev = q.device
    B, T, H, K = q.shape
    Hkv = _kv_heads(k, H, 2)
    if not isinstance(v, torch.Tensor) or v.dim() != 4:
        raise ValueError("v must be a 4-D tensor [B, T, Hkv, V]")
    V = v.shape[-1]
    qkv = _dtype_code(q.dtype, "q")
    _check_dev("q", q, dev)
    _check_dev("k", k, dev, q.dtype, (B, T, Hkv, K))
    _check_dev("v", v, dev, q.dtype, (B, T, Hkv, V))
    if g is not None and g_gamma is not None:
        raise ValueError("g and g_gamma are mutually exclusive; pass at most one")
    _check_dev("g", g, dev, torch.float32, (B, T, H))
    _check_dev("g_gamma", g_gamma, dev, torch.float32, (H,))
    out_dtype = q.dtype if out_dtype is None else out_dtype
    if scale is None:
        scale = K ** -0.5
    args = _chunk_args(B, T, H, K, V, B, 64, qkv, _dtype_code(out_dtype, "out_dtype"), scale, False, Hkv)
    o = torch.empty((B, T, H, V), device=dev, dtype=out_dtype)
    attn = torch.empty((B, H, T, T), device=dev, dtype=torch.float32) if output_attn else None
    st = lib.sgla_parallel_fwd(ctypes.byref(args), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(g_gamma),
                               _ptr(o), _ptr(attn), _stream(dev))
    if st != _OK:
        _raise(st, "sgla_parallel_fwd")
    return o, attn


def recurrent_step_normalizer(q, k, g, z, scale=None, g_gamma=None):
    """One decode step of the running normalizer; ``z`` [N, H, K] float32 is
    updated in place.  q [N, H, K], k [N, Hkv, K]; g [N, H] or None, g_gamma
    [H] or None.  Returns den [N, H] float32."""
    if not isinstance(q, torch.Tensor) or q.dim() != 3:
        raise ValueError("q must be a 3-D tensor [N, H, K]")
    dev = q.device
    N, H, K = q.shape
    Hkv = _kv_heads(k, H, 1)
    qkv = _dtype_code(q.dtype, "q")
    _check_dev("q", q, dev)
    _check_dev("k", k, dev, q.dtype, (N, Hkv, K))
    if g is not None and g_gamma is not None:
        raise ValueError("g and g_gamma are mutually exclusive; pass at most one")
    _check_dev("g", g, dev, torch.float32, (N, H))
    _check_dev("g_gamma", g_gamma, dev, torch.float32, (H,))
    _check_dev("z", z, dev, torch.float32, (N, H, K))
    if scale is None:
        scale = K ** -0.5
    den = torch.empty((N, H), device=dev, dtype=torch.float32)
    st = lib.sgla_recurrent_step_normalizer(N, H, Hkv, K, float(scale), qkv, _ptr(q), _ptr(k), _ptr(g),
                                            _ptr(g_gamma), _ptr(z), _ptr(den), _stream(dev))
    if st != _OK:
        _raise(st, "sgla_recurrent_step_normalizer")
    return den


def chunk_local_cumsum(g, chunk_size=64, cu_seqlens=None):
    """Step (1) alone: chunk-local inclusive cumulative sum of g times 1/ln 2
    (float32 [B, T, H] in, float32 [B, T, H] out)."""
    if not isinstance(g, torch.Tensor) or g.dim() != 3:
        raise ValueError("g must be a 3-D tensor [B, T, H]")
    dev = g.device
    _check_dev("g", g, dev, torch.float32)
    B, T, H = g.shape
    cu = _host_cu(cu_seqlens)
    N = B if cu is None else cu.numel() - 1
    args = _chunk_args(B, T, H, 64, 64, N, chunk_size, _BF16, _F32, 1.0, 0)
    cu_ptr = None if cu is None else ctypes.c_void_p(cu.data_ptr())
    ws_bytes = _workspace_size(args, cu_ptr)
    ws = torch.empty(max(ws_bytes, 1), device=dev, dtype=torch.uint8)
    gc = torch.empty_like(g)
    st = lib.sgla_chunk_local_cumsum(ctypes.byref(args), _ptr(g), cu_ptr, _ptr(gc), _ptr(ws),
                                     ws_bytes, _stream(dev))
    if st != _OK:
        _raise(st, "sgla_chunk_local_cumsum")
    return gc


def recurrent_step(q, k, v, g, state, scale=None, o_dtype=torch.float32, out=None,
                   g_gamma=None, state_v_first=False):
    """One decode step; ``state`` [N, H, K, V] float32 is updated in place.
    q [N, H, K], k [N, Hkv, K], v [N, Hkv, V] (bf16 or float32); g [N, H]
    float32 log gate or None; g_gamma [H] float32 per-head log decay or None
    (at most one; neither means no decay).  Returns o [N, H, V]."""
    if not isinstance(q, torch.Tensor) or q.dim() != 3:
        raise ValueError("q must be a 3-D tensor [N, H, K]")
    dev = q.device
    N, H, K = q.shape
    V = v.shape[-1]
    Hkv = _kv_heads(k, H, 1)
    qkv = _dtype_code(q.dtype, "q")
    _check_dev("q", q, dev)
    _check_dev("k", k, dev, q.dtype, (N, Hkv, K))
    _check_dev("v", v, dev, q.dtype, (N, Hkv, V))
    if g is not None and g_gamma is not None:
        raise ValueError("g and g_gamma are mutually exclusive; pass at most one")
    _check_dev("g", g, dev, torch.float32, (N, H))
    _check_dev("g_gamma", g_gamma, dev, torch.float32, (H,))
    _check_dev("state", state, dev, torch.float32, _state_shape(N, H, K, V, state_v_first))
    if scale is None:
        scale = K ** -0.5
    od = _dtype_code(o_dtype, "o_dtype")
    if out is None:
        o = torch.empty((N, H, V), device=dev, dtype=o_dtype)
    else:
        _check_dev("out", out, dev, o_dtype, (N, H, V))
        o = out
    st = lib.sgla_recurrent_step(N, H, Hkv, K, V, float(scale), qkv, od, int(bool(state_v_first)),
                                 _ptr(q), _ptr(k), _ptr(v),
                                 _ptr(g), _ptr(g_gamma), _ptr(state), _ptr(o), _stream(dev))
    if st != _OK:
        _raise(st, "sgla_recurrent_step")
    return o
