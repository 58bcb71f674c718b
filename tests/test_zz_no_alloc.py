"""The allocation-free forward (sgla_chunk_fwd_noalloc) against the forward
with a caller workspace (sgla_chunk_fwd), through the C ABI: the same
kernels, so the same results bit for bit, on two calls in a row whose second
input is smaller than the first (the fixed scratch array keeps the first
call's contents, which the second call must not depend on)."""
import ctypes

import numpy as np
import pytest
import torch

from gla_workloads import ChunkWorkload, make_chunk_inputs
from gpu_common import DEV, device_inputs

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

if torch.cuda.is_available():
    import gated_linear_attention_amd as sgla
else:  # pragma: no cover - collected on CPU-only hosts, never run
    sgla = None


def _call(inp, noalloc):
    d = device_inputs(inp)
    B, T, H, K, V, N = inp["B"], inp["T"], inp["H"], inp["K"], inp["V"], inp["N"]
    args = sgla._chunk_args(B, T, H, K, V, N, inp["chunk_size"], 1 if inp["dtype"] == "bf16" else 2, 2,
                            inp["scale"], 1, inp["Hkv"])
    cu = None if inp["cu_seqlens"] is None else np.ascontiguousarray(inp["cu_seqlens"], dtype=np.int64)
    cu_ptr = None if cu is None else ctypes.c_void_p(cu.ctypes.data)
    o = torch.full((B, T, H, V), float("nan"), device=DEV, dtype=torch.float32)
    ht = torch.full((N, H, K, V), float("nan"), device=DEV, dtype=torch.float32)
    p = sgla._ptr
    common = (ctypes.byref(args), p(d["q"]), p(d["k"]), p(d["v"]), p(d["g"]), p(d["g_gamma"]),
              p(d["initial_state"]), cu_ptr, p(o), p(ht))
    if noalloc:
        st = sgla.lib.sgla_chunk_fwd_noalloc(*common, sgla._stream(DEV))
    else:
        n = sgla._workspace_size(args, cu_ptr)
        ws = torch.empty(max(n, 1), device=DEV, dtype=torch.uint8)
        st = sgla.lib.sgla_chunk_fwd(*common, p(ws), n, sgla._stream(DEV))
    assert st == 0, sgla.lib.sgla_last_error().decode()
    torch.cuda.synchronize()
    return o.cpu().numpy(), ht.cpu().numpy()


def _w(name, **kw):
    base = dict(B=1, T=0, H=2, K=128, V=64, dtype="bf16", gate="g", initial_state=True, seed=90)
    base.update(kw)
    return ChunkWorkload(name, **base)


PAIRS = [
    # packed K = 128: the scratch holds the sequence and chunk tables
    (_w("packed_big", fixed_lengths=(300, 15, 900, 1, 64)), _w("packed_small", fixed_lengths=(70, 5))),
    # bf16 K = 512: the scratch holds the per-chunk preparation records too
    (_w("k512_big", B=2, T=200, H=2, K=512, V=64, initial_state=False),
     _w("k512_small", B=1, T=90, H=1, K=512, V=64, initial_state=False)),
    # chunk size 32 on packed float32 input
    (_w("c32_big", dtype="f32", K=64, fixed_lengths=(200, 33), chunk_size=32),
     _w("c32_small", dtype="f32", K=64, fixed_lengths=(17,), chunk_size=32)),
]


@pytest.mark.parametrize("big,small", PAIRS, ids=[p[0].name for p in PAIRS])
def test_noalloc_matches_workspace_call(big, small):
    for w in (big, small):
        inp = make_chunk_inputs(w)
        o1, h1 = _call(inp, noalloc=True)
        o2, h2 = _call(inp, noalloc=False)
        assert np.array_equal(o1, o2), w.name
        assert np.array_equal(h1, h2), w.name


def test_noalloc_rejects_oversize():
    """A request needing more scratch than the fixed array holds is refused
    before anything is enqueued (outputs untouched)."""
    inp = make_chunk_inputs(_w("huge", B=1, T=64 * 80, H=2, K=512, V=64, initial_state=False))
    need = sgla._workspace_size(sgla._chunk_args(1, inp["T"], 2, 512, 64, 1, 64, 1, 2, inp["scale"], 1),
                                None)
    assert need > sgla.lib.sgla_chunk_fwd_noalloc_max_bytes()
    d = device_inputs(inp)
    out = torch.full((1, inp["T"], 2, 64), 7.0, device=DEV)
    with pytest.raises(ValueError, match="scratch"):
        sgla.chunk_fwd_noalloc(d["q"], d["k"], d["v"], g=d["g"], scale=inp["scale"], out=out)
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)
