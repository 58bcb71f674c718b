"""GPU parity: libsgla's HIP kernels against the fp64 CPU oracle.

Every test calls the C ABI through the thin ctypes binding and compares with
the oracle on the same seeded inputs.  The bar (one number per output
tensor): max |gpu - oracle| / RMS(oracle) <= 2e-2 for bf16 inputs and 1e-4
for float32 inputs.  Every case compares every element, the full-size named
workloads included (they run the launch the benchmark times).
"""
import numpy as np
import pytest
import torch

import oracle
from gla_workloads import (CHUNK_CONFIGS, DECODE_CONFIGS, ChunkWorkload, DecodeWorkload,
                           make_chunk_inputs, make_decode_inputs)
from gpu_common import DEV, TOL_BF16, TOL_F32, device_inputs, err_ratio, to_dev

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

if torch.cuda.is_available():
    import gated_linear_attention_amd as sgla
else:  # pragma: no cover - collected on CPU-only hosts, never run
    sgla = None


def _tol(dtype):
    return TOL_BF16 if dtype == "bf16" else TOL_F32


def run_chunk(inp, o_dtype=torch.float32, output_final_state=None):
    d = device_inputs(inp)
    ofs = inp["output_final_state"] if output_final_state is None else output_final_state
    o, ht = sgla.chunk_fwd(d["q"], d["k"], d["v"], g=d["g"], g_gamma=d["g_gamma"],
                           scale=inp["scale"], initial_state=d["initial_state"],
                           output_final_state=ofs, cu_seqlens=inp["cu_seqlens"],
                           chunk_size=inp["chunk_size"], o_dtype=o_dtype)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), (None if ht is None else ht.cpu().numpy())


def check_full(inp, o_gpu, ht_gpu):
    o_ref, ht_ref = oracle.fwd(inp["q"], inp["k"], inp["v"], g=inp["g"], g_gamma=inp["g_gamma"],
                               scale=inp["scale"], initial_state=inp["initial_state"],
                               cu_seqlens=inp["cu_seqlens"])
    tol = _tol(inp["dtype"])
    eo = err_ratio(o_gpu, o_ref)
    print(f"[parity {inp['dtype']} K={inp['K']} V={inp['V']}] o err/RMS={eo:.3e}", flush=True)
    assert np.all(np.isfinite(o_gpu))
    assert eo <= tol, f"o: max err / RMS = {eo:.3e} > {tol}"
    if ht_gpu is not None:
        eh = err_ratio(ht_gpu, ht_ref)
        assert eh <= tol, f"final_state: max err / RMS = {eh:.3e} > {tol}"
    return o_ref, ht_ref


def small(name, **kw):
    base = dict(B=2, T=200, H=3, K=64, V=64, dtype="bf16", gate="g", seed=7)
    base.update(kw)
    return ChunkWorkload(name, **base)


# ---------------------------------------------------------------------------
# step (1): chunk-local cumulative gate
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("chunk", [1, 4, 8, 16, 32, 64])
@pytest.mark.parametrize("cu", [None, [0, 15, 100, 300, 1200, 2000], [0, 0, 1, 65, 65, 200]])
def test_gate_cumsum(cu, chunk):
    rng = np.random.default_rng(3)
    if cu is None:
        g = (-np.abs(rng.standard_normal((3, 333, 5)))).astype(np.float32)
    else:
        g = (-np.abs(rng.standard_normal((1, cu[-1], 5)))).astype(np.float32)
    gc = sgla.chunk_local_cumsum(to_dev(g, torch.float32), chunk_size=chunk, cu_seqlens=cu)
    torch.cuda.synchronize()
    ref = oracle.chunk_local_cumsum(g, chunk_size=chunk, cu_seqlens=cu)
    got = gc.cpu().numpy().astype(np.float64)
    # one float32 rounding of a float64 sum
    assert np.all(np.abs(got - ref) <= 1e-6 * np.maximum(1.0, np.abs(ref)))


# ---------------------------------------------------------------------------
# steps (2)+(3): chunked forward, small cases compared element by element
# ---------------------------------------------------------------------------

SMALL_CASES = [
    small("ragged_k64", T=200),
    small("ragged_k128_v128", K=128, V=128, T=131),
    small("k256_v64", K=256, V=64, T=150, H=2),
    small("k512_v128", K=512, V=128, T=140, B=1, H=2),
    small("k512_v96_varlen", B=1, T=0, H=2, K=512, V=96, fixed_lengths=(70, 1, 0, 130),
          initial_state=True),
    small("k256_v32_gamma", K=256, V=32, gate="gamma", T=200, normalize_k=True),
    small("k256_v64_t64", K=256, V=64, T=64, initial_state=True),
    small("k256_no_gate", K=256, V=64, T=150, gate="none", H=2),
    small("k512_strong_gate", K=512, V=64, T=150, B=1, H=2, gate_normalizer=0.1, scale=0.1),
    small("k512_v512_16_tiles", K=512, V=512, T=100, B=1, H=1, initial_state=True),
    small("v192_multi_tile", K=64, V=192, T=97),
    small("gamma", gate="gamma", K=128, V=128, T=300, normalize_k=True),
    small("no_gate", gate="none", K=64, V=64, T=129),
    small("h0", initial_state=True, K=128, V=64, T=77),
    small("norm0.1_scale0.1", gate_normalizer=0.1, scale=0.1, T=190),
    small("norm10_scale1", gate_normalizer=10.0, scale=1.0, T=190),
    small("t1", T=1, initial_state=True),
    small("t63", T=63),
    small("t64", T=64),
    small("t65", T=65, initial_state=True),
    small("empty_T0", T=0, initial_state=True),
    small("varlen_fla", B=1, T=0, H=2, K=128, V=128, fixed_lengths=(15, 85, 200, 900, 800),
          initial_state=True),
    small("varlen_zero_len", B=1, T=0, H=2, K=64, V=64, fixed_lengths=(0, 1, 64, 0, 65, 130),
          initial_state=True),
    small("f32_k16_v32", dtype="f32", K=16, V=32, T=150),
    small("f32_k32_v96", dtype="f32", K=32, V=96, T=70, initial_state=True),
    small("f32_k128_v64", dtype="f32", K=128, V=64, T=130, gate="gamma"),
    small("f32_varlen", dtype="f32", B=1, T=0, K=64, V=64, fixed_lengths=(15, 85, 200),
          initial_state=True),
    # grouped kv heads: query head h reads kv head h // (H // Hkv)
    small("gqa_k64_h4_kv2", H=4, Hkv=2, K=64, V=128, T=150, initial_state=True),
    small("mqa_k128_gamma", H=4, Hkv=1, K=128, V=64, T=200, gate="gamma", normalize_k=True),
    small("gqa_k128_h6_kv2_varlen", B=1, T=0, H=6, Hkv=2, K=128, V=64,
          fixed_lengths=(15, 85, 0, 200), initial_state=True),
    small("gqa_k512_h4_kv2", B=1, T=140, H=4, Hkv=2, K=512, V=96),
    small("mqa_k256_h3", T=130, H=3, Hkv=1, K=256, V=64, initial_state=True),
    small("gqa_k256_h6_kv3_varlen", B=1, T=0, H=6, Hkv=3, K=256, V=32,
          fixed_lengths=(70, 1, 0, 130), initial_state=True),
    small("gqa_f32_k32", dtype="f32", H=4, Hkv=2, K=32, V=64, T=100, initial_state=True),
]


@pytest.mark.parametrize("w", SMALL_CASES, ids=lambda w: w.name)
def test_chunk_small(w):
    inp = make_chunk_inputs(w)
    o, ht = run_chunk(inp)
    check_full(inp, o, ht)


@pytest.mark.parametrize("K", [128, 512])
def test_chunk_bf16_output(K):
    """A bf16 o is the fp32 result rounded once: its error is bounded by the
    fp32 tolerance plus half a bf16 ulp of each element."""
    inp = make_chunk_inputs(small("bf16o", K=K, V=128, T=257, H=2))
    o, _ = run_chunk(inp, o_dtype=torch.bfloat16)
    o_ref, _ = oracle.fwd(inp["q"], inp["k"], inp["v"], g=inp["g"], scale=inp["scale"])
    rms = np.sqrt(np.mean(o_ref ** 2))
    bound = TOL_BF16 * rms + 2.0 ** -8 * np.abs(o_ref)
    assert np.all(np.abs(o - o_ref) <= bound)


# ---------------------------------------------------------------------------
# the named workloads at full size (whole tensors)
# ---------------------------------------------------------------------------

def test_tiny_f32_full():
    inp = make_chunk_inputs(CHUNK_CONFIGS["tiny_f32"])
    o, ht = run_chunk(inp)
    check_full(inp, o, ht)


@pytest.mark.parametrize("cfg", ["dense_bf16_k512", "varlen_bf16_k128", "long_gamma_k128",
                                 "gqa_bf16_k64_h9kv3"])
def test_named_workload_full(cfg):
    """The named workloads at full size, in the launch the benchmark times,
    compared element by element with the oracle over the whole o and
    final_state tensors (RMS taken over the whole tensor)."""
    w = CHUNK_CONFIGS[cfg]
    inp = make_chunk_inputs(w)
    print(f"[{cfg}] B={inp['B']} T={inp['T']} H={inp['H']} K={inp['K']} V={inp['V']} "
          f"N={inp['N']}", flush=True)
    o, ht = run_chunk(inp, output_final_state=True)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(ht))
    o_ref, ht_ref = oracle.fwd(inp["q"], inp["k"], inp["v"], g=inp["g"], g_gamma=inp["g_gamma"],
                               scale=inp["scale"], initial_state=inp["initial_state"],
                               cu_seqlens=inp["cu_seqlens"])
    eo, eh = err_ratio(o, o_ref), err_ratio(ht, ht_ref)
    print(f"[{cfg}] whole-tensor o err/RMS={eo:.3e} final err/RMS={eh:.3e}", flush=True)
    assert eo <= TOL_BF16 and eh <= TOL_BF16


# ---------------------------------------------------------------------------
# cross-path properties
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("K", [128, 512])
def test_varlen_equals_per_sequence_bitwise(K):
    """Packed sequences give exactly the per-sequence results (each sequence
    is processed by the same code from its own start)."""
    w = small("pack", B=1, T=0, H=2, K=K, V=128, fixed_lengths=(100, 64, 257, 1),
              initial_state=True)
    inp = make_chunk_inputs(w)
    o, ht = run_chunk(inp)
    cu = inp["cu_seqlens"]
    for n in range(len(cu) - 1):
        s, e = int(cu[n]), int(cu[n + 1])
        sub = dict(inp)
        for key in ("q", "k", "v", "g"):
            sub[key] = inp[key][:, s:e].copy()
        sub["initial_state"] = inp["initial_state"][n:n + 1].copy()
        sub["cu_seqlens"] = None
        on, hn = run_chunk(sub)
        assert np.array_equal(on[0], o[0, s:e])
        assert np.array_equal(hn[0], ht[n])


@pytest.mark.parametrize("K", [128, 512])
def test_split_at_chunk_boundary_bitwise(K):
    """Running tokens [0, 128) then [128, T) from the carried state equals one
    pass exactly (the split falls on a chunk boundary)."""
    inp = make_chunk_inputs(small("split", B=1, T=300, H=2, K=K, V=64, initial_state=True))
    o, ht = run_chunk(inp)
    a, b = dict(inp), dict(inp)
    for key in ("q", "k", "v", "g"):
        a[key] = inp[key][:, :128].copy()
        b[key] = inp[key][:, 128:].copy()
    oa, ha = run_chunk(a)
    b["initial_state"] = ha
    ob, hb = run_chunk(b)
    assert np.array_equal(np.concatenate([oa, ob], axis=1), o)
    assert np.array_equal(hb, ht)


@pytest.mark.parametrize("K", [128, 512])
def test_deterministic(K):
    inp = make_chunk_inputs(small("det", K=K, V=128, T=333, initial_state=True))
    o1, h1 = run_chunk(inp)
    o2, h2 = run_chunk(inp)
    assert np.array_equal(o1, o2) and np.array_equal(h1, h2)


@pytest.mark.parametrize("K", [64, 512])
def test_in_place_state(K):
    """final_state may alias initial_state exactly."""
    inp = make_chunk_inputs(small("inplace", K=K, V=64, T=100, initial_state=True))
    d = device_inputs(inp)
    o_ref, h_ref = run_chunk(inp)
    state = d["initial_state"]
    args = sgla._chunk_args(inp["B"], inp["T"], inp["H"], inp["K"], inp["V"], inp["N"], 64,
                            1, 2, inp["scale"], 1)
    ws_n = sgla._workspace_size(args, None)
    ws = torch.empty(max(ws_n, 1), device=DEV, dtype=torch.uint8)
    o = torch.empty((inp["B"], inp["T"], inp["H"], inp["V"]), device=DEV, dtype=torch.float32)
    st = sgla.lib.sgla_chunk_fwd(
        __import__("ctypes").byref(args), sgla._ptr(d["q"]), sgla._ptr(d["k"]), sgla._ptr(d["v"]),
        sgla._ptr(d["g"]), None, sgla._ptr(state), None, sgla._ptr(o), sgla._ptr(state),
        sgla._ptr(ws), ws_n, sgla._stream(DEV))
    assert st == 0
    torch.cuda.synchronize()
    assert np.array_equal(o.cpu().numpy(), o_ref)
    assert np.array_equal(state.cpu().numpy(), h_ref)


def test_prefill_then_decode():
    """A chunked prefill of T tokens and T decode steps from the same initial
    state agree (both within tolerance of the oracle and of each other)."""
    w = small("pd", B=3, T=70, H=2, K=128, V=128, initial_state=True)
    inp = make_chunk_inputs(w)
    o_chunk, ht_chunk = run_chunk(inp)
    d = device_inputs(inp)
    state = d["initial_state"].clone()
    outs = []
    for t in range(inp["T"]):
        ot = sgla.recurrent_step(d["q"][:, t].contiguous(), d["k"][:, t].contiguous(),
                                 d["v"][:, t].contiguous(), d["g"][:, t].contiguous(), state,
                                 scale=inp["scale"])
        outs.append(ot)
    torch.cuda.synchronize()
    o_dec = torch.stack(outs, dim=1).cpu().numpy()
    o_ref, ht_ref = check_full(inp, o_chunk, ht_chunk)
    assert err_ratio(o_dec, o_ref) <= TOL_BF16
    assert err_ratio(state.cpu().numpy(), ht_ref) <= TOL_BF16
    assert err_ratio(o_dec, o_chunk) <= TOL_BF16


def test_chunk_then_decode_handoff():
    """The state a prefill leaves behind drives decode exactly like the
    oracle's state (the [N, H, K, V] layout is shared by both entry points)."""
    inp = make_chunk_inputs(small("handoff", B=2, T=130, H=2, K=64, V=64))
    _, ht = run_chunk(inp, output_final_state=True)
    rng = np.random.default_rng(9)
    q, k = [rng.standard_normal((2, 2, 64)).astype(np.float32) for _ in range(2)]
    v = rng.standard_normal((2, 2, 64)).astype(np.float32)
    g = -np.abs(rng.standard_normal((2, 2))).astype(np.float32)
    state = torch.from_numpy(ht).to(DEV)
    o = sgla.recurrent_step(to_dev(q, torch.float32), to_dev(k, torch.float32),
                            to_dev(v, torch.float32), to_dev(g, torch.float32), state)
    torch.cuda.synchronize()
    _, ht_ref = oracle.fwd(inp["q"], inp["k"], inp["v"], g=inp["g"], scale=inp["scale"])
    o_ref, s_ref = oracle.step(q, k, v, g, ht_ref)
    assert err_ratio(o.cpu().numpy(), o_ref) <= TOL_BF16
    assert err_ratio(state.cpu().numpy(), s_ref) <= TOL_BF16


# ---------------------------------------------------------------------------
# step (4): decode
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("K,V,H,Hkv,dtype", [(64, 64, 4, 4, "bf16"), (128, 128, 6, 2, "bf16"),
                                             (128, 256, 4, 1, "f32")])
def test_gqa_equals_repeated_heads_bitwise(K, V, H, Hkv, dtype):
    """Grouped kv heads give bit for bit the result of plain multi-head input
    whose k and v repeat each kv head H // Hkv times in a row (the grouping
    query head h -> kv head h // (H // Hkv)), through every chunk kernel."""
    for KK in ((K, 512) if dtype == "bf16" else (K,)):
        inp = make_chunk_inputs(small("gqa_rep", B=1, T=0, H=H, Hkv=Hkv, K=KK, V=V, dtype=dtype,
                                      fixed_lengths=(100, 7, 64), initial_state=True, seed=21))
        o1, h1 = run_chunk(inp)
        rep_ = dict(inp)
        rep_["k"] = np.repeat(inp["k"], H // Hkv, axis=2)
        rep_["v"] = np.repeat(inp["v"], H // Hkv, axis=2)
        o2, h2 = run_chunk(rep_)
        assert np.array_equal(o1, o2) and np.array_equal(h1, h2), KK
        check_full(inp, o1, h1)


@pytest.mark.parametrize("gate", ["g", "gamma", "none"])
@pytest.mark.parametrize("Hkv", [6, 2, 1])
def test_decode_gate_kinds_and_kv_groups(gate, Hkv):
    """Decode with a per-token gate, a per-head g_gamma or no decay, and with
    grouped kv heads, against the oracle step."""
    w = DecodeWorkload("var", N=5, H=6, K=128, V=128, steps=3, dtype="bf16", Hkv=Hkv, gate=gate,
                       seed=40 + Hkv)
    inp = make_decode_inputs(w)
    bf = torch.bfloat16
    state = to_dev(inp["state"], torch.float32)
    S_ref = inp["state"].astype(np.float64)
    gg = to_dev(inp["g_gamma"], torch.float32)
    for s in range(inp["steps"]):
        g = None if inp["g"] is None else inp["g"][s]
        o = sgla.recurrent_step(to_dev(inp["q"][s], bf), to_dev(inp["k"][s], bf),
                                to_dev(inp["v"][s], bf), to_dev(g, torch.float32), state,
                                scale=inp["scale"], g_gamma=gg)
        o_ref, S_ref = oracle.step(inp["q"][s], inp["k"][s], inp["v"][s], g, S_ref,
                                   scale=inp["scale"], g_gamma=inp["g_gamma"])
        torch.cuda.synchronize()
        assert err_ratio(o.cpu().numpy(), o_ref) <= TOL_F32
    assert err_ratio(state.cpu().numpy(), S_ref) <= TOL_F32

@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("K,V", [(8, 32), (64, 64), (100, 128), (128, 128), (128, 256),
                                 (64, 512)])
def test_decode_small(dtype, K, V):
    w = DecodeWorkload("small", N=3, H=5, K=K, V=V, steps=3, dtype=dtype, seed=K + V)
    inp = make_decode_inputs(w)
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    state = to_dev(inp["state"], torch.float32)
    S_ref = inp["state"].astype(np.float64)
    for s in range(inp["steps"]):
        o = sgla.recurrent_step(to_dev(inp["q"][s], dt), to_dev(inp["k"][s], dt),
                                to_dev(inp["v"][s], dt), to_dev(inp["g"][s], torch.float32),
                                state, scale=inp["scale"])
        o_ref, S_ref = oracle.step(inp["q"][s], inp["k"][s], inp["v"][s], inp["g"][s], S_ref,
                                   scale=inp["scale"])
        torch.cuda.synchronize()
        assert err_ratio(o.cpu().numpy(), o_ref) <= TOL_F32
    assert err_ratio(state.cpu().numpy(), S_ref) <= TOL_F32


def test_decode_named_workload_full():
    """256 sequences x 32 heads, 64 in-place steps: every step's o over all
    8192 units and the whole state after the last step, against the oracle
    step applied to the whole fp64 state."""
    w = DECODE_CONFIGS["decode_n256_h32_k128"]
    inp = make_decode_inputs(w)
    state = to_dev(inp["state"], torch.float32)
    S_ref = inp["state"].astype(np.float64)
    worst = 0.0
    for s in range(inp["steps"]):
        o = sgla.recurrent_step(to_dev(inp["q"][s], torch.bfloat16),
                                to_dev(inp["k"][s], torch.bfloat16),
                                to_dev(inp["v"][s], torch.bfloat16),
                                to_dev(inp["g"][s], torch.float32), state, scale=inp["scale"])
        o_ref, S_ref = oracle.step(inp["q"][s], inp["k"][s], inp["v"][s], inp["g"][s], S_ref,
                                   scale=inp["scale"])
        worst = max(worst, err_ratio(o.cpu().numpy(), o_ref))
    torch.cuda.synchronize()
    es = err_ratio(state.cpu().numpy(), S_ref)
    print(f"[decode] worst step o err/RMS={worst:.3e} state err/RMS={es:.3e}", flush=True)
    assert worst <= TOL_BF16 and es <= TOL_BF16


# ---------------------------------------------------------------------------
# errors surface as exceptions and leave outputs untouched
# ---------------------------------------------------------------------------

def test_errors_leave_outputs_untouched():
    inp = make_chunk_inputs(small("err", K=64, V=64, T=64))
    d = device_inputs(inp)
    out = torch.full((inp["B"], inp["T"], inp["H"], inp["V"]), 7.0, device=DEV)
    with pytest.raises(ValueError, match="chunk_size"):
        sgla.chunk_fwd(d["q"], d["k"], d["v"], g=d["g"], chunk_size=8, out=out)
    with pytest.raises(ValueError):
        sgla.chunk_fwd(d["q"], d["k"], d["v"], g=d["g"], g_gamma=torch.zeros(3, device=DEV),
                       out=out)
    with pytest.raises(ValueError, match="chunk_size"):
        sgla.chunk_fwd(d["q"], d["k"], d["v"], g=d["g"], chunk_size=48, out=out)
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)
    state = torch.full((2, 2, 64, 64), 3.0, device=DEV)
    with pytest.raises(ValueError):
        sgla.recurrent_step(torch.zeros(2, 2, 64, device=DEV), torch.zeros(2, 2, 64, device=DEV),
                            torch.zeros(2, 2, 48, device=DEV), torch.zeros(2, 2, device=DEV),
                            torch.zeros(2, 2, 64, 48, device=DEV))
    torch.cuda.synchronize()
    assert torch.all(state == 3.0)


# ---------------------------------------------------------------------------
# [V, K] state layout (section 二, state_v_first)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("K,V,dtype", [(64, 128, "bf16"), (128, 64, "bf16"), (256, 64, "bf16"),
                                       (512, 96, "bf16"), (32, 64, "f32")])
def test_state_v_first_forward(K, V, dtype):
    """The forward with [V, K] states gives the same o bit for bit and the
    transposed final state of the [K, V] call, and matches the oracle."""
    inp = make_chunk_inputs(small("vf", B=1, T=0, H=2, K=K, V=V, dtype=dtype,
                                  fixed_lengths=(130, 1, 70), initial_state=True, seed=K + V))
    d = device_inputs(inp)
    h0t = d["initial_state"].transpose(-1, -2).contiguous()
    kw = dict(g=d["g"], scale=inp["scale"], output_final_state=True, cu_seqlens=inp["cu_seqlens"])
    o1, h1 = sgla.chunk_fwd(d["q"], d["k"], d["v"], initial_state=d["initial_state"], **kw)
    o2, h2 = sgla.chunk_fwd(d["q"], d["k"], d["v"], initial_state=h0t, state_v_first=True, **kw)
    torch.cuda.synchronize()
    assert tuple(h2.shape) == (3, 2, V, K)
    assert torch.equal(o1, o2) and torch.equal(h1.transpose(-1, -2), h2)
    o_ref, h_ref = oracle.fwd(inp["q"], inp["k"], inp["v"], g=inp["g"], scale=inp["scale"],
                              initial_state=np.swapaxes(inp["initial_state"], -1, -2),
                              cu_seqlens=inp["cu_seqlens"], state_v_first=True)
    tol = _tol(dtype)
    assert err_ratio(o2.cpu().numpy(), o_ref) <= tol
    assert err_ratio(h2.cpu().numpy(), h_ref) <= tol


def test_state_v_first_backward():
    inp = make_chunk_inputs(small("vfb", B=1, T=0, H=2, K=64, V=96, fixed_lengths=(100, 30),
                                  initial_state=True, seed=3))
    d = device_inputs(inp)
    rng = np.random.default_rng(4)
    do = to_dev(rng.standard_normal((1, inp["T"], 2, 96)).astype(np.float32), torch.bfloat16)
    dht = to_dev(rng.standard_normal((2, 2, 64, 96)).astype(np.float32), torch.float32)
    kw = dict(g=d["g"], scale=inp["scale"], cu_seqlens=inp["cu_seqlens"])
    a = sgla.chunk_bwd(d["q"], d["k"], d["v"], do, initial_state=d["initial_state"], dht=dht, **kw)
    b = sgla.chunk_bwd(d["q"], d["k"], d["v"], do,
                       initial_state=d["initial_state"].transpose(-1, -2).contiguous(),
                       dht=dht.transpose(-1, -2).contiguous(), state_v_first=True, **kw)
    torch.cuda.synchronize()
    for name in ("dq", "dk", "dv", "dg"):
        assert torch.equal(a[name], b[name]), name
    assert torch.equal(a["dh0"].transpose(-1, -2), b["dh0"])


@pytest.mark.parametrize("K,V", [(32, 32), (64, 96), (128, 128), (256, 64), (512, 128), (128, 1024)])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_decode_state_v_first(K, V, dtype):
    """Decode on the [V, K] state (its own kernel: rows are value indices and
    q.S reduces along a row) against the oracle step, with grouped kv heads
    and a per-head g_gamma on some cases."""
    Hkv, gate = (2, "gamma") if K in (64, 512) else (4, "g")
    w = DecodeWorkload("vf", N=3, H=4, K=K, V=V, steps=3, dtype=dtype, Hkv=Hkv, gate=gate, seed=K + V)
    inp = make_decode_inputs(w)
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    S_ref = np.swapaxes(inp["state"], -1, -2).astype(np.float64)
    state = to_dev(np.ascontiguousarray(np.swapaxes(inp["state"], -1, -2)), torch.float32)
    gg = to_dev(inp["g_gamma"], torch.float32)
    for s in range(inp["steps"]):
        g = None if inp["g"] is None else inp["g"][s]
        o = sgla.recurrent_step(to_dev(inp["q"][s], dt), to_dev(inp["k"][s], dt), to_dev(inp["v"][s], dt),
                                to_dev(g, torch.float32), state, scale=inp["scale"], g_gamma=gg,
                                state_v_first=True)
        o_ref, S_ref = oracle.step(inp["q"][s], inp["k"][s], inp["v"][s], g, S_ref, scale=inp["scale"],
                                   g_gamma=inp["g_gamma"], state_v_first=True)
        torch.cuda.synchronize()
        assert err_ratio(o.cpu().numpy(), o_ref) <= TOL_F32
    assert err_ratio(state.cpu().numpy(), S_ref) <= TOL_F32


# ---------------------------------------------------------------------------
# degenerate gates: full forget everywhere, and resets inside sequences
# ---------------------------------------------------------------------------

def _reset_gates(inp, kind):
    g = np.array(inp["g"], dtype=np.float32, copy=True)
    if kind == "forget":
        g[:] = -1e4                      # every token forgets all history
    else:
        g[:, ::37, :] = -1e4             # a reset every 37 tokens, normal gates between
    return g


@pytest.mark.parametrize("kind", ["forget", "resets"])
@pytest.mark.parametrize("cfg", [dict(K=64, V=64), dict(K=128, V=128), dict(K=512, V=64, H=1),
                                 dict(dtype="f32", K=32, V=64)],
                         ids=["k64", "k128", "k512", "f32_k32"])
def test_chunk_degenerate_gates(cfg, kind):
    """Gates of -1e4 (a full reset) at every token or every 37th: the forward
    stays finite and matches the oracle (which gives o_t = scale (q_t . k_t)
    v_t for a reset at every token)."""
    inp = make_chunk_inputs(small(f"deg_{kind}", T=150, initial_state=True, **cfg))
    inp["g"] = _reset_gates(inp, kind)
    o, ht = run_chunk(inp)
    check_full(inp, o, ht)


@pytest.mark.parametrize("kind", ["forget", "resets"])
def test_parallel_and_decode_degenerate_gates(kind):
    """The parallel form and the decode step under the same reset gates."""
    inp = make_chunk_inputs(small(f"degp_{kind}", T=150, K=128, V=64, initial_state=False))
    inp["g"] = _reset_gates(inp, kind)
    d = device_inputs(inp)
    o, A = sgla.parallel_fwd(d["q"], d["k"], d["v"], g=d["g"], scale=inp["scale"], out_dtype=torch.float32)
    torch.cuda.synchronize()
    o_ref, A_ref = oracle.parallel(inp["q"], inp["k"], inp["v"], g=inp["g"], scale=inp["scale"])
    assert np.all(np.isfinite(o.cpu().numpy())) and np.all(np.isfinite(A.cpu().numpy()))
    assert err_ratio(o.cpu().numpy(), o_ref) <= TOL_BF16
    assert err_ratio(A.cpu().numpy(), A_ref) <= TOL_BF16
    # decode: the first 8 tokens of every row as 8 steps from a random state
    N, H, K, V = inp["B"], inp["H"], inp["K"], inp["V"]   # one decode step per batch row
    rng = np.random.default_rng(3)
    S0 = (rng.standard_normal((N, H, K, V)) * 0.1).astype(np.float32)
    S = to_dev(S0, torch.float32)
    Sref = S0.astype(np.float64)
    for t in range(8):
        qt, kt, vt = inp["q"][:, t], inp["k"][:, t], inp["v"][:, t]
        gt = inp["g"][:, t]
        ot = sgla.recurrent_step(to_dev(qt, torch.bfloat16), to_dev(kt, torch.bfloat16),
                                 to_dev(vt, torch.bfloat16), to_dev(gt, torch.float32), S,
                                 scale=inp["scale"])
        o_ref_t, Sref = oracle.step(qt, kt, vt, gt, Sref, scale=inp["scale"])
        torch.cuda.synchronize()
        assert np.all(np.isfinite(ot.cpu().numpy()))
        assert err_ratio(ot.cpu().numpy(), o_ref_t) <= TOL_BF16
    assert err_ratio(S.cpu().numpy(), Sref) <= TOL_BF16


# ---------------------------------------------------------------------------
# odd shapes: many heads, many short rows, many tiny packed sequences
# ---------------------------------------------------------------------------

ODD_SHAPES = [
    small("h64_k64", B=1, T=70, H=64, K=64, V=64),
    small("b48_t3", B=48, T=3, H=2, K=128, V=64, initial_state=True),
    small("n200_tiny_varlen", B=1, T=0, H=2, K=64, V=64, initial_state=True,
          fixed_lengths=tuple(int(x) for x in np.random.default_rng(0).integers(0, 6, size=200))),
    small("f32_b40_t2", dtype="f32", B=40, T=2, H=3, K=32, V=32, initial_state=True),
    small("k512_b6_t5", B=6, T=5, H=1, K=512, V=64, initial_state=True),
]


@pytest.mark.parametrize("w", ODD_SHAPES, ids=lambda w: w.name)
def test_chunk_odd_shapes(w):
    inp = make_chunk_inputs(w)
    o, ht = run_chunk(inp)
    check_full(inp, o, ht)


@pytest.mark.parametrize("B,T,H,K,V", [(1, 70, 64, 64, 64), (48, 3, 2, 128, 64), (5, 1, 3, 64, 16)],
                         ids=["h64", "b48_t3", "b5_t1"])
def test_parallel_odd_shapes(B, T, H, K, V):
    inp = make_chunk_inputs(small("par_odd", B=B, T=T, H=H, K=K, V=V))
    d = device_inputs(inp)
    o, A = sgla.parallel_fwd(d["q"], d["k"], d["v"], g=d["g"], scale=inp["scale"], out_dtype=torch.float32)
    torch.cuda.synchronize()
    o_ref, A_ref = oracle.parallel(inp["q"], inp["k"], inp["v"], g=inp["g"], scale=inp["scale"])
    assert err_ratio(o.cpu().numpy(), o_ref) <= TOL_BF16
    assert err_ratio(A.cpu().numpy(), A_ref) <= TOL_BF16


@pytest.mark.parametrize("N,H,Hkv,K,V,vf", [(1, 1, 1, 1, 32, 0), (3000, 1, 1, 16, 32, 0), (7, 5, 5, 96, 64, 0),
                                            (2, 3, 1, 512, 512, 1), (9, 2, 2, 32, 1024, 1)],
                         ids=["k1", "n3000", "k96", "vf_k512_mqa", "vf_v1024"])
def test_decode_odd_shapes(N, H, Hkv, K, V, vf):
    """Decode at the edges of its support: K = 1, thousands of tiny units, a
    non-power-of-two K, and the [V, K] state at its largest K and V."""
    rng = np.random.default_rng(N + K)
    q = rng.standard_normal((N, H, K)).astype(np.float32)
    k = rng.standard_normal((N, Hkv, K)).astype(np.float32)
    v = rng.standard_normal((N, Hkv, V)).astype(np.float32)
    g = np.log(rng.uniform(0.5, 1.0, (N, H))).astype(np.float32)
    S0 = (rng.standard_normal((N, H, K, V)) * 0.1).astype(np.float32)
    S = to_dev(np.swapaxes(S0, -1, -2).copy() if vf else S0, torch.float32)
    o = sgla.recurrent_step(to_dev(q, torch.float32), to_dev(k, torch.float32), to_dev(v, torch.float32),
                            to_dev(g, torch.float32), S, scale=0.3, state_v_first=bool(vf))
    torch.cuda.synchronize()
    o_ref, S_ref = oracle.step(q, k, v, g, S0, scale=0.3)
    S_got = S.cpu().numpy()
    if vf:
        S_got = np.swapaxes(S_got, -1, -2)
    assert err_ratio(o.cpu().numpy(), o_ref) <= TOL_F32
    assert err_ratio(S_got, S_ref) <= TOL_F32


# ---------------------------------------------------------------------------
# chunk sizes 16 and 32 (section 二: any power of two; section 五 runs 16,
# 32 and 64 on packed sequences [0, 15, 100, 300, 1200, 2000])
# ---------------------------------------------------------------------------

FLA_LENGTHS = (15, 85, 200, 900, 800)   # cu_seqlens [0, 15, 100, 300, 1200, 2000]

CHUNK_SIZE_CASES = [
    small("cs_bf16_k64", K=64, V=64, T=200),
    small("cs_bf16_k128_varlen", B=1, T=0, H=2, K=128, V=128, fixed_lengths=FLA_LENGTHS,
          initial_state=True),
    small("cs_bf16_k256_gamma", K=256, V=64, T=150, gate="gamma", normalize_k=True, H=2),
    small("cs_bf16_k512_varlen", B=1, T=0, H=1, K=512, V=96, fixed_lengths=(70, 1, 0, 130),
          initial_state=True),
    small("cs_bf16_no_gate", K=64, V=128, T=97, gate="none"),
    small("cs_gqa_k128", H=4, Hkv=2, K=128, V=64, T=150, initial_state=True),
    small("cs_f32_k16", dtype="f32", K=16, V=32, T=150),
    small("cs_f32_k32_varlen", dtype="f32", B=1, T=0, K=32, V=64, fixed_lengths=FLA_LENGTHS,
          initial_state=True),
    small("cs_f32_k128_gamma", dtype="f32", K=128, V=64, T=130, gate="gamma"),
]


@pytest.mark.parametrize("chunk", [16, 32, 64])
@pytest.mark.parametrize("w", CHUNK_SIZE_CASES, ids=lambda w: w.name)
def test_chunk_sizes(w, chunk):
    inp = make_chunk_inputs(w)
    inp["chunk_size"] = chunk
    o, ht = run_chunk(inp, output_final_state=True)
    check_full(inp, o, ht)


@pytest.mark.parametrize("chunk", [16, 32])
def test_chunk_sizes_named_tiny_f32(chunk):
    inp = make_chunk_inputs(CHUNK_CONFIGS["tiny_f32"])
    inp["chunk_size"] = chunk
    o, ht = run_chunk(inp)
    check_full(inp, o, ht)


@pytest.mark.parametrize("chunk", [16, 32])
@pytest.mark.parametrize("kind", ["forget", "resets"])
def test_chunk_sizes_degenerate_gates(chunk, kind):
    for dtype, K in (("bf16", 128), ("f32", 64)):
        inp = make_chunk_inputs(small(f"csdeg_{kind}", dtype=dtype, K=K, V=64, T=150, initial_state=True))
        inp["g"] = _reset_gates(inp, kind)
        inp["chunk_size"] = chunk
        o, ht = run_chunk(inp)
        check_full(inp, o, ht)


@pytest.mark.parametrize("chunk", [16, 32])
def test_chunk_sizes_state_v_first_and_bf16_out(chunk):
    """[V, K] states give the transposed final state and the same o bit for
    bit; a bf16 o is the float32 result rounded once."""
    inp = make_chunk_inputs(small("cs_vf", B=1, T=0, H=2, K=128, V=64, fixed_lengths=(130, 1, 70),
                                  initial_state=True, seed=5))
    d = device_inputs(inp)
    kw = dict(g=d["g"], scale=inp["scale"], output_final_state=True, cu_seqlens=inp["cu_seqlens"],
              chunk_size=chunk)
    o1, h1 = sgla.chunk_fwd(d["q"], d["k"], d["v"], initial_state=d["initial_state"], **kw)
    o2, h2 = sgla.chunk_fwd(d["q"], d["k"], d["v"],
                            initial_state=d["initial_state"].transpose(-1, -2).contiguous(),
                            state_v_first=True, **kw)
    o3, _ = sgla.chunk_fwd(d["q"], d["k"], d["v"], initial_state=d["initial_state"],
                           o_dtype=torch.bfloat16, **kw)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(h1.transpose(-1, -2), h2)
    o1f, o3f = o1.cpu().numpy().astype(np.float64), o3.float().cpu().numpy().astype(np.float64)
    assert np.all(np.abs(o3f - o1f) <= 2.0 ** -8 * np.abs(o1f) + 1e-30)
    check_full(inp, o1.cpu().numpy(), h1.cpu().numpy())


def test_chunk_sizes_agree():
    """The chunk size changes only the rounding: 16, 32 and 64 agree within
    the fp32 bar on float32 input."""
    inp = make_chunk_inputs(small("cs_agree", dtype="f32", B=1, T=0, H=2, K=64, V=64,
                                  fixed_lengths=FLA_LENGTHS, initial_state=True))
    outs = {}
    for chunk in (16, 32, 64):
        inp["chunk_size"] = chunk
        outs[chunk] = run_chunk(inp, output_final_state=True)
    for chunk in (16, 32):
        assert err_ratio(outs[chunk][0], outs[64][0]) <= TOL_F32
        assert err_ratio(outs[chunk][1], outs[64][1]) <= TOL_F32


def test_back_to_back_varlen_calls():
    """Several packed calls with different cu_seqlens enqueued on one stream
    without a synchronization between them; each host cu_seqlens array is
    overwritten as soon as its call returns (the tables travel in kernel
    arguments, so nothing reads the host array later).  Every call matches
    the oracle."""
    import ctypes
    cases = [(15, 85, 200, 900, 800), (64, 1, 0, 300), (1000, 7), (5,) * 40]
    runs = []
    for i, lens in enumerate(cases):
        inp = make_chunk_inputs(small(f"b2b{i}", B=1, T=0, H=2, K=128, V=64, fixed_lengths=lens,
                                      initial_state=True, seed=50 + i))
        d = device_inputs(inp)
        cu = np.array(inp["cu_seqlens"], dtype=np.int64, copy=True)   # the call's own host array
        N, T = len(cu) - 1, int(cu[-1])
        args = sgla._chunk_args(1, T, 2, 128, 64, N, 64, 1, 2, inp["scale"], 1)
        cu_ptr = ctypes.c_void_p(cu.ctypes.data)
        ws_n = sgla._workspace_size(args, cu_ptr)
        ws = torch.empty(max(ws_n, 1), device=DEV, dtype=torch.uint8)
        o = torch.empty((1, T, 2, 64), device=DEV, dtype=torch.float32)
        ht = torch.empty((N, 2, 128, 64), device=DEV, dtype=torch.float32)
        st = sgla.lib.sgla_chunk_fwd(ctypes.byref(args), sgla._ptr(d["q"]), sgla._ptr(d["k"]),
                                     sgla._ptr(d["v"]), sgla._ptr(d["g"]), None,
                                     sgla._ptr(d["initial_state"]), cu_ptr, sgla._ptr(o), sgla._ptr(ht),
                                     sgla._ptr(ws), ws_n, sgla._stream(DEV))
        assert st == 0, sgla.lib.sgla_last_error()
        cu[:] = 0x7fffffff          # the call has returned: its host array is free again
        runs.append((inp, o, ht, d, ws))
    torch.cuda.synchronize()
    for inp, o, ht, _, _ in runs:
        check_full(inp, o.cpu().numpy(), ht.cpu().numpy())


# ---------------------------------------------------------------------------
# segmented chains: long sequences with little other work are cut into
# segments that run in parallel from entering states computed by a
# state-only pass and a scan (bf16, K <= 128)
# ---------------------------------------------------------------------------

SEGMENT_CASES = [
    small("seg_dense_g", B=1, T=3000, H=2, K=128, V=64),
    small("seg_dense_h0_gamma", B=2, T=2500, H=1, K=128, V=128, gate="gamma", normalize_k=True,
          initial_state=True),
    small("seg_k64_no_gate", B=1, T=2100, H=1, K=64, V=64, gate="none", initial_state=True),
    small("seg_packed", B=1, T=0, H=2, K=128, V=64, fixed_lengths=(15, 2100, 1, 1500, 0, 64),
          initial_state=True),
    small("seg_gqa", B=1, T=2200, H=4, Hkv=2, K=128, V=64, initial_state=True),
    small("seg_strong_gate", B=1, T=2048, H=1, K=64, V=128, gate_normalizer=0.1, scale=0.1),
]


@pytest.mark.parametrize("w", SEGMENT_CASES, ids=lambda w: w.name)
def test_segmented_chains(w):
    inp = make_chunk_inputs(w)
    o, ht = run_chunk(inp, output_final_state=True)
    check_full(inp, o, ht)
    o2, ht2 = run_chunk(inp, output_final_state=True)
    assert np.array_equal(o, o2) and np.array_equal(ht, ht2)   # deterministic


@pytest.mark.parametrize("kind", ["forget", "resets"])
def test_segmented_degenerate_gates(kind):
    inp = make_chunk_inputs(small(f"segdeg_{kind}", B=1, T=2500, H=1, K=128, V=64, initial_state=True))
    inp["g"] = _reset_gates(inp, kind)
    o, ht = run_chunk(inp, output_final_state=True)
    check_full(inp, o, ht)


def test_segmented_state_v_first():
    inp = make_chunk_inputs(small("seg_vf", B=1, T=2300, H=2, K=128, V=64, initial_state=True, seed=8))
    d = device_inputs(inp)
    kw = dict(g=d["g"], scale=inp["scale"], output_final_state=True)
    o1, h1 = sgla.chunk_fwd(d["q"], d["k"], d["v"], initial_state=d["initial_state"], **kw)
    o2, h2 = sgla.chunk_fwd(d["q"], d["k"], d["v"],
                            initial_state=d["initial_state"].transpose(-1, -2).contiguous(),
                            state_v_first=True, **kw)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(h1.transpose(-1, -2), h2)
    check_full(inp, o1.cpu().numpy(), h1.cpu().numpy())
