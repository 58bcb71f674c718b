"""GPU parity of the backward (sgla_chunk_bwd) against the fp64 oracle backward.

Gradients of L = <do, o> + <dht, final_state> with respect to q, k, v, the
gates (dg per token, or dg_gamma per head) and the initial state (page
"flash-linear-attention 中的 Simple GLA", section 五: dq, dk, dv, dg and dh0
are the gradients its tests compare).  The bar, per gradient tensor, is the
forward's: max |gpu - oracle| / RMS(oracle) <= 2e-2 for bf16 inputs and 1e-4
for float32 inputs.  Every case compares every element of every gradient,
the full-size packed workload included.
"""
import numpy as np
import pytest
import torch

import oracle
from gla_workloads import CHUNK_CONFIGS, ChunkWorkload, make_backward_inputs, make_chunk_inputs
from gpu_common import DEV, TOL_BF16, TOL_F32, device_inputs, err_ratio, to_dev

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

if torch.cuda.is_available():
    import gated_linear_attention_amd as sgla
else:  # pragma: no cover - collected on CPU-only hosts, never run
    sgla = None

GRADS = ("dq", "dk", "dv", "dg", "dg_gamma", "dh0")


def small(name, **kw):
    base = dict(B=2, T=150, H=2, K=64, V=64, dtype="bf16", gate="g", seed=31)
    base.update(kw)
    return ChunkWorkload(name, **base)


def run_bwd(inp, bi):
    d = device_inputs(inp)
    dt = d["q"].dtype
    out = sgla.chunk_bwd(d["q"], d["k"], d["v"], to_dev(bi["do"], dt), g=d["g"],
                         g_gamma=d["g_gamma"], scale=inp["scale"], initial_state=d["initial_state"],
                         dht=to_dev(bi["dht"], torch.float32), cu_seqlens=inp["cu_seqlens"],
                         chunk_size=inp["chunk_size"])
    torch.cuda.synchronize()
    return {k: (None if v is None else v.cpu().numpy()) for k, v in out.items()}


def oracle_bwd(inp, bi, **kw):
    return oracle.bwd(inp["q"], inp["k"], inp["v"], bi["do"], g=inp["g"], g_gamma=inp["g_gamma"],
                      scale=inp["scale"], initial_state=inp["initial_state"], dht=bi["dht"],
                      cu_seqlens=inp["cu_seqlens"], **kw)


def compare(got, ref, tol, label=""):
    errs = {}
    for name in GRADS:
        if ref[name] is None:
            assert got[name] is None, name
            continue
        assert np.all(np.isfinite(got[name])), name
        errs[name] = err_ratio(got[name], ref[name])
    print(f"[bwd {label}] " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
    bad = {k: v for k, v in errs.items() if v > tol}
    assert not bad, f"max err / RMS above {tol}: {bad}"


SMALL = [
    small("k64_v64_g"),
    small("k128_v128_h0", K=128, V=128, T=131, initial_state=True),
    small("k16_v32", K=16, V=32, T=97),
    small("k32_v96_gamma", K=32, V=96, T=200, gate="gamma", normalize_k=True),
    small("k128_v64_gamma_h0", K=128, V=64, T=70, gate="gamma", initial_state=True, H=3),
    small("k64_no_gate", K=64, V=64, T=129, gate="none"),
    small("strong_gate", K=64, V=32, T=150, gate_normalizer=0.1, scale=0.1),
    small("t1", T=1, initial_state=True),
    small("t64", T=64),
    small("t65", T=65, initial_state=True),
    small("empty_T0", T=0, initial_state=True),
    small("varlen", B=1, T=0, H=2, K=64, V=64, fixed_lengths=(15, 85, 0, 1, 200, 64),
          initial_state=True),
    small("varlen_k128_gamma", B=1, T=0, H=2, K=128, V=128, fixed_lengths=(70, 130, 5),
          gate="gamma", initial_state=True),
    # bf16 with K in {64, 128} runs the bf16-matrix-core passes: V walked in
    # three 32-column slices, and in one
    small("k64_v96_h0", K=64, V=96, T=100, initial_state=True),
    small("k128_v32_gamma", K=128, V=32, T=90, gate="gamma"),
    small("f32_k32_v64", dtype="f32", K=32, V=64, T=150, initial_state=True),
    small("f32_k128_varlen", dtype="f32", B=1, T=0, K=128, V=32, fixed_lengths=(15, 85, 200),
          initial_state=True),
    # grouped kv heads: dk, dv per kv head, summed over the query heads that read it
    small("gqa_k64_v64", H=4, Hkv=2, K=64, V=64, T=130, initial_state=True),
    small("gqa_k128_gamma_varlen", B=1, T=0, H=6, Hkv=2, K=128, V=128, fixed_lengths=(70, 0, 150),
          gate="gamma", initial_state=True),
    small("gqa_mqa_k64_v96", H=3, Hkv=1, K=64, V=96, T=100),
    small("gqa_f32_k32", dtype="f32", H=4, Hkv=2, K=32, V=64, T=97, initial_state=True),
    small("gqa_bf16_k16", H=4, Hkv=1, K=16, V=32, T=70),
    # K in {256, 512}: key tiles of 128 for dq and dk, dv over 64-key slices,
    # the gate gradient from the key-tile records
    small("k256_v64_h0", K=256, V=64, T=150, initial_state=True),
    small("k512_v128_gamma_h0", K=512, V=128, T=131, gate="gamma", initial_state=True),
    small("k256_no_gate", K=256, V=64, T=70, gate="none"),
    small("k512_varlen", B=1, T=0, H=2, K=512, V=64, fixed_lengths=(15, 85, 0, 1, 200),
          initial_state=True),
    small("gqa_k256_v128", H=4, Hkv=2, K=256, V=128, T=100, initial_state=True),
]


@pytest.mark.parametrize("w", SMALL, ids=lambda w: w.name)
@pytest.mark.parametrize("with_dht", [True, False], ids=["dht", "no_dht"])
def test_bwd_small(w, with_dht):
    inp = make_chunk_inputs(w)
    bi = make_backward_inputs(inp, seed=w.seed + 1, final_state_grad=with_dht)
    got = run_bwd(inp, bi)
    ref = oracle_bwd(inp, bi)
    compare(got, ref, TOL_BF16 if inp["dtype"] == "bf16" else TOL_F32, w.name)


def test_bwd_deterministic():
    inp = make_chunk_inputs(small("det", B=1, T=0, K=128, V=128, fixed_lengths=(300, 77),
                                  gate="gamma", initial_state=True))
    bi = make_backward_inputs(inp, seed=5)
    a, b = run_bwd(inp, bi), run_bwd(inp, bi)
    for name in GRADS:
        if a[name] is not None:
            assert np.array_equal(a[name], b[name]), name


def test_bwd_named_workload_full():
    """The packed workload (8 sequences of 64..4096 tokens, 16 heads, K = V =
    128, bf16, g, h0) in the full launch, every gradient compared with the
    oracle backward over the whole tensor."""
    w = CHUNK_CONFIGS["varlen_bf16_k128"]
    inp = make_chunk_inputs(w)
    bi = make_backward_inputs(inp, seed=w.seed + 100)
    got = run_bwd(inp, bi)
    compare(got, oracle_bwd(inp, bi), TOL_BF16, "varlen_bf16_k128 whole-tensor")


def test_bwd_dense_k512_full():
    """The dense wide-key workload (B=4, T=2048, H=4, K = V = 512, bf16, g)
    with a final-state gradient, every gradient compared with the oracle
    backward over the whole tensor.  The oracle keeps every state of a
    (sequence, head) in fp64 (2 MiB per token at K = V = 512), so it runs on
    8 threads here to bound host memory."""
    w = CHUNK_CONFIGS["dense_bf16_k512"]
    inp = make_chunk_inputs(w)
    bi = make_backward_inputs(inp, seed=w.seed + 100)
    got = run_bwd(inp, bi)
    compare(got, oracle_bwd(inp, bi, nthreads=8), TOL_BF16, "dense_bf16_k512 whole-tensor")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_bwd_grouped_equals_repeated_heads(dtype):
    """With grouped kv heads every query head's gradients are those of the
    same run on k and v repeated per query head, and dk, dv of a kv head are
    the sums over its query heads in head order: bit for bit."""
    K = 64 if dtype == "bf16" else 32
    inp = make_chunk_inputs(small("grp", B=1, T=0, H=4, Hkv=2, K=K, V=64, fixed_lengths=(100, 37),
                                  dtype=dtype, initial_state=True))
    bi = make_backward_inputs(inp, seed=5)
    got = run_bwd(inp, bi)
    rep = dict(inp)
    rep["k"] = np.repeat(inp["k"], 2, axis=2)
    rep["v"] = np.repeat(inp["v"], 2, axis=2)
    full = run_bwd(rep, bi)
    for name in ("dq", "dg", "dh0"):
        assert np.array_equal(got[name], full[name]), name
    for name, D in (("dk", K), ("dv", 64)):
        pairs = full[name].reshape(1, -1, 2, 2, D)
        assert np.array_equal(got[name], pairs[:, :, :, 0] + pairs[:, :, :, 1]), name


@pytest.mark.parametrize("kind", ["forget", "resets"])
@pytest.mark.parametrize("dtype,K", [("bf16", 64), ("bf16", 128), ("bf16", 256), ("f32", 32)],
                         ids=["k64", "k128", "k256", "f32_k32"])
def test_bwd_degenerate_gates(dtype, K, kind):
    """Gates of -1e4 (a full reset) at every token or every 37th token: every
    gradient stays finite and within the bar."""
    inp = make_chunk_inputs(small(f"bdeg_{kind}", dtype=dtype, K=K, V=64, T=150, initial_state=True))
    g = np.array(inp["g"], dtype=np.float32, copy=True)
    if kind == "forget":
        g[:] = -1e4
    else:
        g[:, ::37, :] = -1e4
    inp["g"] = g
    bi = make_backward_inputs(inp, seed=9)
    compare(run_bwd(inp, bi), oracle_bwd(inp, bi), TOL_BF16 if dtype == "bf16" else TOL_F32, f"deg {kind}")


@pytest.mark.parametrize("w", [
    small("b_h32_k64", B=1, T=70, H=32, K=64, V=64),
    small("b_b24_t3", B=24, T=3, H=2, K=128, V=64, initial_state=True),
    small("b_n120_tiny_varlen", B=1, T=0, H=2, K=64, V=32, initial_state=True,
          fixed_lengths=tuple(int(x) for x in np.random.default_rng(1).integers(0, 6, size=120))),
    small("b_f32_b20_t2", dtype="f32", B=20, T=2, H=2, K=32, V=32, initial_state=True),
], ids=lambda w: w.name)
def test_bwd_odd_shapes(w):
    inp = make_chunk_inputs(w)
    bi = make_backward_inputs(inp, seed=12)
    compare(run_bwd(inp, bi), oracle_bwd(inp, bi), TOL_BF16 if inp["dtype"] == "bf16" else TOL_F32, w.name)


# chunk sizes 16 and 32 (section 二: chunk_size is a power of two; section 五
# runs the chunk kernels, gradients included, at 16, 32 and 64 with
# cu_seqlens [0, 15, 100, 300, 1200, 2000])
PAGES_LENGTHS = (15, 85, 200, 900, 800)
CHUNK_CASES = [
    small("cs_k64_varlen_pages", B=1, T=0, K=64, V=64, fixed_lengths=PAGES_LENGTHS, initial_state=True),
    small("cs_k128_gamma", K=128, V=128, T=150, gate="gamma", initial_state=True),
    small("cs_k16_v32", K=16, V=32, T=97),
    small("cs_k256_h0", K=256, V=64, T=150, initial_state=True),
    small("cs_k512_varlen", B=1, T=0, H=1, K=512, V=64, fixed_lengths=(15, 85, 0, 1, 200),
          initial_state=True),
    small("cs_f32_k32_varlen_pages", dtype="f32", B=1, T=0, K=32, V=64, fixed_lengths=PAGES_LENGTHS,
          initial_state=True),
    small("cs_gqa_k64", H=4, Hkv=2, K=64, V=64, T=130, initial_state=True),
]


@pytest.mark.parametrize("chunk", [16, 32])
@pytest.mark.parametrize("w", CHUNK_CASES, ids=lambda w: w.name)
def test_bwd_chunk_sizes(w, chunk):
    """The backward on the chunk grid of the requested size (the state
    records, the gate restarts and the per-chunk gradients all follow
    chunks of 16 or 32 tokens) against the oracle backward."""
    inp = make_chunk_inputs(w)
    inp["chunk_size"] = chunk
    bi = make_backward_inputs(inp, seed=w.seed + 1)
    got = run_bwd(inp, bi)
    ref = oracle_bwd(inp, bi)
    compare(got, ref, TOL_BF16 if inp["dtype"] == "bf16" else TOL_F32, f"{w.name} chunk {chunk}")


@pytest.mark.parametrize("dtype,K", [("bf16", 128), ("f32", 64)])
def test_bwd_chunk_sizes_agree(dtype, K):
    """The three chunk sizes give the same gradients (three different chunk
    grids, one function): within the bar of each other."""
    inp = make_chunk_inputs(small("cs_agree", dtype=dtype, B=1, T=0, K=K, V=64, fixed_lengths=(70, 300, 33),
                                  initial_state=True))
    bi = make_backward_inputs(inp, seed=9)
    outs = {}
    for chunk in (16, 32, 64):
        inp["chunk_size"] = chunk
        outs[chunk] = run_bwd(inp, bi)
    tol = TOL_BF16 if dtype == "bf16" else TOL_F32
    for chunk in (16, 32):
        for name in GRADS:
            if outs[64][name] is not None:
                assert err_ratio(outs[chunk][name], outs[64][name]) <= tol, (chunk, name)


# chunk sizes 16 and 32 at the edges: single tokens, exact multiples of the
# chunk, one token past one, empty packed sequences, the [V, K] state layout
CHUNK_EDGE_CASES = [
    small("cse_t1", T=1, initial_state=True),
    small("cse_t16", T=16, initial_state=True),
    small("cse_t17_gamma", T=17, gate="gamma"),
    small("cse_t33_k512", B=1, T=33, H=1, K=512, V=64, initial_state=True),
    small("cse_tiny_varlen", B=1, T=0, K=128, V=64, fixed_lengths=(0, 1, 16, 17, 0, 32, 33, 2),
          initial_state=True),
    small("cse_f32_t48", dtype="f32", K=16, V=32, T=48, initial_state=True),
]


@pytest.mark.parametrize("chunk", [16, 32])
@pytest.mark.parametrize("w", CHUNK_EDGE_CASES, ids=lambda w: w.name)
def test_bwd_chunk_sizes_edges(w, chunk):
    inp = make_chunk_inputs(w)
    inp["chunk_size"] = chunk
    bi = make_backward_inputs(inp, seed=w.seed + 2)
    got = run_bwd(inp, bi)
    ref = oracle_bwd(inp, bi)
    compare(got, ref, TOL_BF16 if inp["dtype"] == "bf16" else TOL_F32, f"{w.name} chunk {chunk}")


@pytest.mark.parametrize("chunk", [16, 32])
def test_bwd_chunk_sizes_state_v_first(chunk):
    """The [V, K] state layout at the small chunk sizes: the same gradients
    bit for bit, dh0 transposed."""
    inp = make_chunk_inputs(small("cs_vf", B=1, T=0, H=2, K=64, V=96, fixed_lengths=(100, 30),
                                  initial_state=True, seed=3))
    d = device_inputs(inp)
    rng = np.random.default_rng(4)
    do = to_dev(rng.standard_normal((1, inp["T"], 2, 96)).astype(np.float32), torch.bfloat16)
    dht = to_dev(rng.standard_normal((2, 2, 64, 96)).astype(np.float32), torch.float32)
    kw = dict(g=d["g"], scale=inp["scale"], cu_seqlens=inp["cu_seqlens"], chunk_size=chunk)
    a = sgla.chunk_bwd(d["q"], d["k"], d["v"], do, initial_state=d["initial_state"], dht=dht, **kw)
    b = sgla.chunk_bwd(d["q"], d["k"], d["v"], do,
                       initial_state=d["initial_state"].transpose(-1, -2).contiguous(),
                       dht=dht.transpose(-1, -2).contiguous(), state_v_first=True, **kw)
    torch.cuda.synchronize()
    for name in ("dq", "dk", "dv", "dg"):
        assert torch.equal(a[name], b[name]), name
    assert torch.equal(a["dh0"].transpose(-1, -2), b["dh0"])
