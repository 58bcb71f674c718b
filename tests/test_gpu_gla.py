"""GPU parity of elementwise-gate GLA (sgla_gla_chunk_fwd) against the fp64
oracle: per-key log gates gk [B, T, H, K], S_t = diag(exp(gk_t)) S_{t-1} +
k_t v_t^T, o_t = scale S_t^T q_t (the general gate Simple GLA specialises,
page "flash-linear-attention 中的 Simple GLA", section 一).  The bar per
output tensor: max |gpu - oracle| / RMS(oracle) <= 2e-2 for bf16 inputs and
1e-4 for float32 inputs."""
import numpy as np
import pytest
import torch

import oracle
from gla_workloads import CHUNK_CONFIGS, ChunkWorkload, make_chunk_inputs, make_key_gates
from gpu_common import TOL_BF16, TOL_F32, device_inputs, err_ratio, to_dev

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

if torch.cuda.is_available():
    import gated_linear_attention_amd as sgla
else:  # pragma: no cover - collected on CPU-only hosts, never run
    sgla = None


def small(name, **kw):
    base = dict(B=2, T=150, H=2, K=64, V=64, dtype="bf16", gate="none", seed=61)
    base.update(kw)
    return ChunkWorkload(name, **base)


CASES = [
    (small("k64_v64"), 1.0),
    (small("k128_v96_h0", K=128, V=96, T=131, initial_state=True), 1.0),
    (small("k16_v32", K=16, V=32, T=97), 1.0),
    (small("k32_v64_strong", K=32, V=64, T=200), 0.1),
    (small("k128_weak", K=128, V=32, T=70), 10.0),
    (small("t1", T=1, initial_state=True), 1.0),
    (small("t65", T=65), 1.0),
    (small("empty", T=0, initial_state=True), 1.0),
    (small("varlen", B=1, T=0, K=64, V=64, fixed_lengths=(15, 0, 1, 85, 200), initial_state=True), 1.0),
    (small("gqa", H=4, Hkv=2, K=64, V=32, T=130, initial_state=True), 1.0),
    # bf16 inputs with K in {64, 128} and V a multiple of 64 take the bf16
    # chain; the cases above with V = 32 or 96, or K < 64, the fp32 chain
    (small("k128_v128_strong", K=128, V=128, T=150, initial_state=True), 0.1),
    (small("k64_v128_weak", K=64, V=128, T=100, initial_state=True), 10.0),
    (small("gqa_v64", H=4, Hkv=2, K=64, V=64, T=130, initial_state=True), 1.0),
    (small("varlen_k128_v64", B=1, T=0, K=128, V=64, fixed_lengths=(64, 1, 0, 129), initial_state=True), 1.0),
    (small("f32_k32", dtype="f32", K=32, V=64, T=150, initial_state=True), 1.0),
    (small("f32_k128_strong", dtype="f32", K=128, V=32, T=100), 0.1),
]


def run(inp, gk, o_dtype=torch.float32, state_v_first=False):
    d = device_inputs(inp)
    h0 = d["initial_state"]
    if state_v_first and h0 is not None:
        h0 = h0.transpose(-1, -2).contiguous()
    o, ht = sgla.gla_chunk_fwd(d["q"], d["k"], d["v"], to_dev(gk, torch.float32), scale=inp["scale"],
                               initial_state=h0, output_final_state=True, cu_seqlens=inp["cu_seqlens"],
                               chunk_size=inp["chunk_size"], o_dtype=o_dtype, state_v_first=state_v_first)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), ht.cpu().numpy()


@pytest.mark.parametrize("w,norm", CASES, ids=lambda x: x.name if hasattr(x, "name") else str(x))
def test_gla_small(w, norm):
    inp = make_chunk_inputs(w)
    gk = make_key_gates(inp, seed=w.seed + 3, normalizer=norm)
    o, ht = run(inp, gk)
    o_ref, h_ref = oracle.gla_fwd(inp["q"], inp["k"], inp["v"], gk, scale=inp["scale"],
                                  initial_state=inp["initial_state"], cu_seqlens=inp["cu_seqlens"])
    tol = TOL_BF16 if inp["dtype"] == "bf16" else TOL_F32
    eo, eh = err_ratio(o, o_ref), err_ratio(ht, h_ref)
    print(f"[gla {w.name}] o {eo:.2e} final {eh:.2e}", flush=True)
    assert np.all(np.isfinite(o)) and eo <= tol and eh <= tol


def test_gla_scalar_gate_matches_simple_gla():
    """Every key given the head's gate: the GLA kernel agrees with the Simple
    GLA kernel (different paths) within the bf16 bar."""
    inp = make_chunk_inputs(small("scal", B=1, T=0, K=128, V=128, gate="g",
                                  fixed_lengths=(300, 77), initial_state=True))
    gk = np.repeat(inp["g"][..., None], inp["K"], axis=-1)
    o1, h1 = run(inp, gk)
    d = device_inputs(inp)
    o2, h2 = sgla.chunk_fwd(d["q"], d["k"], d["v"], g=d["g"], scale=inp["scale"],
                            initial_state=d["initial_state"], output_final_state=True,
                            cu_seqlens=inp["cu_seqlens"])
    torch.cuda.synchronize()
    assert err_ratio(o1, o2.cpu().numpy()) <= TOL_BF16
    assert err_ratio(h1, h2.cpu().numpy()) <= TOL_BF16


@pytest.mark.parametrize("V", [96, 128], ids=["fp32_chain", "bf16_chain"])
def test_gla_state_v_first_and_bf16_output(V):
    inp = make_chunk_inputs(small("vf", K=64, V=V, T=140, initial_state=True))
    gk = make_key_gates(inp, seed=5)
    o1, h1 = run(inp, gk)
    o2, h2 = run(inp, gk, state_v_first=True)
    assert np.array_equal(o1, o2) and np.array_equal(np.swapaxes(h1, -1, -2), h2)
    # a bf16 o is the fp32 one rounded once: within half a bf16 ulp per element
    o3, _ = run(inp, gk, o_dtype=torch.bfloat16)
    assert np.all(np.abs(o3 - o1) <= 2.0 ** -8 * np.abs(o1))


def test_gla_named_workload_full():
    """The packed K = V = 128 workload (8 sequences of 64..4096 tokens, 16
    heads, h0) with per-key gates, in one launch, compared with the oracle
    over the whole o and final_state tensors."""
    inp = make_chunk_inputs(CHUNK_CONFIGS["varlen_bf16_k128"])
    gk = make_key_gates(inp, seed=77)
    o, ht = run(inp, gk)
    o_ref, h_ref = oracle.gla_fwd(inp["q"], inp["k"], inp["v"], gk, scale=inp["scale"],
                                  initial_state=inp["initial_state"], cu_seqlens=inp["cu_seqlens"])
    eo, eh = err_ratio(o, o_ref), err_ratio(ht, h_ref)
    print(f"[gla varlen] whole-tensor o {eo:.2e} final {eh:.2e}", flush=True)
    assert np.all(np.isfinite(o)) and eo <= TOL_BF16 and eh <= TOL_BF16


@pytest.mark.parametrize("kind", ["forget", "resets"])
@pytest.mark.parametrize("dtype,K,V", [("bf16", 128, 128), ("bf16", 64, 96), ("f32", 32, 64)],
                         ids=["bf16_chain", "fp32_chain", "f32"])
def test_gla_degenerate_gates(dtype, K, V, kind):
    """Per-key gates of -1e4 (a full reset) at every token, or for every key of
    every 37th token.  Float32 inputs carry each key's running gate as hi + lo
    (and form the decays of k from suffix sums in double), so their decays
    stay exact to float32 and the 1e-4 bar holds after a reset."""
    inp = make_chunk_inputs(small(f"gdeg_{kind}", dtype=dtype, K=K, V=V, T=150, initial_state=True))
    gk = np.array(make_key_gates(inp, seed=8), dtype=np.float32, copy=True)
    if kind == "forget":
        gk[:] = -1e4
    else:
        gk[:, ::37] = -1e4
    o, ht = run(inp, gk)
    o_ref, h_ref = oracle.gla_fwd(inp["q"], inp["k"], inp["v"], gk, scale=inp["scale"],
                                  initial_state=inp["initial_state"])
    tol = TOL_BF16 if dtype == "bf16" else TOL_F32
    eo, eh = err_ratio(o, o_ref), err_ratio(ht, h_ref)
    print(f"[gla deg {kind} {dtype} K={K}] o {eo:.2e} final {eh:.2e}", flush=True)
    assert np.all(np.isfinite(o)) and eo <= tol and eh <= tol


@pytest.mark.parametrize("w", [
    small("g_h32_k64", B=1, T=70, H=32, K=64, V=64),
    small("g_b24_t3", B=24, T=3, H=2, K=128, V=128, initial_state=True),
    small("g_n120_tiny_varlen", B=1, T=0, H=2, K=64, V=64, initial_state=True,
          fixed_lengths=tuple(int(x) for x in np.random.default_rng(3).integers(0, 6, size=120))),
    small("g_f32_b20_t2", dtype="f32", B=20, T=2, H=2, K=32, V=32, initial_state=True),
], ids=lambda w: w.name)
def test_gla_odd_shapes(w):
    test_gla_small(w, 1.0)


# chunk sizes 16 and 32 (section 二: a power of two; section 五 runs 16, 32
# and 64 with cu_seqlens [0, 15, 100, 300, 1200, 2000]): both chains
GLA_CHUNK_CASES = [
    (small("cs_varlen_pages_bf16_chain", B=1, T=0, K=64, V=64, fixed_lengths=(15, 85, 200, 900, 800),
           initial_state=True), 1.0),
    (small("cs_k128_v128_strong", K=128, V=128, T=150, initial_state=True), 0.1),
    (small("cs_fp32_chain_k32_v96", K=32, V=96, T=130, initial_state=True), 1.0),
    (small("cs_f32_k64", dtype="f32", K=64, V=64, T=150, initial_state=True), 1.0),
    (small("cs_gqa", H=4, Hkv=2, K=64, V=64, T=130, initial_state=True), 1.0),
]


@pytest.mark.parametrize("chunk", [16, 32])
@pytest.mark.parametrize("w,norm", GLA_CHUNK_CASES, ids=lambda x: x.name if hasattr(x, "name") else str(x))
def test_gla_chunk_sizes(w, norm, chunk):
    inp = make_chunk_inputs(w)
    inp["chunk_size"] = chunk
    gk = make_key_gates(inp, seed=w.seed + 3, normalizer=norm)
    o, ht = run(inp, gk)
    o_ref, h_ref = oracle.gla_fwd(inp["q"], inp["k"], inp["v"], gk, scale=inp["scale"],
                                  initial_state=inp["initial_state"], cu_seqlens=inp["cu_seqlens"])
    tol = TOL_BF16 if inp["dtype"] == "bf16" else TOL_F32
    eo, eh = err_ratio(o, o_ref), err_ratio(ht, h_ref)
    print(f"[gla {w.name} chunk {chunk}] o {eo:.2e} final {eh:.2e}", flush=True)
    assert np.all(np.isfinite(o)) and eo <= tol and eh <= tol



@pytest.mark.parametrize("chunk", [16, 32])
@pytest.mark.parametrize("w,norm", [
    (small("cse_t1", T=1, initial_state=True), 1.0),
    (small("cse_t17_k128", K=128, V=128, T=17, initial_state=True), 1.0),
    (small("cse_tiny_varlen", B=1, T=0, K=64, V=64, fixed_lengths=(0, 1, 16, 17, 0, 33), initial_state=True), 1.0),
    (small("cse_f32_t48", dtype="f32", K=32, V=32, T=48, initial_state=True), 1.0),
], ids=lambda x: x.name if hasattr(x, "name") else str(x))
def test_gla_chunk_sizes_edges(w, norm, chunk):
    inp = make_chunk_inputs(w)
    inp["chunk_size"] = chunk
    gk = make_key_gates(inp, seed=w.seed + 5, normalizer=norm)
    o, ht = run(inp, gk)
    o_ref, h_ref = oracle.gla_fwd(inp["q"], inp["k"], inp["v"], gk, scale=inp["scale"],
                                  initial_state=inp["initial_state"], cu_seqlens=inp["cu_seqlens"])
    tol = TOL_BF16 if inp["dtype"] == "bf16" else TOL_F32
    assert np.all(np.isfinite(o)) and err_ratio(o, o_ref) <= tol and err_ratio(ht, h_ref) <= tol


@pytest.mark.parametrize("chunk", [16, 32])
def test_gla_chunk_sizes_state_v_first(chunk):
    """The [V, K] state layout at the small chunk sizes: the same o bit for
    bit and the final state transposed."""
    inp = make_chunk_inputs(small("cs_gla_vf", B=1, T=0, K=64, V=64, fixed_lengths=(70, 33), initial_state=True))
    inp["chunk_size"] = chunk
    gk = make_key_gates(inp, seed=11)
    o_a, h_a = run(inp, gk)
    o_b, h_b = run(inp, gk, state_v_first=True)
    assert np.array_equal(o_a, o_b)
    assert np.array_equal(h_a, np.swapaxes(h_b, -1, -2))
