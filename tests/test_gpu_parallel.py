"""GPU parity of the parallel form (sgla_parallel_fwd) against the fp64
oracle: the decayed attention matrix A[i, j] = scale (q_i . k_j) exp(G_i -
G_j) for j <= i (0 above the diagonal) and o = A v (page "flash-linear-
attention 中的 Simple GLA", section 二: the parallel entry writes out A;
section 五: its test checks A, float32 inputs among its cases).  The bar per
output tensor: max |gpu - oracle| / RMS(oracle) <= 2e-2 for bf16 inputs and
<= 1e-4 for float32 inputs; entries above the diagonal must be exactly
zero."""
import numpy as np
import pytest
import torch

import oracle
from gla_workloads import CHUNK_CONFIGS, ChunkWorkload, make_chunk_inputs
from gpu_common import TOL_BF16, TOL_F32, device_inputs, err_ratio

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

if torch.cuda.is_available():
    import gated_linear_attention_amd as sgla
else:  # pragma: no cover - collected on CPU-only hosts, never run
    sgla = None


def small(name, **kw):
    base = dict(B=2, T=150, H=2, K=64, V=64, dtype="bf16", gate="g", seed=71, output_final_state=False)
    base.update(kw)
    return ChunkWorkload(name, **base)


CASES = [
    small("k64_v64"),
    small("k128_v128_gamma", B=1, T=200, H=4, K=128, V=128, gate="gamma"),
    small("k256_v256", B=1, T=130, K=256, V=256),
    small("k128_v48_ragged", B=1, T=67, K=128, V=48),          # T % 4 != 0: element stores
    small("gqa", H=4, Hkv=2, K=64, V=32, T=129),
    small("no_gate_t64", B=1, T=64, K=128, V=64, gate="none"),
    small("t1", B=3, T=1, K=64, V=16),
    small("strong_gate", B=1, T=300, K=64, V=128, gate_normalizer=0.1),
    small("weak_gate", B=1, T=300, K=128, V=64, gate_normalizer=10.0),
    small("k64_v256_t190", B=1, T=190, H=3, K=64, V=256),
    small("k256_v80", B=1, T=100, H=2, K=256, V=80),
    small("gqa_gamma_b3", B=3, T=300, H=6, Hkv=3, K=128, V=128, gate="gamma"),
    small("k64_v128_t257", B=1, T=257, H=2, K=64, V=128),        # ragged tail in the second half of a query tile
    small("negative_scale", B=1, T=140, K=128, V=64, scale=-0.3),   # sign carried by q, |scale| by the exponent
    small("zero_scale", B=1, T=70, K=64, V=64, scale=0.0),
]


def run(inp, out_dtype=torch.float32, output_attn=True):
    d = device_inputs(inp)
    o, A = sgla.parallel_fwd(d["q"], d["k"], d["v"], g=d["g"], g_gamma=d["g_gamma"], scale=inp["scale"],
                             output_attn=output_attn, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), None if A is None else A.cpu().numpy()


def check(o, A, o_ref, A_ref, label, tol=TOL_BF16):
    if not np.any(A_ref):  # scale 0: everything is exactly zero
        assert not np.any(A) and not np.any(o), label
        return
    eo, ea = err_ratio(o, o_ref), err_ratio(A, A_ref)
    T = A.shape[-1]
    upper = np.triu(np.ones((T, T), dtype=bool), 1)
    print(f"[parallel {label}] o {eo:.2e} A {ea:.2e}", flush=True)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(A))
    assert eo <= tol and ea <= tol
    assert not np.any(A[..., upper]), "entries above the diagonal must be zero"


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_parallel_small(w):
    inp = make_chunk_inputs(w)
    o, A = run(inp)
    o_ref, A_ref = oracle.parallel(inp["q"], inp["k"], inp["v"], g=inp["g"], g_gamma=inp["g_gamma"],
                                   scale=inp["scale"])
    check(o, A, o_ref, A_ref, w.name)


def test_parallel_bf16_output_and_no_matrix():
    """Without A the kernel computes the same o bit for bit (the matrix is
    optional); a bf16 o is the float32 one rounded once (within half a bf16
    ulp per element)."""
    inp = make_chunk_inputs(small("bf16_out", B=1, T=170, H=2, K=128, V=128))
    o_ref, _ = oracle.parallel(inp["q"], inp["k"], inp["v"], g=inp["g"], scale=inp["scale"],
                               output_attn=False)
    o32, A = run(inp)
    o_noa, none = run(inp, output_attn=False)
    o16, _ = run(inp, out_dtype=torch.bfloat16)
    assert none is None and A is not None
    e32 = err_ratio(o32, o_ref)
    print(f"[parallel bf16_out] o {e32:.2e}", flush=True)
    assert e32 <= TOL_BF16
    assert np.array_equal(o_noa, o32)
    assert np.all(np.abs(o16 - o32) <= 2.0 ** -8 * np.abs(o32))


def test_parallel_matches_chunked_forward():
    """From a zero state the parallel form and the chunked forward compute the
    same o (two different kernels), within the bf16 bar of each other."""
    inp = make_chunk_inputs(small("vs_chunk", B=2, T=257, H=4, Hkv=2, K=128, V=128))
    d = device_inputs(inp)
    o_c, _ = sgla.chunk_fwd(d["q"], d["k"], d["v"], g=d["g"], scale=inp["scale"], output_final_state=False,
                            o_dtype=torch.float32)
    o_p, _ = sgla.parallel_fwd(d["q"], d["k"], d["v"], g=d["g"], scale=inp["scale"], output_attn=False,
                               out_dtype=torch.float32)
    torch.cuda.synchronize()
    e = err_ratio(o_p.cpu().numpy(), o_c.cpu().numpy())
    print(f"[parallel vs chunk] {e:.2e}", flush=True)
    assert e <= TOL_BF16


def test_parallel_empty():
    inp = make_chunk_inputs(small("empty", B=2, T=0))
    o, A = run(inp)
    assert o.shape == (2, 0, 2, 64) and A.shape == (2, 2, 0, 0)


@pytest.mark.parametrize("workload,tol", [("parallel_bf16_k128", TOL_BF16), ("parallel_f32_k128", TOL_F32)])
def test_parallel_full_size_whole_tensor(workload, tol):
    """The benchmark workloads (bf16: B=2, T=4096, H=16, K=V=128; float32: one
    such row; per-token gates) in the benchmark's launch, every element of A
    and o against the oracle.  The oracle runs one batch row at a time (A in
    float64 is 2.1 GB per row); max |err| and the RMS are accumulated over
    the whole tensors."""
    w = CHUNK_CONFIGS[workload]
    inp = make_chunk_inputs(w)
    d = device_inputs(inp)
    o, A = sgla.parallel_fwd(d["q"], d["k"], d["v"], g=d["g"], scale=inp["scale"], output_attn=True,
                             out_dtype=torch.float32)
    torch.cuda.synchronize()
    acc = {"o": [0.0, 0.0, 0], "A": [0.0, 0.0, 0]}   # max |err|, sum ref^2, count

    def add(name, x, ref):
        x = np.asarray(x, dtype=np.float64)
        acc[name][0] = max(acc[name][0], float(np.max(np.abs(x - ref))))
        acc[name][1] += float(np.sum(ref * ref))
        acc[name][2] += ref.size

    for b in range(inp["B"]):
        sl = slice(b, b + 1)
        o_ref, A_ref = oracle.parallel(inp["q"][sl], inp["k"][sl], inp["v"][sl], g=inp["g"][sl],
                                       scale=inp["scale"])
        A_got = A[b].cpu().numpy()
        T = inp["T"]
        upper = np.triu(np.ones((T, T), dtype=bool), 1)
        assert not np.any(A_got[:, upper]), f"row {b}: nonzero entries above the diagonal"
        add("A", A_got, A_ref[0])
        del A_got, A_ref
        add("o", o[b].cpu().numpy(), o_ref[0])
    errs = {k: v[0] / np.sqrt(v[1] / v[2]) for k, v in acc.items()}
    print(f"[parallel full {workload}] whole-tensor o {errs['o']:.2e} A {errs['A']:.2e}", flush=True)
    assert errs["o"] <= tol and errs["A"] <= tol


# float32 inputs: the fp32 matrix-core kernel, held to the float32 bar
F32_CASES = [
    small("f32_k64_v64", dtype="f32"),
    small("f32_k128_v128_gamma", dtype="f32", B=1, T=200, H=4, K=128, V=128, gate="gamma"),
    small("f32_k256_v256", dtype="f32", B=1, T=130, K=256, V=256),
    small("f32_k32_v48_ragged", dtype="f32", B=1, T=67, K=32, V=48),      # T % 4 != 0: element stores
    small("f32_k16_v16", dtype="f32", B=2, T=33, H=3, K=16, V=16),
    small("f32_k96_v80", dtype="f32", B=1, T=129, H=2, K=96, V=80),
    small("f32_gqa", dtype="f32", H=4, Hkv=2, K=64, V=32, T=129),
    small("f32_no_gate", dtype="f32", B=1, T=64, K=128, V=64, gate="none"),
    small("f32_t1", dtype="f32", B=3, T=1, K=64, V=16),
    small("f32_strong_gate", dtype="f32", B=1, T=300, K=64, V=128, gate_normalizer=0.1),
    small("f32_weak_gate", dtype="f32", B=1, T=300, K=128, V=64, gate_normalizer=10.0),
    small("f32_k256_v64_t300", dtype="f32", B=2, T=300, H=3, Hkv=1, K=256, V=64, gate="gamma"),
    small("f32_k256_v128", dtype="f32", B=1, T=150, H=2, K=256, V=128),
    small("f32_negative_scale", dtype="f32", B=1, T=140, K=128, V=64, scale=-0.3),
    small("f32_zero_scale", dtype="f32", B=1, T=70, K=64, V=64, scale=0.0),
]


@pytest.mark.parametrize("w", F32_CASES, ids=lambda w: w.name)
def test_parallel_f32(w):
    inp = make_chunk_inputs(w)
    o, A = run(inp)
    o_ref, A_ref = oracle.parallel(inp["q"], inp["k"], inp["v"], g=inp["g"], g_gamma=inp["g_gamma"],
                                   scale=inp["scale"])
    check(o, A, o_ref, A_ref, w.name, tol=TOL_F32)


@pytest.mark.parametrize("kind", ["forget", "resets"])
def test_parallel_f32_degenerate_gates(kind):
    """Gates of -1e4 at every token, or at every 37th token with ordinary gates
    between: the decay exponents after a reset stay exact to float32, so A and
    o keep the float32 bar."""
    inp = make_chunk_inputs(small(f"f32_deg_{kind}", dtype="f32", B=2, T=200, H=2, K=64, V=64))
    g = np.array(inp["g"], dtype=np.float32, copy=True)
    if kind == "forget":
        g[:] = -1e4
    else:
        g[:, ::37, :] = -1e4
    inp["g"] = g
    o, A = run(inp)
    o_ref, A_ref = oracle.parallel(inp["q"], inp["k"], inp["v"], g=inp["g"], scale=inp["scale"])
    check(o, A, o_ref, A_ref, f"f32_deg_{kind}", tol=TOL_F32)


def test_parallel_f32_outputs_and_chunk_agreement():
    """float32 inputs: without A the kernel computes the same o bit for bit; a
    bf16 o is the float32 one rounded once; and the parallel form agrees with
    the float32 chunked forward (a different kernel) within the float32 bar."""
    inp = make_chunk_inputs(small("f32_vs_chunk", dtype="f32", B=2, T=257, H=4, Hkv=2, K=64, V=64))
    o32, A = run(inp)
    o_noa, none = run(inp, output_attn=False)
    o16, _ = run(inp, out_dtype=torch.bfloat16)
    assert none is None and A is not None
    assert np.array_equal(o_noa, o32)
    assert np.all(np.abs(o16 - o32) <= 2.0 ** -8 * np.abs(o32))
    d = device_inputs(inp)
    o_c, _ = sgla.chunk_fwd(d["q"], d["k"], d["v"], g=d["g"], scale=inp["scale"], output_final_state=False,
                            o_dtype=torch.float32)
    torch.cuda.synchronize()
    e = err_ratio(o32, o_c.cpu().numpy())
    print(f"[parallel f32 vs chunk] {e:.2e}", flush=True)
    assert e <= TOL_F32


def test_parallel_f32_empty():
    inp = make_chunk_inputs(small("f32_empty", dtype="f32", B=2, T=0))
    o, A = run(inp)
    assert o.shape == (2, 0, 2, 64) and A.shape == (2, 2, 0, 0)
