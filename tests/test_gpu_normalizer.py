"""GPU parity of the running normalizer (sgla_chunk_normalizer and
sgla_recurrent_step_normalizer) against the oracle: the output of a ones
column appended to v (page "relinear": the normalizer q . z of normalized
linear attention via the augmented value).  Inputs are used exactly and the
recurrence runs in fp32, so both dtypes are held to the float32 bar (1e-4);
the cross-check against the augmented forward uses the bf16 bar."""
import numpy as np
import pytest
import torch

import oracle
from gla_workloads import ChunkWorkload, DecodeWorkload, make_chunk_inputs, make_decode_inputs
from gpu_common import TOL_BF16, TOL_F32, device_inputs, err_ratio, to_dev

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

if torch.cuda.is_available():
    import gated_linear_attention_amd as sgla
else:  # pragma: no cover - collected on CPU-only hosts, never run
    sgla = None


def small(name, **kw):
    base = dict(B=2, T=150, H=2, K=64, V=64, dtype="bf16", gate="g", seed=51)
    base.update(kw)
    return ChunkWorkload(name, **base)


CASES = [
    small("k64"),
    small("k16_f32", K=16, dtype="f32", T=97),
    small("k128_gamma_h0", K=128, gate="gamma", initial_state=True, normalize_k=True, T=300),
    small("k256_no_gate", K=256, gate="none", T=129),
    small("k32_varlen", B=1, T=0, K=32, fixed_lengths=(15, 0, 1, 64, 200), initial_state=True),
    small("gqa_k64", H=6, Hkv=2, K=64, T=140, initial_state=True),
    small("empty", T=0, initial_state=True),
    # more than 32 chunks in a sequence: the chunk scan takes several batches
    small("long_k64", B=1, T=2600, K=64, initial_state=True),
    small("long_varlen_k128_gamma", B=1, T=0, K=128, gate="gamma", fixed_lengths=(2100, 5, 0, 700),
          initial_state=True),
]


def check_chunk_normalizer(w, chunk=64):
    inp = make_chunk_inputs(w)
    d = device_inputs(inp)
    rng = np.random.default_rng(w.seed + 7)
    z0 = (rng.standard_normal((inp["N"], inp["H"], inp["K"])).astype(np.float32)
          if inp["initial_state"] is not None else None)
    den, zt = sgla.chunk_normalizer(d["q"], d["k"], g=d["g"], g_gamma=d["g_gamma"], scale=inp["scale"],
                                    initial_z=to_dev(z0, torch.float32), output_final_state=True,
                                    cu_seqlens=inp["cu_seqlens"], chunk_size=chunk)
    torch.cuda.synchronize()
    den_ref, z_ref = oracle.normalizer(inp["q"], inp["k"], g=inp["g"], g_gamma=inp["g_gamma"],
                                       scale=inp["scale"], initial_z=z0, cu_seqlens=inp["cu_seqlens"])
    assert err_ratio(den.cpu().numpy(), den_ref) <= TOL_F32
    assert err_ratio(zt.cpu().numpy(), z_ref) <= TOL_F32


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_chunk_normalizer(w):
    check_chunk_normalizer(w)


# chunk sizes 16 and 32 (section 二: a power of two; section 五 runs 16, 32
# and 64 with cu_seqlens [0, 15, 100, 300, 1200, 2000])
CHUNK_CASES = [
    small("cs_varlen_pages", B=1, T=0, K=64, fixed_lengths=(15, 85, 200, 900, 800), initial_state=True),
    small("cs_k128_gamma_h0", K=128, gate="gamma", initial_state=True, normalize_k=True, T=300),
    small("cs_k16_f32", K=16, dtype="f32", T=97),
    small("cs_gqa_k64", H=6, Hkv=2, K=64, T=140, initial_state=True),
    # more than 32 chunks of 16 tokens: the chunk scan takes several batches
    small("cs_long_varlen_k128", B=1, T=0, K=128, fixed_lengths=(1100, 5, 0, 700), initial_state=True),
    small("cs_t1", T=1, initial_state=True),
    small("cs_tiny_varlen", B=1, T=0, K=64, fixed_lengths=(0, 1, 16, 17, 0, 33), initial_state=True),
    small("cs_empty", T=0, initial_state=True),
]


@pytest.mark.parametrize("chunk", [16, 32])
@pytest.mark.parametrize("w", CHUNK_CASES, ids=lambda w: w.name)
def test_chunk_normalizer_chunk_sizes(w, chunk):
    check_chunk_normalizer(w, chunk)


def test_normalizer_is_the_ones_column_of_the_augmented_forward():
    """chunk_fwd on v extended by a ones column (padded to the kernel's V
    granularity with zero columns) gives the normalizer in that column."""
    inp = make_chunk_inputs(small("aug", B=1, T=0, K=64, V=64, fixed_lengths=(200, 70)))
    d = device_inputs(inp)
    T = inp["T"]
    extra = np.zeros((1, T, 2, 64), dtype=np.float32)
    extra[..., 0] = 1.0
    v_aug = to_dev(np.concatenate([inp["v"], extra], axis=-1), torch.bfloat16)
    o, _ = sgla.chunk_fwd(d["q"], d["k"], v_aug, g=d["g"], scale=inp["scale"], cu_seqlens=inp["cu_seqlens"])
    den, _ = sgla.chunk_normalizer(d["q"], d["k"], g=d["g"], scale=inp["scale"], cu_seqlens=inp["cu_seqlens"])
    torch.cuda.synchronize()
    assert err_ratio(o[..., 64].cpu().numpy(), den.cpu().numpy()) <= TOL_BF16


@pytest.mark.parametrize("gate,Hkv,K", [("g", 4, 128), ("gamma", 2, 64), ("none", 1, 100)])
def test_step_normalizer(gate, Hkv, K):
    w = DecodeWorkload("nrm", N=5, H=4, K=K, V=32, steps=3, Hkv=Hkv, gate=gate, seed=K)
    inp = make_decode_inputs(w)
    rng = np.random.default_rng(2)
    z_np = rng.standard_normal((5, 4, K)).astype(np.float32)
    z = to_dev(z_np, torch.float32)
    z_ref = z_np.astype(np.float64)
    gg = to_dev(inp["g_gamma"], torch.float32)
    for s in range(inp["steps"]):
        g = None if inp["g"] is None else inp["g"][s]
        den = sgla.recurrent_step_normalizer(to_dev(inp["q"][s], torch.bfloat16), to_dev(inp["k"][s], torch.bfloat16),
                                             to_dev(g, torch.float32), z, scale=inp["scale"], g_gamma=gg)
        den_ref, z_ref = oracle.normalizer(inp["q"][s][:, None], inp["k"][s][:, None],
                                           g=None if g is None else g[:, None], g_gamma=inp["g_gamma"],
                                           scale=inp["scale"], initial_z=z_ref)
        torch.cuda.synchronize()
        assert err_ratio(den.cpu().numpy(), den_ref[:, 0]) <= TOL_F32
    assert err_ratio(z.cpu().numpy(), z_ref) <= TOL_F32


@pytest.mark.parametrize("kind", ["forget", "resets"])
@pytest.mark.parametrize("dtype,K", [("bf16", 128), ("f32", 32)], ids=["k128", "f32_k32"])
def test_chunk_normalizer_degenerate_gates(dtype, K, kind):
    """Gates of -1e4 (a full reset) at every token or every 37th token."""
    inp = make_chunk_inputs(small(f"ndeg_{kind}", dtype=dtype, K=K, T=150))
    g = np.array(inp["g"], dtype=np.float32, copy=True)
    if kind == "forget":
        g[:] = -1e4
    else:
        g[:, ::37, :] = -1e4
    d = device_inputs(inp)
    z0 = np.random.default_rng(4).standard_normal((inp["N"], inp["H"], K)).astype(np.float32)
    den, zt = sgla.chunk_normalizer(d["q"], d["k"], g=to_dev(g, torch.float32), scale=inp["scale"],
                                    initial_z=to_dev(z0, torch.float32), output_final_state=True)
    torch.cuda.synchronize()
    den_ref, z_ref = oracle.normalizer(inp["q"], inp["k"], g=g, scale=inp["scale"], initial_z=z0)
    e1, e2 = err_ratio(den.cpu().numpy(), den_ref), err_ratio(zt.cpu().numpy(), z_ref)
    print(f"[norm deg {kind} {dtype}] den {e1:.2e} z {e2:.2e}", flush=True)
    assert e1 <= TOL_F32 and e2 <= TOL_F32


@pytest.mark.parametrize("w", [
    small("n_h48_k64", B=1, T=70, H=48, K=64),
    small("n_b40_t3", B=40, T=3, H=2, K=128, initial_state=True),
    small("n_n150_tiny_varlen", B=1, T=0, H=2, K=64, initial_state=True,
          fixed_lengths=tuple(int(x) for x in np.random.default_rng(2).integers(0, 6, size=150))),
], ids=lambda w: w.name)
def test_chunk_normalizer_odd_shapes(w):
    test_chunk_normalizer(w)
