"""Pins for the CPU fp64 oracle (CPU only).

Each pin checks the oracle against something other than itself: a hand-worked
example, a closed form, a textbook special case, an independent brute-force
or chunked formulation, or an invariant the recurrence must satisfy.  The
operator is Simple GLA (page "flash-linear-attention 中的 Simple GLA",
section 一: S_t = exp(g_t) S_{t-1} + k_t v_t^T, o_t = scale S_t^T q_t; section
二: shapes, g / g_gamma, initial/final state, cu_seqlens; section 五: the test
axes -- chunk sizes 16/32/64, cu_seqlens [0,15,100,300,1200,2000], scales and
gate normalisers).

The pin functions take the oracle library handle so that
``test_planted_mistakes_are_caught`` can run them against deliberately broken
builds of the oracle.
"""
import json
import os

import numpy as np
import pytest

import oracle
from gla_workloads import logsigmoid, retnet_gamma, round_to_bf16

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
TIGHT = 1e-12


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def _rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    den = max(np.max(np.abs(b)), 1e-300)
    return float(np.max(np.abs(a - b)) / den)


# ---------------------------------------------------------------------------
# independent formulations used as pins (written from the mathematics, not
# from the oracle's loop)
# ---------------------------------------------------------------------------

def brute_force_parallel(q, k, v, g, scale, S0):
    """O(T^2) decay-weighted attention for one sequence and one head:
    o_t = scale * [ sum_{j<=t} exp(G_t - G_j) (q_t . k_j) v_j + exp(G_t) S0^T q_t ],
    G_t = g_0 + ... + g_t.  This is the explicit attention-matrix form the page
    calls parallel_simple_gla (section 二) written out in full."""
    T = q.shape[0]
    G = np.cumsum(g)
    o = np.zeros((T, v.shape[1]))
    for t in range(T):
        for j in range(t + 1):
            o[t] += np.exp(G[t] - G[j]) * np.dot(q[t], k[j]) * v[j]
        o[t] += np.exp(G[t]) * (S0.T @ q[t])
    return scale * o


def chunked_form(q, k, v, g, scale, S0, C):
    """Chunk form of the same operator for one sequence/head (section 一's
    naive_chunk_simple_gla idea and section 三's split into a chunk-local
    cumulative gate, an inter-chunk state pass and an output pass), in fp64.
    Within a chunk b is the inclusive cumulative log gate; the intra-chunk
    weight for j <= i is exp(b_i - b_j) and zero for j > i."""
    T = q.shape[0]
    S = S0.copy()
    o = np.zeros((T, v.shape[1]))
    for s in range(0, T, C):
        e = min(s + C, T)
        Q, Kc, Vc = q[s:e], k[s:e], v[s:e]
        b = np.cumsum(g[s:e])
        L = e - s
        expo = b[:, None] - b[None, :]
        mask = np.tril(np.ones((L, L), dtype=bool))
        M = np.where(mask, np.exp(np.where(mask, expo, 0.0)), 0.0)
        A = (Q @ Kc.T) * M
        o[s:e] = scale * (A @ Vc + np.exp(b)[:, None] * (Q @ S))
        S = np.exp(b[-1]) * S + (Kc * np.exp(b[-1] - b)[:, None]).T @ Vc
    return o, S


# ---------------------------------------------------------------------------
# pins as functions of the library handle
# ---------------------------------------------------------------------------

def pin_hand_example(lib):
    with open(os.path.join(GOLDEN, "hand_worked_example.json")) as f:
        ex = json.load(f)
    q = np.array(ex["q"], dtype=np.float64)[None, :, None, :]
    k = np.array(ex["k"], dtype=np.float64)[None, :, None, :]
    v = np.array(ex["v"], dtype=np.float64)[None, :, None, :]
    g = np.log(np.array(ex["gate_multiplier"], dtype=np.float64))[None, :, None]
    h0 = np.array(ex["initial_state"], dtype=np.float64)[:, None]
    o, ht = oracle.fwd(q, k, v, g=g, scale=ex["scale"], initial_state=h0,
                       cu_seqlens=ex["cu_seqlens"], lib=lib)
    ok_o = np.allclose(o[0, :, 0], np.array(ex["expected_o"]), rtol=0, atol=1e-13)
    ok_s = np.allclose(ht[:, 0], np.array(ex["expected_final_state"]), rtol=0, atol=1e-13)
    return ok_o and ok_s


def pin_brute_force(lib, seed=0, T=97, H=3, K=5, V=4, scale=0.37, normalizer=1.0):
    """P1: random q, k, v, g, S0 against the O(T^2) form, every head."""
    rng = np.random.default_rng(seed)
    q, k, v = _rand(rng, 1, T, H, K), _rand(rng, 1, T, H, K), _rand(rng, 1, T, H, V)
    g = logsigmoid(_rand(rng, 1, T, H)) / normalizer
    S0 = _rand(rng, 1, H, K, V)
    o, ht = oracle.fwd(q, k, v, g=g, scale=scale, initial_state=S0, lib=lib)
    for h in range(H):
        ref = brute_force_parallel(q[0, :, h], k[0, :, h], v[0, :, h], g[0, :, h], scale, S0[0, h])
        if _rel(o[0, :, h], ref) > TIGHT:
            return False
    # final state: S_T = exp(G_T) S0 + sum_j exp(G_T - G_j) k_j v_j^T
    for h in range(H):
        G = np.cumsum(g[0, :, h])
        ref = np.exp(G[-1]) * S0[0, h]
        for j in range(T):
            ref = ref + np.exp(G[-1] - G[j]) * np.outer(k[0, j, h], v[0, j, h])
        if _rel(ht[0, h], ref) > TIGHT:
            return False
    return True


def pin_zero_gate(lib, seed=1, T=50, H=2, K=4, V=6):
    """P2: g = 0 is causal linear attention: S_t = S0 + sum_{j<=t} k_j v_j^T."""
    rng = np.random.default_rng(seed)
    q, k, v = _rand(rng, 1, T, H, K), _rand(rng, 1, T, H, K), _rand(rng, 1, T, H, V)
    S0 = _rand(rng, 1, H, K, V)
    scale = 0.5
    o_none, ht_none = oracle.fwd(q, k, v, scale=scale, initial_state=S0, lib=lib)
    o_zero, ht_zero = oracle.fwd(q, k, v, g=np.zeros((1, T, H)), scale=scale, initial_state=S0,
                                 lib=lib)
    kv = np.einsum("bthk,bthv->bthkv", k, v)
    S = S0[:, None] + np.cumsum(kv, axis=1)          # [1, T, H, K, V]
    ref = scale * np.einsum("bthkv,bthk->bthv", S, q)
    return (_rel(o_none, ref) < TIGHT and _rel(o_zero, ref) < TIGHT
            and _rel(ht_none, S[:, -1]) < TIGHT and _rel(ht_zero, S[:, -1]) < TIGHT)


def pin_full_forget(lib, seed=2, T=33, H=2, K=3, V=5):
    """P3: g -> -inf forgets everything before the current token:
    o_t = scale (q_t . k_t) v_t and the final state is k_last v_last^T."""
    rng = np.random.default_rng(seed)
    q, k, v = _rand(rng, 1, T, H, K), _rand(rng, 1, T, H, K), _rand(rng, 1, T, H, V)
    S0 = _rand(rng, 1, H, K, V)
    scale = 1.3
    o, ht = oracle.fwd(q, k, v, g=np.full((1, T, H), -1e4), scale=scale, initial_state=S0,
                       lib=lib)
    ref = scale * np.sum(q * k, axis=-1, keepdims=True) * v
    ref_s = np.einsum("hk,hv->hkv", k[0, -1], v[0, -1])
    return _rel(o, ref) < TIGHT and _rel(ht[0], ref_s) < TIGHT


def pin_split_sequence(lib, seed=3, T=80, split=29, H=2, K=4, V=3):
    """P4: running [0, split) then [split, T) from the carried state equals one
    pass, bit for bit."""
    rng = np.random.default_rng(seed)
    q, k, v = _rand(rng, 1, T, H, K), _rand(rng, 1, T, H, K), _rand(rng, 1, T, H, V)
    g = logsigmoid(_rand(rng, 1, T, H))
    S0 = _rand(rng, 1, H, K, V)
    o, ht = oracle.fwd(q, k, v, g=g, initial_state=S0, lib=lib)
    o1, h1 = oracle.fwd(q[:, :split], k[:, :split], v[:, :split], g=g[:, :split],
                        initial_state=S0, lib=lib)
    o2, h2 = oracle.fwd(q[:, split:], k[:, split:], v[:, split:], g=g[:, split:],
                        initial_state=h1, lib=lib)
    return (np.array_equal(np.concatenate([o1, o2], axis=1), o) and np.array_equal(h2, ht))


def pin_varlen_equals_per_sequence(lib, seed=4, H=2, K=4, V=5):
    """P5: a packed batch equals separate runs of its sequences, bit for bit
    (section 五's cu_seqlens [0,15,100,300,1200,2000], shortened here)."""
    rng = np.random.default_rng(seed)
    cu = np.array([0, 15, 100, 300, 301, 301, 420], dtype=np.int64)   # incl. len 1 and len 0
    T = int(cu[-1])
    N = len(cu) - 1
    q, k, v = _rand(rng, 1, T, H, K), _rand(rng, 1, T, H, K), _rand(rng, 1, T, H, V)
    g = logsigmoid(_rand(rng, 1, T, H))
    S0 = _rand(rng, N, H, K, V)
    o, ht = oracle.fwd(q, k, v, g=g, initial_state=S0, cu_seqlens=cu, lib=lib)
    for n in range(N):
        s, e = cu[n], cu[n + 1]
        on, hn = oracle.fwd(q[:, s:e], k[:, s:e], v[:, s:e], g=g[:, s:e],
                            initial_state=S0[n:n + 1], lib=lib)
        if not (np.array_equal(on, o[:, s:e]) and np.array_equal(hn[0], ht[n])):
            return False
    # an empty sequence hands its initial state straight through
    return np.array_equal(ht[4], S0[4])


def pin_chunk_form(lib, seed=5, H=2, K=6, V=5):
    """P6: the chunked formulation (chunk sizes 16, 32, 64; partial chunks;
    packed cu_seqlens [0,15,100,300,1200,2000]) equals the recurrence."""
    rng = np.random.default_rng(seed)
    cu = np.array([0, 15, 100, 300, 1200, 2000], dtype=np.int64)
    T = int(cu[-1])
    N = len(cu) - 1
    q, k, v = _rand(rng, 1, T, H, K), _rand(rng, 1, T, H, K), _rand(rng, 1, T, H, V)
    g = logsigmoid(_rand(rng, 1, T, H))
    S0 = _rand(rng, N, H, K, V)
    scale = 0.21
    o, ht = oracle.fwd(q, k, v, g=g, scale=scale, initial_state=S0, cu_seqlens=cu, lib=lib)
    for C in (16, 32, 64):
        for n in range(N):
            s, e = cu[n], cu[n + 1]
            for h in range(H):
                oc, Sc = chunked_form(q[0, s:e, h], k[0, s:e, h], v[0, s:e, h], g[0, s:e, h],
                                      scale, S0[n, h], C)
                if _rel(o[0, s:e, h], oc) > 1e-11 or _rel(ht[n, h], Sc) > 1e-11:
                    return False
    return True


def pin_gamma_is_broadcast_g(lib, seed=6, T=70, H=4, K=3, V=3):
    """P7: a per-head decay g_gamma[h] equals the per-token gate g[t, h] =
    g_gamma[h], bit for bit (section 二: g and g_gamma are alternatives)."""
    rng = np.random.default_rng(seed)
    q, k, v = _rand(rng, 2, T, H, K), _rand(rng, 2, T, H, K), _rand(rng, 2, T, H, V)
    gam = retnet_gamma(H).astype(np.float64)
    o1, h1 = oracle.fwd(q, k, v, g_gamma=gam, lib=lib)
    o2, h2 = oracle.fwd(q, k, v, g=np.broadcast_to(gam, (2, T, H)).copy(), lib=lib)
    return np.array_equal(o1, o2) and np.array_equal(h1, h2)


def pin_retnet_closed_form(lib, T=300):
    """P8: K = V = 1, q = k = v = 1, constant decay gamma:
    S_t = sum_{j<=t} gamma^(t-j) = (1 - gamma^(t+1)) / (1 - gamma)."""
    H = 3
    gam = np.array([0.5, 0.9, 0.999])
    ones = np.ones((1, T, H, 1))
    scale = 0.75
    o, ht = oracle.fwd(ones, ones, ones, g_gamma=np.log(gam), scale=scale, lib=lib)
    t = np.arange(T)[:, None]
    ref = scale * (1 - gam[None, :] ** (t + 1)) / (1 - gam[None, :])
    return _rel(o[0, :, :, 0], ref) < 1e-12 and _rel(ht[0, :, 0, 0], ref[-1] / scale) < 1e-12


def pin_invariants(lib, seed=7, T=40, H=3, K=4, V=4):
    """P9: o is linear in v; the final state ignores q and scale; scale = 0
    gives o = 0; permuting heads permutes the outputs."""
    rng = np.random.default_rng(seed)
    q, k = _rand(rng, 1, T, H, K), _rand(rng, 1, T, H, K)
    v1, v2 = _rand(rng, 1, T, H, V), _rand(rng, 1, T, H, V)
    g = logsigmoid(_rand(rng, 1, T, H))
    oa, ha = oracle.fwd(q, k, v1, g=g, lib=lib)
    ob, hb = oracle.fwd(q, k, v2, g=g, lib=lib)
    oc, hc = oracle.fwd(q, k, v1 + 2.0 * v2, g=g, lib=lib)
    if _rel(oc, oa + 2.0 * ob) > 1e-12 or _rel(hc, ha + 2.0 * hb) > 1e-12:
        return False
    oq, hq = oracle.fwd(_rand(rng, 1, T, H, K), k, v1, g=g, scale=3.0, lib=lib)
    if not np.array_equal(hq, ha):
        return False
    oz, _ = oracle.fwd(q, k, v1, g=g, scale=0.0, lib=lib)
    if np.any(oz != 0.0):
        return False
    perm = np.array([2, 0, 1])
    op, hp = oracle.fwd(q[:, :, perm], k[:, :, perm], v1[:, :, perm], g=g[:, :, perm], lib=lib)
    return np.array_equal(op, oa[:, :, perm]) and np.array_equal(hp, ha[:, perm])


def pin_prefill_then_decode(lib, seed=8, T=24, N=3, H=2, K=4, V=5):
    """P10/P11: T single-token decode steps from S0 equal one forward over the
    T tokens (and T = 1 forward equals one step)."""
    rng = np.random.default_rng(seed)
    q, k, v = _rand(rng, N, T, H, K), _rand(rng, N, T, H, K), _rand(rng, N, T, H, V)
    g = logsigmoid(_rand(rng, N, T, H))
    S0 = _rand(rng, N, H, K, V)
    o, ht = oracle.fwd(q, k, v, g=g, initial_state=S0, lib=lib)
    S = S0
    for t in range(T):
        ot, S = oracle.step(q[:, t], k[:, t], v[:, t], g[:, t], S, lib=lib)
        if _rel(ot, o[:, t]) > 1e-12:
            return False
    if _rel(S, ht) > 1e-12:
        return False
    o1, h1 = oracle.fwd(q[:, :1], k[:, :1], v[:, :1], g=g[:, :1], initial_state=S0, lib=lib)
    os_, Ss = oracle.step(q[:, 0], k[:, 0], v[:, 0], g[:, 0], S0, lib=lib)
    return np.allclose(o1[:, 0], os_, rtol=0, atol=1e-14) and np.allclose(h1, Ss, rtol=0, atol=1e-14)


def pin_step_brute_force(lib, seed=9, N=2, H=3, K=3, V=2):
    """Decode step written out for one unit: S' = exp(g) S + k v^T, o = scale S'^T q."""
    rng = np.random.default_rng(seed)
    q, k, v = _rand(rng, N, H, K), _rand(rng, N, H, K), _rand(rng, N, H, V)
    g = logsigmoid(_rand(rng, N, H))
    S = _rand(rng, N, H, K, V)
    o, S1 = oracle.step(q, k, v, g, S, scale=0.4, lib=lib)
    for n in range(N):
        for h in range(H):
            ref_S = np.exp(g[n, h]) * S[n, h] + np.outer(k[n, h], v[n, h])
            if _rel(S1[n, h], ref_S) > TIGHT:
                return False
            if _rel(o[n, h], 0.4 * ref_S.T @ q[n, h]) > TIGHT:
                return False
    return True


def pin_chunk_local_cumsum(lib, seed=10, H=3):
    """Gate prep: with g = ln 2 everywhere the scaled chunk-local sum counts
    tokens since the chunk start (1, 2, ..., restarting at every chunk and every
    sequence); for random gates 2^gc equals the product of exp(g_j) over the
    chunk prefix."""
    cu = np.array([0, 15, 100, 300, 301, 301, 420], dtype=np.int64)
    T = int(cu[-1])
    gc = oracle.chunk_local_cumsum(np.full((1, T, H), np.log(2.0)), chunk_size=32,
                                   cu_seqlens=cu, lib=lib)
    for n in range(len(cu) - 1):
        for t in range(cu[n], cu[n + 1]):
            if abs(gc[0, t, 0] - ((t - cu[n]) % 32 + 1)) > 1e-12:
                return False
    rng = np.random.default_rng(seed)
    g = logsigmoid(_rand(rng, 2, 130, H))
    gc = oracle.chunk_local_cumsum(g, chunk_size=64, lib=lib)
    for b in range(2):
        for t in range(130):
            c0 = (t // 64) * 64
            prod = np.prod(np.exp(g[b, c0:t + 1]), axis=0)
            if np.max(np.abs(np.exp2(gc[b, t]) - prod) / prod) > 1e-12:
                return False
    return True


def pin_gqa_is_repeated_mha(lib, seed=11, H=6, Hkv=2, K=4, V=3):
    """Grouped kv heads (page "relinear", its GQA target; page "flash-linear-
    attention 中的 Simple GLA", section 四, num_kv_heads dividing num_heads):
    query head h reads kv head h // (H // Hkv), the contiguous grouping of
    repeat_kv.  So the forward with Hkv kv heads equals, bit for bit, the
    (brute-force pinned) multi-head forward on k and v whose every head is
    repeated H // Hkv times in a row -- for packed sequences, per-token gates,
    g_gamma and one shared kv head (MQA) alike."""
    rng = np.random.default_rng(seed)
    cu = np.array([0, 13, 50, 71], dtype=np.int64)
    T = int(cu[-1])
    q = _rand(rng, 1, T, H, K)
    g = logsigmoid(_rand(rng, 1, T, H))
    S0 = _rand(rng, 3, H, K, V)
    for hkv in (Hkv, 1):
        rep = H // hkv
        k, v = _rand(rng, 1, T, hkv, K), _rand(rng, 1, T, hkv, V)
        kr, vr = np.repeat(k, rep, axis=2), np.repeat(v, rep, axis=2)
        o, ht = oracle.fwd(q, k, v, g=g, initial_state=S0, cu_seqlens=cu, lib=lib)
        om, hm = oracle.fwd(q, kr, vr, g=g, initial_state=S0, cu_seqlens=cu, lib=lib)
        if not (np.array_equal(o, om) and np.array_equal(ht, hm)):
            return False
        gam = retnet_gamma(H).astype(np.float64)
        o, ht = oracle.fwd(q, k, v, g_gamma=gam, scale=0.3, lib=lib)
        om, hm = oracle.fwd(q, kr, vr, g_gamma=gam, scale=0.3, lib=lib)
        if not (np.array_equal(o, om) and np.array_equal(ht, hm)):
            return False
    return True


def pin_step_variants(lib, seed=12, N=3, H=4, Hkv=2, K=3, V=5):
    """Decode step with a per-head decay g_gamma (section 二: g and g_gamma are
    alternatives) and with grouped kv heads: it equals the one-token forward
    from the same state (forward pinned above), g_gamma equals the broadcast
    per-token gate bit for bit, no gate at all equals g = 0, and Hkv kv heads
    equal the repeated multi-head step bit for bit."""
    rng = np.random.default_rng(seed)
    q, k, v = _rand(rng, N, H, K), _rand(rng, N, Hkv, K), _rand(rng, N, Hkv, V)
    S = _rand(rng, N, H, K, V)
    gam = retnet_gamma(H).astype(np.float64)
    o1, S1 = oracle.step(q, k, v, None, S, scale=0.6, g_gamma=gam, lib=lib)
    of, hf = oracle.fwd(q[:, None], k[:, None], v[:, None], g_gamma=gam, scale=0.6,
                        initial_state=S, lib=lib)
    if _rel(o1, of[:, 0]) > 1e-14 or _rel(S1, hf) > 1e-14:
        return False
    o2, S2 = oracle.step(q, k, v, np.broadcast_to(gam, (N, H)).copy(), S, scale=0.6, lib=lib)
    if not (np.array_equal(o1, o2) and np.array_equal(S1, S2)):
        return False
    o3, S3 = oracle.step(q, k, v, None, S, lib=lib)
    o4, S4 = oracle.step(q, k, v, np.zeros((N, H)), S, lib=lib)
    if not (np.array_equal(o3, o4) and np.array_equal(S3, S4)):
        return False
    rep = H // Hkv
    o5, S5 = oracle.step(q, np.repeat(k, rep, axis=1), np.repeat(v, rep, axis=1), None, S,
                         scale=0.6, g_gamma=gam, lib=lib)
    return np.array_equal(o1, o5) and np.array_equal(S1, S5)


def _loss(lib, q, k, v, g, gg, scale, S0, cu, do, dht):
    o, ht = oracle.fwd(q, k, v, g=g, g_gamma=gg, scale=scale, initial_state=S0, cu_seqlens=cu,
                       nthreads=1, lib=lib)
    return float(np.sum(o * do) + np.sum(ht * dht))


def pin_bwd_finite_differences(lib, seed=13, H=2, K=3, V=2):
    """Backward (page "flash-linear-attention 中的 Simple GLA", section 三 and
    the gradient tests of section 五): every gradient -- dq, dk, dv, dg or
    dg_gamma, dh0 -- equals the central finite difference of L = <do, o> +
    <dht, final_state> computed with the (pinned) forward, on packed sequences
    with an empty one, for a per-token gate, a per-head g_gamma and no gate."""
    rng = np.random.default_rng(seed)
    cu = np.array([0, 5, 5, 13], dtype=np.int64)
    T, N = 13, 3
    q, k, v = _rand(rng, 1, T, H, K), _rand(rng, 1, T, H, K), _rand(rng, 1, T, H, V)
    do = _rand(rng, 1, T, H, V)
    dht = _rand(rng, N, H, K, V)
    S0 = _rand(rng, N, H, K, V)
    scale, eps = 0.7, 1e-6
    for kind in ("g", "gamma", "none"):
        g = logsigmoid(_rand(rng, 1, T, H)) if kind == "g" else None
        gg = np.log([0.9, 0.6]) if kind == "gamma" else None
        gr = oracle.bwd(q, k, v, do, g=g, g_gamma=gg, scale=scale, initial_state=S0, dht=dht,
                        cu_seqlens=cu, nthreads=1, lib=lib)
        args = dict(q=q, k=k, v=v, g=g, gg=gg, S0=S0)
        want = dict(q="dq", k="dk", v="dv", g="dg", gg="dg_gamma", S0="dh0")
        for name, gname in want.items():
            x = args[name]
            if x is None:
                if gr.get(gname) is not None:
                    return False
                continue
            fd = np.zeros_like(x)
            for idx in np.ndindex(x.shape):
                a = dict(args)
                xp = x.copy(); xp[idx] += eps
                xm = x.copy(); xm[idx] -= eps
                a[name] = xp
                lp = _loss(lib, a["q"], a["k"], a["v"], a["g"], a["gg"], scale, a["S0"], cu, do, dht)
                a[name] = xm
                lm = _loss(lib, a["q"], a["k"], a["v"], a["g"], a["gg"], scale, a["S0"], cu, do, dht)
                fd[idx] = (lp - lm) / (2 * eps)
            if _rel(gr[gname], fd) > 1e-6:
                return False
    return True


def pin_bwd_gqa_finite_differences(lib, seed=21, H=4, Hkv=2, K=3, V=2):
    """Backward with grouped kv heads (query head h reads kv head h // (H //
    Hkv)): dq, dk [T, Hkv, K], dv [T, Hkv, V], dg and dh0 equal the central
    finite differences of the grouped forward, which evaluates the kv rows of
    each group directly (no repeat), on packed sequences."""
    rng = np.random.default_rng(seed)
    cu = np.array([0, 4, 9], dtype=np.int64)
    T, N = 9, 2
    q, k, v = _rand(rng, 1, T, H, K), _rand(rng, 1, T, Hkv, K), _rand(rng, 1, T, Hkv, V)
    do = _rand(rng, 1, T, H, V)
    dht = _rand(rng, N, H, K, V)
    S0 = _rand(rng, N, H, K, V)
    g = logsigmoid(_rand(rng, 1, T, H))
    scale, eps = 0.6, 1e-6
    gr = oracle.bwd(q, k, v, do, g=g, scale=scale, initial_state=S0, dht=dht, cu_seqlens=cu,
                    nthreads=1, lib=lib)
    if gr["dk"].shape != k.shape or gr["dv"].shape != v.shape:
        return False
    args = dict(q=q, k=k, v=v, g=g, S0=S0)
    want = dict(q="dq", k="dk", v="dv", g="dg", S0="dh0")
    for name, gname in want.items():
        x = args[name]
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            a = dict(args)
            xp = x.copy(); xp[idx] += eps
            xm = x.copy(); xm[idx] -= eps
            a[name] = xp
            lp = _loss(lib, a["q"], a["k"], a["v"], a["g"], None, scale, a["S0"], cu, do, dht)
            a[name] = xm
            lm = _loss(lib, a["q"], a["k"], a["v"], a["g"], None, scale, a["S0"], cu, do, dht)
            fd[idx] = (lp - lm) / (2 * eps)
        if _rel(gr[gname], fd) > 1e-6:
            return False
    return True


def pin_bwd_gate_identity(lib, seed=14, B=2, T=150, H=2, K=5, V=4):
    """The gate gradient from the mathematics of the scalar gate: every term of
    o_t and of the final state depends on the log gates only through
    differences of their running sums G, so dL/dG_t = q_t . dq_t - k_t . dk_t
    (+ <dht, S_T> at the last token), and dg_j is the reverse cumulative sum of
    that over t >= j -- the relation behind section 三's reverse cumsum for dg.
    Checked against the oracle's dg (computed as gamma_t <D, S_{t-1}>) and, for
    g_gamma, the sum of dg over tokens."""
    rng = np.random.default_rng(seed)
    q, k, v = _rand(rng, B, T, H, K), _rand(rng, B, T, H, K), _rand(rng, B, T, H, V)
    do, dht = _rand(rng, B, T, H, V), _rand(rng, B, H, K, V)
    g = logsigmoid(_rand(rng, B, T, H))
    S0 = _rand(rng, B, H, K, V)
    _, ht = oracle.fwd(q, k, v, g=g, scale=0.5, initial_state=S0, lib=lib)
    gr = oracle.bwd(q, k, v, do, g=g, scale=0.5, initial_state=S0, dht=dht, lib=lib)
    r = np.sum(q * gr["dq"], axis=-1) - np.sum(k * gr["dk"], axis=-1)      # [B, T, H]
    r[:, -1, :] += np.einsum("bhkv,bhkv->bh", dht, ht)
    ref = np.flip(np.cumsum(np.flip(r, axis=1), axis=1), axis=1)
    if _rel(gr["dg"], ref) > 1e-10:
        return False
    gam = retnet_gamma(H).astype(np.float64)
    g2 = oracle.bwd(q, k, v, do, g=np.broadcast_to(gam, (B, T, H)).copy(), scale=0.5,
                    initial_state=S0, dht=dht, lib=lib)
    g3 = oracle.bwd(q, k, v, do, g_gamma=gam, scale=0.5, initial_state=S0, dht=dht, lib=lib)
    return (_rel(g3["dg_gamma"], g2["dg"].sum(axis=(0, 1))) < 1e-12
            and all(np.array_equal(g2[x], g3[x]) for x in ("dq", "dk", "dv", "dh0")))


def pin_state_v_first(lib, seed=15, N=2, H=2, K=3, V=4):
    """The [V, K] state layout (section 二, state_v_first): one token from a
    zero state with g = 0 leaves the state v k^T (rows indexed by v); a
    forward, a backward and a decode step in that layout equal the [K, V] ones
    with every state transposed."""
    rng = np.random.default_rng(seed)
    q, k, v = _rand(rng, N, 1, H, K), _rand(rng, N, 1, H, K), _rand(rng, N, 1, H, V)
    _, ht = oracle.fwd(q, k, v, g=np.zeros((N, 1, H)), lib=lib, state_v_first=True)
    want = np.einsum("nhv,nhk->nhvk", v[:, 0], k[:, 0])
    if _rel(ht, want) > TIGHT:
        return False
    T = 30
    q, k, v = _rand(rng, N, T, H, K), _rand(rng, N, T, H, K), _rand(rng, N, T, H, V)
    g = logsigmoid(_rand(rng, N, T, H))
    S0 = _rand(rng, N, H, K, V)
    S0t = np.ascontiguousarray(np.swapaxes(S0, -1, -2))
    o1, h1 = oracle.fwd(q, k, v, g=g, initial_state=S0, lib=lib)
    o2, h2 = oracle.fwd(q, k, v, g=g, initial_state=S0t, lib=lib, state_v_first=True)
    if not (np.array_equal(o1, o2) and np.array_equal(np.swapaxes(h1, -1, -2), h2)):
        return False
    do, dht = _rand(rng, N, T, H, V), _rand(rng, N, H, K, V)
    b1 = oracle.bwd(q, k, v, do, g=g, initial_state=S0, dht=dht, lib=lib)
    b2 = oracle.bwd(q, k, v, do, g=g, initial_state=S0t, dht=np.swapaxes(dht, -1, -2), lib=lib,
                    state_v_first=True)
    if not (np.array_equal(b1["dq"], b2["dq"]) and np.array_equal(np.swapaxes(b1["dh0"], -1, -2), b2["dh0"])):
        return False
    s1, S1 = oracle.step(q[:, 0], k[:, 0], v[:, 0], g[:, 0], S0, lib=lib)
    s2, S2 = oracle.step(q[:, 0], k[:, 0], v[:, 0], g[:, 0], S0t, lib=lib, state_v_first=True)
    return np.array_equal(s1, s2) and np.array_equal(np.swapaxes(S1, -1, -2), S2)


def pin_normalizer(lib, seed=16, H=3, K=4, V=5):
    """The running normalizer (relinear pages: the output of a ones column
    appended to v is q . z).  With no gate it is scale * q_t . (k_0 + ... +
    k_t) (closed form); with gates it equals the last output column and last
    state column of a forward on [v, 1] bit for bit, on packed sequences with
    an initial z."""
    rng = np.random.default_rng(seed)
    T = 40
    q, k = _rand(rng, 1, T, H, K), _rand(rng, 1, T, H, K)
    den, z = oracle.normalizer(q, k, scale=0.3, lib=lib)
    cs = np.cumsum(k, axis=1)
    if _rel(den, 0.3 * np.sum(q * cs, axis=-1)) > TIGHT or _rel(z[0], cs[0, -1]) > TIGHT:
        return False
    cu = np.array([0, 11, 11, 40], dtype=np.int64)
    v = _rand(rng, 1, T, H, V)
    g = logsigmoid(_rand(rng, 1, T, H))
    z0 = _rand(rng, 3, H, K)
    S0 = np.concatenate([_rand(rng, 3, H, K, V), z0[..., None]], axis=-1)
    o, ht = oracle.fwd(q, k, np.concatenate([v, np.ones((1, T, H, 1))], axis=-1), g=g, scale=0.3,
                       initial_state=S0, cu_seqlens=cu, lib=lib)
    den, z = oracle.normalizer(q, k, g=g, scale=0.3, initial_z=z0, cu_seqlens=cu, lib=lib)
    return np.array_equal(den, o[..., V]) and np.array_equal(z, ht[..., V])


def pin_gla_scalar_gate_is_simple_gla(lib, seed=17, H=4, Hkv=2, K=3, V=5):
    """Elementwise-gate GLA with every key's gate equal to the head's scalar
    gate is Simple GLA (the pages: the head-wise gate is the special case of
    the key-vector gate), bit for bit, on packed sequences with grouped kv
    heads and an initial state."""
    rng = np.random.default_rng(seed)
    cu = np.array([0, 9, 9, 50], dtype=np.int64)
    T = 50
    q, k, v = _rand(rng, 1, T, H, K), _rand(rng, 1, T, Hkv, K), _rand(rng, 1, T, Hkv, V)
    g = logsigmoid(_rand(rng, 1, T, H))
    S0 = _rand(rng, 3, H, K, V)
    o1, h1 = oracle.fwd(q, k, v, g=g, scale=0.4, initial_state=S0, cu_seqlens=cu, lib=lib)
    gk = np.repeat(g[..., None], K, axis=-1)
    o2, h2 = oracle.gla_fwd(q, k, v, gk, scale=0.4, initial_state=S0, cu_seqlens=cu, lib=lib)
    return np.array_equal(o1, o2) and np.array_equal(h1, h2)


def pin_gla_brute_force(lib, seed=18, T=60, H=2, K=4, V=3):
    """Elementwise-gate GLA against its explicit attention form (one sequence):
    o_t = scale [ sum_{j<=t} sum_a q_t[a] k_j[a] exp(G_t[a] - G_j[a]) v_j
                  + sum_a q_t[a] exp(G_t[a]) S0[a, :] ],  G = cumsum of gk
    (different gates on different keys, so a gate applied to the wrong index
    changes the result)."""
    rng = np.random.default_rng(seed)
    q, k, v = _rand(rng, 1, T, H, K), _rand(rng, 1, T, H, K), _rand(rng, 1, T, H, V)
    gk = logsigmoid(_rand(rng, 1, T, H, K)) * np.linspace(0.2, 2.0, K)
    S0 = _rand(rng, 1, H, K, V)
    o, ht = oracle.gla_fwd(q, k, v, gk, scale=0.6, initial_state=S0, lib=lib)
    for h in range(H):
        G = np.cumsum(gk[0, :, h], axis=0)                        # [T, K]
        for t in range(T):
            w = np.exp(G[t][None, :] - G[: t + 1]) * q[0, t, h][None, :] * k[0, : t + 1, h]   # [t+1, K]
            ref = w.sum(axis=1) @ v[0, : t + 1, h] + (q[0, t, h] * np.exp(G[t])) @ S0[0, h]
            if _rel(o[0, t, h], 0.6 * ref) > 1e-11:
                return False
        Sref = np.exp(G[-1])[:, None] * S0[0, h] + sum(
            np.exp(G[-1] - G[j])[:, None] * np.outer(k[0, j, h], v[0, j, h]) for j in range(T))
        if _rel(ht[0, h], Sref) > 1e-11:
            return False
    return True


def pin_parallel_equals_recurrence(lib, seed=19, B=2, T=45, H=4, Hkv=2, K=5, V=3):
    """The parallel form (explicit decayed attention matrix) equals the
    token-by-token recurrence from a zero state, with per-token gates and with
    a per-head g_gamma, on grouped kv heads; its o is A v."""
    rng = np.random.default_rng(seed)
    q, k, v = _rand(rng, B, T, H, K), _rand(rng, B, T, Hkv, K), _rand(rng, B, T, Hkv, V)
    g = logsigmoid(_rand(rng, B, T, H)) * 0.7
    gg = np.log1p(-np.exp2(-np.arange(1, H + 1, dtype=np.float64)))
    for kw in ({"g": g}, {"g_gamma": gg}, {}):
        o_r, _ = oracle.fwd(q, k, v, scale=0.45, output_final_state=False, lib=lib, **kw)
        o_p, A = oracle.parallel(q, k, v, scale=0.45, lib=lib, **kw)
        if _rel(o_p, o_r) > TIGHT:
            return False
        vq = np.repeat(v, H // Hkv, axis=2)                     # kv head of each query head
        if _rel(np.einsum("bhij,bjhv->bihv", A, vq), o_p) > TIGHT:
            return False
    return True


def pin_parallel_special_gates(lib, seed=20, T=37, H=2, K=4, V=3):
    """Closed forms of the attention matrix: g = 0 gives scale * tril(Q K^T)
    (causal linear attention); g -> -inf leaves only the diagonal
    scale * q_i . k_i.  Entries above the diagonal are exactly zero."""
    rng = np.random.default_rng(seed)
    q, k, v = _rand(rng, 1, T, H, K), _rand(rng, 1, T, H, K), _rand(rng, 1, T, H, V)
    _, A0 = oracle.parallel(q, k, v, g=np.zeros((1, T, H)), scale=0.8, lib=lib)
    _, Af = oracle.parallel(q, k, v, g=np.full((1, T, H), -1e4), scale=0.8, lib=lib)
    for h in range(H):
        qk = q[0, :, h] @ k[0, :, h].T
        if _rel(A0[0, h], 0.8 * np.tril(qk)) > TIGHT:
            return False
        if _rel(Af[0, h], 0.8 * np.diag(np.diag(qk))) > TIGHT:
            return False
        if np.any(np.triu(A0[0, h], 1) != 0):
            return False
    return True


ALL_PINS = [pin_chunk_local_cumsum, pin_hand_example, pin_brute_force, pin_zero_gate, pin_full_forget,
            pin_split_sequence, pin_varlen_equals_per_sequence, pin_chunk_form,
            pin_gamma_is_broadcast_g, pin_retnet_closed_form, pin_invariants,
            pin_prefill_then_decode, pin_step_brute_force, pin_gqa_is_repeated_mha,
            pin_step_variants, pin_bwd_finite_differences, pin_bwd_gate_identity,
            pin_state_v_first, pin_normalizer, pin_gla_scalar_gate_is_simple_gla,
            pin_gla_brute_force, pin_parallel_equals_recurrence, pin_parallel_special_gates,
            pin_bwd_gqa_finite_differences]


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    assert pin(oracle.load())


@pytest.mark.parametrize("normalizer", [0.1, 1.0, 10.0])
@pytest.mark.parametrize("scale", [0.1, 1.0])
def test_brute_force_axes(normalizer, scale):
    """Section 五's axes: scale in {0.1, 1} and gate normaliser in {0.1, 1, 10}."""
    assert pin_brute_force(oracle.load(), seed=11, T=64, H=2, K=8, V=8, scale=scale,
                           normalizer=normalizer)


def test_bf16_inputs_are_read_exactly():
    """The oracle consumes the rounded bf16 values exactly (upcast is exact)."""
    rng = np.random.default_rng(12)
    x = rng.standard_normal(1000).astype(np.float32)
    r = round_to_bf16(x)
    bits = r.view(np.uint32)
    assert np.all(bits & 0xFFFF == 0)
    # round-to-nearest: error within half a bf16 ulp (2^-8 relative for the 8-bit significand)
    assert np.all(np.abs(r - x) <= np.abs(x) * 2.0 ** -8)


def test_retnet_gamma_values():
    """log(1 - 2^(-5 - 5h/H)) for H = 16: h = 0 gives log(31/32)."""
    gam = retnet_gamma(16).astype(np.float64)
    assert abs(gam[0] - np.log(31.0 / 32.0)) < 1e-7
    assert abs(gam[15] - np.log1p(-2.0 ** (-5.0 - 75.0 / 16.0))) < 1e-9
    assert np.all(np.diff(gam) > 0)


MUTANTS = {
    1: "gate applied after the outer product is added",
    2: "output read from the state before the update",
    3: "initial state taken from the wrong head",
    4: "per-token gate indexed as [H, T] instead of [T, H]",
    5: "scale dropped from the output",
    6: "output contracts the state with k instead of q",
    7: "decode step forms v k^T instead of k v^T",
    8: "query head h reads kv head h % Hkv (interleaved) instead of h // (H / Hkv)",
    9: "decode step reads g_gamma by sequence instead of by head",
    10: "backward: state gradient not decayed between tokens",
    11: "backward: gate gradient pairs with the state after the token",
    12: "backward: k and v gradients miss the token's own output term",
    13: "elementwise GLA: interleaved kv grouping",
    14: "elementwise GLA: gate indexed by the value column instead of the key",
    15: "parallel form: strictly causal mask (the token's own term dropped)",
    16: "parallel form: the key token's own gate counted in the decay",
}


@pytest.mark.parametrize("mutant", sorted(MUTANTS), ids=lambda m: f"mutant{m}")
def test_planted_mistakes_are_caught(mutant, tmp_path):
    """Each plausible mistake planted in a copy of the oracle fails at least
    one pin, so the pins above really constrain the oracle."""
    path = oracle.build(str(tmp_path / f"liboracle_m{mutant}.so"), mutant=mutant)
    lib = oracle.load(path)
    failed = []
    for pin in ALL_PINS:
        try:
            ok = pin(lib)
        except Exception:
            ok = False
        if not ok:
            failed.append(pin.__name__)
    assert failed, f"no pin caught mutant {mutant}: {MUTANTS[mutant]}"
