"""CPU tests of the C ABI boundary (no GPU needed).

libsgla.so is loaded and checked to export every function include/sgla.h
declares.  Argument validation runs on the host before anything is enqueued,
so every error path can be exercised here: the calls below pass HOST buffers
in place of device pointers and confirm both the status code and that not a
byte of any buffer changed (section 二 of page "flash-linear-attention 中的
Simple GLA": g xor g_gamma, B == 1 with cu_seqlens, one initial state per
sequence, chunk_size a power of two; no silent fallback)."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sgla.h")

OK, INVALID, SHAPE, DTYPE, UNSUPPORTED, WORKSPACE, HIP = range(7)
BF16, F32 = 1, 2


@pytest.fixture(scope="module")
def G():
    import gated_linear_attention_amd as G
    return G


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sgla_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_entry_points():
    names = declared_functions()
    for n in ("sgla_chunk_fwd", "sgla_recurrent_step", "sgla_chunk_fwd_workspace_size",
              "sgla_chunk_bwd", "sgla_chunk_bwd_workspace_size",
              "sgla_chunk_local_cumsum", "sgla_last_error", "sgla_abi_version", "sgla_parallel_fwd"):
        assert n in names


def test_library_exports_every_declared_symbol(G):
    out = subprocess.run(["nm", "-D", "--defined-only", G.library_path()], capture_output=True,
                         text=True, check=True).stdout
    exported = set(line.split()[-1] for line in out.splitlines() if line.strip())
    missing = [n for n in declared_functions() if n not in exported]
    assert not missing, f"declared but not exported: {missing}"
    for n in declared_functions():
        assert hasattr(G.lib, n)


def test_single_hip_runtime_in_process(G):
    maps = open("/proc/self/maps").read()
    libs = {l.split()[-1] for l in maps.splitlines() if "libamdhip64" in l}
    assert len(libs) == 1, libs


def test_abi_version(G):
    assert G.lib.sgla_abi_version() == G.ABI_VERSION == 5


class Buffers:
    """Host buffers standing in for device pointers; snapshot() / unchanged()
    detect any write."""

    def __init__(self, B=1, T=128, H=2, K=64, V=64, N=None):
        N = B if N is None else N
        rng = np.random.default_rng(0)
        self.arrs = {}
        for name, shape, dt in [("q", (B, T, H, K), np.uint16), ("k", (B, T, H, K), np.uint16),
                                ("v", (B, T, H, V), np.uint16), ("g", (B, T, H), np.float32),
                                ("gg", (H,), np.float32), ("h0", (N, H, K, V), np.float32),
                                ("o", (B, T, H, V), np.float32), ("ht", (N, H, K, V), np.float32),
                                ("do", (B, T, H, V), np.uint16), ("dq", (B, T, H, K), np.float32),
                                ("dk", (B, T, H, K), np.float32), ("dv", (B, T, H, V), np.float32),
                                ("dg", (B, T, H), np.float32), ("dgg", (H,), np.float32),
                                ("dh0", (N, H, K, V), np.float32),
                                ("ws", (1 << 22,), np.uint8)]:
            n = int(np.prod(shape)) * np.dtype(dt).itemsize
            raw = rng.integers(0, 255, size=n + 256, dtype=np.uint8)
            off = (-raw.ctypes.data) % 256          # 256-byte aligned view, like device memory
            self.arrs[name] = raw[off:off + n]
        self.snap = {k: a.copy() for k, a in self.arrs.items()}

    def p(self, name, offset=0):
        return ctypes.c_void_p(self.arrs[name].ctypes.data + offset)

    def unchanged(self):
        return all(np.array_equal(self.arrs[k], self.snap[k]) for k in self.arrs)


def chunk_call(G, args, b, cu=None, g=True, gg=False, h0=True, ht=True, ws_bytes=1 << 20,
               ht_ptr=None, **ptr_override):
    cu_arr = None if cu is None else np.asarray(cu, dtype=np.int64)
    ptrs = dict(q=b.p("q"), k=b.p("k"), v=b.p("v"), g=b.p("g") if g else None,
                gg=b.p("gg") if gg else None, h0=b.p("h0") if h0 else None,
                o=b.p("o"), ht=b.p("ht") if ht else None, ws=b.p("ws"))
    ptrs.update(ptr_override)
    if ht_ptr is not None:
        ptrs["ht"] = ht_ptr
    st = G.lib.sgla_chunk_fwd(
        None if args is None else ctypes.byref(args), ptrs["q"], ptrs["k"], ptrs["v"], ptrs["g"],
        ptrs["gg"], ptrs["h0"],
        None if cu_arr is None else ctypes.c_void_p(cu_arr.ctypes.data),
        ptrs["o"], ptrs["ht"], ptrs["ws"], ws_bytes, None)
    return st, G.lib.sgla_last_error().decode()


def mkargs(G, B=1, T=128, H=2, K=64, V=64, N=1, chunk=64, qkv=BF16, od=F32, scale=0.125, fs=1,
           Hkv=0):
    return G._ChunkArgs(B, T, H, K, V, N, chunk, qkv, od, scale, fs, Hkv, 0)


CASES = [
    # (description, args overrides, call overrides, expected status, message fragment)
    ("null args", None, {}, INVALID, "args"),
    ("both gates", {}, dict(gg=True), INVALID, "mutually exclusive"),
    ("B != 1 with cu_seqlens", dict(B=2, N=2), dict(cu=[0, 64, 128]), SHAPE, "B == 1"),
    ("cu not from 0", dict(N=2), dict(cu=[1, 64, 128]), SHAPE, "cu_seqlens[0]"),
    ("cu decreasing", dict(N=2), dict(cu=[0, 100, 90]), SHAPE, "non-decreasing"),
    ("cu not ending at T", dict(N=2), dict(cu=[0, 64, 127]), SHAPE, "equal T"),
    ("chunk not power of 2", dict(chunk=48), {}, UNSUPPORTED, "power of two"),
    ("chunk 8 unsupported", dict(chunk=8), {}, UNSUPPORTED, "16, 32 or 64"),
    ("chunk 128 unsupported", dict(chunk=128), {}, UNSUPPORTED, "at most 64"),
    ("bf16 K=96", dict(K=96), {}, UNSUPPORTED, "K in"),
    ("bf16 V=96", dict(V=96), {}, UNSUPPORTED, "V a multiple"),
    ("bf16 K=512 V=48", dict(K=512, V=48), {}, UNSUPPORTED, "V a multiple"),
    ("f32 K=256", dict(qkv=F32, K=256), {}, UNSUPPORTED, "K in"),
    ("f32 V=48", dict(qkv=F32, V=48), {}, UNSUPPORTED, "V a multiple"),
    ("fp16 inputs", dict(qkv=3), {}, DTYPE, "qkv_dtype"),
    ("bad o dtype", dict(od=0), {}, DTYPE, "o_dtype"),
    ("nan scale", dict(scale=float("nan")), {}, INVALID, "scale"),
    ("inf scale", dict(scale=float("inf")), {}, INVALID, "scale"),
    ("H = 0", dict(H=0), {}, SHAPE, "H must"),
    ("negative T", dict(T=-1), {}, SHAPE, ">= 0"),
    ("NULL q", {}, dict(q=None), INVALID, "non-NULL"),
    ("final requested, NULL", {}, dict(ht=False), INVALID, "final_state is NULL"),
    ("workspace small", dict(N=2), dict(cu=[0, 64, 128], ws_bytes=16), WORKSPACE, "workspace"),
    ("workspace NULL", dict(N=2), dict(cu=[0, 64, 128], ws=None), WORKSPACE, "workspace"),
    ("misaligned q", {}, dict(q="misaligned"), INVALID, "aligned"),
    ("partial state overlap", {}, dict(ht="overlap"), INVALID, "overlap"),
    ("num_seqs 0 with cu", dict(N=0), dict(cu=[0]), SHAPE, "num_seqs"),
    ("num_kv_heads not dividing H", dict(H=2, Hkv=3), {}, SHAPE, "num_kv_heads"),
    ("negative num_kv_heads", dict(Hkv=-1), {}, SHAPE, "num_kv_heads"),
]


@pytest.mark.parametrize("desc,aover,cover,status,frag", CASES, ids=[c[0] for c in CASES])
def test_chunk_fwd_rejects_without_writing(G, desc, aover, cover, status, frag):
    # state buffers sized for the case's sequence count, so no check sees
    # two unrelated host buffers as overlapping states
    b = Buffers(N=max(1, (aover or {}).get("N", 1)))
    args = None if aover is None else mkargs(G, **aover)
    cover = dict(cover)
    kw = {}
    if cover.pop("gg", False):
        kw["gg"] = True
    if "ht" in cover and cover["ht"] is False:
        kw["ht"] = False
        cover.pop("ht")
    if cover.get("q") == "misaligned":
        cover["q"] = b.p("q", 2)
    if cover.get("ht") == "overlap":
        cover.pop("ht")
        kw["ht_ptr"] = b.p("h0", 256)
    for key in ("cu", "ws_bytes"):
        if key in cover:
            kw[key] = cover.pop(key)
    st, msg = chunk_call(G, args, b, **kw, **cover)
    assert st == status, (st, msg)
    assert frag in msg, msg
    assert b.unchanged()


def test_workspace_size(G):
    """Dense input needs no workspace; packed input needs room for the
    sequence and chunk tables (256-byte aligned pieces)."""
    a = mkargs(G, B=2, T=100, H=3)
    assert G.lib.sgla_chunk_fwd_workspace_size(ctypes.byref(a), None) == 0
    assert G.lib.sgla_last_error() == b""
    cu = np.array([0, 15, 100, 300], dtype=np.int64)
    a = mkargs(G, B=1, T=300, H=3, N=3)
    n2 = G.lib.sgla_chunk_fwd_workspace_size(ctypes.byref(a), ctypes.c_void_p(cu.ctypes.data))
    assert n2 >= 3 * 16 + 6 * 8 and n2 % 256 == 0
    bad = mkargs(G, K=96)
    assert G.lib.sgla_chunk_fwd_workspace_size(ctypes.byref(bad), None) == 0
    assert "K in" in G.lib.sgla_last_error().decode()


def test_normalizer_and_gla_workspace_size(G):
    """Normalizer: the tables, then per (chunk, head) K floats of z records and
    one float of log2 decay, each piece 256-byte aligned.  Elementwise-gate
    GLA: the tables, then per (chunk, head) a 64 x 64 float32 A (fp32 chain:
    float32 inputs, K < 64 or V not a multiple of 64) or bf16 hi/lo planes of
    q~, k~ (64 x K each) and A plus K floats of decay (bf16 chain)."""
    al = lambda x: (x + 255) // 256 * 256
    a = mkargs(G, B=2, T=100, H=3, K=64)
    tasks = 2 * 2 * 3
    assert G.lib.sgla_chunk_normalizer_workspace_size(ctypes.byref(a), None) == al(tasks * 64 * 4) + al(tasks * 4)
    bf16_chain = lambda K: 4 * 64 * K * 2 + 2 * 64 * 64 * 2 + K * 4
    assert G.lib.sgla_gla_chunk_fwd_workspace_size(ctypes.byref(a), None) == tasks * bf16_chain(64)
    for over in (dict(qkv=F32), dict(V=96), dict(K=32)):
        af = mkargs(G, **dict(dict(B=2, T=100, H=3, K=64), **over))
        assert G.lib.sgla_gla_chunk_fwd_workspace_size(ctypes.byref(af), None) == tasks * 64 * 64 * 4, over
    a0 = mkargs(G, B=2, T=0, H=3)
    assert G.lib.sgla_chunk_normalizer_workspace_size(ctypes.byref(a0), None) == 0
    assert G.lib.sgla_gla_chunk_fwd_workspace_size(ctypes.byref(a0), None) == 0
    cu = np.array([0, 15, 100, 300], dtype=np.int64)
    a = mkargs(G, B=1, T=300, H=3, N=3, K=128)
    cup = ctypes.c_void_p(cu.ctypes.data)
    tables = G.lib.sgla_chunk_fwd_workspace_size(ctypes.byref(a), cup)
    assert tables > 0
    tasks = (1 + 2 + 4) * 3
    assert G.lib.sgla_gla_chunk_fwd_workspace_size(ctypes.byref(a), cup) == tables + tasks * bf16_chain(128)
    assert G.lib.sgla_chunk_normalizer_workspace_size(ctypes.byref(a), cup) == \
        tables + al(tasks * 128 * 4) + al(tasks * 4)


def test_workspace_size_wide_keys(G):
    """bf16 K = 512: per (chunk, query head) 768 bytes of gates, 16 KiB of
    A and K * 128 bytes of Q; per (chunk, kv head) K * 128 bytes of K^T."""
    for H, Hkv in ((4, 4), (4, 2), (4, 1)):
        a = mkargs(G, B=2, T=130, H=H, K=512, V=64, Hkv=Hkv)
        n = G.lib.sgla_chunk_fwd_workspace_size(ctypes.byref(a), None)
        chunks = 2 * 3
        assert n == chunks * H * (768 + 16384 + 512 * 128) + chunks * Hkv * 512 * 128


STEP_CASES = [
    ("V=48", dict(V=48), UNSUPPORTED, "V in"),
    ("both gates", dict(gg="gg"), INVALID, "mutually exclusive"),
    ("num_kv_heads not dividing H", dict(Hkv=3), SHAPE, "num_kv_heads"),
    ("null k", dict(k=None), INVALID, "non-NULL"),
    ("[V, K] state with K=100", dict(vf=1, K=100), UNSUPPORTED, "[V, K]"),
    ("[V, K] state with V=48", dict(vf=1, V=48), UNSUPPORTED, "[V, K]"),
    ("K=0", dict(K=0), UNSUPPORTED, "K <="),
    ("K=2048", dict(K=2048), UNSUPPORTED, "K <="),
    ("H=0", dict(H=0), SHAPE, "H > 0"),
    ("fp16", dict(qkv=3), DTYPE, "qkv_dtype"),
    ("o dtype", dict(od=9), DTYPE, "o_dtype"),
    ("nan scale", dict(scale=float("nan")), INVALID, "scale"),
    ("o aliases state", dict(o="state"), INVALID, "alias"),
    ("misaligned state", dict(state="misaligned"), INVALID, "aligned"),
]


@pytest.mark.parametrize("desc,over,status,frag", STEP_CASES, ids=[c[0] for c in STEP_CASES])
def test_recurrent_step_rejects_without_writing(G, desc, over, status, frag):
    b = Buffers(B=1, T=4, H=2, K=64, V=64, N=4)
    kw = dict(N=4, H=2, Hkv=0, K=64, V=64, scale=0.125, qkv=BF16, od=F32, vf=0, q=b.p("q"),
              k=b.p("k"), v=b.p("v"), g=b.p("g"), gg=None, state=b.p("h0"), o=b.p("o"))
    for key, val in over.items():
        if val == "state":
            val = b.p("h0", 64)
        elif val == "misaligned":
            val = b.p("h0", 4)
        elif val == "gg":
            val = b.p("gg")
        kw[key] = val
    st = G.lib.sgla_recurrent_step(kw["N"], kw["H"], kw["Hkv"], kw["K"], kw["V"], kw["scale"],
                                   kw["qkv"], kw["od"], kw["vf"], kw["q"], kw["k"], kw["v"], kw["g"],
                                   kw["gg"], kw["state"], kw["o"], None)
    msg = G.lib.sgla_last_error().decode()
    assert st == status, (st, msg)
    assert frag in msg, msg
    assert b.unchanged()


def test_binding_checks_initial_state_rows(G):
    """initial_state must have one row per sequence (len(cu_seqlens) - 1)."""
    import torch
    q = torch.zeros(1, 10, 2, 64, dtype=torch.bfloat16)
    v = torch.zeros(1, 10, 2, 64, dtype=torch.bfloat16)
    h0 = torch.zeros(3, 2, 64, 64)
    with pytest.raises(ValueError, match="initial_state"):
        G.chunk_fwd(q, q, v, initial_state=h0, cu_seqlens=[0, 4, 10])
    with pytest.raises(ValueError, match="B == 1"):
        G.chunk_fwd(torch.zeros(2, 5, 2, 64, dtype=torch.bfloat16),
                    torch.zeros(2, 5, 2, 64, dtype=torch.bfloat16),
                    torch.zeros(2, 5, 2, 64, dtype=torch.bfloat16), cu_seqlens=[0, 4, 10])
    with pytest.raises(ValueError, match="mutually exclusive"):
        G.chunk_fwd(q, q, v, g=torch.zeros(1, 10, 2), g_gamma=torch.zeros(2))
    with pytest.raises(ValueError, match="float16|bfloat16"):
        G.chunk_fwd(q.half(), q.half(), v.half())
    q4 = torch.zeros(1, 10, 4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="must divide"):
        G.chunk_fwd(q4, torch.zeros(1, 10, 3, 64, dtype=torch.bfloat16),
                    torch.zeros(1, 10, 3, 64, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="shape"):
        G.chunk_fwd(q4, torch.zeros(1, 10, 2, 64, dtype=torch.bfloat16),
                    torch.zeros(1, 10, 1, 64, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="must divide"):
        G.recurrent_step(torch.zeros(2, 4, 64), torch.zeros(2, 3, 64), torch.zeros(2, 3, 64),
                         None, torch.zeros(2, 4, 64, 64))
    with pytest.raises(ValueError, match="mutually exclusive"):
        G.recurrent_step(torch.zeros(2, 4, 64), torch.zeros(2, 2, 64), torch.zeros(2, 2, 64),
                         torch.zeros(2, 4), torch.zeros(2, 4, 64, 64), g_gamma=torch.zeros(4))


def bwd_call(G, args, b, cu=None, g=True, gg=False, dg=True, dgg=False, ws_bytes=1 << 22, **over):
    cu_arr = None if cu is None else np.asarray(cu, dtype=np.int64)
    ptrs = dict(q=b.p("q"), k=b.p("k"), v=b.p("v"), g=b.p("g") if g else None,
                gg=b.p("gg") if gg else None, h0=b.p("h0"), do=b.p("do"), dht=b.p("ht"),
                dq=b.p("dq"), dk=b.p("dk"), dv=b.p("dv"), dg=b.p("dg") if dg else None,
                dgg=b.p("dgg") if dgg else None, dh0=b.p("dh0"), ws=b.p("ws"))
    ptrs.update(over)
    st = G.lib.sgla_chunk_bwd(
        ctypes.byref(args), ptrs["q"], ptrs["k"], ptrs["v"], ptrs["g"], ptrs["gg"], ptrs["h0"],
        None if cu_arr is None else ctypes.c_void_p(cu_arr.ctypes.data), ptrs["do"], ptrs["dht"],
        ptrs["dq"], ptrs["dk"], ptrs["dv"], ptrs["dg"], ptrs["dgg"], ptrs["dh0"], ptrs["ws"],
        ws_bytes, None)
    return st, G.lib.sgla_last_error().decode()


BWD_CASES = [
    ("K=384", dict(K=384), {}, UNSUPPORTED, "K in"),
    ("V=48", dict(V=48), {}, UNSUPPORTED, "V a multiple"),
    ("f32 K=256", dict(qkv=F32, K=256), {}, UNSUPPORTED, "bf16 inputs only"),
    ("K=512 V=96", dict(K=512, V=96), {}, UNSUPPORTED, "multiple of 64"),
    ("fp16", dict(qkv=3), {}, DTYPE, "qkv_dtype"),
    ("both gates", {}, dict(gg=True), INVALID, "mutually exclusive"),
    ("g without dg", {}, dict(dg=False), INVALID, "dg is NULL"),
    ("g_gamma without dg_gamma", {}, dict(g=False, gg=True), INVALID, "dg_gamma is NULL"),
    ("NULL dout", {}, dict(do=None), INVALID, "non-NULL"),
    ("chunk 128", dict(chunk=128), {}, UNSUPPORTED, "chunk_size"),
    ("chunk 48", dict(chunk=48), {}, UNSUPPORTED, "power of two"),
    ("cu not ending at T", dict(N=2), dict(cu=[0, 64, 100]), SHAPE, "equal T"),
    ("workspace small", dict(N=2), dict(cu=[0, 64, 128], ws_bytes=64), WORKSPACE, "workspace"),
    ("nan scale", dict(scale=float("nan")), {}, INVALID, "scale"),
]


@pytest.mark.parametrize("desc,aover,cover,status,frag", BWD_CASES, ids=[c[0] for c in BWD_CASES])
def test_chunk_bwd_rejects_without_writing(G, desc, aover, cover, status, frag):
    b = Buffers()
    args = mkargs(G, **aover)
    st, msg = bwd_call(G, args, b, **cover)
    assert st == status, (st, msg)
    assert frag in msg, msg
    assert b.unchanged()


def test_chunk_bwd_workspace_size_wide(G):
    """K > 128 adds one gate record of 132 floats per (chunk, head, 128-key
    tile) after the per-chunk gate sums."""
    def align(n):
        return (n + 255) // 256 * 256
    for K in (256, 512):
        a = mkargs(G, B=2, T=130, H=4, K=K, V=64)
        tasks = 2 * 3 * 4
        rec = tasks * K * 64 * 4
        want = 2 * align(rec) + align(tasks * 4) + align(tasks * (K // 128) * 132 * 4)
        assert G.lib.sgla_chunk_bwd_workspace_size(ctypes.byref(a), None) == want, K


def test_chunk_bwd_workspace_size_grouped(G):
    """Grouped kv heads add the per-query-head k and v gradients (4 (K + V)
    bytes per token and query head) after the records."""
    a1 = mkargs(G, B=2, T=130, H=4, K=64, V=96)
    a2 = mkargs(G, B=2, T=130, H=4, K=64, V=96, Hkv=2)
    n1 = G.lib.sgla_chunk_bwd_workspace_size(ctypes.byref(a1), None)
    n2 = G.lib.sgla_chunk_bwd_workspace_size(ctypes.byref(a2), None)
    th = 2 * 130 * 4
    up = lambda x: (x + 255) // 256 * 256
    assert n2 == n1 + up(th * 64 * 4) + up(th * 96 * 4)


def test_chunk_bwd_workspace_size(G):
    """Two fp32 K x V records per (chunk, head) plus 4 bytes per (chunk, head)."""
    a = mkargs(G, B=2, T=130, H=3, K=64, V=96)
    n = G.lib.sgla_chunk_bwd_workspace_size(ctypes.byref(a), None)
    tasks = 2 * 3 * 3
    rec = tasks * 64 * 96 * 4
    assert n == 2 * rec + ((tasks * 4 + 255) // 256) * 256


@pytest.mark.parametrize("chunk", [16, 32])
def test_chunk_bwd_workspace_size_small_chunks(G, chunk):
    """At chunk_size 16 or 32 the backward's records follow the requested
    chunk grid: one pair per chunk of that size (dense and packed)."""
    up = lambda x: (x + 255) // 256 * 256
    a = mkargs(G, B=2, T=130, H=3, K=64, V=96, chunk=chunk)
    tasks = 2 * ((130 + chunk - 1) // chunk) * 3
    assert G.lib.sgla_chunk_bwd_workspace_size(ctypes.byref(a), None) == \
        2 * up(tasks * 64 * 96 * 4) + up(tasks * 4)
    cu = np.array([0, 15, 100, 300], dtype=np.int64)
    a = mkargs(G, B=1, T=300, H=3, N=3, K=64, V=96, chunk=chunk)
    nch = sum((int(cu[i + 1] - cu[i]) + chunk - 1) // chunk for i in range(3))
    tables = up(3 * 16) + up(nch * 8)
    assert G.lib.sgla_chunk_bwd_workspace_size(ctypes.byref(a), ctypes.c_void_p(cu.ctypes.data)) == \
        tables + 2 * up(nch * 3 * 64 * 96 * 4) + up(nch * 3 * 4)


@pytest.mark.parametrize("chunk", [16, 32])
def test_normalizer_and_gla_workspace_size_small_chunks(G, chunk):
    """At chunk_size 16 or 32 the normalizer's and the elementwise-gate GLA's
    per-chunk records follow the requested chunk grid (one record per chunk
    of that size, each still a 64-row tile's worth)."""
    al = lambda x: (x + 255) // 256 * 256
    a = mkargs(G, B=2, T=100, H=3, K=64, chunk=chunk)
    tasks = 2 * ((100 + chunk - 1) // chunk) * 3
    assert G.lib.sgla_chunk_normalizer_workspace_size(ctypes.byref(a), None) == al(tasks * 64 * 4) + al(tasks * 4)
    bf16_chain = lambda K: 4 * 64 * K * 2 + 2 * 64 * 64 * 2 + K * 4
    assert G.lib.sgla_gla_chunk_fwd_workspace_size(ctypes.byref(a), None) == tasks * bf16_chain(64)
    af = mkargs(G, B=2, T=100, H=3, K=64, qkv=F32, chunk=chunk)
    assert G.lib.sgla_gla_chunk_fwd_workspace_size(ctypes.byref(af), None) == tasks * 64 * 64 * 4


NORM_CASES = [
    ("chunk 128", dict(chunk=128), {}, UNSUPPORTED, "chunk_size"),
    ("chunk 24", dict(chunk=24), {}, UNSUPPORTED, "power of two"),
    ("K=512", dict(K=512), {}, UNSUPPORTED, "K in"),
    ("K=48", dict(K=48), {}, UNSUPPORTED, "K in"),
    ("both gates", {}, dict(gg=True), INVALID, "mutually exclusive"),
    ("fp16", dict(qkv=3), {}, DTYPE, "qkv_dtype"),
    ("kv heads not dividing", dict(H=2, Hkv=3), {}, SHAPE, "num_kv_heads"),
    ("final without pointer", {}, dict(zt=None), INVALID, "final_z is NULL"),
    ("workspace small", dict(N=2), dict(cu=[0, 64, 128], ws_bytes=8), WORKSPACE, "workspace"),
    ("dense workspace small", {}, dict(ws_bytes=8), WORKSPACE, "workspace"),
]


@pytest.mark.parametrize("desc,aover,cover,status,frag", NORM_CASES, ids=[c[0] for c in NORM_CASES])
def test_chunk_normalizer_rejects_without_writing(G, desc, aover, cover, status, frag):
    b = Buffers()
    args = mkargs(G, **aover)
    cu = cover.get("cu")
    cu_arr = None if cu is None else np.asarray(cu, dtype=np.int64)
    ptrs = dict(q=b.p("q"), k=b.p("k"), g=b.p("g"), gg=b.p("gg") if cover.get("gg") else None,
                z0=b.p("h0"), den=b.p("dg"), zt=b.p("ht"), ws=b.p("ws"))
    if "zt" in cover:
        ptrs["zt"] = cover["zt"]
    st = G.lib.sgla_chunk_normalizer(
        ctypes.byref(args), ptrs["q"], ptrs["k"], ptrs["g"], ptrs["gg"], ptrs["z0"],
        None if cu_arr is None else ctypes.c_void_p(cu_arr.ctypes.data), ptrs["den"], ptrs["zt"],
        ptrs["ws"], cover.get("ws_bytes", 1 << 22), None)
    msg = G.lib.sgla_last_error().decode()
    assert st == status, (st, msg)
    assert frag in msg, msg
    assert b.unchanged()


def test_step_normalizer_rejects_without_writing(G):
    b = Buffers(B=1, T=4, H=2, K=64, V=64, N=4)
    cases = [(dict(K=0), UNSUPPORTED), (dict(K=5000), UNSUPPORTED), (dict(qkv=3), DTYPE),
             (dict(gg="gg"), INVALID), (dict(Hkv=3), SHAPE), (dict(z=None), INVALID)]
    for over, status in cases:
        kw = dict(N=4, H=2, Hkv=0, K=64, scale=0.125, qkv=BF16, q=b.p("q"), k=b.p("k"), g=b.p("g"),
                  gg=None, z=b.p("h0"), den=b.p("dg"))
        for key, val in over.items():
            kw[key] = b.p("gg") if val == "gg" else val
        st = G.lib.sgla_recurrent_step_normalizer(kw["N"], kw["H"], kw["Hkv"], kw["K"], kw["scale"],
                                                  kw["qkv"], kw["q"], kw["k"], kw["g"], kw["gg"],
                                                  kw["z"], kw["den"], None)
        assert st == status, (over, st, G.lib.sgla_last_error())
        assert b.unchanged()


def test_gate_cumsum_chunk_sizes(G):
    """The standalone gate cumsum takes any power-of-two chunk size up to 64;
    larger sizes and non-powers of two are unsupported; the chunked forward
    takes 16, 32 and 64 (the case list above)."""
    b = Buffers()
    for chunk, status, frag in ((128, UNSUPPORTED, "at most 64"), (48, UNSUPPORTED, "power of two")):
        a = mkargs(G, chunk=chunk)
        st = G.lib.sgla_chunk_local_cumsum(ctypes.byref(a), b.p("g"), None, b.p("dg"), None, 0, None)
        assert st == status and frag in G.lib.sgla_last_error().decode()
    assert b.unchanged()
    cu = np.array([0, 15, 100, 300], dtype=np.int64)
    for chunk in (1, 16, 32, 64):
        a = mkargs(G, B=1, T=300, H=3, N=3, chunk=chunk)
        assert G.lib.sgla_chunk_fwd_workspace_size(ctypes.byref(a), ctypes.c_void_p(cu.ctypes.data)) > 0


PAR_CASES = [
    ("null args", None, {}, INVALID, "args"),
    ("K=96", dict(K=96), {}, UNSUPPORTED, "K in"),
    ("K=512", dict(K=512), {}, UNSUPPORTED, "K in"),
    ("V=24", dict(V=24), {}, UNSUPPORTED, "V a multiple"),
    ("V=272", dict(V=272), {}, UNSUPPORTED, "V a multiple"),
    ("float32 K=40", dict(qkv=F32, K=40), {}, UNSUPPORTED, "float32 inputs"),
    ("float32 K=272", dict(qkv=F32, K=272), {}, UNSUPPORTED, "float32 inputs"),
    ("float32 V=8", dict(qkv=F32, V=8), {}, UNSUPPORTED, "float32 inputs"),
    ("bf16 K=96", dict(K=96), {}, UNSUPPORTED, "bf16 inputs"),
    ("fp16", dict(qkv=3), {}, DTYPE, "qkv_dtype"),
    ("o dtype", dict(od=3), {}, DTYPE, "o_dtype"),
    ("both gates", {}, dict(gg=True), INVALID, "mutually exclusive"),
    ("kv heads not dividing", dict(H=2, Hkv=3), {}, SHAPE, "num_kv_heads"),
    ("negative T", dict(T=-1), {}, SHAPE, "B and T"),
    ("o NULL", {}, dict(o=None), INVALID, "non-NULL"),
    ("attn misaligned", {}, dict(attn_off=4), INVALID, "aligned"),
    ("A rows past 32-bit offsets", dict(T=(1 << 22) + 64), {}, UNSUPPORTED, "T <= 4194304"),
]


@pytest.mark.parametrize("desc,aover,cover,status,frag", PAR_CASES, ids=[c[0] for c in PAR_CASES])
def test_parallel_fwd_rejects_without_writing(G, desc, aover, cover, status, frag):
    b = Buffers()
    args = None if aover is None else ctypes.byref(mkargs(G, **aover))
    o = cover.get("o", b.p("o"))
    attn = ctypes.c_void_p(b.p("ht").value + cover.get("attn_off", 0))
    st = G.lib.sgla_parallel_fwd(args, b.p("q"), b.p("k"), b.p("v"), b.p("g"),
                                 b.p("gg") if cover.get("gg") else None, o, attn, None)
    msg = G.lib.sgla_last_error().decode()
    assert st == status, (st, msg)
    assert frag in msg, msg
    assert b.unchanged()


def test_parallel_fwd_empty_is_ok(G):
    """No tokens (or no batch rows) is a valid call that launches nothing."""
    b = Buffers()
    for over in (dict(T=0), dict(B=0)):
        st = G.lib.sgla_parallel_fwd(ctypes.byref(mkargs(G, **over)), None, None, None, None, None,
                                     None, None, None)
        assert st == OK, G.lib.sgla_last_error()
    assert b.unchanged()


def test_chunk_fwd_noalloc_rejects_without_device(G):
    """sgla_chunk_fwd_noalloc validates everything on the host before it looks
    up its scratch array (no device call is made): a request needing more
    scratch than the fixed array holds and every invalid argument return
    their status with nothing written."""
    b = Buffers()
    cap = G.lib.sgla_chunk_fwd_noalloc_max_bytes()
    assert cap == 16 << 20
    # bf16 K = 512, 5120 tokens x 2 heads: ~24 MB of preparation records
    a = mkargs(G, B=1, T=64 * 80, H=2, K=512, V=64)
    assert G.lib.sgla_chunk_fwd_workspace_size(ctypes.byref(a), None) > cap
    st = G.lib.sgla_chunk_fwd_noalloc(ctypes.byref(a), b.p("q"), b.p("k"), b.p("v"), b.p("g"), None,
                                      None, None, b.p("o"), b.p("ht"), None)
    assert st == WORKSPACE and "scratch" in G.lib.sgla_last_error().decode()
    cu = np.array([0, 64, 128], dtype=np.int64)
    cases = [(mkargs(G, N=2), dict(gg=b.p("gg")), INVALID, "mutually exclusive"),
             (mkargs(G, N=2, chunk=8), {}, UNSUPPORTED, "chunk_size"),
             (mkargs(G, N=2), dict(q=None), INVALID, "non-NULL")]
    for args, over, status, frag in cases:
        kw = dict(q=b.p("q"), gg=None)
        kw.update(over)
        st = G.lib.sgla_chunk_fwd_noalloc(ctypes.byref(args), kw["q"], b.p("k"), b.p("v"), b.p("g"), kw["gg"],
                                          b.p("h0"), ctypes.c_void_p(cu.ctypes.data), b.p("o"), b.p("ht"), None)
        msg = G.lib.sgla_last_error().decode()
        assert st == status and frag in msg, (st, msg)
    assert b.unchanged()
