"""C-ABI checks that need no GPU: the library loads, exports every declared
entry point, computes layouts, and rejects bad arguments before any HIP call."""
import ctypes as ct
import os
import re

import pytest

from tree_indexed_sparse_zha_amd import zha

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "zha.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(zha_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return zha.load()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert len(names) >= 11
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_status(lib):
    assert zha.version() == 1
    assert lib.zha_status_string(0) == b"ok"
    assert lib.zha_status_string(-4).startswith(b"capacity")


def cfg_deep(**kw):
    base = dict(batch=1, n_kv_heads=8, q_per_kv=4, head_dim=128, n_ref=16, chunk=4, levels=6, dtype="bf16", capacity=32768)
    base.update(kw)
    return zha.ZhaConfig(**base)


def test_tree_layout_sizes():
    cfg = cfg_deep()
    tl = zha.tree_layout(cfg)
    assert tl.levels == 6
    assert [tl.node_cap[i] for i in range(6)] == [8192, 2048, 512, 128, 32, 8]
    assert all(tl.g_bytes[i] == 16 * 128 * 2 for i in range(6))
    # node = R*d*2 (g) + 4R (L) + 4R (c) = 4224 bytes
    nodes = sum(tl.node_cap[i] for i in range(6)) * 8
    # plus the append scratch: fp32 children of 2 top nodes per cache
    scratch = 8 * 2 * 4 * 16 * (128 + 2) * 4
    assert tl.scratch_offset >= 0 and tl.scratch_offset % 256 == 0
    assert tl.total_bytes >= nodes * 4224 + scratch
    assert tl.total_bytes < nodes * 4224 + scratch + 7 * 3 * 256
    for i in range(6):
        assert tl.g_offset[i] % 256 == 0 and tl.L_offset[i] % 256 == 0 and tl.c_offset[i] % 256 == 0


def test_tree_layout_weights_form():
    cfg = cfg_deep(leaf_form="weights")
    tl = zha.tree_layout(cfg)
    assert tl.g_bytes[0] == 16 * 4 * 4
    assert all(tl.g_bytes[i] == 16 * 128 * 2 for i in range(1, 6))
    mean = zha.tree_layout(cfg_deep())
    assert tl.total_bytes < mean.total_bytes * 0.35


def test_tree_layout_weights2_form():
    """Level 1 holds the weights of its keys ([R][C] fp32), level 2 its
    children's mass shares ([R][C] fp32): a level-2 node shrinks from R*d*2
    to R*C*4 bytes."""
    cfg = cfg_deep(leaf_form="weights2")
    tl = zha.tree_layout(cfg)
    assert tl.g_bytes[0] == 16 * 4 * 4
    assert tl.g_bytes[1] == 16 * 4 * 4
    assert all(tl.g_bytes[i] == 16 * 128 * 2 for i in range(2, 6))
    w1 = zha.tree_layout(cfg_deep(leaf_form="weights"))
    assert [int(tl.node_cap[i]) for i in range(6)] == [int(w1.node_cap[i]) for i in range(6)]
    assert tl.total_bytes < w1.total_bytes
    # the reference queries ([H][R][d] fp32) kept for the fused level-2 pass:
    # a 256-byte aligned block inside the tree, past every level's arrays
    assert tl.ref_offset > 0 and tl.ref_offset % 256 == 0
    assert tl.ref_offset + cfg.n_kv_heads * 16 * 128 * 4 <= tl.total_bytes
    for i in range(6):
        assert tl.ref_offset >= tl.c_offset[i] + 8 * int(tl.node_cap[i]) * 16 * 4  # 8 caches
    assert w1.ref_offset == -1 and zha.tree_layout(cfg_deep()).ref_offset == -1
    # the route's key-range slots of level 2 follow its 256-key tiles (16 nodes each)
    r2, r1 = zha.route_layout(cfg, 1), zha.route_layout(cfg_deep(leaf_form="weights"), 1)
    assert r2.logits_floats == r1.logits_floats
    assert r2.workspace_min_bytes > r1.workspace_min_bytes


def test_tree_layout_fp8():
    for leaf_form in ("mean", "weights", "weights2"):
        tl = zha.tree_layout(cfg_deep(leaf_form=leaf_form, g_dtype="fp8"))
        kv = zha.tree_layout(cfg_deep(leaf_form=leaf_form))
        for i in range(6):
            weights = (leaf_form == "weights" and i == 0) or (leaf_form == "weights2" and i <= 1)
            assert tl.g_bytes[i] == (16 * 4 * 4 if weights else 16 * 128)
            assert (tl.s_offset[i] == -1) if weights else (tl.s_offset[i] % 256 == 0 and tl.s_offset[i] > tl.c_offset[i])
            assert kv.s_offset[i] == -1
        assert all(tl.s_offset[i] == -1 for i in range(6, zha.MAX_LEVELS))
        # fp8 nodes: R*d (g) + 3 * 4R (L, c, scale) bytes
        assert tl.total_bytes < kv.total_bytes


def test_tree_layout_mxfp4():
    """MXFP4 levels (>= 3 with levels 1-2 as weights): R*d/2 bytes of codes per
    node and an E8M0 scale block of R*d/32 bytes per node."""
    tl = zha.tree_layout(cfg_deep(leaf_form="weights2", g_dtype="fp4"))
    w2 = zha.tree_layout(cfg_deep(leaf_form="weights2"))
    assert tl.g_bytes[0] == tl.g_bytes[1] == 16 * 4 * 4
    assert tl.s_offset[0] == tl.s_offset[1] == -1
    for i in range(2, 6):
        assert tl.g_bytes[i] == 16 * 128 // 2
        assert tl.s_offset[i] % 256 == 0 and tl.s_offset[i] > tl.c_offset[i]
        nxt = tl.g_offset[i + 1] if i + 1 < 6 else tl.total_bytes
        assert nxt - tl.s_offset[i] >= 8 * tl.node_cap[i] * 16 * 4  # caches x nodes x R x d/32
    assert tl.total_bytes < w2.total_bytes


def test_route_layout_logits():
    assert zha.route_layout(cfg_deep(), 1).logits_floats == 0
    rl = zha.route_layout(cfg_deep(leaf_form="weights"), 1)
    # caches x ceil(QC/16) x quads x 4 keys x QW (QW = QC rounded up to 4, at most 16; QC = 4 here)
    assert rl.logits_floats == 8 * 1 * (32768 // 4) * 4 * 4
    rl = zha.route_layout(cfg_deep(leaf_form="weights"), 8)  # QC = 32: two groups of 16
    assert rl.logits_floats == 8 * 2 * (32768 // 4) * 16 * 4


def test_route_workspace_split_select():
    """Few queries over many candidates: the full workspace adds, after the
    key-range slots, one 128-byte state per query and one slot of 2,056
    64-bit words per (query, segment), segments of >= 32,768 candidates and
    at most 2,048 workgroups per level, at most 64 queries."""
    cfg = cfg_deep(capacity=1 << 20, batch=1)  # 8 caches x 4 query heads, T = 1: 32 queries
    rl = zha.route_layout(cfg, 1)
    assert rl.n_queries == 32
    S = min(2048 // 32, (1 << 18) // 32768)  # level 1: 262,144 chunks -> 8 segments
    split = 32 * 128 + 32 * S * 2056 * 8
    assert rl.workspace_bytes == rl.workspace_min_bytes + (split + 255) // 256 * 256
    assert rl.workspace_min_bytes % 256 == 0
    many = zha.route_layout(cfg, 4)  # 128 queries: one workgroup per query
    assert many.workspace_bytes == many.workspace_min_bytes


def test_route_layout_sizes():
    cfg = cfg_deep()
    rl = zha.route_layout(cfg, 64)
    assert rl.n_queries == 8 * 4 * 64
    assert rl.words[0] == 8192 // 32
    assert rl.score_floats_total == rl.n_queries * (8192 + 2048 + 512 + 128 + 32 + 8)
    assert rl.stats_total == 6 * rl.n_queries
    assert [rl.score_stride[i] for i in range(6)] == [8192, 2048, 512, 128, 32, 8]
    assert rl.workspace_min_bytes >= 6 * rl.n_queries * 16
    # 2,048 queries: every level keeps one select workgroup per query
    assert rl.workspace_bytes == rl.workspace_min_bytes
    odd = zha.route_layout(cfg_deep(capacity=32768 + 4 * 4096 * 3 + 4), 1)
    for i in range(6):
        assert odd.score_stride[i] % 4 == 0 and odd.score_stride[i] >= zha.tree_layout(cfg_deep(capacity=32768 + 4 * 4096 * 3 + 4)).node_cap[i]


@pytest.mark.parametrize(
    "kw,code",
    [
        (dict(head_dim=96), zha.ZHA_ERR_UNSUPPORTED),
        (dict(head_dim=0), zha.ZHA_ERR_ARG),
        (dict(n_ref=17), zha.ZHA_ERR_UNSUPPORTED),
        (dict(chunk=3), zha.ZHA_ERR_UNSUPPORTED),
        (dict(chunk=512, levels=1), zha.ZHA_ERR_UNSUPPORTED),
        (dict(levels=9), zha.ZHA_ERR_UNSUPPORTED),
        (dict(chunk=16, levels=7), zha.ZHA_ERR_UNSUPPORTED),  # span 2^28
        (dict(batch=0), zha.ZHA_ERR_ARG),
        (dict(capacity=0), zha.ZHA_ERR_ARG),
        (dict(dtype="f32", head_dim=64, n_ref=4, chunk=4, levels=3), 0),
        (dict(leaf_form="weights"), 0),
        (dict(leaf_form="weights", chunk=8, levels=4), 0),
        (dict(leaf_form="weights", dtype="f32"), zha.ZHA_ERR_UNSUPPORTED),
        (dict(leaf_form="weights", chunk=256, levels=1), zha.ZHA_ERR_UNSUPPORTED),
        (dict(leaf_form="weights", chunk=2, levels=6), zha.ZHA_ERR_UNSUPPORTED),
        (dict(g_dtype="fp8"), 0),
        (dict(g_dtype="fp8", leaf_form="weights"), 0),
        (dict(g_dtype="fp8", dtype="f32", head_dim=64, n_ref=4, chunk=4, levels=3), zha.ZHA_ERR_UNSUPPORTED),
        (dict(leaf_form="weights2"), 0),
        (dict(leaf_form="weights2", levels=3, n_ref=1, head_dim=64), 0),
        (dict(leaf_form="weights2", levels=2), zha.ZHA_ERR_UNSUPPORTED),
        (dict(leaf_form="weights2", chunk=8, levels=4), zha.ZHA_ERR_UNSUPPORTED),
        (dict(leaf_form="weights2", g_dtype="fp8"), 0),
        (dict(leaf_form="weights2", g_dtype="fp4"), 0),
        (dict(g_dtype="fp4"), zha.ZHA_ERR_UNSUPPORTED),
        (dict(leaf_form="weights", g_dtype="fp4"), zha.ZHA_ERR_UNSUPPORTED),
        (dict(leaf_form="weights2", g_dtype="fp4", head_dim=64), zha.ZHA_ERR_UNSUPPORTED),
        (dict(leaf_form="weights2", dtype="f32", head_dim=64, n_ref=4, levels=3), zha.ZHA_ERR_UNSUPPORTED),
    ],
)
def test_config_validation(kw, code):
    cfg = cfg_deep(**kw)
    if code == 0:
        zha.tree_layout(cfg)
        return
    with pytest.raises(zha.ZhaError) as e:
        zha.tree_layout(cfg)
    assert e.value.code == code


def _call_route(lib, cfg, **over):
    a = dict(tree=16, n_tokens=32768, Q=16, qs=zha._i64(1 << 20, 1 << 16, 1 << 12, 128), T=1, p=0.95,
             K=None, ks=None, sel=16, score=16, stats=16, ws=16, ws_bytes=0)
    a.update(over)
    c = cfg.c()
    return lib.zha_route(ct.byref(c), a["tree"], a["n_tokens"], a["Q"], a["qs"], a["T"], a["p"], a["K"], a["ks"], a["sel"],
                         a["score"], a["stats"], a.get("logits"), a["ws"], a["ws_bytes"], a.get("prof"), None)


def _call_route_levels(lib, cfg, pl, top=0, **over):
    a = dict(tree=16, n_tokens=32768, Q=16, qs=zha._i64(1 << 20, 1 << 16, 1 << 12, 128), T=1,
             K=None, ks=None, sel=16, score=16, stats=16, ws=16, ws_bytes=1 << 30)
    a.update(over)
    c = cfg.c()
    arr = None if pl is None else (ct.c_float * len(pl))(*pl)
    return lib.zha_route_levels(ct.byref(c), a["tree"], a["n_tokens"], a["Q"], a["qs"], a["T"], arr, top, a["K"],
                                a["ks"], a["sel"], a["score"], a["stats"], None, a["ws"], a["ws_bytes"], None, None)


def test_route_levels_argument_errors(lib):
    cfg = cfg_deep()
    assert _call_route_levels(lib, cfg, None) == zha.ZHA_ERR_NULL
    assert b"p_levels" in lib.zha_last_error()
    assert _call_route_levels(lib, cfg, [0.9] * 5 + [0.0]) == zha.ZHA_ERR_ARG
    assert b"level 6" in lib.zha_last_error()
    assert _call_route_levels(lib, cfg, [float("nan")] + [0.9] * 5) == zha.ZHA_ERR_ARG
    assert _call_route_levels(lib, cfg, [0.9] * 6, top=7) == zha.ZHA_ERR_ARG
    assert _call_route_levels(lib, cfg, [0.9] * 6, top=-1) == zha.ZHA_ERR_ARG
    # valid schedules pass validation and reach the capacity check
    assert _call_route_levels(lib, cfg, [0.9] * 6, top=3, n_tokens=32769) == zha.ZHA_ERR_CAPACITY


def test_prefill_argument_errors(lib):
    cfg = cfg_deep()
    c = cfg.c()
    assert zha.spine_bytes(cfg, 64) > 0
    # a spine record per (state, level >= 2): states = T / C + 2
    rec = (16 * 128 * 2 + 12 * 16 + 15) // 16 * 16
    assert zha.spine_bytes(cfg, 64) >= 8 * (64 // 4 + 2) * 5 * rec
    ks = zha._i64(1 << 22, 1 << 19, 128)
    # T beyond n_tokens, NULL spine, f32 keys
    assert lib.zha_build_spine(ct.byref(c), 16, ks, 100, 200, 16, 16, None, None) == zha.ZHA_ERR_ARG
    assert lib.zha_build_spine(ct.byref(c), 16, ks, 1000, 64, 16, None, None, None) == zha.ZHA_ERR_NULL
    cf = cfg_deep(dtype="f32", head_dim=64, n_ref=4, chunk=4, levels=3).c()
    assert lib.zha_build_spine(ct.byref(cf), 16, zha._i64(1 << 20, 1 << 16, 64), 1000, 64, 16, 16, None,
                               None) == zha.ZHA_ERR_UNSUPPORTED
    qs = zha._i64(1 << 20, 1 << 16, 1 << 12, 128)
    args = (16, 16, 1000, 16, qs, 64, 0.9, None, None, 16, 16, 16, None, 16, 1 << 30, None, None)
    # missing spine with an upper level is an error before any launch
    bad = (16, None) + args[2:]
    assert lib.zha_route_prefill(ct.byref(c), *bad) == zha.ZHA_ERR_NULL
    big = (16, 16, 40) + args[3:]  # T = 64 > n_tokens = 40
    assert lib.zha_route_prefill(ct.byref(c), *big) == zha.ZHA_ERR_ARG


def test_route_argument_errors(lib):
    cfg = cfg_deep()
    # fake but aligned addresses: every case fails validation before any HIP call
    assert _call_route(lib, cfg, tree=None) == zha.ZHA_ERR_NULL
    assert _call_route(lib, cfg, Q=8) == zha.ZHA_ERR_ALIGN
    assert _call_route(lib, cfg, p=0.0) == zha.ZHA_ERR_ARG
    assert _call_route(lib, cfg, p=float("nan")) == zha.ZHA_ERR_ARG
    assert _call_route(lib, cfg, p=-0.5) == zha.ZHA_ERR_ARG
    assert _call_route(lib, cfg, T=0) == zha.ZHA_ERR_ARG
    assert _call_route(lib, cfg, T=512) == zha.ZHA_ERR_UNSUPPORTED
    assert _call_route(lib, cfg, n_tokens=32769) == zha.ZHA_ERR_CAPACITY
    assert b"n_tokens exceeds capacity" in lib.zha_last_error()
    assert _call_route(lib, cfg, qs=zha._i64(1, 1, 1, 1)) == zha.ZHA_ERR_ALIGN
    assert _call_route(lib, cfg, ws_bytes=0) == zha.ZHA_ERR_CAPACITY
    assert b"workspace" in lib.zha_last_error()
    assert _call_route(lib, cfg, ws=None, ws_bytes=1 << 20) == zha.ZHA_ERR_NULL
    # the leaf weights form scores level 1 from the keys: K is required
    cw = cfg_deep(leaf_form="weights")
    assert _call_route(lib, cw, ws_bytes=1 << 20) == zha.ZHA_ERR_NULL
    assert b"K" in lib.zha_last_error()
    assert _call_route(lib, cfg, logits=16, ws_bytes=1 << 20) == zha.ZHA_ERR_ARG
    assert _call_route(lib, cw, K=16, ks=zha._i64(0, 0, 128), logits=8, ws_bytes=1 << 20) == zha.ZHA_ERR_ALIGN
    bad = zha.Profile()
    bad.n_pairs = 40
    assert _call_route(lib, cfg, prof=ct.byref(bad)) == zha.ZHA_ERR_ARG
    bad.n_pairs = 1  # events left NULL
    assert _call_route(lib, cfg, prof=ct.byref(bad)) == zha.ZHA_ERR_NULL


def test_build_argument_errors(lib):
    cfg = cfg_deep()
    c = cfg.c()
    ks = zha._i64(8 * 32768 * 128, 32768 * 128, 128)
    assert lib.zha_build(ct.byref(c), None, ks, 100, 16, 16, None, None) == zha.ZHA_ERR_NULL
    assert lib.zha_build(ct.byref(c), 16, ks, 40000, 16, 16, None, None) == zha.ZHA_ERR_CAPACITY
    assert b"exceed capacity" in lib.zha_last_error()
    assert lib.zha_build(ct.byref(c), 16, ks, -1, 16, 16, None, None) == zha.ZHA_ERR_ARG
    assert lib.zha_build(ct.byref(c), 16, zha._i64(0, 0, 4), 10, 16, 16, None, None) == zha.ZHA_ERR_ALIGN
    assert lib.zha_append(ct.byref(c), 16, ks, 30000, 5000, 16, 16, None, None) == zha.ZHA_ERR_CAPACITY
    assert lib.zha_append(ct.byref(c), 16, ks, -4, 5, 16, 16, None, None) == zha.ZHA_ERR_ARG
    # no new complete chunk: nothing to do, succeeds without touching the GPU
    assert lib.zha_append(ct.byref(c), 16, ks, 100, 3, 16, 16, None, None) == zha.ZHA_OK


def test_attend_argument_errors(lib):
    cfg = cfg_deep()
    c = cfg.c()
    qs = zha._i64(1 << 20, 1 << 16, 1 << 12, 128)
    ks = zha._i64(8 * 32768 * 128, 32768 * 128, 128)
    ws = zha.attend_workspace_bytes(cfg, 1)
    assert ws > 0

    def call(**o):
        a = dict(Q=16, T=1, K=16, V=16, n=32768, sel=16, words=256, flags=3, out=16, ws=16, wsb=ws)
        a.update(o)
        return lib.zha_attend(ct.byref(c), a["Q"], qs, a["T"], a["K"], a["V"], ks, a["n"], a["sel"], a["words"],
                              a.get("logits"), a["flags"], a["out"], None, a["ws"], a["wsb"], None, None)

    assert call(sel=None) == zha.ZHA_ERR_NULL
    assert call(words=255) == zha.ZHA_ERR_CAPACITY
    assert call(wsb=ws - 1) == zha.ZHA_ERR_CAPACITY
    assert call(n=0) == zha.ZHA_ERR_ARG
    assert call(n=40000) == zha.ZHA_ERR_CAPACITY
    assert call(flags=16) == zha.ZHA_ERR_ARG
    assert call(flags=8 | 3, T=2, n=1) == zha.ZHA_ERR_ARG  # causal block longer than the context
    assert call(V=24) == zha.ZHA_ERR_ALIGN
    assert call(out=None) == zha.ZHA_ERR_NULL
    assert call(logits=16) == zha.ZHA_ERR_ARG  # logits need the weights form
    assert b"weights" in lib.zha_last_error()


def test_bit_helpers_roundtrip():
    import torch

    m = torch.rand(3, 77) < 0.4
    w = zha.pack_bits(m, 3)
    assert w.dtype == torch.int32 and w.shape == (3, 3)
    assert torch.equal(zha.unpack_bits(w, 77), m)


def test_attend_noalloc_rejects_oversized_configuration(lib):
    """zha_attend_noalloc checks on the host that the split-K partials fit its
    static scratch (before touching any pointer or the GPU)."""
    import torch

    cfg = zha.ZhaConfig(8, 8, 4, 128, 16, 4, 6, "bf16", 1 << 20, "weights")
    assert zha.attend_workspace_bytes(cfg, 256) > zha.ZHA_NOALLOC_SCRATCH_BYTES
    q = torch.empty(8, 8, 4, 256, 128, dtype=torch.bfloat16)
    k = torch.empty(1, 1, 16, 128, dtype=torch.bfloat16)
    out = torch.empty(16, 128)
    with pytest.raises(zha.ZhaError) as ei:
        zha.attend_noalloc(cfg, q, 256, k, k, 1 << 20, None, zha.ZHA_ALL_KEYS, out, None)
    assert ei.value.code == zha.ZHA_ERR_CAPACITY
    assert "static scratch" in str(ei.value)
    # the header's limit is the binding's
    text = open(HEADER).read()
    assert "#define ZHA_NOALLOC_SCRATCH_BYTES (32ll << 20)" in text


def test_stream_probe_rejects_bad_arguments(lib):
    """The measurement probe checks mode, size, alignment, overlap and the
    destination's size on the host before any launch."""
    import torch

    src = torch.empty(1024, dtype=torch.int32)
    dst = torch.empty(1024, dtype=torch.int32)
    with pytest.raises(zha.ZhaError) as ei:
        lib_mode = 9
        zha._check(lib.zha_stream_probe(lib_mode, zha._ptr(src), zha._ptr(dst), 4096, 4096, None, None))
    assert ei.value.code == zha.ZHA_ERR_ARG
    for n in (0, 100):
        with pytest.raises(zha.ZhaError) as ei:
            zha.stream_probe("copy", src, dst, n)
        assert ei.value.code == zha.ZHA_ERR_ARG
    with pytest.raises(zha.ZhaError) as ei:  # a copy writes n_bytes
        zha.stream_probe("copy", src, dst[:512], 4096)
    assert ei.value.code == zha.ZHA_ERR_CAPACITY
    with pytest.raises(zha.ZhaError) as ei:  # read-only probes write one word per workgroup
        zha.stream_probe("read", src, dst, 4096)
    assert ei.value.code == zha.ZHA_ERR_CAPACITY
    with pytest.raises(zha.ZhaError) as ei:  # the tile mix writes 16 bytes per 256 read
        zha.stream_probe("tile_mix", src, dst[:60], 4096)
    assert ei.value.code == zha.ZHA_ERR_CAPACITY
    with pytest.raises(zha.ZhaError) as ei:
        zha.stream_probe("mix", src, src, 4096)
    assert ei.value.code == zha.ZHA_ERR_ARG
    with pytest.raises(zha.ZhaError) as ei:
        zha._check(lib.zha_stream_probe(2, ct.c_void_p(src.data_ptr() + 4), zha._ptr(dst), 64, 4096, None, None))
    assert ei.value.code == zha.ZHA_ERR_ALIGN


def test_selected_chunks_rejects_bad_arguments(lib):
    """The chunk-id export checks pointers, alignment, counts and the row
    width on the host before any launch (fake, aligned addresses)."""
    A = ct.c_void_p(1 << 20)

    def call(sel=A, words=4, nq=2, n=100, ids=A, cnt=A, cap=8):
        return lib.zha_selected_chunks(sel, words, nq, n, ids, cnt, cap, None)

    assert call(sel=None) == zha.ZHA_ERR_NULL
    assert call(cnt=None) == zha.ZHA_ERR_NULL
    assert call(ids=None) == zha.ZHA_ERR_NULL
    assert call(sel=ct.c_void_p((1 << 20) + 2)) == zha.ZHA_ERR_ALIGN
    assert call(nq=0) == zha.ZHA_ERR_ARG
    assert call(n=-1) == zha.ZHA_ERR_ARG
    assert call(n=1 << 31) == zha.ZHA_ERR_ARG
    assert call(cap=-1) == zha.ZHA_ERR_ARG
    assert call(words=3, n=97) == zha.ZHA_ERR_CAPACITY  # 97 chunks need 4 words


def test_single_number_size_queries_match_the_layouts(lib):
    """zha_tree_bytes / zha_route_workspace_bytes / zha_dense_workspace_bytes
    are the layouts' totals; an invalid configuration gives a negative code."""
    for kw in (dict(), dict(leaf_form="weights2"), dict(g_dtype="fp8", leaf_form="weights2")):
        cfg = cfg_deep(**kw)
        c = cfg.c()
        assert lib.zha_tree_bytes(ct.byref(c)) == zha.tree_layout(cfg).total_bytes
        for T in (1, 16):
            assert lib.zha_route_workspace_bytes(ct.byref(c), T) == zha.route_layout(cfg, T).workspace_bytes
            assert lib.zha_dense_workspace_bytes(ct.byref(c), T) == zha.attend_workspace_bytes(cfg, T)
    bad = cfg_deep()
    c = bad.c()
    c.head_dim = 96
    assert lib.zha_tree_bytes(ct.byref(c)) < 0
    assert lib.zha_route_workspace_bytes(ct.byref(c), 1) < 0
    assert lib.zha_dense_workspace_bytes(ct.byref(c), 1) < 0
