"""GPU parity: the HIP library (through the C ABI) against the CPU oracle.

Every input comes from the seeded generators; the oracle takes CPU copies of
the very same tensors.  Tolerances: attention outputs within 1e-5 (fp32 K/V)
or 1e-2 (bf16 K/V, fp32 accumulation) max abs error; selected sets identical
up to ambiguous nodes (see tests/parity.py); tree fields as documented in
each test.
"""
import math
import sys

import numpy as np
import pytest
import torch

import scipy.special as sps

import oracle.zha_oracle as O
from tests import parity as PAR
from tree_indexed_sparse_zha_amd import workloads as W
from tree_indexed_sparse_zha_amd import zha

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[gpu-test] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm device")
    zha.load()
    torch.manual_seed(0)
    yield
    torch.cuda.synchronize()


def cfg_of(w: W.Workload, capacity=None, **kw) -> zha.ZhaConfig:
    d = dict(
        batch=w.batch, n_kv_heads=w.n_kv_heads, q_per_kv=w.q_per_kv, head_dim=w.head_dim, n_ref=w.n_ref,
        chunk=w.chunk, levels=w.levels, dtype=w.dtype, capacity=capacity or w.n_tokens,
    )
    d.update(kw)
    return zha.ZhaConfig(**d)


def np64(t):
    return t.detach().to(torch.float64).cpu().numpy()


def random_inputs(cfg: zha.ZhaConfig, T, seed=0, n_tokens=None):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    B, H, G, d = cfg.batch, cfg.n_kv_heads, cfg.q_per_kv, cfg.head_dim
    cap = cfg.capacity
    K = torch.randn(B, H, cap, d, generator=g, device="cuda").to(cfg.torch_dtype)
    V = torch.randn(B, H, cap, d, generator=g, device="cuda").to(cfg.torch_dtype)
    Q = torch.randn(B, H, G, T, d, generator=g, device="cuda").to(cfg.torch_dtype)
    ref = (torch.randn(H, cfg.n_ref, d, generator=g, device="cuda") / math.sqrt(d)).to(cfg.torch_dtype).float()
    return K, V, Q, ref


def query_list(cfg, T):
    return [(b, h, gq, t) for b in range(cfg.batch) for h in range(cfg.n_kv_heads) for gq in range(cfg.q_per_kv) for t in range(T)]


# ---------------------------------------------------------------------------
# attention over given chunk sets


ATTEND_CASES = [
    # name, cfg kwargs, T, n_tokens
    ("f32-d64-C4", dict(batch=1, n_kv_heads=2, q_per_kv=3, head_dim=64, n_ref=4, chunk=4, levels=3, dtype="f32", capacity=5000), 2, 4999),
    ("bf16-d128-C4", dict(batch=2, n_kv_heads=2, q_per_kv=4, head_dim=128, n_ref=16, chunk=4, levels=6, dtype="bf16", capacity=9000), 1, 8999),
    ("bf16-d64-C256", dict(batch=1, n_kv_heads=2, q_per_kv=4, head_dim=64, n_ref=16, chunk=256, levels=1, dtype="bf16", capacity=4200), 3, 4133),
    ("f32-d128-C8", dict(batch=1, n_kv_heads=1, q_per_kv=5, head_dim=128, n_ref=1, chunk=8, levels=4, dtype="f32", capacity=3000), 1, 2997),
]


@pytest.mark.parametrize("name,kw,T,N", ATTEND_CASES, ids=[c[0] for c in ATTEND_CASES])
@pytest.mark.parametrize("flags", [zha.ZHA_SINK | zha.ZHA_LAST_CHUNK, 0, zha.ZHA_ALL_KEYS])
def test_attend_matches_oracle(name, kw, T, N, flags):
    _say(f"attend {name} flags={flags}")
    cfg = zha.ZhaConfig(**kw)
    K, V, Q, _ = random_inputs(cfg, T, seed=1)
    nq = cfg.n_caches * cfg.q_per_kv * T
    n_chunks = N // cfg.chunk
    words = (n_chunks + 31) // 32 + 1
    gsel = torch.Generator(device="cpu")
    gsel.manual_seed(2)
    density = torch.rand(nq, 1, generator=gsel) * 0.5
    mask = torch.rand(nq, n_chunks, generator=gsel) < density
    mask[0, :] = False  # one query with no routed chunk: only the forced keys
    sel = zha.pack_bits(mask, words).cuda()
    out = torch.full((nq, cfg.head_dim), float("nan"), device="cuda")
    lse = torch.full((nq,), float("nan"), device="cuda")
    ws = torch.empty(zha.attend_workspace_bytes(cfg, T), dtype=torch.uint8, device="cuda")
    zha.attend(cfg, Q, T, K, V, N, sel, flags, out, lse, ws)
    torch.cuda.synchronize()
    out_c, lse_c = out.cpu().numpy(), lse.cpu().numpy()
    tol = PAR.OUT_TOL[cfg.dtype]
    for qi, (b, h, gq, t) in enumerate(query_list(cfg, T)):
        Kn, Vn = np64(K[b, h, :N]), np64(V[b, h, :N])
        q = np64(Q[b, h, gq, t])
        if flags & zha.ZHA_ALL_KEYS:
            idx = np.arange(N)
        else:
            chunks = np.nonzero(mask[qi].numpy())[0]
            idx = O.attend_set(chunks, N, cfg.chunk, bool(flags & zha.ZHA_SINK), bool(flags & zha.ZHA_LAST_CHUNK))
        if idx.size == 0:
            assert np.all(out_c[qi] == 0) and np.isneginf(lse_c[qi])
            continue
        o, l = O.attend(q, Kn, Vn, idx)
        np.testing.assert_allclose(out_c[qi], o, rtol=0, atol=tol, err_msg=f"query {qi}")
        np.testing.assert_allclose(lse_c[qi], l, rtol=0, atol=tol, err_msg=f"query {qi}")


# attention reading the route's cached level-1 logits (leaf-weights form):
# query groups of 4, 8 and 16 with a ragged last group, d = 64 and 128,
# chunk sizes 4, 8, 16, ragged token counts, several key tiles, every forced-
# key flag combination
CACHED_CASES = [
    # name, cfg kwargs, T, n_tokens, p
    ("qg4-d128-C4", dict(batch=2, n_kv_heads=2, q_per_kv=4, head_dim=128, n_ref=16, chunk=4, levels=4, capacity=9000), 1, 8998, 0.9),
    ("qg8-d64-C8", dict(batch=1, n_kv_heads=2, q_per_kv=3, head_dim=64, n_ref=4, chunk=8, levels=3, capacity=6000), 2, 5995, 0.7),
    ("qg16-d128-C16", dict(batch=1, n_kv_heads=1, q_per_kv=4, head_dim=128, n_ref=2, chunk=16, levels=2, capacity=5000), 5, 4992, 0.95),
    ("qg4-d64-C4-p1", dict(batch=1, n_kv_heads=1, q_per_kv=2, head_dim=64, n_ref=3, chunk=4, levels=3, capacity=2100), 1, 2051, 1.0),
    ("qg4-d128-C8", dict(batch=1, n_kv_heads=2, q_per_kv=4, head_dim=128, n_ref=16, chunk=8, levels=3, capacity=7000), 1, 6999, 0.9),
    ("qg4-d64-C16-R1", dict(batch=1, n_kv_heads=1, q_per_kv=3, head_dim=64, n_ref=1, chunk=16, levels=2, capacity=5000), 1, 4990, 0.8),
    # levels 1 and 2 as weights: <= 4 queries per cache score level 1 from the level-2 pass's
    # logits; 6 queries per cache score it from the keys
    ("w2-qg4-d128-C4", dict(batch=2, n_kv_heads=2, q_per_kv=4, head_dim=128, n_ref=16, chunk=4, levels=4, capacity=9000, leaf_form="weights2"), 1, 8998, 0.9),
    ("w2-qg4-d64-C4-p1", dict(batch=1, n_kv_heads=1, q_per_kv=2, head_dim=64, n_ref=3, chunk=4, levels=3, capacity=2100, leaf_form="weights2"), 1, 2051, 1.0),
    ("w2-qg8-d64-C4", dict(batch=1, n_kv_heads=2, q_per_kv=3, head_dim=64, n_ref=5, chunk=4, levels=3, capacity=6000, leaf_form="weights2"), 2, 5995, 0.8),
    ("w2-qg4-d128-R1", dict(batch=1, n_kv_heads=2, q_per_kv=4, head_dim=128, n_ref=1, chunk=4, levels=4, capacity=9000, leaf_form="weights2"), 1, 8990, 0.8),
    ("w2-fp8-qg4-d128-C4", dict(batch=2, n_kv_heads=2, q_per_kv=4, head_dim=128, n_ref=16, chunk=4, levels=5, capacity=9000, leaf_form="weights2", g_dtype="fp8"), 1, 8998, 0.9),
    ("w2-fp4-qg4-d128-C4", dict(batch=2, n_kv_heads=2, q_per_kv=4, head_dim=128, n_ref=16, chunk=4, levels=5, capacity=9000, leaf_form="weights2", g_dtype="fp4"), 1, 8998, 0.9),
]


@pytest.mark.parametrize("name,kw,T,N,p", CACHED_CASES, ids=[c[0] for c in CACHED_CASES])
@pytest.mark.parametrize("flags", [zha.ZHA_SINK | zha.ZHA_LAST_CHUNK, 0, zha.ZHA_SINK, zha.ZHA_LAST_CHUNK])
def test_attend_cached_logits_matches_oracle(name, kw, T, N, p, flags):
    _say(f"attend with cached logits {name} flags={flags}")
    cfg = zha.ZhaConfig(**{"dtype": "bf16", "leaf_form": "weights", **kw})
    K, V, Q, ref = random_inputs(cfg, T, seed=5)
    tree = zha.alloc_tree(cfg)
    zha.build(cfg, K, ref, tree, N)
    buf = zha.alloc_route(cfg, T, logits=True)
    zha.route(cfg, tree, N, Q, T, p, buf, K=K)
    nq = int(buf.layout.n_queries)
    out = torch.full((nq, cfg.head_dim), float("nan"), device="cuda")
    lse = torch.full((nq,), float("nan"), device="cuda")
    ws = torch.empty(zha.attend_workspace_bytes(cfg, T), dtype=torch.uint8, device="cuda")
    zha.attend(cfg, Q, T, K, V, N, zha.level1_sel(buf), flags, out, lse, ws, logits=buf.logits)
    torch.cuda.synchronize()
    out_c, lse_c = out.cpu().numpy(), lse.cpu().numpy()
    tol = PAR.OUT_TOL[cfg.dtype]
    n_chunks = N // cfg.chunk
    if flags == zha.ZHA_SINK | zha.ZHA_LAST_CHUNK:
        # the routing itself (level-1 scores from raw keys and weights), teacher-forced
        QC = cfg.q_per_kv * T
        for cache in sorted({0, cfg.n_caches - 1}):
            b, h = divmod(cache, cfg.n_kv_heads)
            Kn, rn = np64(K[b, h, :N]), np64(ref[h])
            l2d = "f64" if cfg.weight_keys(2) else None
            gd = cfg.g_dtype if cfg.g_dtype in ("fp8", "fp4") else cfg.dtype
            to = O.build_tree(Kn, rn, cfg.chunk, cfg.levels, gd, keep_g=False, leaf_dtype="f64", level2_dtype=l2d)
            for ql in range(QC):
                bits, scores = gpu_levels(cfg, buf, N, cache * QC + ql)
                q = np64(Q[b, h, ql // T, ql % T])
                PAR.check_route_teacher_forced(q, to, rn, cfg.chunk, p, PAR.gpu_kept_from_bits(bits), gd,
                                               scores, leaf_dtype="f64", level2_dtype=l2d)
        PAR.check_stats_all(zha, cfg, buf, N, p, range(int(buf.layout.n_queries)))
    for qi, (b, h, gq, t) in enumerate(query_list(cfg, T)):
        bits, _ = gpu_levels(cfg, buf, N, qi)
        chunks = np.nonzero(bits[1][:n_chunks])[0]
        idx = O.attend_set(chunks, N, cfg.chunk, bool(flags & zha.ZHA_SINK), bool(flags & zha.ZHA_LAST_CHUNK))
        if idx.size == 0:
            assert np.all(out_c[qi] == 0) and np.isneginf(lse_c[qi])
            continue
        o, l = O.attend(np64(Q[b, h, gq, t]), np64(K[b, h, :N]), np64(V[b, h, :N]), idx)
        np.testing.assert_allclose(out_c[qi], o, rtol=0, atol=tol, err_msg=f"query {qi}")
        np.testing.assert_allclose(lse_c[qi], l, rtol=0, atol=tol, err_msg=f"query {qi}")


# ---------------------------------------------------------------------------
# tree build


BUILD_CASES = [
    ("tiny-f32", dict(batch=1, n_kv_heads=1, q_per_kv=1, head_dim=64, n_ref=4, chunk=4, levels=3, dtype="f32", capacity=4096), 4096),
    ("deep-bf16-ragged", dict(batch=1, n_kv_heads=2, q_per_kv=4, head_dim=128, n_ref=16, chunk=4, levels=6, dtype="bf16", capacity=9000), 8192 + 4 * 37 + 2),
    ("wide-bf16", dict(batch=1, n_kv_heads=2, q_per_kv=4, head_dim=128, n_ref=16, chunk=256, levels=1, dtype="bf16", capacity=3000), 2560 + 100),
    ("light-bf16", dict(batch=1, n_kv_heads=1, q_per_kv=4, head_dim=128, n_ref=1, chunk=8, levels=4, dtype="bf16", capacity=5000), 4096 + 8 * 5 + 3),
    ("c32-f32-d64", dict(batch=1, n_kv_heads=1, q_per_kv=1, head_dim=64, n_ref=5, chunk=32, levels=2, dtype="f32", capacity=2200), 2048 + 70),
    ("c1-f32", dict(batch=1, n_kv_heads=1, q_per_kv=1, head_dim=64, n_ref=3, chunk=1, levels=1, dtype="f32", capacity=300), 300),
    ("c2-f32-5lv", dict(batch=1, n_kv_heads=2, q_per_kv=1, head_dim=128, n_ref=3, chunk=2, levels=5, dtype="f32", capacity=1000), 32 * 7 + 2 * 5 + 1),
    ("deep-bf16-weights", dict(batch=1, n_kv_heads=2, q_per_kv=4, head_dim=128, n_ref=16, chunk=4, levels=6, dtype="bf16", capacity=9000, leaf_form="weights"), 8192 + 4 * 37 + 2),
    ("light-bf16-weights", dict(batch=1, n_kv_heads=1, q_per_kv=4, head_dim=128, n_ref=1, chunk=8, levels=4, dtype="bf16", capacity=5000, leaf_form="weights"), 4096 + 8 * 5 + 3),
    ("c16-bf16-d64-weights", dict(batch=2, n_kv_heads=1, q_per_kv=2, head_dim=64, n_ref=7, chunk=16, levels=2, dtype="bf16", capacity=3000, leaf_form="weights"), 2048 + 16 * 9 + 5),
    ("deep-bf16-fp8", dict(batch=1, n_kv_heads=2, q_per_kv=4, head_dim=128, n_ref=16, chunk=4, levels=6, dtype="bf16", capacity=9000, g_dtype="fp8"), 8192 + 4 * 37 + 2),
    ("deep-bf16-weights-fp8", dict(batch=1, n_kv_heads=2, q_per_kv=4, head_dim=128, n_ref=16, chunk=4, levels=6, dtype="bf16", capacity=9000, leaf_form="weights", g_dtype="fp8"), 8192 + 4 * 37 + 2),
    ("c8-bf16-d64-fp8", dict(batch=1, n_kv_heads=1, q_per_kv=2, head_dim=64, n_ref=5, chunk=8, levels=3, dtype="bf16", capacity=5000, g_dtype="fp8"), 4096 + 8 * 7 + 3),
    # matrix-core build (bf16, chunk 4, weights form): d = 64 with 3 levels (no level above the round's),
    # 4 levels (one open level, append split), 8 levels (five open levels, a partial second top span)
    ("mf-d64-r5-l3", dict(batch=2, n_kv_heads=1, q_per_kv=2, head_dim=64, n_ref=5, chunk=4, levels=3, dtype="bf16", capacity=3000, leaf_form="weights"), 2048 + 4 * 37 + 2),
    ("mf-d128-r7-l4", dict(batch=1, n_kv_heads=2, q_per_kv=4, head_dim=128, n_ref=7, chunk=4, levels=4, dtype="bf16", capacity=5000, leaf_form="weights"), 4096 + 64 * 3 + 16 * 2 + 4 * 3 + 1),
    ("mf-mean-d64-r16-l4", dict(batch=1, n_kv_heads=2, q_per_kv=2, head_dim=64, n_ref=16, chunk=4, levels=4, dtype="bf16", capacity=5000), 4096 + 64 * 2 + 4 * 5 + 3),
    ("mf-c8-d64-r16-l2", dict(batch=1, n_kv_heads=2, q_per_kv=2, head_dim=64, n_ref=16, chunk=8, levels=2, dtype="bf16", capacity=3000, leaf_form="weights"), 2048 + 64 + 8 * 3 + 5),
    ("mf-c8-mean-d128-r5-l5", dict(batch=1, n_kv_heads=1, q_per_kv=4, head_dim=128, n_ref=5, chunk=8, levels=5, dtype="bf16", capacity=40000), 32768 + 8 * 100 + 3),
    ("mf-d128-r3-l8", dict(batch=1, n_kv_heads=1, q_per_kv=1, head_dim=128, n_ref=3, chunk=4, levels=8, dtype="bf16", capacity=70000, leaf_form="weights"), 65536 + 4 * 100 + 1),
    # levels 1 and 2 as weights: a trailing level-2 node of one and of three chunks
    ("w2-d128-r16-l6", dict(batch=1, n_kv_heads=2, q_per_kv=4, head_dim=128, n_ref=16, chunk=4, levels=6, dtype="bf16", capacity=9000, leaf_form="weights2"), 8192 + 4 * 37 + 2),
    ("w2-d64-r5-l3", dict(batch=2, n_kv_heads=1, q_per_kv=2, head_dim=64, n_ref=5, chunk=4, levels=3, dtype="bf16", capacity=3000, leaf_form="weights2"), 2048 + 4 * 39 + 3),
    ("w2-d128-r1-l5", dict(batch=1, n_kv_heads=2, q_per_kv=4, head_dim=128, n_ref=1, chunk=4, levels=5, dtype="bf16", capacity=5000, leaf_form="weights2"), 4096 + 16 * 7 + 4 * 3 + 1),
    # levels 1 and 2 as weights, fp8 rows (power-of-two scales) from level 3 up: d = 128 (8 values
    # per lane) and d = 64 (4 per lane), trailing partial nodes, a partial second top span
    ("w2-fp8-d128-r16-l6", dict(batch=1, n_kv_heads=2, q_per_kv=4, head_dim=128, n_ref=16, chunk=4, levels=6, dtype="bf16", capacity=9000, leaf_form="weights2", g_dtype="fp8"), 8192 + 4 * 37 + 2),
    ("w2-fp8-d64-r5-l4", dict(batch=2, n_kv_heads=1, q_per_kv=2, head_dim=64, n_ref=5, chunk=4, levels=4, dtype="bf16", capacity=5000, leaf_form="weights2", g_dtype="fp8"), 4096 + 64 * 3 + 16 * 2 + 4 * 3 + 1),
    # levels 1 and 2 as weights, OCP MXFP4 from level 3 up (d = 128): R = 16 and R = 5, ragged
    ("w2-fp4-d128-r16-l6", dict(batch=1, n_kv_heads=2, q_per_kv=4, head_dim=128, n_ref=16, chunk=4, levels=6, dtype="bf16", capacity=9000, leaf_form="weights2", g_dtype="fp4"), 8192 + 4 * 37 + 2),
    ("w2-fp4-d128-r5-l4", dict(batch=2, n_kv_heads=1, q_per_kv=2, head_dim=128, n_ref=5, chunk=4, levels=4, dtype="bf16", capacity=5000, leaf_form="weights2", g_dtype="fp4"), 4096 + 64 * 3 + 16 * 2 + 4 * 3 + 1),
]
APPEND_CASES = [c for c in BUILD_CASES if c[0] != "c1-f32"]


def _segmented_keys(cfg, seed):
    """Clustered keys (segments of 64) so that reference softmaxes are not flat."""
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    B, H, cap, d = cfg.batch, cfg.n_kv_heads, cfg.capacity, cfg.head_dim
    mu = torch.randn(B, H, (cap + 63) // 64, d, generator=g, device="cuda")
    idx = torch.arange(cap, device="cuda") // 64
    K = mu[:, :, idx] + 0.5 * torch.randn(B, H, cap, d, generator=g, device="cuda")
    ref = torch.randn(H, cfg.n_ref, d, generator=g, device="cuda")  # larger than N(0, I/d): sharper weights
    return K.to(cfg.torch_dtype), ref.to(cfg.torch_dtype).float()


def check_tree(cfg, tree, K, ref, N):
    sizes = O.level_sizes(N, cfg.chunk, cfg.levels)
    d = cfg.head_dim
    for b in range(cfg.batch):
        for h in range(cfg.n_kv_heads):
            cache = b * cfg.n_kv_heads + h
            Kn, rn = np64(K[b, h, :N]), np64(ref[h])
            gd = cfg.g_dtype if cfg.g_dtype in ("fp8", "fp4") else cfg.dtype
            to = O.build_tree(Kn, rn, cfg.chunk, cfg.levels, gd, n_tokens=N,
                              leaf_dtype="f64" if cfg.weights else None,
                              level2_dtype="f64" if cfg.weight_keys(2) else None)
            for lv in range(1, cfg.levels + 1):
                n = sizes[lv - 1]
                got = zha.read_level(cfg, tree, lv, n)
                lvl = to[lv - 1]
                if lv == 2 and cfg.leaf_form == "weights2":
                    # each child's share of the node's mass: exp(L(child) - L) from the oracle's
                    # level-1 and level-2 L (0 for the children a trailing node lacks)
                    gr, gL, gc = np64(got["rho"][cache]), np64(got["L"][cache]), np64(got["c"][cache])
                    L1p = np.full((n * cfg.chunk, cfg.n_ref), -np.inf)
                    L1p[: sizes[0]] = to[0].L
                    rho = np.exp(L1p.reshape(n, cfg.chunk, cfg.n_ref) - lvl.L[:, None, :]).transpose(0, 2, 1)
                    np.testing.assert_allclose(gr, rho, rtol=1e-5, atol=2e-6, err_msg="rho level 2")
                    np.testing.assert_allclose(gL, lvl.L, rtol=1e-5, atol=3e-5, err_msg="L level 2")
                    np.testing.assert_allclose(gc, lvl.c, rtol=1e-5, atol=3e-5, err_msg="c level 2")
                    continue
                wk = cfg.weight_keys(lv)
                if wk:
                    # w is the softmax of r_j . k_i / sqrt(d) over the node's own keys (scipy),
                    # zeros for the keys a trailing node lacks; c = L - sum w z
                    gw, gL, gc = np64(got["w"][cache]), np64(got["L"][cache]), np64(got["c"][cache])
                    nk = sizes[0] * cfg.chunk  # keys of complete chunks
                    kpad = np.zeros((n * wk, d))
                    kpad[:nk] = Kn[:nk]
                    z = np.einsum("ncd,rd->nrc", kpad.reshape(n, wk, d), rn) / math.sqrt(d)
                    have = (np.arange(n * wk) < nk).reshape(n, 1, wk)
                    z = np.where(have, z, -np.inf)
                    np.testing.assert_allclose(gw, sps.softmax(z, axis=2), rtol=0, atol=2e-6, err_msg=f"w level {lv}")
                    np.testing.assert_allclose(gL, lvl.L, rtol=1e-5, atol=3e-5, err_msg=f"L level {lv}")
                    np.testing.assert_allclose(gc, lvl.c, rtol=1e-5, atol=3e-5, err_msg=f"c level {lv}")
                    continue
                gg, gL, gc = np64(got["g"][cache]), np64(got["L"][cache]), np64(got["c"][cache])
                np.testing.assert_allclose(gL, lvl.L, rtol=1e-5, atol=3e-5, err_msg=f"L level {lv}")
                # c is consistent with the GPU's own stored g ...
                c_self = gL - np.einsum("nrd,rd->nr", gg, rn) / math.sqrt(d)
                np.testing.assert_allclose(gc, c_self, rtol=0, atol=3e-5, err_msg=f"c/g level {lv}")
                # ... and with the oracle's L given that g
                c_or = lvl.L - np.einsum("nrd,rd->nr", gg, rn) / math.sqrt(d)
                np.testing.assert_allclose(gc, c_or, rtol=1e-5, atol=5e-5, err_msg=f"c level {lv}")
                if cfg.dtype == "f32":
                    scale = np.abs(lvl.g).max() + 1e-30
                    np.testing.assert_allclose(gg, lvl.g, rtol=0, atol=2e-6 * scale, err_msg=f"g level {lv}")
                elif cfg.g_dtype == "fp8":
                    check_fp8_level(lv, np64(got["g"][cache]), np64(got["scale"][cache]), lvl)
                elif cfg.g_dtype == "fp4":
                    check_fp4_level(lv, np64(got["g"][cache]), np64(got["scale"][cache]), lvl)
                else:
                    mism = gg != lvl.ghat
                    # at most 1e-3 of the values, and never fewer than 2 allowed (a level of a few
                    # hundred values, such as an 8-level tree's top, may hold one boundary flip)
                    assert mism.sum() <= max(2, 1e-3 * mism.size), f"level {lv}: {int(mism.sum())} of {mism.size} bf16 g differ"
                    if mism.any():
                        # A mismatch is a rounding-boundary flip: the GPU's fp32 value and the
                        # oracle's fp64 value round to neighbouring bf16 numbers.  Allowed: one
                        # bf16 spacing at the value, plus the fp32 accumulation error of the
                        # node row (relative 4e-6 of the row's largest element).
                        row_scale = np.abs(lvl.g).max(axis=2, keepdims=True)
                        row_scale = np.broadcast_to(row_scale, lvl.g.shape)[mism]
                        spacing = np.maximum(np.abs(lvl.ghat[mism]), np.abs(gg[mism])) * 2.0**-7
                        allowed = spacing + 4e-6 * row_scale
                        dev = np.abs(gg[mism] - lvl.ghat[mism])
                        bad = dev > allowed
                        assert not bad.any(), (
                            f"level {lv}: {int(bad.sum())} g flips beyond one spacing: gpu {gg[mism][bad][:5]} "
                            f"oracle {lvl.ghat[mism][bad][:5]} exact {lvl.g[mism][bad][:5]}"
                        )


def check_fp8_level(lv, gg, gs, lvl):
    """fp8 rows: the GPU's power-of-two scale equals the oracle's except where
    the row max sits at a power of two (fp32 and fp64 may then pick
    neighbouring exponents); codes differ only at rounding boundaries, by one
    E4M3 spacing, on at most 1e-3 of the elements."""
    m = np.abs(lvl.g).max(axis=-1)
    f, _ = np.frexp(np.maximum(m, 1e-300))
    near_pow2 = np.abs(f - 0.5) < 1e-5
    same = gs == lvl.scale
    assert np.all(same | near_pow2), f"level {lv}: {int((~same & ~near_pow2).sum())} row scales differ"
    assert np.all(np.log2(gs) == np.round(np.log2(gs)))
    a, b = gg[same], lvl.ghat[same]
    sc = np.broadcast_to(gs[..., None], gg.shape)[same]
    mism = a != b
    frac = mism.mean() if mism.size else 0.0
    assert frac <= 1e-3, f"level {lv}: {frac:.2e} of fp8 g differ"
    if mism.any():
        row = np.broadcast_to(np.abs(lvl.g).max(axis=-1, keepdims=True), lvl.g.shape)[same][mism]
        x = np.maximum(np.abs(a[mism]), np.abs(b[mism])) / sc[mism]
        spacing = np.maximum(2.0 ** (np.floor(np.log2(np.maximum(x, 2.0**-6))) - 3), 2.0**-9) * sc[mism]
        dev = np.abs(a[mism] - b[mism])
        bad = dev > spacing + 4e-6 * row
        assert not bad.any(), f"level {lv}: {int(bad.sum())} fp8 flips beyond one spacing"


def check_fp4_level(lv, gg, gs, lvl):
    """MXFP4 blocks: the GPU's E8M0 scale equals the oracle's except where the
    block max sits at a power of two (fp32 and fp64 may then pick neighbouring
    exponents); E2M1 codes differ only at rounding boundaries, by one spacing
    (0.5, 1 or 2 scale units), on at most 1e-3 of the elements."""
    n, R, d = gg.shape
    m = np.abs(lvl.g).reshape(n, R, d // 32, 32).max(axis=-1)
    f, _ = np.frexp(np.maximum(m, 1e-300))
    near_pow2 = np.abs(f - 0.5) < 1e-5
    same = gs == lvl.scale
    assert np.all(same | near_pow2), f"level {lv}: {int((~same & ~near_pow2).sum())} block scales differ"
    assert np.all(np.log2(gs) == np.round(np.log2(gs)))
    blk = np.repeat(same, 32, axis=-1)
    sc = np.repeat(gs, 32, axis=-1)
    a, b = gg[blk], lvl.ghat[blk]
    mism = a != b
    frac = mism.mean() if mism.size else 0.0
    assert frac <= 1e-3, f"level {lv}: {frac:.2e} of MXFP4 g differ"
    if mism.any():
        u = np.maximum(np.abs(a[mism]), np.abs(b[mism])) / sc[blk][mism]
        spacing = np.where(u <= 2, 0.5, np.where(u <= 4, 1.0, 2.0)) * sc[blk][mism]
        bad = np.abs(a[mism] - b[mism]) > spacing * (1 + 1e-6)
        assert not bad.any(), f"level {lv}: {int(bad.sum())} MXFP4 flips beyond one spacing"


@pytest.mark.parametrize("name,kw,N", BUILD_CASES, ids=[c[0] for c in BUILD_CASES])
def test_build_matches_oracle(name, kw, N):
    _say(f"build {name}")
    cfg = zha.ZhaConfig(**kw)
    K, ref = _segmented_keys(cfg, 3)
    tree = zha.alloc_tree(cfg)
    zha.build(cfg, K, ref, tree, N)
    torch.cuda.synchronize()
    check_tree(cfg, tree, K, ref, N)


REF_ROUNDING_CASES = [c for c in BUILD_CASES if c[0] in ("w2-d128-r16-l6", "c16-bf16-d64-weights", "deep-bf16-fp8")]


@pytest.mark.parametrize("name,kw,N", REF_ROUNDING_CASES, ids=[c[0] for c in REF_ROUNDING_CASES])
def test_build_takes_bf16_rounded_reference_queries(name, kw, N):
    """Reference queries that are not bf16 values: with bf16 keys the tree is
    that of the bf16-rounded reference queries (matrix-core logits and plane
    offsets alike), checked against the oracle given round_bf16(ref); level 2
    of the weights2 form is then routed (fused pass) teacher-forced."""
    _say(f"bf16-rounded reference queries {name}")
    cfg = zha.ZhaConfig(**kw)
    K, _ = _segmented_keys(cfg, 7)
    g = torch.Generator(device="cuda")
    g.manual_seed(8)
    ref = torch.randn(cfg.n_kv_heads, cfg.n_ref, cfg.head_dim, generator=g, device="cuda")
    assert not torch.equal(ref, ref.to(torch.bfloat16).float())
    tree = zha.alloc_tree(cfg)
    zha.build(cfg, K, ref, tree, N)
    torch.cuda.synchronize()
    ref_r = torch.from_numpy(O.round_bf16(np64(ref))).float().cuda()
    check_tree(cfg, tree, K, ref_r, N)
    if cfg.leaf_form == "weights2":
        Q = torch.randn(cfg.batch, cfg.n_kv_heads, cfg.q_per_kv, 1, cfg.head_dim, generator=g,
                        device="cuda").to(torch.bfloat16)
        buf = zha.alloc_route(cfg, 1, logits=True)
        zha.route(cfg, tree, N, Q, 1, 0.9, buf, K=K)
        torch.cuda.synchronize()
        Kn, rn = np64(K[0, 0, :N]), np64(ref_r[0])
        to = O.build_tree(Kn, rn, cfg.chunk, cfg.levels, cfg.dtype, keep_g=False, leaf_dtype="f64", level2_dtype="f64")
        for ql in range(cfg.q_per_kv):
            bits, scores = gpu_levels(cfg, buf, N, ql)
            PAR.check_route_teacher_forced(np64(Q[0, 0, ql, 0]), to, rn, cfg.chunk, 0.9, PAR.gpu_kept_from_bits(bits),
                                           cfg.dtype, scores, leaf_dtype="f64", level2_dtype="f64")


@pytest.mark.parametrize("name,kw,N", APPEND_CASES, ids=[c[0] for c in APPEND_CASES])
def test_append_equals_build(name, kw, N):
    _say(f"append {name}")
    cfg = zha.ZhaConfig(**kw)
    K, ref = _segmented_keys(cfg, 4)
    fresh = zha.alloc_tree(cfg)
    zha.build(cfg, K, ref, fresh, N)
    grown = zha.alloc_tree(cfg)
    grown.fill_(0x7F)
    steps = [N // 3, 1, 2 * cfg.chunk + 1, 0, N // 4]
    n = 0
    zha.build(cfg, K, ref, grown, steps[0])
    n = steps[0]
    for s in steps[1:]:
        zha.append(cfg, K, ref, grown, n, s)
        n += s
    zha.append(cfg, K, ref, grown, n, N - n)
    torch.cuda.synchronize()
    sizes = O.level_sizes(N, cfg.chunk, cfg.levels)
    for lv in range(1, cfg.levels + 1):
        a = zha.read_level(cfg, fresh, lv, sizes[lv - 1])
        b = zha.read_level(cfg, grown, lv, sizes[lv - 1])
        for f in a:
            ba = a[f].contiguous().view(torch.uint8)
            bb = b[f].contiguous().view(torch.uint8)
            assert torch.equal(ba, bb), f"{f} level {lv} differs between append and build"


# ---------------------------------------------------------------------------
# routing + attention end to end on the workloads


def check_cached_logits(cfg, buf, K, Q, N, T, n_queries=3, max_chunks=48):
    """The level-1 logits the route keeps, on sampled routed chunks, against
    q.k / sqrt(d) in fp64 (products of bf16 values are exact in fp32; the
    only error is the fp32 accumulation)."""
    QC = cfg.q_per_kv * T
    QB, QW = (QC + 15) // 16, min((QC + 3) // 4 * 4, 16)
    nquads = buf.logits.numel() // (cfg.n_caches * QB * QW * 4)
    lg = buf.logits.view(cfg.n_caches, QB, nquads, 4, QW)
    rng = np.random.default_rng(11)
    d = cfg.head_dim
    for cache in sorted({0, cfg.n_caches - 1}):
        bb, h = divmod(cache, cfg.n_kv_heads)
        for ql in rng.choice(QC, size=min(n_queries, QC), replace=False):
            qi = cache * QC + int(ql)
            bits, _ = gpu_levels(cfg, buf, N, qi)
            kept = np.nonzero(bits[1])[0]
            kept = kept[rng.permutation(kept.size)[:max_chunks]]
            keys = (kept[:, None] * cfg.chunk + np.arange(cfg.chunk)[None, :]).reshape(-1)
            kt = torch.as_tensor(keys, device=lg.device)
            got = lg[cache, int(ql) // 16, kt // 4, kt % 4, int(ql) % 16].double().cpu().numpy()
            q = np64(Q[bb, h, int(ql) // T, int(ql) % T])
            Kk = np64(K[bb, h, kt])
            ref = Kk @ q / math.sqrt(d)
            tol = 4 * d * 2.0**-24 * (np.abs(Kk) @ np.abs(q)) / math.sqrt(d) + 1e-6
            assert np.all(np.abs(got - ref) <= tol), (cache, int(ql), float(np.max(np.abs(got - ref) - tol)))


def run_path(cfg, K, V, Q, ref, N, T, p, flags=zha.ZHA_SINK | zha.ZHA_LAST_CHUNK):
    """build + route + attend.  In the weights form the route also keeps the
    level-1 logits: they are checked against q.k in fp64, and attention runs
    twice, without them (logits from its own MFMA) and with them (the
    streaming kernel); the two agree to fp32 summation order and the second
    is returned."""
    tree = zha.alloc_tree(cfg)
    zha.build(cfg, K, ref, tree, N)
    buf = zha.alloc_route(cfg, T, logits=cfg.weights)
    zha.route(cfg, tree, N, Q, T, p, buf, K=K)
    nq = int(buf.layout.n_queries)
    out = torch.empty(nq, cfg.head_dim, device="cuda")
    lse = torch.empty(nq, device="cuda")
    ws = torch.empty(zha.attend_workspace_bytes(cfg, T), dtype=torch.uint8, device="cuda")
    zha.attend(cfg, Q, T, K, V, N, zha.level1_sel(buf), flags, out, lse, ws)
    if buf.logits is not None:
        torch.cuda.synchronize()
        check_cached_logits(cfg, buf, K, Q, N, T)
        out2, lse2 = torch.empty_like(out), torch.empty_like(lse)
        zha.attend(cfg, Q, T, K, V, N, zha.level1_sel(buf), flags, out2, lse2, ws, logits=buf.logits)
        torch.cuda.synchronize()
        assert float((out - out2).abs().max()) <= 2e-5, float((out - out2).abs().max())
        assert float((lse - lse2).abs().max()) <= 2e-5, float((lse - lse2).abs().max())
        out, lse = out2, lse2
    torch.cuda.synchronize()
    return tree, buf, out, lse


def gpu_levels(cfg, buf, N, qi):
    """Per level: kept bits [n_l] and score row [n_l] of query qi."""
    rl = buf.layout
    sizes = O.level_sizes(N, cfg.chunk, cfg.levels)
    nq = int(rl.n_queries)
    bits, scores = {}, {}
    for lv in range(1, cfg.levels + 1):
        i = lv - 1
        w = int(rl.words[i])
        words = buf.sel[int(rl.sel_offset[i]) + qi * w : int(rl.sel_offset[i]) + (qi + 1) * w]
        bits[lv] = zha.unpack_bits(words.cpu(), sizes[i]).numpy()
        cap = int(rl.score_stride[i])
        off = int(rl.score_offset[i]) + qi * cap
        scores[lv] = buf.score[off : off + sizes[i]].cpu().numpy()
    return bits, scores


ROUTE_WORKLOADS = [
    ("tiny", None, "mean", 16, "kv"),  # all queries of the tiny workload
    ("deep32k", 2, "mean", 6, "kv"),  # 2 of 8 caches, 6 sampled queries each
    ("deep32k", 2, "weights", 6, "kv"),
    ("wide256k", 2, "mean", 4, "kv"),
    ("deep32k", 2, "weights", 6, "fp8"),
    ("deep32k", 1, "mean", 6, "fp8"),
    ("deep32k", 2, "weights2", 6, "kv"),
    ("deep32k", 2, "weights2", 6, "fp8"),
    ("deep32k", 2, "weights2", 6, "fp4"),
]


@pytest.mark.parametrize(
    "wname,n_caches_checked,leaf_form,q_per_cache,g_dtype",
    ROUTE_WORKLOADS,
    ids=[f"{r[0]}-{r[2]}" + ("" if r[4] == "kv" else "-" + r[4]) for r in ROUTE_WORKLOADS],
)
def test_route_and_attend_match_oracle(wname, n_caches_checked, leaf_form, q_per_cache, g_dtype):
    w = W.WORKLOADS[wname]
    _say(f"route {wname} {leaf_form} {g_dtype}")
    cfg = cfg_of(w, leaf_form=leaf_form, g_dtype=g_dtype)
    batch = W.make_batch(w, device="cuda")
    N, T, p = w.n_tokens, w.queries_per_head, w.p[0]
    tree, buf, out, lse = run_path(cfg, batch.K, batch.V, batch.Q, batch.ref, N, T, p)
    tol = PAR.OUT_TOL[cfg.dtype]
    QC = cfg.q_per_kv * T
    caches = list(range(cfg.n_caches))
    if n_caches_checked:
        caches = [0, cfg.n_caches - 1][:n_caches_checked]
    rng = np.random.default_rng(5)
    out_c, lse_c = out.cpu().numpy(), lse.cpu().numpy()
    n_same = n_checked = 0
    for cache in caches:
        b, h = divmod(cache, cfg.n_kv_heads)
        Kn, Vn, rn = np64(batch.K[b, h, :N]), np64(batch.V[b, h, :N]), np64(batch.ref[h])
        leaf_dtype = "f64" if cfg.weights else None
        l2d = "f64" if cfg.weight_keys(2) else None
        gd = g_dtype if g_dtype in ("fp8", "fp4") else cfg.dtype
        to = O.build_tree(Kn, rn, cfg.chunk, cfg.levels, gd, keep_g=False, leaf_dtype=leaf_dtype, level2_dtype=l2d)
        qis = list(range(QC)) if q_per_cache >= QC else sorted(rng.choice(QC, q_per_cache, replace=False).tolist())
        for qi_local in qis:
            gq, t = divmod(qi_local, T)
            qi = cache * QC + qi_local
            q = np64(batch.Q[b, h, gq, t])
            bits, scores = gpu_levels(cfg, buf, N, qi)
            kept = PAR.gpu_kept_from_bits(bits)
            reps = PAR.check_route_teacher_forced(q, to, rn, cfg.chunk, p, kept, gd, scores, leaf_dtype=leaf_dtype,
                                                  level2_dtype=l2d)
            # attention over the GPU's set (R21)
            idx = O.attend_set(kept[1], N, cfg.chunk, True, True)
            o, l = O.attend(q, Kn, Vn, idx)
            np.testing.assert_allclose(out_c[qi], o, rtol=0, atol=tol)
            np.testing.assert_allclose(lse_c[qi], l, rtol=0, atol=tol)
            # end to end: with no ambiguous node at any level the oracle's own
            # routing must reach exactly the GPU's set
            o2, l2, idx2, _ = O.route_and_attend(q, Kn, Vn, to, rn, cfg.chunk, p, N)
            n_checked += 1
            if all(r.n_diff == 0 for r in reps):
                assert np.array_equal(idx, idx2), f"query {qi}: free-running oracle set differs"
                n_same += 1
                np.testing.assert_allclose(out_c[qi], o2, rtol=0, atol=tol)
    PAR.check_stats_all(zha, cfg, buf, N, p, range(int(buf.layout.n_queries)))
    # ambiguous nodes are rare: most queries match the oracle end to end
    assert n_same >= max(1, (9 * n_checked) // 10), (n_same, n_checked)


def test_route_stats_consistent():
    """The selection records of every level and query against the GPU's own
    score rows and bits: kept mass >= ceil(p M), minimality, the cut rule."""
    w = W.WORKLOADS["tiny"]
    cfg = cfg_of(w)
    batch = W.make_batch(w, device="cuda")
    N, T, p = w.n_tokens, w.queries_per_head, w.p[0]
    tree, buf, out, lse = run_path(cfg, batch.K, batch.V, batch.Q, batch.ref, N, T, p)
    PAR.check_stats_all(zha, cfg, buf, N, p, range(int(buf.layout.n_queries)))


def test_p1_is_dense():
    w = W.WORKLOADS["tiny"]
    cfg = cfg_of(w)
    batch = W.make_batch(w, device="cuda")
    N, T = w.n_tokens, w.queries_per_head
    tree, buf, out, lse = run_path(cfg, batch.K, batch.V, batch.Q, batch.ref, N, T, 1.0)
    sel1 = zha.unpack_bits(zha.level1_sel(buf).cpu(), N // cfg.chunk)
    assert bool(sel1.all())
    dense = torch.empty_like(out)
    dl = torch.empty_like(lse)
    ws = torch.empty(zha.attend_workspace_bytes(cfg, T), dtype=torch.uint8, device="cuda")
    zha.dense_decode(cfg, batch.Q, T, batch.K, batch.V, N, dense, dl, ws)
    torch.cuda.synchronize()
    Kn, Vn = np64(batch.K[0, 0, :N]), np64(batch.V[0, 0, :N])
    for t in range(T):
        o, l = O.attend(np64(batch.Q[0, 0, 0, t]), Kn, Vn, np.arange(N))
        np.testing.assert_allclose(out[t].cpu().numpy(), o, atol=1e-5, rtol=0)
        np.testing.assert_allclose(dense[t].cpu().numpy(), o, atol=1e-5, rtol=0)


def test_route_levels_schedule_and_start_level():
    """zha_route_levels: a depth-aware schedule and a lower start level,
    teacher-forced against the oracle; keep-all at the top equals starting
    one level lower, bit for bit."""
    w = W.WORKLOADS["deep32k"]
    cfg = cfg_of(w, leaf_form="weights")
    batch = W.make_batch(w, device="cuda")
    N, T, L = w.n_tokens, w.queries_per_head, w.levels
    _say("route_levels deep32k")
    tree = zha.alloc_tree(cfg)
    zha.build(cfg, batch.K, batch.ref, tree, N)
    QC = cfg.q_per_kv * T
    cache = cfg.n_caches - 1
    b, h = divmod(cache, cfg.n_kv_heads)
    Kn, rn = np64(batch.K[b, h, :N]), np64(batch.ref[h])
    to = O.build_tree(Kn, rn, cfg.chunk, L, cfg.dtype, keep_g=False, leaf_dtype="f64")
    sched = O.depth_schedule(0.8, L)
    for pl, top in ((sched, 0), ([0.9, 0.95, 0.97, 0.99, 1.0, 1.0], 4), ([0.5] * L, 1)):
        buf = zha.alloc_route(cfg, T)
        zha.route_levels(cfg, tree, N, batch.Q, T, pl, buf, top_level=top, K=batch.K)
        torch.cuda.synchronize()
        for ql in (0, QC // 2, QC - 1):
            bits, scores = gpu_levels(cfg, buf, N, cache * QC + ql)
            t = top or L
            kept = PAR.gpu_kept_from_bits({lv: bits[lv] for lv in range(1, t + 1)})
            q = np64(batch.Q[b, h, ql // T, ql % T])
            PAR.check_route_teacher_forced(q, to, rn, cfg.chunk, pl, kept, cfg.dtype,
                                           {lv: scores[lv] for lv in range(1, t + 1)}, leaf_dtype="f64", top=t)
        PAR.check_stats_all(zha, cfg, buf, N, pl, range(int(buf.layout.n_queries)), top=top or L)
    a, c = zha.alloc_route(cfg, T), zha.alloc_route(cfg, T)
    zha.route_levels(cfg, tree, N, batch.Q, T, [0.9] * (L - 1) + [1.0], a, K=batch.K)
    zha.route_levels(cfg, tree, N, batch.Q, T, [0.9] * L, c, top_level=L - 1, K=batch.K)
    torch.cuda.synchronize()
    rl = a.layout
    for lv in range(1, L):
        o, n = int(rl.sel_offset[lv - 1]), int(rl.words[lv - 1]) * int(rl.n_queries)
        assert torch.equal(a.sel[o : o + n], c.sel[o : o + n]), f"level {lv}"


@pytest.mark.parametrize("leaf_form", ["mean", "weights", "weights2"])
def test_route_is_deterministic(leaf_form):
    w = W.WORKLOADS["deep32k"]
    cfg = cfg_of(w, leaf_form=leaf_form)
    batch = W.make_batch(w, device="cuda")
    N, T, p = w.n_tokens, w.queries_per_head, w.p[0]
    tree, buf, out, lse = run_path(cfg, batch.K, batch.V, batch.Q, batch.ref, N, T, p)
    sel0, sc0, st0, out0 = buf.sel.clone(), buf.score.clone(), buf.stats.clone(), out.clone()
    zha.route(cfg, tree, N, batch.Q, T, p, buf, K=batch.K)
    ws = torch.empty(zha.attend_workspace_bytes(cfg, T), dtype=torch.uint8, device="cuda")
    zha.attend(cfg, batch.Q, T, batch.K, batch.V, N, zha.level1_sel(buf), 3, out, lse, ws, logits=buf.logits)
    torch.cuda.synchronize()
    assert torch.equal(sel0, buf.sel)
    assert torch.equal(sc0.nan_to_num(), buf.score.nan_to_num())
    assert torch.equal(st0, buf.stats)
    assert torch.equal(out0, out)


CHUNK_ID_CASES = [
    # name, n_queries, n_chunks, words (>= ceil(n_chunks / 32)), keep probability, cap
    ("ragged-dense", 5, 1000, 40, 0.5, 1000),
    ("many-segments", 3, 100003, 3126, 0.3, 100003),
    ("cap-cut", 4, 5000, 157, 0.6, 777),
    ("empty-and-full", 2, 4097, 129, None, 4097),
    ("no-chunks", 2, 0, 1, 0.5, 4),
]


@pytest.mark.parametrize("name,nq,n,words,prob,cap", CHUNK_ID_CASES, ids=[c[0] for c in CHUNK_ID_CASES])
def test_selected_chunks_lists_the_set_bits(name, nq, n, words, prob, cap):
    """zha_selected_chunks returns, per query, the ids of the set bits below
    n_chunks in increasing order (bits past n_chunks set on purpose must be
    ignored), the full count even when it exceeds cap, and writes nothing
    past min(count, cap)."""
    _say(f"selected chunks {name}")
    g = torch.Generator().manual_seed(77)
    if prob is None:
        mask = torch.zeros(nq, n, dtype=torch.bool)
        mask[1] = True  # query 0 keeps nothing, query 1 everything
    else:
        mask = torch.rand(nq, n, generator=g) < prob
    full = torch.zeros(nq, words * 32, dtype=torch.bool)
    full[:, :n] = mask
    full[:, n:] = True  # garbage past n_chunks
    words_t = zha.pack_bits(full, words).cuda()
    ids, count = zha.selected_chunks(words_t, n, cap)
    torch.cuda.synchronize()
    ids, count = ids.cpu(), count.cpu()
    for q in range(nq):
        want = torch.nonzero(mask[q]).flatten().to(torch.int32)
        assert int(count[q]) == want.numel(), (q, int(count[q]), want.numel())
        k = min(want.numel(), cap)
        assert torch.equal(ids[q, :k], want[:k]), q
        assert bool((ids[q, k:] == -1).all()), f"query {q}: entries written past its count"


def test_selected_chunks_of_a_route_match_its_bits():
    """On a real route's level-1 rows the lists are exactly the kept chunks."""
    _say("selected chunks of a route")
    cfg = zha.ZhaConfig(batch=1, n_kv_heads=2, q_per_kv=4, head_dim=128, n_ref=16, chunk=4, levels=5, dtype="bf16",
                        capacity=70000, leaf_form="weights2")
    N, T = 65536 + 4 * 301 + 3, 1
    K, V, Q, ref = random_inputs(cfg, T, seed=21)
    tree = zha.alloc_tree(cfg)
    zha.build(cfg, K, ref, tree, N)
    buf = zha.alloc_route(cfg, T, logits=True)
    zha.route(cfg, tree, N, Q, T, 0.9, buf, K=K)
    sel = zha.level1_sel(buf)
    n1 = N // cfg.chunk
    ids, count = zha.selected_chunks(sel, n1, n1)
    torch.cuda.synchronize()
    bits = zha.unpack_bits(sel.cpu(), n1)
    for q in range(sel.shape[0]):
        want = torch.nonzero(bits[q]).flatten().to(torch.int32)
        assert int(count[q]) == want.numel() > 0
        assert torch.equal(ids[q, : want.numel()].cpu(), want)


W2_LOGIT_CASES = [
    # name, cfg kwargs, T, n_tokens, p, top level (0 = the tree's top)
    ("qc4-l5", dict(batch=2, n_kv_heads=2, q_per_kv=4, head_dim=128, n_ref=16, chunk=4, levels=5, capacity=70000), 1, 65536 + 4 * 301 + 3, 0.9, 0),
    ("qc2-l3-d64", dict(batch=1, n_kv_heads=3, q_per_kv=2, head_dim=64, n_ref=5, chunk=4, levels=3, capacity=9000), 1, 8999, 0.8, 0),
    ("qc4-top2", dict(batch=1, n_kv_heads=2, q_per_kv=4, head_dim=128, n_ref=16, chunk=4, levels=4, capacity=9000), 1, 8998, 0.9, 2),
    ("qc3-top1", dict(batch=1, n_kv_heads=2, q_per_kv=3, head_dim=128, n_ref=7, chunk=4, levels=4, capacity=9000), 1, 8997, 0.9, 1),
]


@pytest.mark.parametrize("name,kw,T,N,p,top", W2_LOGIT_CASES, ids=[c[0] for c in W2_LOGIT_CASES])
def test_fused_level1_scores_match_the_key_path(name, kw, T, N, p, top):
    """Levels 1 and 2 as weights, at most 4 queries per cache: the level-2
    pass writes the level-1 scores of its candidates' chunks from the same
    MFMA logits and level-1 rows the level-1 kernel of the leaf-weights form
    uses, so on every chunk both trees hold as a candidate the two level-1
    scores agree (to fp32 rounding of the same expression); the fused rows
    hold -inf exactly off the kept parents' children; attention reading the
    kept logits agrees with attention computing its own."""
    _say(f"w2 fused level 1 {name}")
    cfg2 = zha.ZhaConfig(dtype="bf16", leaf_form="weights2", **kw)
    cfg1 = zha.ZhaConfig(dtype="bf16", leaf_form="weights", **kw)
    K, V, Q, ref = random_inputs(cfg2, T, seed=9)
    pl = [p] * cfg2.levels
    bufs = {}
    for cfg in (cfg2, cfg1):
        tree = zha.alloc_tree(cfg)
        zha.build(cfg, K, ref, tree, N)
        buf = zha.alloc_route(cfg, T, logits=True)
        buf.score.fill_(float("nan"))
        zha.route_levels(cfg, tree, N, Q, T, pl, buf, top_level=top, K=K)
        bufs[cfg.leaf_form] = buf
    torch.cuda.synchronize()
    b2, b1 = bufs["weights2"], bufs["weights"]
    n1 = N // cfg2.chunk
    nq = int(b2.layout.n_queries)
    both = 0
    for qi in range(nq):
        bits2, s2 = gpu_levels(cfg2, b2, N, qi)
        bits1, s1 = gpu_levels(cfg1, b1, N, qi)
        # candidates of the fused row: children of the kept level-2 nodes (all chunks when level 1 is the top)
        cand = np.ones(n1, bool) if top == 1 else np.repeat(bits2[2], cfg2.chunk)[:n1].astype(bool)
        assert np.all(np.isfinite(s2[1][cand])), f"query {qi}: a candidate without a score"
        assert np.all(np.isneginf(s2[1][~cand])), f"query {qi}: a non-candidate with a score"
        common = cand & np.isfinite(s1[1])
        both += int(common.sum())
        d = np.abs(s2[1][common].astype(np.float64) - s1[1][common].astype(np.float64))
        tol = 4e-6 * (1.0 + np.abs(s1[1][common]))
        assert np.all(d <= tol), f"query {qi}: level-1 scores differ by {float(d.max())}"
    assert both > 0
    check_cached_logits(cfg2, b2, K, Q, N, T)
    ws = torch.empty(zha.attend_workspace_bytes(cfg2, T), dtype=torch.uint8, device="cuda")
    outs = []
    for lg in (None, b2.logits):
        out, lse = torch.empty(nq, cfg2.head_dim, device="cuda"), torch.empty(nq, device="cuda")
        zha.attend(cfg2, Q, T, K, V, N, zha.level1_sel(b2), 3, out, lse, ws, logits=lg)
        outs.append((out, lse))
    torch.cuda.synchronize()
    assert float((outs[0][0] - outs[1][0]).abs().max()) <= 2e-5
    assert float((outs[0][1] - outs[1][1]).abs().max()) <= 2e-5


SPLIT_CASES = [
    # name, leaf form, n_tokens, p, keys repeat with period 4096 (exact score ties)
    ("weights-ragged", "weights", (1 << 19) - 1003, 0.95, False),
    ("weights-keep-all", "weights", 1 << 19, 1.0, False),
    ("mean-ties", "mean", 1 << 19, 0.9, True),
    ("mean-ties-small-p", "mean", (1 << 19) - 64, 0.05, True),
]


@pytest.mark.parametrize("name,leaf_form,N,p,repeat", SPLIT_CASES, ids=[c[0] for c in SPLIT_CASES])
def test_split_select_is_bit_identical(name, leaf_form, N, p, repeat):
    """With few queries and many candidates a level's selection may run
    split over several workgroups per query; it must reach exactly what the
    one-workgroup kernel reaches on the same score rows (bits, statistics)."""
    _say(f"split select {name}")
    cap = 1 << 19
    cfg = zha.ZhaConfig(batch=1, n_kv_heads=2, q_per_kv=4, head_dim=128, n_ref=16, chunk=4, levels=5, dtype="bf16",
                        capacity=cap, leaf_form=leaf_form)
    T = 1
    rl = zha.route_layout(cfg, T)
    assert int(rl.workspace_bytes) > int(rl.workspace_min_bytes)
    K = torch.empty(1, 2, cap, 128, dtype=torch.bfloat16)
    Q = torch.empty(1, 2, 4, T, 128, dtype=torch.bfloat16)
    ref = torch.empty(2, 16, 128)
    for h in range(2):
        k, _, r, q = W.random_cache(cap, 128, 16, "bf16", seed=71 + h, n_queries=4, segment_len=16)
        if repeat:
            k = k[:4096].repeat(cap // 4096, 1)
        q[::2] = (1.5 * k[[777, 300001]].float()).to(torch.bfloat16)  # two needle queries per head
        K[0, h], ref[h], Q[0, h, :, 0] = k, r, q
    K, Q, ref = K.cuda(), Q.cuda(), ref.cuda()
    tree = zha.alloc_tree(cfg)
    zha.build(cfg, K, ref, tree, N)
    weights = leaf_form == "weights"
    bufs = []
    for split in (True, False):
        buf = zha.alloc_route(cfg, T, logits=weights, split_select=split)
        zha.route(cfg, tree, N, Q, T, p, buf, K=K)
        bufs.append(buf)
    torch.cuda.synchronize()
    sizes = O.level_sizes(N, cfg.chunk, cfg.levels)
    n_cut = 0
    for lv in range(1, cfg.levels + 1):
        i = lv - 1
        nw, st = int(rl.words[i]), int(rl.score_stride[i])
        for qi in range(int(rl.n_queries)):
            rows = []
            for b in bufs:
                w0 = int(rl.sel_offset[i]) + qi * nw
                s0 = int(rl.score_offset[i]) + qi * st
                rows.append((b.sel[w0 : w0 + nw].cpu(), b.score[s0 : s0 + sizes[i]].cpu()))
            assert torch.equal(rows[0][1].view(torch.int32), rows[1][1].view(torch.int32)), (lv, qi, "scores")
            assert torch.equal(rows[0][0], rows[1][0]), (lv, qi, "bits")
            # the kept set is a prefix of the candidates ordered by score
            # descending, then id ascending (ties at the cut go to lower ids)
            sc = rows[0][1].numpy()
            kept = zha.unpack_bits(rows[0][0], sizes[i]).numpy()
            cand = np.nonzero(np.isfinite(sc))[0]
            order = cand[np.lexsort((cand, -sc[cand]))]
            ks = kept[order].astype(np.int8)
            assert not kept[np.isinf(sc)].any(), (lv, qi, "kept a non-candidate")
            assert ks.sum() >= 1 and np.all(ks[: ks.sum()] == 1), (lv, qi, "kept set is not a prefix")
        ra, rb = zha.stats_records(bufs[0], lv), zha.stats_records(bufs[1], lv)
        for qi, (a, b) in enumerate(zip(ra, rb)):
            assert bytes(a) == bytes(b), (lv, qi, "stats")
            n_cut += a.cut_id != 2**31 - 1
    if repeat and p < 1.0:
        assert n_cut > 0, "no level split its ties at the cut"
    PAR.check_stats_all(zha, cfg, bufs[0], N, p, range(int(rl.n_queries)))


SMALL_CASES = [
    # name, cfg kwargs (capacity 300), token counts: below one chunk, one chunk, one 16-key block,
    # one 64-key round, ragged rounds, several top nodes
    ("mf-weights-C4", dict(batch=1, n_kv_heads=2, q_per_kv=2, head_dim=64, n_ref=4, chunk=4, levels=3, dtype="bf16",
                           leaf_form="weights"), [1, 3, 4, 5, 16, 63, 64, 65, 257]),
    ("mf-mean-C8", dict(batch=1, n_kv_heads=1, q_per_kv=3, head_dim=128, n_ref=1, chunk=8, levels=2, dtype="bf16"),
     [7, 8, 9, 64, 65, 200]),
    ("f32-C4", dict(batch=1, n_kv_heads=1, q_per_kv=2, head_dim=64, n_ref=3, chunk=4, levels=3, dtype="f32"), [1, 4, 65, 299]),
]


@pytest.mark.parametrize("name,kw,sizes", SMALL_CASES, ids=[c[0] for c in SMALL_CASES])
def test_small_and_degenerate_token_counts(name, kw, sizes):
    """Build, route and attend at token counts around the chunk, block, round
    and top-node boundaries, down to fewer tokens than one chunk (no node at
    all: attention over the forced keys alone)."""
    _say(f"small token counts {name}")
    cfg = zha.ZhaConfig(capacity=300, **kw)
    K, V, Q, ref = random_inputs(cfg, 1, seed=9)
    weights = cfg.leaf_form == "weights"
    leaf_dtype = "f64" if weights else None
    tol = PAR.OUT_TOL[cfg.dtype]
    p = 0.9
    for N in sizes:
        tree = zha.alloc_tree(cfg)
        zha.build(cfg, K, ref, tree, N)
        buf = zha.alloc_route(cfg, 1, logits=weights)
        zha.route(cfg, tree, N, Q, 1, p, buf, K=K)
        nq = int(buf.layout.n_queries)
        out = torch.full((nq, cfg.head_dim), float("nan"), device="cuda")
        lse = torch.full((nq,), float("nan"), device="cuda")
        ws = torch.empty(zha.attend_workspace_bytes(cfg, 1), dtype=torch.uint8, device="cuda")
        zha.attend(cfg, Q, 1, K, V, N, zha.level1_sel(buf), zha.ZHA_SINK | zha.ZHA_LAST_CHUNK, out, lse, ws,
                   logits=buf.logits)
        torch.cuda.synchronize()
        if N >= cfg.chunk:
            check_tree(cfg, tree, K, ref, N)
        out_c, lse_c = out.cpu().numpy(), lse.cpu().numpy()
        for qi, (b, h, gq, t) in enumerate(query_list(cfg, 1)):
            Kn, Vn, rn = np64(K[b, h, :N]), np64(V[b, h, :N]), np64(ref[h])
            q = np64(Q[b, h, gq, t])
            bits, scores = gpu_levels(cfg, buf, N, qi)
            kept = PAR.gpu_kept_from_bits(bits)
            if N >= cfg.chunk:
                gd = cfg.dtype
                to = O.build_tree(Kn, rn, cfg.chunk, cfg.levels, gd, keep_g=False, leaf_dtype=leaf_dtype)
                PAR.check_route_teacher_forced(q, to, rn, cfg.chunk, p, kept, gd, scores, leaf_dtype=leaf_dtype)
            else:
                assert all(k.size == 0 for k in kept.values()), f"N={N}: a node kept with no complete chunk"
            idx = O.attend_set(kept[1], N, cfg.chunk, True, True)
            o, l = O.attend(q, Kn, Vn, idx)
            np.testing.assert_allclose(out_c[qi], o, rtol=0, atol=tol, err_msg=f"N={N} query {qi}")
            np.testing.assert_allclose(lse_c[qi], l, rtol=0, atol=tol, err_msg=f"N={N} query {qi}")
        PAR.check_stats_all(zha, cfg, buf, N, p, range(nq))


WAVE_CASES = [
    # name, n_tokens, p, keys repeat with period 512 (exact score ties); rows of up to 2,048
    # candidates take the one-wave form, up to 8,192 the one-workgroup row form
    ("ragged", 4096 + 4 * 37 + 3, 0.9, False),
    ("keep-all", 4096, 1.0, False),
    ("ties", 4096, 0.9, True),
    ("ties-small-p", 4096 + 64, 0.05, True),
    ("rows-ragged", 32768 - 1003, 0.9, False),
    ("rows-ties", 32768, 0.9, True),
]


@pytest.mark.parametrize("name,N,p,repeat", WAVE_CASES, ids=[c[0] for c in WAVE_CASES])
def test_wave_select_is_bit_identical(name, N, p, repeat):
    """Rows of at most 2,048 (8,192) candidates at levels with 64 or more
    queries are selected by one wave (one 256-thread workgroup holding the row
    in registers) per query; the same queries routed among fewer queries (one
    1,024-thread workgroup per query, reading the row per pass) must give the
    same bits and statistics on the same score rows."""
    _say(f"wave select {name}")
    cap = N + 256
    cfg = zha.ZhaConfig(batch=1, n_kv_heads=2, q_per_kv=4, head_dim=128, n_ref=16, chunk=4, levels=4, dtype="bf16",
                        capacity=cap)
    K = torch.empty(1, 2, cap, 128, dtype=torch.bfloat16)
    ref = torch.empty(2, 16, 128)
    Q16 = torch.empty(1, 2, 4, 16, 128, dtype=torch.bfloat16)
    for h in range(2):
        k, _, r, q = W.random_cache(cap, 128, 16, "bf16", seed=31 + h, n_queries=64, segment_len=16)
        if repeat:
            k = k[:512].repeat(cap // 512 + 1, 1)[:cap]
        q[::3] = (1.5 * k[(torch.arange(q.shape[0])[::3] * 61) % N].float()).to(torch.bfloat16)
        K[0, h], ref[h], Q16[0, h] = k, r, q.view(4, 16, 128)
    Q1 = Q16[:, :, :, :1].contiguous()
    K, ref, Q1, Q16 = K.cuda(), ref.cuda(), Q1.cuda(), Q16.cuda()
    tree = zha.alloc_tree(cfg)
    zha.build(cfg, K, ref, tree, N)
    b1 = zha.alloc_route(cfg, 1)
    zha.route(cfg, tree, N, Q1, 1, p, b1, K=K)
    b16 = zha.alloc_route(cfg, 16)
    zha.route(cfg, tree, N, Q16, 16, p, b16, K=K)
    torch.cuda.synchronize()
    assert int(b16.layout.n_queries) >= 64
    sizes = O.level_sizes(N, cfg.chunk, cfg.levels)
    n_cut = 0
    for lv in range(1, cfg.levels + 1):
        assert sizes[lv - 1] <= 8192
        s1 = zha.stats_records(b1, lv)
        s16 = zha.stats_records(b16, lv)
        for cache in range(cfg.n_caches):
            for gq in range(cfg.q_per_kv):
                qa = cache * cfg.q_per_kv + gq          # T = 1
                qb = (cache * cfg.q_per_kv + gq) * 16   # T = 16, t = 0
                ba, sa = gpu_levels(cfg, b1, N, qa)
                bb, sb = gpu_levels(cfg, b16, N, qb)
                assert np.array_equal(sa[lv].view(np.int32), sb[lv].view(np.int32)), (lv, qa, "scores")
                assert np.array_equal(ba[lv], bb[lv]), (lv, qa, "bits")
                assert bytes(s1[qa]) == bytes(s16[qb]), (lv, qa, "stats")
                n_cut += s1[qa].cut_id != 2**31 - 1
    if repeat and p < 1.0:
        assert n_cut > 0, "no level split its ties at the cut"
    PAR.check_stats_all(zha, cfg, b16, N, p, range(int(b16.layout.n_queries)))


CUT_CASES = [
    # name, leaf form, n_tokens, p, keys repeat with period 4096 (exact score ties), queries per head
    ("weights", "weights", (1 << 18) - 1003, 0.95, False, 1),
    ("weights2-fused", "weights2", (1 << 18) - 64, 0.9, False, 1),
    ("mean-ties", "mean", 1 << 18, 0.9, True, 1),
    ("mean-small-p", "mean", (1 << 18) - 4 * 37, 0.05, False, 1),
    ("mean-keep-all", "mean", 1 << 17, 1.0, False, 1),
    ("weights-16q", "weights", 1 << 17, 0.95, False, 4),
    # level 1 with 131,008 parents: their bits take 4,094 words of LDS
    ("weights2-2m", "weights2", (1 << 21) - 1003, 0.95, False, 1),
]


@pytest.mark.parametrize("name,leaf_form,N,p,repeat,T", CUT_CASES, ids=[c[0] for c in CUT_CASES])
def test_select_cut_bin_matches_radix(name, leaf_form, N, p, repeat, T, monkeypatch):
    """The one-workgroup select resolves the cut among the candidates of one
    score bin held in LDS (two reads of the row, children of dropped parents
    skipped); forced onto its radix passes (ZHA_SELECT_CUT_CAP=0) it must
    reach the same bits and statistics, and both agree with the selection
    records' exact rule."""
    _say(f"select cut bin {name}")
    cap = max(1 << 18, N)
    cfg = zha.ZhaConfig(batch=1, n_kv_heads=2, q_per_kv=4, head_dim=128, n_ref=16, chunk=4, levels=5, dtype="bf16",
                        capacity=cap, leaf_form=leaf_form)
    K = torch.empty(1, 2, cap, 128, dtype=torch.bfloat16)
    Q = torch.empty(1, 2, 4, T, 128, dtype=torch.bfloat16)
    ref = torch.empty(2, 16, 128)
    for h in range(2):
        k, _, r, q = W.random_cache(cap, 128, 16, "bf16", seed=171 + h, n_queries=4 * T, segment_len=16)
        if repeat:
            k = k[:4096].repeat(cap // 4096, 1)
        n_even = q[::2].shape[0]  # needle queries: half of each head's queries
        pos = (torch.arange(n_even) * 48611 + 777) % N
        q[::2] = (1.5 * k[pos].float()).to(torch.bfloat16)
        K[0, h], ref[h], Q[0, h] = k, r, q.view(4, T, 128)
    K, Q, ref = K.cuda(), Q.cuda(), ref.cuda()
    tree = zha.alloc_tree(cfg)
    zha.build(cfg, K, ref, tree, N)
    bufs = []
    for cut in (None, "0"):
        if cut is None:
            monkeypatch.delenv("ZHA_SELECT_CUT_CAP", raising=False)
        else:
            monkeypatch.setenv("ZHA_SELECT_CUT_CAP", cut)
        buf = zha.alloc_route(cfg, T, logits=cfg.weights, split_select=False)
        buf.sel.fill_(-1)  # every word must be written
        buf.score.zero_()  # entries past a level's nodes are never written
        zha.route(cfg, tree, N, Q, T, p, buf, K=K)
        torch.cuda.synchronize()
        bufs.append(buf)
    monkeypatch.delenv("ZHA_SELECT_CUT_CAP", raising=False)
    a, b = bufs
    assert torch.equal(a.sel, b.sel), "bits differ between the LDS cut bin and the radix passes"
    assert torch.equal(a.stats, b.stats), "statistics differ between the LDS cut bin and the radix passes"
    assert torch.equal(a.score.nan_to_num(), b.score.nan_to_num())
    PAR.check_stats_all(zha, cfg, a, N, p, range(int(a.layout.n_queries)))
