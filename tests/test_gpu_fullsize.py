"""GPU parity at full size, in both storage forms the bench can time.

The bench times the 1M-token workload with levels 1 and 2 scored from their
keys (leaf form "weights2": one pass reads a candidate level-2 node's keys,
writes its chunks' level-1 scores and the keys' logits, and attention reads
those logits), with the capacity it allocates (room for every warm-up and
timed append step) and the logits buffer it passes.  Each test runs both
that form and the leaf-weights form ("weights").

1M-token deep tree (8 x 8 caches, one 4,096-token append step, p = 0.95):
the oracle builds the full fp64 tree of two sampled caches and checks
routing teacher-forced, the GPU's selection records and attention for all
their queries.

10M-token deep tree (2 x 2 caches): the oracle cannot hold fp64 trees of
that size, so the checks use properties that hold at any size:
  * sampled nodes of every level against statistics computed directly from
    their keys (merge exactness makes these the defined values);
  * sampled candidate scores against the oracle's plane scores of those nodes;
  * the top-p selection re-done in fp64 from the GPU's own scores: every
    differing node must have a cumulative-mass boundary within 1e-4 of p;
  * the GPU's selection records (kept mass, minimality, cut rule);
  * attention over the GPU's routed set against the oracle.
"""
import gc
import math
import sys

import numpy as np
import pytest
import torch

import oracle.zha_oracle as O
from tests import parity as PAR
from tree_indexed_sparse_zha_amd import workloads as W
from tree_indexed_sparse_zha_amd import zha

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[gpu-fullsize] {msg}", flush=True)
    sys.stdout.flush()


def np64(t):
    return t.detach().to(torch.float64).cpu().numpy()


def _cfg(w, capacity, leaf_form="weights"):
    return zha.ZhaConfig(
        w.batch, w.n_kv_heads, w.q_per_kv, w.head_dim, w.n_ref, w.chunk, w.levels, w.dtype, capacity, leaf_form
    )


def _levels(cfg, buf, N, qi):
    rl = buf.layout
    sizes = O.level_sizes(N, cfg.chunk, cfg.levels)
    bits, scores = {}, {}
    for lv in range(1, cfg.levels + 1):
        i = lv - 1
        w = int(rl.words[i])
        words = buf.sel[int(rl.sel_offset[i]) + qi * w : int(rl.sel_offset[i]) + (qi + 1) * w]
        bits[lv] = zha.unpack_bits(words.cpu(), sizes[i]).numpy()
        st = int(rl.score_stride[i])
        off = int(rl.score_offset[i]) + qi * st
        scores[lv] = buf.score[off : off + sizes[i]].cpu().numpy()
    return bits, scores


FORMS = ["weights2", "weights"]
# the bench's form with fp8 rows or MXFP4 blocks from level 3 up (the low-precision router variants)
FORMS_1M = FORMS + ["weights2-fp8", "weights2-fp4"]
# the bench's default run: 2 warm-up + 8 timed append steps sized into the capacity
BENCH_STEPS = 10


def _run_step(cfg, b, N0, A, T, p):
    """The bench's step: build over N0, append A, route (keeping the level-1
    logits), attend (reading them)."""
    tree = zha.alloc_tree(cfg)
    zha.build(cfg, b.K, b.ref, tree, N0)
    if A:
        zha.append(cfg, b.K, b.ref, tree, N0, A)
    N = N0 + A
    buf = zha.alloc_route(cfg, T, logits=True)
    zha.route(cfg, tree, N, b.Q, T, p, buf, K=b.K)
    nq = int(buf.layout.n_queries)
    out = torch.empty(nq, cfg.head_dim, device="cuda")
    lse = torch.empty(nq, device="cuda")
    ws = torch.empty(zha.attend_workspace_bytes(cfg, T), dtype=torch.uint8, device="cuda")
    zha.attend(cfg, b.Q, T, b.K, b.V, N, zha.level1_sel(buf), zha.ZHA_SINK | zha.ZHA_LAST_CHUNK, out, lse, ws,
               logits=buf.logits)
    torch.cuda.synchronize()
    return tree, buf, out, lse


@pytest.mark.parametrize("form", FORMS_1M)
def test_deep1m_full_size_two_caches(form):
    w = W.WORKLOADS["deep1m"]
    N0, A, T, p = w.n_tokens, w.append_tokens, w.queries_per_head, 0.95
    leaf_form, _, g8 = form.partition("-")
    cfg = _cfg(w, N0 + BENCH_STEPS * A, leaf_form)
    if g8:
        cfg.g_dtype = g8  # fp8 rows or MXFP4 blocks from level 3 up
    gd = g8 or w.dtype
    _say(f"deep1m {form}: generating and running the bench step")
    b = W.make_batch(w, device="cuda", capacity=cfg.capacity, append_steps=1)
    tree, buf, out, lse = _run_step(cfg, b, N0, A, T, p)
    assert buf.logits is not None
    N = N0 + A
    QC = cfg.q_per_kv * T
    l2d = "f64" if cfg.weight_keys(2) else None
    PAR.check_stats_all(zha, cfg, buf, N, p, [c * QC + i for c in (0, cfg.n_caches - 1) for i in range(QC)])
    out_c, lse_c = out.cpu().numpy(), lse.cpu().numpy()
    for cache in (0, cfg.n_caches - 1):
        bb, h = divmod(cache, cfg.n_kv_heads)
        _say(f"deep1m {form}: oracle tree of cache {cache}")
        Kn, Vn, rn = np64(b.K[bb, h, :N]), np64(b.V[bb, h, :N]), np64(b.ref[h])
        to = O.build_tree(Kn, rn, w.chunk, w.levels, gd, keep_g=False, leaf_dtype="f64", level2_dtype=l2d)
        # sampled tree fields, including the appended span
        sizes = O.level_sizes(N, w.chunk, w.levels)
        for lv in range(1, w.levels + 1):
            got = zha.read_level(cfg, tree, lv, sizes[lv - 1])
            n = sizes[lv - 1]
            idx = np.unique(np.r_[0, n // 2, n - 1, np.random.default_rng(lv).integers(0, n, 16)])
            np.testing.assert_allclose(np64(got["L"][cache][idx]), to[lv - 1].L[idx], rtol=1e-5, atol=3e-5)
            if "g" in got:
                # c against the oracle's L and the GPU's own stored g (an fp8 or bf16 rounding-boundary
                # flip of g moves both sides' c alike)
                gg = np64(got["g"][cache][idx])
                c_ref = to[lv - 1].L[idx] - np.einsum("nrd,rd->nr", gg, rn) / math.sqrt(w.head_dim)
                np.testing.assert_allclose(np64(got["c"][cache][idx]), c_ref, rtol=1e-5, atol=5e-5)
            else:
                np.testing.assert_allclose(np64(got["c"][cache][idx]), to[lv - 1].c[idx], rtol=1e-5, atol=2e-4)
        for qi_local in range(QC):
            gq, t = divmod(qi_local, T)
            qi = cache * QC + qi_local
            q = np64(b.Q[bb, h, gq, t])
            bits, scores = _levels(cfg, buf, N, qi)
            kept = PAR.gpu_kept_from_bits(bits)
            reps = PAR.check_route_teacher_forced(q, to, rn, w.chunk, p, kept, gd, scores, leaf_dtype="f64",
                                                  level2_dtype=l2d)
            idx = O.attend_set(kept[1], N, w.chunk)
            o, l = O.attend(q, Kn, Vn, idx)
            np.testing.assert_allclose(out_c[qi], o, rtol=0, atol=PAR.OUT_TOL[w.dtype])
            np.testing.assert_allclose(lse_c[qi], l, rtol=0, atol=PAR.OUT_TOL[w.dtype])
            _say(f"deep1m {form} cache {cache} query {qi_local}: share {idx.size / N:.3f}, level diffs "
                 f"{[r.n_diff for r in reps]}, score errors {[f'{r.max_score_err:.1e}' for r in reps]}")
        del to
        gc.collect()
    del tree, buf, b
    torch.cuda.empty_cache()


@pytest.mark.parametrize("leaf_form", FORMS)
def test_deep10m_full_size_sampled(leaf_form):
    w = W.WORKLOADS["deep10m"]
    N, T, p = w.n_tokens, w.queries_per_head, w.p[0]
    cfg = _cfg(w, N, leaf_form)
    _say(f"deep10m {leaf_form}: generating and running build + route + attend")
    b = W.make_batch(w, device="cuda", capacity=N)
    tree, buf, out, lse = _run_step(cfg, b, N, 0, T, p)
    QC = cfg.q_per_kv * T
    # levels stored as weights of their own keys: planes with g unrounded
    wl = 2 if cfg.weight_keys(2) else 1
    PAR.check_stats_all(zha, cfg, buf, N, p, range(int(buf.layout.n_queries)))
    sizes = O.level_sizes(N, w.chunk, w.levels)
    cache = cfg.n_caches - 1
    bb, h = divmod(cache, cfg.n_kv_heads)
    K = b.K[bb, h, :N]
    rn = np64(b.ref[h])
    rng = np.random.default_rng(7)
    d = w.head_dim
    # 1) sampled nodes of every level against their keys
    for lv in range(1, w.levels + 1):
        n = sizes[lv - 1]
        idx = np.unique(np.r_[0, n - 1, rng.integers(0, n, 12)])
        got = zha.read_level(cfg, tree, lv, n)
        for node in idx:
            a0, a1 = O.node_token_range(lv, int(node), w.chunk, N)
            Lx, gx = O.node_stats_direct(np64(K[a0:a1]), rn, 0, a1 - a0)
            np.testing.assert_allclose(np64(got["L"][cache][node]), Lx, rtol=1e-5, atol=3e-5)
            # levels held as weights keep g unrounded; upper levels store bf16 g
            gh = gx if lv <= wl else O.round_storage(gx, w.dtype)
            c_ref = Lx - np.einsum("rd,rd->r", gh, rn) / math.sqrt(d)
            np.testing.assert_allclose(np64(got["c"][cache][node]), c_ref, rtol=1e-5, atol=2e-4)
    _say("deep10m: sampled nodes ok")
    out_c = out.cpu().numpy()
    Kn, Vn = np64(K), np64(b.V[bb, h, :N])
    for qi_local in range(QC):
        gq, t = divmod(qi_local, T)
        qi = cache * QC + qi_local
        q = np64(b.Q[bb, h, gq, t])
        bits, scores = _levels(cfg, buf, N, qi)
        for lv in range(w.levels, 0, -1):
            n = sizes[lv - 1]
            cand = np.arange(n) if lv == w.levels else O.children(np.nonzero(bits[lv + 1])[0], w.chunk, n)
            s_gpu = scores[lv][cand].astype(np.float64)
            assert np.all(np.isfinite(s_gpu))
            assert np.all(~np.isfinite(np.delete(scores[lv], cand)))  # non-candidates are -inf
            # 2) sampled candidate scores against the oracle's planes of directly built nodes
            for m in rng.choice(cand, size=min(8, cand.size), replace=False):
                a0, a1 = O.node_token_range(lv, int(m), w.chunk, N)
                Lx, gx = O.node_stats_direct(Kn[a0:a1], rn, 0, a1 - a0)
                gh = gx if lv <= wl else O.round_storage(gx, w.dtype)
                lvl = O.Level(L=Lx[None], g=None, ghat=gh[None], c=None)
                s_or = O.plane_scores(q, lvl, rn)[0]
                eps = PAR.eps_score("f64" if lv <= wl else w.dtype, q, lvl)
                assert abs(scores[lv][m] - s_or) <= eps, (lv, m, scores[lv][m], s_or)
            # 3) the selection re-done in fp64 from the GPU's own scores
            sel = O.top_p_select(cand, s_gpu, p)
            diff = set(sel.kept_ids.tolist()) ^ set(np.nonzero(bits[lv])[0].tolist())
            pos = {int(x): i for i, x in enumerate(cand.tolist())}
            assert len(diff) <= PAR.MAX_DIFF, (lv, len(diff))
            for m in diff:
                i = pos[m]
                lo = sel.prefix_excl[i] / sel.total
                hi = (sel.prefix_excl[i] + sel.mass[i]) / sel.total
                assert min(abs(lo - p), abs(hi - p)) <= PAR.MASS_WINDOW, (lv, m, lo, hi)
        # 4) attention over the GPU's set
        idx = O.attend_set(np.nonzero(bits[1])[0], N, w.chunk)
        o, l = O.attend(q, Kn, Vn, idx)
        np.testing.assert_allclose(out_c[qi], o, rtol=0, atol=PAR.OUT_TOL[w.dtype])
        _say(f"deep10m {leaf_form} query {qi_local}: share {idx.size / N:.3f}")
    del tree, buf, b
    torch.cuda.empty_cache()
