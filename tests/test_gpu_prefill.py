"""GPU parity of chunked prefill (causal) against the oracle.

A block of T positions [N - T, N) of every sequence is routed and attended at
once; query t of a head sits at position N - T + t and must match the oracle
decoding against the tree of its own prefix of N - T + t + 1 tokens
(teacher-forced routing, attention over the GPU's set).  The partial nodes
of those prefix trees come from the spine; their log masses are also checked
directly against the statistics of the keys they hold.
"""
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
    print(f"[gpu-prefill] {msg}", flush=True)
    sys.stdout.flush()


def np64(t):
    return t.detach().to(torch.float64).cpu().numpy()


CASES = [
    # name, cfg kwargs, N, T, p (, queries sampled per cache, caches checked)
    ("weights-C4-d128", dict(batch=1, n_kv_heads=2, q_per_kv=2, head_dim=128, n_ref=16, chunk=4, levels=4,
                             leaf_form="weights"), 3000, 96, 0.9),
    ("mean-fp8-C8-d64", dict(batch=1, n_kv_heads=1, q_per_kv=2, head_dim=64, n_ref=5, chunk=8, levels=3,
                             g_dtype="fp8"), 2100, 64, 0.85),
    ("weights-C16-start", dict(batch=1, n_kv_heads=1, q_per_kv=2, head_dim=128, n_ref=4, chunk=16, levels=2,
                               leaf_form="weights"), 300, 300, 0.9),
    # enough tiles that levels 1 and 2 walk several query blocks per workgroup
    ("weights-many-tiles", dict(batch=1, n_kv_heads=4, q_per_kv=2, head_dim=128, n_ref=16, chunk=4, levels=5,
                                leaf_form="weights"), 65536 + 100, 16, 0.9, 2, [0, 3]),
]


def _inputs(cfg, N, T, seed):
    """Clustered keys per cache; half of the queries point at an earlier key."""
    B, H, G, d = cfg.batch, cfg.n_kv_heads, cfg.q_per_kv, cfg.head_dim
    K = torch.empty(B, H, N, d)
    V = torch.empty(B, H, N, d)
    Q = torch.empty(B, H, G, T, d)
    ref = torch.empty(H, cfg.n_ref, d)
    g = torch.Generator().manual_seed(seed)
    for b in range(B):
        for h in range(H):
            k, v, r, q = W.random_cache(N, d, cfg.n_ref, "bf16", seed=seed + 7 * b + h, n_queries=G * T,
                                        segment_len=64)
            K[b, h], V[b, h], ref[h] = k.float(), v.float(), r
            q = q.float().view(G, T, d)
            for t in range(0, T, 2):
                pos = N - T + t
                src = int(torch.randint(0, pos + 1, (1,), generator=g))
                q[:, t] = 1.5 * K[b, h, src]
            Q[b, h] = q
    bf = torch.bfloat16
    return K.to(bf).cuda(), V.to(bf).cuda(), Q.to(bf).cuda(), ref.cuda()


def _level_rows(cfg, buf, N, qi):
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


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_prefill_matches_prefix_decode(case):
    name, kw, N, T, p = case[:5]
    n_pick = case[5] if len(case) > 5 else 10
    caches_checked = case[6] if len(case) > 6 else None
    _say(f"prefill {name}")
    cfg = zha.ZhaConfig(dtype="bf16", capacity=N, **kw)
    K, V, Q, ref = _inputs(cfg, N, T, seed=41)
    C, L = cfg.chunk, cfg.levels
    weights = cfg.leaf_form == "weights"
    gd = "fp8" if cfg.g_dtype == "fp8" else "bf16"
    tree = zha.alloc_tree(cfg)
    zha.build(cfg, K, ref, tree, N)
    spine = zha.alloc_spine(cfg, T)
    zha.build_spine(cfg, K, ref, spine, N, T)
    buf = zha.alloc_route(cfg, T, logits=weights)
    zha.route_prefill(cfg, tree, spine, N, Q, T, p, buf, K=K)
    nq = int(buf.layout.n_queries)
    out = torch.full((nq, cfg.head_dim), float("nan"), device="cuda")
    lse = torch.full((nq,), float("nan"), device="cuda")
    dense = torch.full((nq, cfg.head_dim), float("nan"), device="cuda")
    ws = torch.empty(zha.attend_workspace_bytes(cfg, T), dtype=torch.uint8, device="cuda")
    flags = zha.ZHA_SINK | zha.ZHA_LAST_CHUNK | zha.ZHA_CAUSAL
    zha.attend(cfg, Q, T, K, V, N, zha.level1_sel(buf), flags, out, lse, ws, logits=buf.logits)
    zha.attend(cfg, Q, T, K, V, N, None, zha.ZHA_ALL_KEYS | zha.ZHA_CAUSAL, dense, None, ws)
    torch.cuda.synchronize()
    out_c, lse_c, dense_c = out.cpu().numpy(), lse.cpu().numpy(), dense.cpu().numpy()
    QC = cfg.q_per_kv * T
    tol = PAR.OUT_TOL["bf16"]
    rng = np.random.default_rng(3)
    for cache in (caches_checked if caches_checked is not None else range(cfg.n_caches)):
        b, h = divmod(cache, cfg.n_kv_heads)
        Kn, Vn, rn = np64(K[b, h]), np64(V[b, h]), np64(ref[h])
        picks = sorted(set([0, QC - 1, QC // 2] + rng.choice(QC, size=min(n_pick, QC), replace=False).tolist()))
        for ql in picks:
            gq, t = divmod(ql, T)
            pos = N - T + t
            qi = cache * QC + ql
            q = np64(Q[b, h, gq, t])
            # dense causal decode over [0, pos]
            od, _ = O.attend(q, Kn, Vn, np.arange(pos + 1))
            np.testing.assert_allclose(dense_c[qi], od, rtol=0, atol=tol, err_msg=f"dense causal q{ql}")
            sizes = O.level_sizes(pos + 1, C, L)
            bits, scores = _level_rows(cfg, buf, N, qi)
            if sizes[0] == 0:
                idx = O.attend_set(np.zeros(0, np.int64), pos + 1, C)
            else:
                tree_t = O.build_tree(Kn[: pos + 1], rn, C, L, gd, n_tokens=pos + 1, keep_g=False,
                                      leaf_dtype="f64" if weights else None)
                kept, sc = {}, {}
                for lv in range(1, L + 1):
                    n = sizes[lv - 1]
                    assert not bits[lv][n:].any(), f"q{ql} level {lv}: bit beyond the prefix"
                    assert np.all(np.isneginf(scores[lv][n:])), f"q{ql} level {lv}: score beyond the prefix"
                    kept[lv] = np.nonzero(bits[lv][:n])[0].astype(np.int64)
                    sc[lv] = scores[lv][:n]
                PAR.check_route_teacher_forced(q, tree_t, rn, C, p, kept, gd, sc,
                                               leaf_dtype="f64" if weights else None)
                idx = O.attend_set(kept[1], pos + 1, C)
            assert idx.max() <= pos
            o, l = O.attend(q, Kn, Vn, idx)
            np.testing.assert_allclose(out_c[qi], o, rtol=0, atol=tol, err_msg=f"q{ql}")
            np.testing.assert_allclose(lse_c[qi], l, rtol=0, atol=tol, err_msg=f"q{ql}")
    # the GPU's own selection records of every query of the block
    PAR.check_stats_all(zha, cfg, buf, N, p, range(nq))
    _say(f"prefill {name}: {cfg.n_caches} caches checked")


def test_spine_partial_nodes_are_key_statistics():
    """The spine's partial nodes hold the log mass of exactly the complete
    chunks they contain (checked on the L field of every record written)."""
    cfg = zha.ZhaConfig(batch=1, n_kv_heads=1, q_per_kv=1, head_dim=128, n_ref=8, chunk=4, levels=4, dtype="bf16",
                        capacity=1500, leaf_form="weights")
    N, T = 1500, 200
    K, V, Q, ref = _inputs(cfg, N, T, seed=5)
    spine = zha.alloc_spine(cfg, T)
    spine.fill_(0xFF)  # NaN pattern: records never written stay NaN
    zha.build_spine(cfg, K, ref, spine, N, T)
    torch.cuda.synchronize()
    C, L, R, d = cfg.chunk, cfg.levels, cfg.n_ref, cfg.head_dim
    k0 = (N - T + 1) // C
    states = T // C + 2
    rec = (R * d * 2 + 12 * R + 15) // 16 * 16
    raw = spine.cpu()
    Kn, rn = np64(K[0, 0]), np64(ref[0])
    n_checked = 0
    for k in range(k0, N // C + 1):
        for lv in range(2, L + 1):
            per = C ** (lv - 1)  # chunks under a level-lv node
            off = ((k - k0) * (L - 1) + (lv - 2)) * rec
            Lg = raw[off + R * d * 2 : off + R * d * 2 + 4 * R].view(torch.float32).double().numpy()
            if k % per == 0:
                continue  # complete node: lives in the tree, no record
            a = (k - 1) // per * per * C
            Lx, _ = O.node_stats_direct(Kn, rn, a, k * C)
            np.testing.assert_allclose(Lg, Lx, rtol=1e-5, atol=3e-5, err_msg=f"state {k} level {lv}")
            n_checked += 1
    assert n_checked > 100
    assert states >= N // C + 1 - k0
