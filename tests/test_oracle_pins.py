"""Pins for the CPU oracle: checks against things other than the oracle itself.

Each pin compares the oracle with a closed form, a library routine (scipy,
torch's attention), a brute-force search, or an invariant of the mathematics.
The planted-mistake tests at the end patch a plausible bug into the oracle and
show that a pin fails.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import scipy.special as sps
import scipy.stats as sst
import torch

import oracle.zha_oracle as O
from tree_indexed_sparse_zha_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_cache(N, d, R, seed, seg=8):
    K, V, ref, Q = W.random_cache(N, d, R, "f32", seed=seed, n_queries=6, segment_len=seg)
    f = lambda t: t.double().numpy()
    return f(K), f(V), f(ref), f(Q)


# ----------------------------------------------------------------------------
# pin checks, written as functions so the planted-mistake tests can reuse them


def pin_dense_at_p1(o=O, N=203, d=16, R=3, C=4, levels=3, seed=1):
    """P1: p = 1 keeps every key; the output is torch's dense attention."""
    K, V, ref, Q = _rand_cache(N, d, R, seed)
    tree = o.build_tree(K, ref, C, levels, "f64", n_tokens=N)
    for q in Q:
        out, lse, idx, recs = o.route_and_attend(q, K, V, tree, ref, C, 1.0, N)
        assert np.array_equal(idx, np.arange(N))
        ref_o = torch.nn.functional.scaled_dot_product_attention(
            torch.tensor(q)[None, None, None], torch.tensor(K)[None, None], torch.tensor(V)[None, None]
        )[0, 0, 0].numpy()
        np.testing.assert_allclose(out, ref_o, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse, sps.logsumexp(K @ q / math.sqrt(d)), rtol=0, atol=1e-12)


def pin_chunk1_exact_logit(o=O, N=37, d=8, R=5, seed=2):
    """P2: C = 1, one level: the plane score is the exact logit q.k/sqrt(d)."""
    K, V, ref, Q = _rand_cache(N, d, R, seed)
    tree = o.build_tree(K, ref, 1, 1, "f64")
    for q in Q:
        s = o.plane_scores(q, tree[0], ref)
        np.testing.assert_allclose(s, K @ q / math.sqrt(d), rtol=0, atol=1e-12)


def pin_merge_equals_direct(o=O, N=150, d=8, R=3, C=3, levels=4, seed=3):
    """P3: every node equals logsumexp / softmax mean over all its keys."""
    K, V, ref, Q = _rand_cache(N, d, R, seed)
    tree = o.build_tree(K, ref, C, levels, "f64", n_tokens=N)
    sizes = o.level_sizes(N, C, levels)
    for lv in range(1, levels + 1):
        assert tree[lv - 1].L.shape[0] == sizes[lv - 1]
        for n in range(sizes[lv - 1]):
            a, b = o.node_token_range(lv, n, C, N)
            z = (K[a:b] @ ref.T) / math.sqrt(d)  # [keys, R]
            L = sps.logsumexp(z, axis=0)
            w = sps.softmax(z, axis=0)
            g = w.T @ K[a:b]
            np.testing.assert_allclose(tree[lv - 1].L[n], L, rtol=0, atol=1e-12)
            np.testing.assert_allclose(tree[lv - 1].g[n], g, rtol=0, atol=1e-12)


def pin_tangent_point(o=O, N=96, d=8, R=4, C=4, levels=3, seed=4):
    """P4: at q = r_j the score is L_j (planes touch there; others lie below)."""
    K, V, ref, Q = _rand_cache(N, d, R, seed)
    tree = o.build_tree(K, ref, C, levels, "f64")
    for lvl in tree:
        for j in range(R):
            s = o.plane_scores(ref[j], lvl, ref)
            # the max over planes at r_j is exactly L_j (convexity: other planes <= f(r_j) = L_j)
            np.testing.assert_allclose(s, lvl.L[:, j], rtol=0, atol=1e-12)


def pin_gibbs_bound(o=O, N=128, d=8, R=4, C=4, levels=3, seed=5):
    """P5: every plane, hence the score, is <= the exact log mass of the node."""
    K, V, ref, Q = _rand_cache(N, d, R, seed)
    tree = o.build_tree(K, ref, C, levels, "f64")
    rng = np.random.default_rng(seed)
    for q in np.concatenate([Q, rng.normal(size=(10, d)) * 2.0]):
        for lv, lvl in enumerate(tree, start=1):
            s = o.plane_scores(q, lvl, ref)
            for n in range(lvl.L.shape[0]):
                a, b = o.node_token_range(lv, n, C, N)
                exact = sps.logsumexp(K[a:b] @ q / math.sqrt(d))
                assert s[n] <= exact + 1e-12


def pin_entropy(o=O, N=128, d=8, R=4, C=4, levels=3, seed=6):
    """P6: c_j is the Shannon entropy of r_j's softmax over the node, in [0, ln|node|]."""
    K, V, ref, Q = _rand_cache(N, d, R, seed)
    tree = o.build_tree(K, ref, C, levels, "f64")
    for lv, lvl in enumerate(tree, start=1):
        for n in range(lvl.L.shape[0]):
            a, b = o.node_token_range(lv, n, C, N)
            z = (K[a:b] @ ref.T) / math.sqrt(d)
            H = sst.entropy(sps.softmax(z, axis=0), axis=0)
            np.testing.assert_allclose(lvl.c[n], H, rtol=0, atol=1e-11)
            assert np.all(lvl.c[n] >= -1e-12) and np.all(lvl.c[n] <= math.log(b - a) + 1e-12)


def pin_zero_reference(o=O, N=64, d=8, C=4, levels=3, seed=7):
    """P7: r = 0 gives uniform weights: c = ln|node|, g = centroid."""
    K, V, ref, Q = _rand_cache(N, d, 1, seed)
    ref = np.zeros((1, d))
    tree = o.build_tree(K, ref, C, levels, "f64")
    for lv, lvl in enumerate(tree, start=1):
        for n in range(lvl.L.shape[0]):
            a, b = o.node_token_range(lv, n, C, N)
            np.testing.assert_allclose(lvl.c[n, 0], math.log(b - a), atol=1e-12)
            np.testing.assert_allclose(lvl.g[n, 0], K[a:b].mean(axis=0), atol=1e-12)
            for q in Q:
                s = o.plane_scores(q, lvl, ref, [n])[0]
                np.testing.assert_allclose(s, math.log(b - a) + q @ K[a:b].mean(0) / math.sqrt(d), atol=1e-12)


def pin_top_p_invariants(o=O, seed=8):
    """P8: kept mass >= pM; removing the smallest kept drops below pM; kept >= dropped."""
    rng = np.random.default_rng(seed)
    for trial in range(200):
        n = int(rng.integers(1, 300))
        s = rng.normal(size=n) * rng.uniform(0.1, 4)
        if trial % 5 == 0:  # exact ties
            s = np.round(s, 1)
        ids = rng.permutation(10 * n)[:n]
        p = float(rng.uniform(0.05, 0.999))
        sel = o.top_p_select(ids, s, p)
        m = np.exp(s - s.max())
        M = m.sum()
        kept = sel.kept
        assert kept.any()
        assert m[kept].sum() >= p * M * (1 - 1e-12)
        smallest = np.min(m[kept])
        assert m[kept].sum() - smallest < p * M * (1 + 1e-12)
        if (~kept).any():
            assert m[~kept].max() <= m[kept].min()
        # ties: among equal scores the lower ids are kept first
        for v in np.unique(s):
            eq = s == v
            if kept[eq].any() and (~kept[eq]).any():
                assert ids[eq & kept].max() < ids[eq & ~kept].min()
    # p = 1 keeps everything, even masses that underflow
    s = np.array([0.0, -800.0, -900.0])
    assert o.top_p_select(np.arange(3), s, 1.0).kept.all()


def pin_brute_force_minimal(o=O, seed=9):
    """P9: on tiny trees the kept set is the minimum-cardinality set with mass >= pM."""
    rng = np.random.default_rng(seed)
    checked = 0
    for trial in range(40):
        N = int(rng.integers(8, 65))
        C, levels, d, R = 2, int(rng.integers(1, 4)), 6, int(rng.integers(1, 4))
        K, V, ref, Q = _rand_cache(N, d, R, 100 + trial, seg=4)
        tree = o.build_tree(K, ref, C, levels, "f64")
        p = float(rng.uniform(0.3, 0.99))
        for q in Q[:2]:
            for rec in o.route(q, tree, ref, C, p):
                sel = rec.sel
                n = sel.ids.size
                if n == 0 or n > 16:
                    continue
                m = sel.mass
                target = p * sel.total
                best = None
                for k in range(1, n + 1):
                    sets = [c for c in itertools.combinations(range(n), k) if m[list(c)].sum() >= target]
                    if sets:
                        best = k
                        break
                assert best == int(sel.kept.sum())
                # with distinct masses the minimal set of max mass is unique: the kept one
                top = np.argsort(-m, kind="stable")[:best]
                if len(np.unique(m)) == n:
                    assert set(top) == set(np.nonzero(sel.kept)[0])
                checked += 1
    assert checked > 50


def pin_structure(o=O, N=1000, d=8, R=3, C=4, levels=4, seed=10):
    """P10: kept nodes lie under kept parents; A holds the sink and the current chunk."""
    K, V, ref, Q = _rand_cache(N + 3, d, R, seed)
    for n_tok in (N, N + 3):
        tree = o.build_tree(K, ref, C, levels, "f64", n_tokens=n_tok)
        for q in Q:
            out, lse, idx, recs = o.route_and_attend(q, K, V, tree, ref, C, 0.8, n_tok)
            for up, down in zip(recs[:-1], recs[1:]):
                parents = set(up.sel.kept_ids.tolist())
                assert all(int(x) // C in parents for x in down.sel.ids)
                assert set(down.sel.kept_ids.tolist()) <= set(down.sel.ids.tolist())
            assert 0 in idx
            last = C * ((n_tok - 1) // C)
            assert set(range(last, n_tok)) <= set(idx.tolist())
            forced = {0} | set(range(last, n_tok))
            rest = [i for i in idx.tolist() if i not in forced]
            chunks = {i // C for i in rest}
            assert all(set(range(c * C, c * C + C)) <= set(idx.tolist()) for c in chunks)


def pin_prefix_stable(o=O, d=8, R=3, C=4, levels=3, seed=11):
    """P11 (oracle side): nodes complete in a prefix are unchanged when keys are appended."""
    K, V, ref, Q = _rand_cache(300, d, R, seed)
    small = o.build_tree(K, ref, C, levels, "f64", n_tokens=170)
    big = o.build_tree(K, ref, C, levels, "f64", n_tokens=300)
    for lv in range(1, levels + 1):
        span = C ** lv
        n_full = 168 // span  # nodes whose whole span lies in the complete chunks of the prefix
        np.testing.assert_array_equal(small[lv - 1].L[:n_full], big[lv - 1].L[:n_full])
        np.testing.assert_array_equal(small[lv - 1].ghat[:n_full], big[lv - 1].ghat[:n_full])


def pin_subset_attention(o=O, N=90, d=8, seed=12):
    """P12: attention over any index set is torch's softmax attention over the gathered keys."""
    K, V, ref, Q = _rand_cache(N, d, 2, seed)
    rng = np.random.default_rng(seed)
    for q in Q:
        idx = np.sort(rng.choice(N, size=int(rng.integers(1, N)), replace=False))
        out, lse = o.attend(q, K, V, idx)
        ref_o = torch.nn.functional.scaled_dot_product_attention(
            torch.tensor(q)[None, None, None], torch.tensor(K[idx])[None, None], torch.tensor(V[idx])[None, None]
        )[0, 0, 0].numpy()
        np.testing.assert_allclose(out, ref_o, rtol=0, atol=1e-12)


PINS = [
    pin_dense_at_p1,
    pin_chunk1_exact_logit,
    pin_merge_equals_direct,
    pin_tangent_point,
    pin_gibbs_bound,
    pin_entropy,
    pin_zero_reference,
    pin_top_p_invariants,
    pin_brute_force_minimal,
    pin_structure,
    pin_prefix_stable,
    pin_subset_attention,
]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin()


# ----------------------------------------------------------------------------
# storage rounding and geometry


def test_bf16_rounding_matches_torch_on_fp32_inputs():
    rng = np.random.default_rng(0)
    x32 = (rng.normal(size=20000) * np.exp(rng.normal(size=20000) * 5)).astype(np.float32)
    mine = O.round_bf16(x32.astype(np.float64))
    theirs = torch.tensor(x32).to(torch.bfloat16).double().numpy()
    np.testing.assert_array_equal(mine, theirs)


def test_bf16_rounding_single_rounding_from_fp64():
    # 1 + 2^-8 is the midpoint between 1 and 1 + 2^-7: ties go to the even mantissa (1.0)
    assert O.round_bf16(np.array([1.0 + 2.0**-8]))[0] == 1.0
    # just above the midpoint rounds up, even though fp32 would first round it to the midpoint
    x = 1.0 + 2.0**-8 + 2.0**-40
    assert O.round_bf16(np.array([x]))[0] == 1.0 + 2.0**-7
    assert O.round_bf16(np.array([3.0 * 2.0**-8 + 1.0]))[0] == 1.0 + 2.0**-6


def test_per_level_p_and_start_level():
    """Depth-aware routing: p per level (index l-1 for level l) and a start
    level.  Keeping everything at the top makes every node one level down a
    candidate, which is routing from that level; a small p at the top only,
    with 1 below, keeps exactly the descendants of the kept top nodes."""
    K, V, ref, Q = _rand_cache(1024, 16, 4, 21)
    C, L = 4, 4
    tree = O.build_tree(K, ref, C, L, "f64")
    for q in Q:
        a = O.route(q, tree, ref, C, [0.9] * (L - 1) + [1.0])
        b = O.route(q, tree, ref, C, 0.9, top=L - 1)
        assert len(b) == L - 1
        for ra, rb in zip(a[1:], b):
            assert ra.level == rb.level
            np.testing.assert_array_equal(ra.sel.kept_ids, rb.sel.kept_ids)
        c = O.route(q, tree, ref, C, [1.0] * (L - 1) + [0.3])
        top_kept = c[0].sel.kept_ids
        assert 0 < top_kept.size < tree[-1].L.shape[0]
        desc = top_kept
        for lv in range(L - 1, 0, -1):
            desc = O.children(desc, C, tree[lv - 1].L.shape[0])
        np.testing.assert_array_equal(c[-1].sel.kept_ids, desc)
        # a scalar p is the same p at every level
        d1 = O.route(q, tree, ref, C, 0.8)
        d2 = O.route(q, tree, ref, C, [0.8] * L)
        for x, y in zip(d1, d2):
            np.testing.assert_array_equal(x.sel.kept_ids, y.sel.kept_ids)
    sched = O.depth_schedule(0.9, 6)
    assert len(sched) == 6 and abs(np.prod(sched) - 0.9) < 1e-12


def test_prefill_is_decode_of_the_prefix():
    """Chunked prefill, causal: the query at position t routes on the tree of
    tokens [0, t] and never attends a later key; at the last position it is
    the decode query; the tree's straddling (partial) nodes are the direct
    statistics of the keys they hold; complete nodes equal the full tree's."""
    K, V, ref, Q = _rand_cache(700, 16, 3, 31)
    C, L, p = 4, 3, 0.9
    full = O.build_tree(K, ref, C, L, "f64", n_tokens=700)
    for t in (0, 2, 3, 4, 63, 64, 65, 130, 255, 256, 450, 699):
        q = Q[t % len(Q)]
        o, lse, idx, recs, tree = O.prefill_query(q, K, V, ref, C, L, p, t)
        assert idx.max() <= t and 0 in idx and t in idx
        if t == 699:
            o2, l2, idx2, _ = O.route_and_attend(q, K, V, full, ref, C, p, 700)
            np.testing.assert_array_equal(idx, idx2)
        sizes = O.level_sizes(t + 1, C, L)
        for lv in range(1, L + 1):
            n = sizes[lv - 1]
            for m in range(n):
                a, b = O.node_token_range(lv, m, C, t + 1)
                Lx, gx = O.node_stats_direct(K, ref, a, b)
                np.testing.assert_allclose(tree[lv - 1].L[m], Lx, rtol=0, atol=1e-12)
                complete = b - a == C**lv
                if complete:
                    np.testing.assert_allclose(tree[lv - 1].L[m], full[lv - 1].L[m], rtol=0, atol=1e-12)


def _e4m3_table():
    """All finite E4M3 values by code, from the bit layout alone: sign, 4
    exponent bits (bias 7), 3 mantissa bits; exponent 0 is subnormal; code
    0x7F / 0xFF (exponent 15, mantissa 7) is NaN."""
    vals = {}
    for code in range(256):
        sgn = -1.0 if code & 0x80 else 1.0
        e, m = (code >> 3) & 15, code & 7
        if e == 15 and m == 7:
            continue
        vals[code] = sgn * (m / 8.0 * 2.0**-6 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7))
    return vals


def _e4m3_brute(x):
    """Nearest E4M3 value by exhaustive search; ties go to the even code."""
    table = _e4m3_table()
    best = min(table.items(), key=lambda kv: (abs(kv[1] - x), kv[0] & 1, kv[0]))
    return best[1]


def test_e4m3_rounding_matches_brute_force():
    table = _e4m3_table()
    pos = sorted(set(abs(v) for v in table.values()))
    assert max(pos) == 448.0 and min(v for v in pos if v > 0) == 2.0**-9 and len(pos) == 127
    xs = [0.0]
    for a, b in zip(pos[:-1], pos[1:]):
        mid = 0.5 * (a + b)
        xs += [a, mid, np.nextafter(mid, 0.0), np.nextafter(mid, 1e9)]
    rng = np.random.default_rng(3)
    xs += list(rng.uniform(-448, 448, 3000)) + list(rng.normal(0, 0.02, 2000))
    xs = np.array(xs + [-v for v in xs])
    got = O.round_e4m3(xs)
    want = np.array([_e4m3_brute(float(x)) for x in xs])
    np.testing.assert_array_equal(np.abs(got), np.abs(want))
    assert np.all((got == 0) | (np.sign(got) == np.sign(xs)))


def test_fp8_rows_scale_and_error():
    rng = np.random.default_rng(4)
    g = rng.normal(size=(50, 16, 64)) * np.exp(rng.normal(size=(50, 16, 1)) * 3)
    g[0, 0] = 0.0
    g[1, 1, :] = 0.0
    g[1, 1, 5] = 2.0**-3  # max exactly a power of two: row max maps to 256
    ghat, scale = O.round_fp8_rows(g)
    m = np.abs(g).max(axis=-1)
    nz = m > 0
    r = m[nz] / scale[nz]
    assert np.all((r > 128) & (r <= 256))
    assert scale[0, 0] == 1.0 and np.all(ghat[0, 0] == 0)
    assert ghat[1, 1, 5] == 2.0**-3 and scale[1, 1] == 2.0**-11
    assert np.all(np.log2(scale) == np.round(np.log2(scale)))
    # each element is within half a spacing of its exact value (spacing 2^-3
    # relative in a binade, 2^-9 * scale below the normal range)
    spacing = np.maximum(2.0 ** (np.floor(np.log2(np.maximum(np.abs(g) / scale[..., None], 2.0**-6))) - 3), 2.0**-9)
    assert np.all(np.abs(ghat - g) <= 0.5 * spacing * scale[..., None] * (1 + 1e-12))


def test_fp8_tree_keeps_tangent_point():
    """With fp8 storage plane j still passes through (r_j, L_j): c absorbs the
    rounding of g.  The other planes are no longer exact tangents, so the max
    at r_j is >= L_j, by at most the rounding's reach."""
    K, V, ref, Q = _rand_cache(256, 16, 4, 11)
    d = ref.shape[1]
    tree = O.build_tree(K, ref, 4, 3, "fp8")
    for lvl in tree:
        assert lvl.scale is not None
        np.testing.assert_array_equal(lvl.ghat, O.round_fp8_rows(lvl.g)[0])
        for j in range(4):
            plane_j = lvl.c[:, j] + lvl.ghat[:, j] @ ref[j] / math.sqrt(d)
            np.testing.assert_allclose(plane_j, lvl.L[:, j], rtol=0, atol=1e-12)
            s = O.plane_scores(ref[j], lvl, ref)
            assert np.all(s >= lvl.L[:, j] - 1e-12)
            reach = np.abs(ref[j] - ref).sum(axis=1).max() * np.abs(lvl.ghat - lvl.g).max() / math.sqrt(d)
            assert np.all(s - lvl.L[:, j] <= reach + 1e-12)


def _e2m1_table():
    """All 16 FP4 E2M1 codes by value, from the bit layout alone: sign, 2
    exponent bits (bias 1), 1 mantissa bit; exponent 0 is subnormal
    (m * 2**-1).  No code is infinite or NaN."""
    vals = {}
    for code in range(16):
        sgn = -1.0 if code & 8 else 1.0
        e, m = (code >> 1) & 3, code & 1
        vals[code] = sgn * (m * 0.5 if e == 0 else (1.0 + m / 2.0) * 2.0 ** (e - 1))
    return vals


def _e2m1_brute(x):
    """Nearest E2M1 value by exhaustive search over the 16 codes, ties to the
    even code, magnitudes past the largest value saturating to it."""
    table = _e2m1_table()
    top = max(table.values())
    x = min(max(x, -top), top)
    best = min(table.items(), key=lambda kv: (abs(kv[1] - x), kv[0] & 1, kv[0]))
    return best[1]


def test_e2m1_rounding_matches_brute_force():
    table = _e2m1_table()
    pos = sorted(set(abs(v) for v in table.values()))
    assert pos == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    xs = [0.0, 6.5, 7.0, 7.999, 8.0, 100.0, 1e30]
    for a, b in zip(pos[:-1], pos[1:]):
        mid = 0.5 * (a + b)
        xs += [a, mid, np.nextafter(mid, 0.0), np.nextafter(mid, 1e9)]
    rng = np.random.default_rng(5)
    xs += list(rng.uniform(-9, 9, 3000)) + list(rng.normal(0, 0.3, 1000))
    xs = np.array(xs + [-v for v in xs])
    got = O.round_e2m1(xs)
    want = np.array([_e2m1_brute(float(x)) for x in xs])
    np.testing.assert_array_equal(np.abs(got), np.abs(want))
    assert np.all((got == 0) | (np.sign(got) == np.sign(xs)))


def test_e2m1_pin_rejects_ties_away_from_zero(monkeypatch):
    """Planted mistake: rounding half away from zero (np.round is half-even,
    floor(a / q + 0.5) is not) must fail the brute-force pin."""
    def bad(x):
        x = np.asarray(x, dtype=np.float64)
        a = np.abs(x)
        _, e = np.frexp(a)
        q = np.ldexp(1.0, np.maximum(e - 1, 0) - 1)
        return np.copysign(np.minimum(np.floor(a / q + 0.5) * q, 6.0), x)

    monkeypatch.setattr(O, "round_e2m1", bad)
    with pytest.raises(AssertionError):
        test_e2m1_rounding_matches_brute_force()


def test_mxfp4_block_scale_rule_and_error():
    """OCP MXFP4: per block of 32 elements an E8M0 scale 2**(floor(log2 max) - 2),
    so the block max sits in [4, 8) scale units; each element is the nearest
    E2M1 value (half a spacing of error) unless it saturates at 6 units."""
    rng = np.random.default_rng(6)
    g = rng.normal(size=(40, 16, 128)) * np.exp(rng.normal(size=(40, 16, 1)) * 2)
    g[0, 0] = 0.0
    g[1, 1, :64] = 0.0
    g[1, 1, 40] = 2.0**-3  # block max exactly a power of two: 4 scale units
    ghat, scale = O.round_mxfp4_rows(g)
    assert scale.shape == (40, 16, 4)
    assert np.all(np.log2(scale) == np.round(np.log2(scale)))
    blocks = np.abs(g).reshape(40, 16, 4, 32)
    m = blocks.max(axis=-1)
    nz = m > 0
    r = m[nz] / scale[nz]
    assert np.all((r >= 4) & (r < 8))
    assert np.all(scale[0, 0] == 2.0**-127) and np.all(ghat[0, 0] == 0)
    assert scale[1, 1, 0] == 2.0**-127 and scale[1, 1, 1] == 2.0**-5 and ghat[1, 1, 40] == 2.0**-3
    sc = np.repeat(scale, 32, axis=-1)
    u = np.abs(g) / sc  # scale units
    spacing = np.where(u < 2, 0.5, np.where(u < 4, 1.0, 2.0))
    err = np.abs(ghat - g) / sc
    ok = np.where(u <= 6, err <= 0.5 * spacing * (1 + 1e-12), np.abs(ghat) / sc == 6.0)
    assert np.all(ok)
    # storage rounding is the same function
    np.testing.assert_array_equal(O.round_storage(g, "fp4"), ghat)


def test_fp4_tree_keeps_tangent_point():
    """With MXFP4 storage plane j still passes through (r_j, L_j): c absorbs
    the rounding of g."""
    K, V, ref, Q = _rand_cache(256, 16, 4, 13)
    ref = np.concatenate([ref, ref], axis=1)  # d = 128 (blocks of 32)
    K = np.concatenate([K, K[::-1]], axis=1)
    d = ref.shape[1]
    tree = O.build_tree(K, ref, 4, 3, "fp4")
    for lvl in tree:
        assert lvl.scale.shape == lvl.L.shape + (d // 32,)
        np.testing.assert_array_equal(lvl.ghat, O.round_mxfp4_rows(lvl.g)[0])
        for j in range(4):
            plane_j = lvl.c[:, j] + lvl.ghat[:, j] @ ref[j] / math.sqrt(d)
            np.testing.assert_allclose(plane_j, lvl.L[:, j], rtol=0, atol=1e-12)


def test_level2_weights_form_is_scored_from_its_own_keys():
    """Levels 1 and 2 held as weights (f64) over bf16 mean keys above: each
    level-2 node's plane j is H(w_j) + E_{w_j}[q . k / sqrt(d)] with w_j the
    softmax of r_j over the node's own keys (the Gibbs form of the tangent
    plane, from the keys directly, not from the merge), while level 3 still
    holds bf16-rounded mean keys."""
    K, V, ref, Q = _rand_cache(16 * 37 + 8, 16, 4, 12)
    N, d = K.shape[0], ref.shape[1]
    tree = O.build_tree(K, ref, 4, 3, "bf16", n_tokens=N, leaf_dtype="f64", level2_dtype="f64")
    lv2 = tree[1]
    n2 = lv2.L.shape[0]
    assert n2 == 38  # 150 chunks: the last level-2 node holds 2 of them
    for n in range(n2):
        keys = K[16 * n : min(16 * n + 16, (N // 4) * 4)]
        z = keys @ ref.T / math.sqrt(d)  # [keys, R]
        w = sps.softmax(z, axis=0)
        H = -(w * np.log(w)).sum(axis=0)
        np.testing.assert_allclose(lv2.c[n], H, rtol=0, atol=1e-12)
        for q in Q[:3]:
            planes = H + w.T @ (keys @ q) / math.sqrt(d)
            np.testing.assert_allclose(O.plane_scores(q, lv2, ref, [n]), [planes.max()], rtol=0, atol=1e-12)
    # level 3 keeps bf16 storage, and its c uses the rounded values
    lv3 = tree[2]
    np.testing.assert_array_equal(lv3.ghat, O.round_bf16(lv3.g))
    assert np.any(lv3.ghat != lv3.g)
    np.testing.assert_allclose(lv3.c, lv3.L - np.einsum("nrd,rd->nr", lv3.ghat, ref) / math.sqrt(d), rtol=0, atol=1e-12)


def test_golden_geometry():
    gold = json.load(open(os.path.join(GOLDEN, "geometry.json")))
    for t in gold["trees"]:
        C, lv = t["chunk"], t["levels"]
        # a top node spans the tokens of C**levels: one top node per top_span keys
        sizes = O.level_sizes(t["top_span"], C, lv)
        assert sizes[-1] == 1 and sizes[0] == t["top_span"] // C
        assert O.level_sizes(t["top_span"] + C, C, lv)[-1] == 2
    anim = gold["animation"]
    C = anim["chunk"]
    counts = {int(k): v for k, v in anim["nodes_per_level"].items()}
    assert O.level_sizes(counts[1] * C, C, 3) == [counts[1], counts[2], counts[3]]
    kept = {int(k): v for k, v in anim["kept"].items()}
    for lv in (2, 1):
        cand = O.children(np.array(kept[lv + 1]), C, counts[lv])
        assert set(kept[lv]) <= set(cand.tolist())


def test_workload_geometry():
    for w in W.WORKLOADS.values():
        assert w.top_span == w.chunk ** w.levels
    assert W.WORKLOADS["deep1m"].top_span == 4096
    assert W.WORKLOADS["wide256k"].top_span == 256
    assert int(W.WORKLOADS["deep1m"].needle_counts().sum()) == 256
    assert int(W.WORKLOADS["deep32k"].needle_counts().sum()) == 32
    assert int(W.WORKLOADS["tiny"].needle_counts().sum()) == 8


def test_tiny_workload_routes_needles():
    """On the tiny workload the oracle finds planted needles through the tree."""
    w = W.WORKLOADS["tiny"]
    b = W.make_batch(w)
    K = b.K[0, 0, : w.n_tokens].double().numpy()
    V = b.V[0, 0, : w.n_tokens].double().numpy()
    ref = b.ref[0].double().numpy()
    tree = O.build_tree(K, ref, w.chunk, w.levels, "f32")
    found = 0
    for t in range(w.queries_per_head):
        q = b.Q[0, 0, 0, t].double().numpy()
        o, lse, idx, recs = O.route_and_attend(q, K, V, tree, ref, w.chunk, w.p[0], w.n_tokens)
        assert 0 < idx.size < w.n_tokens
        for pos in b.needles[0][t]:
            found += int(pos in set(idx.tolist()))
    assert found >= 1


# ----------------------------------------------------------------------------
# planted mistakes: each must make at least one pin fail


def _fails(pin, monkeypatch, name, bad):
    with monkeypatch.context() as mp:
        mp.setattr(O, name, bad)
        with pytest.raises(AssertionError):
            pin()


def test_planted_score_sign_error_is_caught(monkeypatch):
    def bad(q, level, ref, ids=None):
        q = np.asarray(q, float)
        ids = np.arange(level.L.shape[0]) if ids is None else np.asarray(ids)
        d = q.shape[-1]
        planes = level.L[ids] + np.einsum("nrd,rd->nr", level.ghat[ids], q[None] + ref) / math.sqrt(d)
        return planes.max(1)

    _fails(pin_tangent_point, monkeypatch, "plane_scores", bad)


def test_planted_missing_scale_is_caught(monkeypatch):
    def bad(q, level, ref, ids=None):
        q = np.asarray(q, float)
        ids = np.arange(level.L.shape[0]) if ids is None else np.asarray(ids)
        planes = level.L[ids] + np.einsum("nrd,rd->nr", level.ghat[ids], q[None] - ref)
        return planes.max(1)

    _fails(pin_chunk1_exact_logit, monkeypatch, "plane_scores", bad)


def test_planted_merge_weight_error_is_caught(monkeypatch):
    orig = O._logsumexp

    def bad_lse(a, axis):  # mean instead of logsumexp
        return np.mean(a, axis=axis)

    _fails(pin_merge_equals_direct, monkeypatch, "_logsumexp", bad_lse)


def test_planted_selection_order_error_is_caught(monkeypatch):
    orig = O.top_p_select

    def bad(ids, score, p):  # keeps the lowest-scoring candidates first
        return orig(ids, -np.asarray(score), p)

    _fails(pin_top_p_invariants, monkeypatch, "top_p_select", bad)


def test_planted_children_index_error_is_caught(monkeypatch):
    def bad(ids, chunk, n_below):
        ids = np.asarray(ids, dtype=np.int64)
        kids = (ids[:, None] + np.arange(chunk)[None, :]).reshape(-1)
        return np.unique(kids[kids < n_below])

    _fails(pin_structure, monkeypatch, "children", bad)


def test_planted_sink_dropped_is_caught(monkeypatch):
    orig = O.attend_set

    def bad(kept, n, chunk, sink=True, last_chunk=True):
        return orig(kept, n, chunk, False, last_chunk)

    _fails(pin_structure, monkeypatch, "attend_set", bad)
