"""The parity checker itself, on the CPU: planted selection mistakes must fail.

The set-parity rule (tests/parity.py) exempts a differing node only if one
of its cumulative-mass boundaries lies within 1e-4 of p (widened by the
measured score error's effect on mass ratios) or if a candidate on the other
side of the cut has a score within twice the measured score error.  These
tests feed the checker selections that a correct GPU could produce (pass)
and selections with plausible select bugs (fail): the cut node dropped
("keep iff prefix_incl < pM"), one node too many, a swap of nodes far apart
in score.  check_select_stats is fed records made by a host rendering of
the kernels' documented fixed-point rule, and the same records with the
same bugs.
"""
import math
import types

import numpy as np
import pytest

import oracle.zha_oracle as O
from tests import parity as PAR


def _tree(seed=0, N=4096, C=4, L=3, d=64, R=4):
    rng = np.random.default_rng(seed)
    seg = np.repeat(rng.normal(size=(N // 256, d)), 256, axis=0)
    K = seg + 0.5 * rng.normal(size=(N, d))
    ref = rng.normal(size=(R, d)) / math.sqrt(d)
    return K, ref, O.build_tree(K, ref, C, L, "f32")


def _oracle_kept(q, tree, ref, C, p):
    return {r.level: r.sel.kept_ids for r in O.route(q, tree, ref, C, p)}


def _boundary_margin(sel, p):
    """Distance of the cut node's boundaries from p (fraction of M)."""
    cut = sel.order[int(sel.kept.sum()) - 1]
    lo = sel.prefix_excl[cut] / sel.total
    hi = (sel.prefix_excl[cut] + sel.mass[cut]) / sel.total
    return cut, min(abs(lo - p), abs(hi - p))


def test_oracle_routing_passes_itself():
    K, ref, tree = _tree()
    rng = np.random.default_rng(1)
    for _ in range(8):
        q = rng.normal(size=64)
        kept = _oracle_kept(q, tree, ref, 4, 0.9)
        reps = PAR.check_route_teacher_forced(q, tree, ref, 4, 0.9, kept, "f32")
        assert all(r.n_diff == 0 for r in reps)


def _first_clear_cut(tree, ref, p, seed=2):
    """A query and level whose cut node has both boundaries well away from p."""
    rng = np.random.default_rng(seed)
    for _ in range(50):
        q = rng.normal(size=64)
        for r in O.route(q, tree, ref, 4, p):
            if r.sel.kept.sum() >= 2:
                cut, margin = _boundary_margin(r.sel, p)
                s = np.sort(r.sel.score)
                if margin > 1e-3 and np.min(np.abs(np.diff(s))) > 1e-5:
                    return q, r.level, r.sel, cut
    raise AssertionError("no query with a clear cut")


def test_dropping_the_cut_node_fails():
    """'keep iff prefix_incl < pM' drops the cut node: not exempt."""
    K, ref, tree = _tree()
    p = 0.9
    q, lv, sel, cut = _first_clear_cut(tree, ref, p)
    kept = _oracle_kept(q, tree, ref, 4, p)
    bad = dict(kept)
    bad[lv] = np.setdiff1d(kept[lv], [sel.ids[cut]])
    # teacher forcing: the levels below see the candidates of the bad level
    for below in range(lv - 1, 0, -1):
        cand = O.children(bad[below + 1], 4, tree[below - 1].L.shape[0])
        s = O.plane_scores(q, tree[below - 1], ref, cand)
        bad[below] = O.top_p_select(cand, s, p).kept_ids
    with pytest.raises(AssertionError):
        PAR.check_route_teacher_forced(q, tree, ref, 4, p, bad, "f32")


def test_one_node_too_many_fails():
    K, ref, tree = _tree()
    p = 0.9
    q, lv, sel, cut = _first_clear_cut(tree, ref, p)
    kept = _oracle_kept(q, tree, ref, 4, p)
    nxt = sel.order[int(sel.kept.sum())] if sel.kept.sum() < sel.ids.size else None
    assert nxt is not None
    bad = dict(kept)
    bad[lv] = np.sort(np.r_[kept[lv], sel.ids[nxt]])
    for below in range(lv - 1, 0, -1):
        cand = O.children(bad[below + 1], 4, tree[below - 1].L.shape[0])
        s = O.plane_scores(q, tree[below - 1], ref, cand)
        bad[below] = O.top_p_select(cand, s, p).kept_ids
    with pytest.raises(AssertionError):
        PAR.check_route_teacher_forced(q, tree, ref, 4, p, bad, "f32")


def _sel(scores, p):
    ids = np.arange(len(scores))
    return O.top_p_select(ids, np.asarray(scores, float), p)


def test_swap_rule_needs_close_scores():
    # two candidates 1e-7 apart straddle the cut: a swap is explained by a
    # score error of 1e-6, not by a score error of 0
    scores = [3.0, 2.5, 1.0, 1.0 + 1e-7, -2.0, -3.0]
    sel = _sel(scores, 0.9)
    assert sel.kept[3] and not sel.kept[2]
    why = PAR.ambiguous_nodes(sel, 0.9, 1e-6, {2, 3})
    assert why[2] == "swap" and why[3] == "swap"
    why0 = PAR.ambiguous_nodes(sel, 0.9, 0.0, {2, 3})
    assert why0[2] == "" and why0[3] == ""
    # nodes far apart in score are never a swap
    why_far = PAR.ambiguous_nodes(sel, 0.9, 1e-6, {1, 4})
    assert why_far[1] == "" and why_far[4] == ""


def test_boundary_rule_is_the_target_window():
    # cut node with prefix_excl / M within 1e-4 of p: exempt; a margin of 1e-3: not
    m = np.array([0.5, 0.39995, 0.1, 0.00005])  # prefixes 0, .5, .89995, .99995
    scores = np.log(m)
    sel = _sel(scores, 0.9)
    why = PAR.ambiguous_nodes(sel, 0.9, 0.0, {2})
    assert why[2] == "boundary"
    m2 = np.array([0.5, 0.399, 0.1, 0.001])
    sel2 = _sel(np.log(m2), 0.9)
    assert PAR.ambiguous_nodes(sel2, 0.9, 0.0, {2})[2] == ""


# ---------------------------------------------------------------------------
# the selection records


def _kernel_record(row, p, drop_cut=False, extra=False):
    """Host rendering of the select kernels' rule: fixed-point masses
    round(exp(s - max) * 2^shift), P = ceil(p * M), keep the descending
    prefix (ties to lower ids) up to the first rank whose inclusive mass
    reaches P; returns (record, bits)."""
    row = np.asarray(row, np.float32)
    cand = np.isfinite(row)
    n = row.size
    lg = 0
    while (1 << lg) < n:
        lg += 1
    shift = 62 - lg
    mx = float(row[cand].max())
    m = np.zeros(n)
    m[cand] = PAR.fixed_masses(row[cand], mx, shift)
    M = int(m.sum())
    P = min(max(math.ceil(float(np.float32(p)) * M), 1), M)
    ids = np.nonzero(cand)[0]
    order = ids[np.lexsort((ids, -row[ids]))]
    cum = np.cumsum(m[order])
    k = int(np.searchsorted(cum, P) + 1)  # first rank with cum >= P
    if drop_cut:
        k -= 1
    if extra:
        k += 1
    keep = order[:k]
    bits = np.zeros(n, bool)
    bits[keep] = True
    last = keep[-1]
    tau = int(PAR.order_key(row[last]))
    same = keep[PAR.order_key(row[keep]) == tau]
    ties_all = ids[PAR.order_key(row[ids]) == tau]
    cut_id = 2**31 - 1 if same.size == ties_all.size else int(same.max()) + 1
    rec = types.SimpleNamespace(max_score=mx, n_cand=int(cand.sum()), n_kept=int(k), cut_key=tau, cut_id=cut_id,
                                shift=shift, mass_total=M, mass_kept=int(m[keep].sum()))
    return rec, bits


@pytest.mark.parametrize("seed", range(4))
def test_kernel_rule_passes_the_stats_check(seed):
    rng = np.random.default_rng(seed)
    row = rng.normal(size=500).astype(np.float32) * 3
    row[rng.random(500) < 0.3] = -np.inf
    row[10] = row[11] = row[12] = row[40]  # exact ties
    for p in (0.5, 0.9, 0.95, 0.999):
        rec, bits = _kernel_record(row, p)
        PAR.check_select_stats(rec, row, bits, p)


def test_stats_check_catches_select_bugs():
    rng = np.random.default_rng(7)
    row = rng.normal(size=300).astype(np.float32) * 2
    for p in (0.6, 0.9):
        rec, bits = _kernel_record(row, p, drop_cut=True)
        with pytest.raises(AssertionError):
            PAR.check_select_stats(rec, row, bits, p)
        rec, bits = _kernel_record(row, p, extra=True)
        with pytest.raises(AssertionError):
            PAR.check_select_stats(rec, row, bits, p)
        rec, bits = _kernel_record(row, p)
        bits2 = bits.copy()
        bits2[np.nonzero(~bits)[0][0]] = True  # a bit outside the cut rule
        with pytest.raises(AssertionError):
            PAR.check_select_stats(rec, row, bits2, p)
