"""Parity helpers: compare the HIP path with the CPU oracle.

Set parity is judged teacher-forced, level by level: at each level the oracle
re-selects from the GPU's own candidate set (children of the GPU's kept
parents) using its own fp64 tree, and every node on which the two selections
differ must be ambiguous in one of two ways:

  * boundary: one of its two cumulative-mass boundaries (the oracle's mass
    ranked before it, prefix_excl / M, or that plus its own mass,
    prefix_incl / M) lies within 1e-4 of p -- the pages' exemption, taken
    from the target's wording -- widened only by the shift 2 * err that the
    *measured* score error err of this level (GPU against oracle, max over
    the candidates) can cause in a mass ratio (every mass scales by a factor
    in [exp(-err), exp(err)]);
  * order swap: on the other side of the oracle's cut there is a candidate
    whose oracle score lies within 2 * err of its own, so the two sides may
    rank the pair differently.

The oracle's own cut node is *not* exempt by construction: dropping it (a
"keep iff prefix_incl < pM" off-by-one) fails unless its boundary is really
within the window.  At most ``MAX_DIFF`` nodes per level may differ.

check_select_stats() checks the GPU's own selection records exactly:
kept mass >= P = ceil(p * M) in the GPU's fixed-point masses, minimality
(kept mass minus the last kept node's mass < P), the cut's order and tie
rule, and the counts.

eps_score (below) bounds the GPU-oracle score error that the tests accept:
5e-5 when g is effectively fp32; with bf16, fp8 or MXFP4 storage it bounds
two rounding flips of g at the level's largest magnitudes.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List

import numpy as np

import oracle.zha_oracle as O

MASS_WINDOW = 1e-4
MAX_DIFF = 4
OUT_TOL = {"f32": 1e-5, "bf16": 1e-2}


def eps_score(dtype: str, q: np.ndarray, level) -> float:
    """Score tolerance between the GPU (fp32 arithmetic on its stored g) and the
    oracle (fp64 on its own stored g).

    fp32 storage: accumulation error only, 5e-5.  bf16 storage: the two sides
    may round a g element to neighbouring bf16 values (spacing <= 2^-7 |g|);
    each such flip moves a plane by |q_i - r_ji| * spacing / sqrt(d).  The
    bound allows two flips of the largest |q_i| and |g| of the level, plus
    the fp32 term.
    """
    if dtype in ("f32", "f64"):
        return 5e-5
    d = q.shape[-1]
    gmax = float(np.abs(level.ghat).max()) if level.ghat.size else 0.0
    # relative spacing of the stored format: bf16 2^-7, fp8 E4M3 2^-3; MXFP4 at
    # most 2 scale units where the block max is at least 4 units: 1/2 of the max
    rel = {"fp8": 2.0**-3, "fp4": 0.5}.get(dtype, 2.0**-7)
    return 2.0 * (float(np.abs(q).max()) + 1.0) * gmax * rel / np.sqrt(d) + 5e-5


@dataclasses.dataclass
class LevelReport:
    level: int
    n_cand: int
    n_kept_oracle: int
    n_kept_gpu: int
    n_diff: int
    max_score_err: float


def ambiguous_nodes(sel: "O.Selection", p: float, err: float, diff) -> Dict[int, str]:
    """Classify each node id of ``diff`` (the symmetric difference of two
    selections from the same candidates) as "boundary", "swap" or "" (not
    ambiguous), given the oracle's Selection and the level's score error."""
    pos = {int(n): i for i, n in enumerate(sel.ids.tolist())}
    win = MASS_WINDOW + 2.0 * err
    kept_s = sel.score[sel.kept]
    drop_s = sel.score[~sel.kept]
    out = {}
    for n in diff:
        i = pos[int(n)]
        lo = sel.prefix_excl[i] / sel.total
        hi = (sel.prefix_excl[i] + sel.mass[i]) / sel.total
        if abs(lo - p) <= win or abs(hi - p) <= win:
            out[int(n)] = "boundary"
            continue
        other = drop_s if sel.kept[i] else kept_s  # the far side of the oracle's cut
        if other.size and float(np.min(np.abs(other - sel.score[i]))) <= 2.0 * err:
            out[int(n)] = "swap"
            continue
        out[int(n)] = ""
    return out


def check_route_teacher_forced(q, tree, ref, chunk, p, gpu_kept: Dict[int, np.ndarray], dtype, gpu_score=None,
                               leaf_dtype=None, top=None, level2_dtype=None, max_diff=MAX_DIFF):
    """Returns per-level reports; raises AssertionError on an unexplained difference.

    gpu_kept[level] = sorted kept node ids of the GPU; gpu_score[level] =
    the GPU's score row for that level (or None: the score error is then
    taken as eps_score).  p is a scalar or one value per level (index l-1
    for level l); routing starts at ``top`` (default: the top level).
    leaf_dtype and level2_dtype are the storage precisions of levels 1 and 2
    when they differ from dtype ("f64" for a level scored from its own keys).
    """
    levels = len(tree)
    top = levels if top is None else top
    pl = O.level_p(p, levels)
    reports: List[LevelReport] = []
    for lv in range(top, 0, -1):
        p = pl[lv - 1]
        n_lv = tree[lv - 1].L.shape[0]
        if lv == top:
            cand = np.arange(n_lv, dtype=np.int64)
        else:
            cand = O.children(gpu_kept[lv + 1], chunk, n_lv)
        gk = np.asarray(gpu_kept[lv], dtype=np.int64)
        assert set(gk.tolist()) <= set(cand.tolist()), f"level {lv}: GPU kept a non-candidate"
        s = O.plane_scores(q, tree[lv - 1], ref, cand)
        lv_dtype = {1: leaf_dtype, 2: level2_dtype}.get(lv) or dtype
        eps = eps_score(lv_dtype, q, tree[lv - 1])
        err = eps
        if gpu_score is not None and cand.size:
            gs = np.asarray(gpu_score[lv], dtype=np.float64)[cand]
            err = float(np.max(np.abs(gs - s)))
            assert err <= eps, f"level {lv}: score error {err} > {eps}"
        sel = O.top_p_select(cand, s, p)
        ok = set(sel.kept_ids.tolist())
        gs_set = set(gk.tolist())
        diff = ok ^ gs_set
        assert len(diff) <= max_diff, f"level {lv}: {len(diff)} nodes differ (at most {max_diff} allowed)"
        if diff:
            why = ambiguous_nodes(sel, p, err, diff)
            s_cut = float(s[sel.kept].min()) if sel.kept.any() else float("nan")
            for n, reason in why.items():
                if reason:
                    continue
                i = int(np.nonzero(cand == n)[0][0])
                lo = sel.prefix_excl[i] / sel.total
                hi = (sel.prefix_excl[i] + sel.mass[i]) / sel.total
                raise AssertionError(
                    f"level {lv}: node {n} differs (oracle kept={n in ok}) with prefix {lo:.6f}..{hi:.6f}, "
                    f"p={p}, score {s[i]:.6f} vs cut {s_cut:.6f}, score error {err:.2e}"
                )
        reports.append(LevelReport(lv, int(cand.size), len(ok), len(gs_set), len(diff), err))
    return reports


def gpu_kept_from_bits(bits_by_level: Dict[int, np.ndarray]) -> Dict[int, np.ndarray]:
    return {lv: np.nonzero(b)[0].astype(np.int64) for lv, b in bits_by_level.items()}


# ---------------------------------------------------------------------------
# the GPU's own selection records


def order_key(s: np.ndarray) -> np.ndarray:
    """The select kernels' total order on fp32 scores as uint32 keys
    (larger key = larger score; -0 below +0)."""
    u = np.asarray(s, dtype=np.float32).view(np.uint32)
    return np.where(u & np.uint32(0x80000000), ~u, u | np.uint32(0x80000000)).astype(np.uint32)


def fixed_masses(s: np.ndarray, mx: float, shift: int) -> np.ndarray:
    """round(exp(s - max) * 2^shift) with the difference and the exponential
    in fp32, as the select kernels form them (numpy's fp32 exp may differ from
    the device's by an ulp; callers allow for it)."""
    e = np.exp(np.asarray(s, dtype=np.float32) - np.float32(mx), dtype=np.float32).astype(np.float64)
    return np.rint(e * 2.0**shift)


def check_select_stats(rec, score_row: np.ndarray, bits: np.ndarray, p: float):
    """One (level, query) record of the GPU's top-p selection, checked exactly
    against its own score row and bitset: counts, the cut's order rule (kept
    iff key > cut_key, or == cut_key with id < cut_id), kept fixed-point mass
    >= P = ceil(p * M) (p as the fp32 the kernel reads), and minimality: the
    kept mass minus the last kept node's mass is < P.  The last kept node's
    mass is recomputed on the host, so it is allowed 2^-21 of itself (one
    fp32 ulp of exp) plus one unit; every other figure is the kernel's own
    integer."""
    row = np.asarray(score_row, dtype=np.float32)
    cand = np.isfinite(row)
    kept = np.asarray(bits, dtype=bool)
    n_cand = int(cand.sum())
    assert rec.n_cand == n_cand, (rec.n_cand, n_cand)
    assert rec.n_kept == int(kept.sum()), (rec.n_kept, int(kept.sum()))
    assert not (kept & ~cand).any(), "a non-candidate is kept"
    if n_cand == 0:
        assert rec.n_kept == 0 and rec.mass_total == 0
        return
    M = int(rec.mass_total)
    if float(np.float32(p)) >= 1.0:
        assert rec.n_kept == n_cand and int(rec.mass_kept) == M
        return
    assert 1 <= rec.n_kept <= n_cand
    P = math.ceil(float(np.float32(p)) * float(M))
    P = min(max(P, 1), M)
    assert int(rec.mass_kept) >= P, f"kept mass {rec.mass_kept} < P {P} (M {M})"
    keys = order_key(row)
    ids = np.arange(row.size)
    tau, cut_id = np.uint32(rec.cut_key), int(rec.cut_id)
    want = cand & ((keys > tau) | ((keys == tau) & (ids < cut_id)))
    assert np.array_equal(want, kept), "bitset differs from the cut rule"
    s_cut = float(row[kept].min())
    assert order_key(np.float32(s_cut)) == tau, "cut key is not the smallest kept score's"
    m = fixed_masses(row[cand], rec.max_score, rec.shift)
    assert float(np.float32(rec.max_score)) == float(row[cand].max())
    m_cut = float(fixed_masses(np.float32(s_cut), rec.max_score, rec.shift))
    slack = m_cut * 2.0**-21 + 1.0
    assert int(rec.mass_kept) - m_cut < P + slack, (
        f"not minimal: kept {rec.mass_kept} - last {m_cut:.0f} >= P {P}")
    # the records' totals agree with the row up to the host's exp rounding
    assert abs(float(m.sum()) - M) <= float(m.sum()) * 2.0**-20 + n_cand
    assert abs(float(m[kept[cand]].sum()) - int(rec.mass_kept)) <= float(m.sum()) * 2.0**-20 + n_cand


def check_stats_all(zha, cfg, buf, n_tokens, p, queries, top=None):
    """check_select_stats for every level from ``top`` down and every query
    index in ``queries`` of a route call's buffers (``zha`` is the binding
    module; p a scalar or one value per level)."""
    levels = cfg.levels
    top = top or levels
    pl = O.level_p(p, levels)
    sizes = O.level_sizes(n_tokens, cfg.chunk, levels)
    rl = buf.layout
    score = buf.score.cpu().numpy()
    sel = buf.sel.cpu()
    for lv in range(top, 0, -1):
        i = lv - 1
        recs = zha.stats_records(buf, lv)
        w, st = int(rl.words[i]), int(rl.score_stride[i])
        for qi in queries:
            off = int(rl.sel_offset[i]) + qi * w
            bits = zha.unpack_bits(sel[off : off + w], sizes[i]).numpy()
            so = int(rl.score_offset[i]) + qi * st
            check_select_stats(recs[qi], score[so : so + sizes[i]], bits, pl[i])
