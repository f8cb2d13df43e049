"""Parity helpers: compare the HIP path with the CPU oracle.

Set parity is judged teacher-forced, level by level: at each level the oracle
re-selects from the GPU's own candidate set (children of the GPU's kept
parents) using its own fp64 tree, and every node on which the two selections
differ must be ambiguous:
  * its cumulative-mass boundary lies within 1e-4 of p, i.e. the oracle's
    [prefix_excl, prefix_incl] / M interval, widened by 1e-4, contains p; or
  * its oracle score is within eps_score of the score of the oracle's last
    kept node (an order swap caused by rounding of near-equal scores).
eps_score (below) is 5e-5 when g is stored in fp32; with bf16 or fp8 storage
it bounds two rounding flips of g at the level's largest magnitudes.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List

import numpy as np

import oracle.zha_oracle as O

MASS_WINDOW = 1e-4
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
    # relative spacing of the stored format: bf16 2^-7, fp8 E4M3 2^-3
    rel = 2.0**-3 if dtype == "fp8" else 2.0**-7
    return 2.0 * (float(np.abs(q).max()) + 1.0) * gmax * rel / np.sqrt(d) + 5e-5


@dataclasses.dataclass
class LevelReport:
    level: int
    n_cand: int
    n_kept_oracle: int
    n_kept_gpu: int
    n_diff: int
    max_score_err: float


def check_route_teacher_forced(q, tree, ref, chunk, p, gpu_kept: Dict[int, np.ndarray], dtype, gpu_score=None,
                               leaf_dtype=None, top=None, level2_dtype=None):
    """Returns per-level reports; raises AssertionError on an unexplained difference.

    gpu_kept[level] = sorted kept node ids of the GPU; gpu_score[level] =
    the GPU's score row for that level (or None).  p is a scalar or one
    value per level (index l-1 for level l); routing starts at ``top``
    (default: the top level).  leaf_dtype and level2_dtype are the storage
    precisions of levels 1 and 2 when they differ from dtype ("f64" for a
    level scored from its own keys).
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
        err = 0.0
        if gpu_score is not None and cand.size:
            gs = np.asarray(gpu_score[lv], dtype=np.float64)[cand]
            err = float(np.max(np.abs(gs - s)))
            assert err <= eps, f"level {lv}: score error {err} > {eps}"
        sel = O.top_p_select(cand, s, p)
        ok = set(sel.kept_ids.tolist())
        gs_set = set(gk.tolist())
        diff = ok ^ gs_set
        if diff:
            pos = {int(n): i for i, n in enumerate(cand.tolist())}
            s_cut = float(s[sel.kept].min())
            for n in diff:
                i = pos[n]
                lo = sel.prefix_excl[i] / sel.total
                hi = (sel.prefix_excl[i] + sel.mass[i]) / sel.total
                amb = (lo - MASS_WINDOW <= p <= hi + MASS_WINDOW) or abs(s[i] - s_cut) <= eps
                assert amb, (
                    f"level {lv}: node {n} differs (oracle kept={n in ok}) with prefix {lo:.6f}..{hi:.6f}, "
                    f"p={p}, score {s[i]:.6f} vs cut {s_cut:.6f}"
                )
        reports.append(LevelReport(lv, int(cand.size), len(ok), len(gs_set), len(diff), err))
    return reports


def gpu_kept_from_bits(bits_by_level: Dict[int, np.ndarray]) -> Dict[int, np.ndarray]:
    return {lv: np.nonzero(b)[0].astype(np.int64) for lv, b in bits_by_level.items()}
