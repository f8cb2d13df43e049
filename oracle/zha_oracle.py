"""Plain fp64 CPU oracle for the ZHA decode path (tree build, routing, attention).

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite, the smoke check
and the CPU-baseline leg of the benchmark may import this module.  It shares no
code with the HIP library: it is written directly from the method's
description, in fp64, one node and one query at a time where that is the
plain reading, with numpy for the library steps (matmul, sort, cumsum).

Sources (web pages; cited by title and section):
  MTP   = "Zyphra AI Introduces Zyphra Hierarchical Attention (ZHA): A Path to
          True Subquadratic Attention" (MarkTechPost article and its embedded
          explainer widget).
  LC    = "Zyphra Hierarchical Attention" news article on lesscarbs.net,
          section "What happened?".

What is computed, for one cache (one sequence x one KV head):

* Nodes.  Level 1 cuts the keys into contiguous chunks of C keys; a node at
  level l groups C nodes of level l-1 (MTP "Building the tree": chunk 4 with
  6 levels gives 4,096 tokens per top node, i.e. a top node spans C**levels
  tokens).  n_1 = floor(N / C): a trailing incomplete chunk is not a node (it
  is reached through the current-chunk rule below); n_l = ceil(n_{l-1} / C),
  an incomplete upper node merges the children that exist.
* Node statistics per reference query r_j (MTP "Building the tree": each
  reference query gives a tangent-plane estimate of the chunk's log
  attention mass).  With z_ji = r_j . k_i / sqrt(d) over the node's keys:
    L_j = logsumexp_i z_ji                 (log attention mass at r_j)
    g_j = sum_i softmax_i(z_j) k_i         (= sqrt(d) * dL_j/dr_j)
  so the tangent plane of f(q) = logsumexp_i q.k_i/sqrt(d) at r_j is
  L_j + (q - r_j) . g_j / sqrt(d).
* Merge ("summaries are grouped and compressed again, level by level"):
  parents are computed from their children's statistics,
    L_j(P) = logsumexp_c L_j(c),   g_j(P) = sum_c exp(L_j(c) - L_j(P)) g_j(c),
  which is exactly the statistic of all descendant keys.
* Storage.  g is stored in the KV dtype (rounded once, round-to-nearest-even,
  from the unrounded merge value), or, in the low-precision router variants
  (MTP TL;DR "FP4 router"; the pages name no format), per row j as a
  power-of-two scale times FP8 E4M3 values, or as OCP MXFP4: blocks of 32
  elements of d, each an E8M0 power-of-two scale times FP4 E2M1 values
  (ties to even, saturating); L in fp32-or-better; the plane offset
  c_j = L_j - r_j . ghat_j / sqrt(d) makes c_j + q . ghat_j / sqrt(d) equal the
  tangent plane written with the stored ghat.
* Score (MTP "Building the tree": the max over the planes approximates the
  attention any future query would give the node):
    s(q, node) = max_j [ L_j + (q - r_j) . ghat_j / sqrt(d) ].
* Routing (MTP "How does top-p routing pick tokens?" and widget
  "1 . How it works", steps 2-4): score every top-level node; the estimated
  mass of a candidate is exp(s), renormalised over all current candidates of
  this query; keep the smallest set holding fraction p of that mass; the
  children of the kept nodes are the next candidates; repeat down to level 1,
  whose nodes are raw KV chunks.
* Attention (MTP widget step 5 and "How does top-p routing pick tokens?"):
  exact softmax attention over the keys of the kept level-1 chunks, plus
  token 0 (the attention sink) and the current chunk.

Readings taken where the pages are silent:
  R3  smallest set: order candidates by (score desc, node id asc) and keep
      rank i iff the mass of the ranks before it is < p * M.  This prefix is a
      minimum-cardinality set with mass >= p * M (checked by brute force).
  R5  p >= 1 keeps every candidate.
  R6  the renormalisation pools all candidates of the query at that level.
  R10 current chunk = tokens [C * floor((N-1)/C), N).
  R16 decode queries see all N keys: no causal mask, no positional encoding.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional, Sequence

import numpy as np

# ---------------------------------------------------------------------------
# storage rounding


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round fp64 values to the nearest bfloat16 (ties to even), returned as fp64.

    bfloat16 keeps 8 significant bits and the fp32 exponent range; the
    rounding is done once, directly from fp64, so no double rounding occurs.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.empty_like(x)
    finite = np.isfinite(x)
    xf = x[finite]
    m, e = np.frexp(xf)  # xf = m * 2**e, 0.5 <= |m| < 1
    e = np.maximum(e, -125)  # below 2**-126 the quantum stays 2**-133
    quantum = np.ldexp(1.0, e - 8)
    r = np.rint(xf / quantum) * quantum  # np.rint rounds half to even
    big = np.abs(r) > 3.3895313892515355e38  # beyond the largest bfloat16
    r[big] = np.copysign(np.inf, r[big])
    out[finite] = r
    out[~finite] = x[~finite]
    return out


def round_e4m3(x: np.ndarray) -> np.ndarray:
    """Round fp64 values to the nearest OCP FP8 E4M3 value (ties to even), as fp64.

    E4M3: 1 sign, 4 exponent (bias 7) and 3 mantissa bits; normal values
    (1 + m/8) * 2**(e-7) for e = 1..15 (largest 448), subnormals m * 2**-9.
    In every binade [2**E, 2**(E+1)) the spacing is 2**(E-3); below 2**-6 it
    stays 2**-9.  Inputs must satisfy |x| <= 448 (callers scale first).
    """
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    if np.any(a > 448.0):
        raise ValueError("round_e4m3: |x| > 448")
    _, e = np.frexp(a)  # a = f * 2**e, 0.5 <= f < 1, so a lies in [2**(e-1), 2**e)
    quantum = np.ldexp(1.0, np.maximum(e - 1, -6) - 3)
    return np.copysign(np.rint(a / quantum) * quantum, x)  # np.rint: half to even


def fp8_row_scale(g: np.ndarray) -> np.ndarray:
    """Power-of-two scale 2**s per row (last axis) with max|row| / 2**s in (128, 256].

    s = ceil(log2 max|row|) - 8; a row whose max is below 2**-126 gets 1.
    """
    m = np.max(np.abs(np.asarray(g, dtype=np.float64)), axis=-1)
    f, e = np.frexp(m)  # m = f * 2**e, 0.5 <= f < 1
    ceil_log2 = np.where(f == 0.5, e - 1, e)
    s = np.where(m < 2.0**-126, 0, ceil_log2 - 8)
    return np.ldexp(1.0, s)


def round_fp8_rows(g: np.ndarray):
    """(ghat, scale): each row of g (last axis) stored as scale * E4M3(g / scale)."""
    scale = fp8_row_scale(g)
    return scale[..., None] * round_e4m3(np.asarray(g, dtype=np.float64) / scale[..., None]), scale


def round_e2m1(x: np.ndarray) -> np.ndarray:
    """Round fp64 values to the nearest OCP FP4 E2M1 value (ties to even),
    saturating at +-6, as fp64.

    E2M1: 1 sign, 2 exponent (bias 1) and 1 mantissa bit: 0 and 0.5
    (exponent field 0), (1 + m/2) * 2**(e-1) for e = 1..3: 1, 1.5, 2, 3, 4, 6.
    The spacing is 0.5 below 2, 1 in [2, 4) and 2 from 4 on; the format has
    no infinity, so magnitudes past 6 saturate to 6.
    """
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    _, e = np.frexp(a)  # a lies in [2**(e-1), 2**e)
    quantum = np.ldexp(1.0, np.maximum(e - 1, 0) - 1)
    r = np.minimum(np.rint(a / quantum) * quantum, 6.0)  # np.rint: half to even
    return np.copysign(r, x)


MX_BLOCK = 32  # elements sharing one scale in the OCP MX formats


def mxfp4_block_scale(g: np.ndarray) -> np.ndarray:
    """E8M0 scale 2**s per block of 32 consecutive elements of the last axis
    (shape [..., d / 32]): s = floor(log2 max|block|) - 2, the OCP MX rule
    (the largest E2M1 exponent is 2, so the block max lands in [4, 8) and
    saturates above 6), clamped to the E8M0 range [-127, 127]; an all-zero
    block gets 2**-127."""
    g = np.asarray(g, dtype=np.float64)
    blocks = g.reshape(*g.shape[:-1], g.shape[-1] // MX_BLOCK, MX_BLOCK)
    m = np.max(np.abs(blocks), axis=-1)
    _, e = np.frexp(m)  # m in [2**(e-1), 2**e): floor(log2 m) = e - 1
    s = np.where(m > 0, np.clip(e - 1 - 2, -127, 127), -127)
    return np.ldexp(1.0, s)


def round_mxfp4_rows(g: np.ndarray):
    """(ghat, scale): the last axis of g in blocks of 32, each stored as
    scale * E2M1(g / scale) (OCP MXFP4)."""
    g = np.asarray(g, dtype=np.float64)
    scale = mxfp4_block_scale(g)
    sc = np.repeat(scale, MX_BLOCK, axis=-1)
    return sc * round_e2m1(g / sc), scale


def round_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return round_bf16(x)
    if dtype == "fp8":
        return round_fp8_rows(x)[0]
    if dtype == "fp4":
        return round_mxfp4_rows(x)[0]
    if dtype == "f32":
        return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)
    if dtype == "f64":
        return np.asarray(x, dtype=np.float64)
    raise ValueError(dtype)


# ---------------------------------------------------------------------------
# tree geometry


def level_sizes(n_tokens: int, chunk: int, levels: int) -> List[int]:
    """Node counts [n_1, ..., n_levels] for a prefix of n_tokens keys."""
    sizes = [n_tokens // chunk]
    for _ in range(1, levels):
        sizes.append(-(-sizes[-1] // chunk))
    return sizes


def children(ids: np.ndarray, chunk: int, n_below: int) -> np.ndarray:
    """Children of nodes ``ids`` one level down: C*n .. C*n+C-1 that exist."""
    ids = np.asarray(ids, dtype=np.int64)
    if ids.size == 0:
        return ids
    kids = (ids[:, None] * chunk + np.arange(chunk)[None, :]).reshape(-1)
    return kids[kids < n_below]


def node_token_range(level: int, node: int, chunk: int, n_tokens: int):
    """Token range [a, b) covered by a node (level 1 = raw chunks)."""
    span = chunk ** level
    a = node * span
    b = min(a + span, (n_tokens // chunk) * chunk)
    return a, b


# ---------------------------------------------------------------------------
# build


@dataclasses.dataclass
class Level:
    L: np.ndarray  # [n, R] log mass per reference query
    g: Optional[np.ndarray]  # [n, R, d] unrounded softmax-weighted mean key
    ghat: np.ndarray  # [n, R, d] stored (rounded) g
    c: np.ndarray  # [n, R] plane offset L - r . ghat / sqrt(d)
    scale: Optional[np.ndarray] = None  # [n, R] fp8 row scales, or [n, R, d/32] fp4 block scales


def _logsumexp(a: np.ndarray, axis: int) -> np.ndarray:
    m = np.max(a, axis=axis, keepdims=True)
    m = np.where(np.isfinite(m), m, 0.0)
    return np.squeeze(m, axis=axis) + np.log(np.sum(np.exp(a - m), axis=axis))


def leaf_stats(keys: np.ndarray, ref: np.ndarray):
    """(L [R], g [R, d]) of one chunk of raw keys [C, d]."""
    d = keys.shape[-1]
    z = (ref @ keys.T) / math.sqrt(d)  # [R, C]
    L = _logsumexp(z, axis=1)
    w = np.exp(z - L[:, None])  # softmax over the chunk, per reference query
    g = w @ keys  # [R, d]
    return L, g


def merge_stats(L_children: np.ndarray, g_children: np.ndarray):
    """(L [R], g [R, d]) of a parent from children L [k, R], g [k, R, d]."""
    L = _logsumexp(L_children, axis=0)
    a = np.exp(L_children - L[None, :])  # [k, R] mass share of each child
    g = np.einsum("kr,krd->rd", a, g_children)
    return L, g


def _finish(L, g, ref, g_dtype, keep_g, block=8192):
    """Round g to its storage dtype and derive the plane offsets c."""
    d = ref.shape[-1]
    ghat = np.empty_like(g)
    c = np.empty_like(L)
    scale = None
    if g_dtype == "fp8":
        scale = np.empty_like(L)
    elif g_dtype == "fp4":
        scale = np.empty(L.shape + (d // MX_BLOCK,))
    for a in range(0, L.shape[0], block):
        b = min(L.shape[0], a + block)
        if g_dtype == "fp8":
            ghat[a:b], scale[a:b] = round_fp8_rows(g[a:b])
        elif g_dtype == "fp4":
            ghat[a:b], scale[a:b] = round_mxfp4_rows(g[a:b])
        else:
            ghat[a:b] = round_storage(g[a:b], g_dtype)
        c[a:b] = L[a:b] - np.einsum("nrd,rd->nr", ghat[a:b], ref) / math.sqrt(d)
    return Level(L=L, g=g if keep_g else None, ghat=ghat, c=c, scale=scale)


def build_tree(
    K: np.ndarray,
    ref: np.ndarray,
    chunk: int,
    levels: int,
    g_dtype: str = "f64",
    n_tokens: Optional[int] = None,
    keep_g: bool = True,
    block: int = 8192,
    leaf_dtype: Optional[str] = None,
    level2_dtype: Optional[str] = None,
) -> List[Level]:
    """Build every level for keys K[:n_tokens] (fp64 [N, d]) and ref [R, d].

    Returns levels[0] = level 1 (chunks) ... levels[-1] = top level.  Nodes
    are processed in batches of ``block`` only to bound memory; each node's
    arithmetic is the per-node definition above.  ``g_dtype`` is the storage
    precision of g; ``leaf_dtype`` (default: g_dtype) that of level 1 alone,
    "f64" when level-1 planes are evaluated from the chunk's own keys so that
    g is never rounded there; ``level2_dtype`` (default: g_dtype) likewise
    for level 2, "f64" when level 2 too is evaluated from its own keys.
    """
    K = np.asarray(K, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    N = K.shape[0] if n_tokens is None else n_tokens
    sizes = level_sizes(N, chunk, levels)
    R, d = ref.shape
    out: List[Level] = []
    # level 1 from raw keys
    n1 = sizes[0]
    L1 = np.empty((n1, R))
    g1 = np.empty((n1, R, d))
    for a in range(0, n1, block):
        b = min(n1, a + block)
        keys = K[a * chunk : b * chunk].reshape(b - a, chunk, d)
        z = np.einsum("rd,ncd->nrc", ref, keys) / math.sqrt(d)
        L = _logsumexp(z, axis=2)
        w = np.exp(z - L[:, :, None])
        L1[a:b] = L
        g1[a:b] = np.einsum("nrc,ncd->nrd", w, keys)
    out.append(_finish(L1, g1, ref, leaf_dtype or g_dtype, True))
    # upper levels from the unrounded children
    for lv in range(1, levels):
        n = sizes[lv]
        Lc, gc = out[-1].L, out[-1].g
        nc = Lc.shape[0]
        Lp = np.empty((n, R))
        gp = np.empty((n, R, d))
        full = nc // chunk
        for a in range(0, full, block):
            b = min(full, a + block)
            Lk = Lc[a * chunk : b * chunk].reshape(b - a, chunk, R)
            gk = gc[a * chunk : b * chunk].reshape(b - a, chunk, R, d)
            L = _logsumexp(Lk, axis=1)
            wgt = np.exp(Lk - L[:, None, :])
            Lp[a:b] = L
            gp[a:b] = np.einsum("nkr,nkrd->nrd", wgt, gk)
        if full < n:  # incomplete trailing parent: merge the children that exist
            Lp[full], gp[full] = merge_stats(Lc[full * chunk :], gc[full * chunk :])
        out.append(_finish(Lp, gp, ref, (level2_dtype or g_dtype) if lv == 1 else g_dtype, True))
        if not keep_g:
            out[-2].g = None
    if not keep_g:
        out[-1].g = None
    return out


def node_stats_direct(K: np.ndarray, ref: np.ndarray, a: int, b: int):
    """(L, g) computed directly from all keys K[a:b] of a node (no merging)."""
    return leaf_stats(np.asarray(K[a:b], dtype=np.float64), np.asarray(ref, dtype=np.float64))


# ---------------------------------------------------------------------------
# scoring and routing


def plane_scores(q: np.ndarray, level: Level, ref: np.ndarray, ids=None) -> np.ndarray:
    """s(q, n) = max_j [L_j + (q - r_j) . ghat_j / sqrt(d)] for nodes ``ids``."""
    q = np.asarray(q, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    d = q.shape[-1]
    if ids is None:
        ids = np.arange(level.L.shape[0])
    ids = np.asarray(ids, dtype=np.int64)
    if ids.size == 0:
        return np.zeros(0)
    gh = level.ghat[ids]  # [n, R, d]
    planes = level.L[ids] + np.einsum("nrd,rd->nr", gh, q[None, :] - ref) / math.sqrt(d)
    return planes.max(axis=1)


@dataclasses.dataclass
class Selection:
    ids: np.ndarray  # candidates, in input order
    score: np.ndarray  # their scores
    order: np.ndarray  # permutation: (score desc, id asc)
    mass: np.ndarray  # exp(s - max s) per candidate (input order)
    total: float  # M = sum of mass
    prefix_excl: np.ndarray  # mass of the ranks before each candidate (input order)
    kept: np.ndarray  # bool per candidate (input order)

    @property
    def kept_ids(self) -> np.ndarray:
        return np.sort(self.ids[self.kept])


def top_p_select(ids: np.ndarray, score: np.ndarray, p: float) -> Selection:
    """Smallest set of candidates holding fraction p of the renormalised mass."""
    ids = np.asarray(ids, dtype=np.int64)
    score = np.asarray(score, dtype=np.float64)
    n = ids.size
    if n == 0:
        z = np.zeros(0)
        return Selection(ids, score, np.zeros(0, np.int64), z, 0.0, z, np.zeros(0, bool))
    mass = np.exp(score - score.max())
    total = float(mass.sum())
    order = np.lexsort((ids, -score))
    sorted_mass = mass[order]
    before = np.concatenate(([0.0], np.cumsum(sorted_mass)[:-1]))
    prefix_excl = np.empty(n)
    prefix_excl[order] = before
    if p >= 1.0:
        kept = np.ones(n, dtype=bool)
    else:
        kept = prefix_excl < p * total
    return Selection(ids, score, order, mass, total, prefix_excl, kept)


@dataclasses.dataclass
class RouteLevel:
    level: int  # 1 = chunks
    sel: Selection


def level_p(p, levels: int) -> List[float]:
    """p per level (index l-1 for level l) from a scalar or a per-level sequence."""
    if np.ndim(p) == 0:
        return [float(p)] * levels
    p = [float(x) for x in p]
    if len(p) != levels:
        raise ValueError("one p per level")
    return p


def depth_schedule(coverage: float, depth: int) -> List[float]:
    """Per-level p whose product is ``coverage``: p_l = coverage ** (1 / depth).

    MTP widget "5 . Caveats" ("Top-p must scale with depth"): with the same p
    at every level the mass kept down to the leaves shrinks roughly like
    p ** depth; spreading a target coverage over the routed levels keeps it
    independent of the depth.
    """
    return [float(coverage) ** (1.0 / depth)] * depth


def route(q: np.ndarray, tree: List[Level], ref: np.ndarray, chunk: int, p, top: Optional[int] = None) -> List[RouteLevel]:
    """Top-down routing of one query; returns records from the start level down.

    ``p`` is a scalar or one value per level (index l-1 for level l).  ``top``
    (default: the tree's top level) is the level routing starts from: every
    node of that level is a candidate and the levels above it are not used,
    so the routing depth can follow the context length (MTP "depth can grow
    iteratively").
    """
    levels = len(tree)
    top = levels if top is None else top
    if not 1 <= top <= levels:
        raise ValueError("top must be in 1..levels")
    pl = level_p(p, levels)
    cand = np.arange(tree[top - 1].L.shape[0], dtype=np.int64)
    out: List[RouteLevel] = []
    for lv in range(top, 0, -1):
        lvl = tree[lv - 1]
        s = plane_scores(q, lvl, ref, cand)
        sel = top_p_select(cand, s, pl[lv - 1])
        out.append(RouteLevel(lv, sel))
        if lv > 1:
            cand = children(sel.kept_ids, chunk, tree[lv - 2].L.shape[0])
    return out


# ---------------------------------------------------------------------------
# attention


def attend_set(
    kept_chunks: Sequence[int], n_tokens: int, chunk: int, sink: bool = True, last_chunk: bool = True
) -> np.ndarray:
    """Sorted key indices attended: kept chunks' keys, token 0, current chunk."""
    kc = np.asarray(kept_chunks, dtype=np.int64)
    parts = [(kc[:, None] * chunk + np.arange(chunk)[None, :]).reshape(-1)]
    if sink and n_tokens > 0:
        parts.append(np.array([0], dtype=np.int64))
    if last_chunk and n_tokens > 0:
        parts.append(np.arange(chunk * ((n_tokens - 1) // chunk), n_tokens, dtype=np.int64))
    idx = np.unique(np.concatenate(parts))
    return idx[idx < n_tokens]


def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, key_idx: np.ndarray):
    """Exact softmax attention of q over keys K[key_idx]; returns (o [d], lse)."""
    q = np.asarray(q, dtype=np.float64)
    d = q.shape[-1]
    idx = np.asarray(key_idx, dtype=np.int64)
    if idx.size == 0:
        return np.zeros(V.shape[-1]), -np.inf
    k = np.asarray(K[idx], dtype=np.float64)
    v = np.asarray(V[idx], dtype=np.float64)
    z = k @ q / math.sqrt(d)
    m = z.max()
    w = np.exp(z - m)
    l = w.sum()
    return (w @ v) / l, float(m + math.log(l))


def route_and_attend(q, K, V, tree, ref, chunk, p, n_tokens, sink=True, last_chunk=True, top=None):
    """Full decode path for one query: (o, lse, key set, route records)."""
    recs = route(q, tree, ref, chunk, p, top)
    kept = recs[-1].sel.kept_ids
    idx = attend_set(kept, n_tokens, chunk, sink, last_chunk)
    o, lse = attend(q, K, V, idx)
    return o, lse, idx, recs


# ---------------------------------------------------------------------------
# chunked prefill (causal)


def prefill_query(q, K, V, ref, chunk, levels, p, position, g_dtype="f64", leaf_dtype=None,
                  sink=True, last_chunk=True, top=None):
    """One prefill query at ``position`` t, causal: it sees tokens [0, t].

    The plain reading of routing under a causal limit (the pages' claim of
    sub-quadratic cost is about this regime, MTP TL;DR): the query decodes
    against the tree of its own prefix of t + 1 tokens.  Complete nodes of
    that tree are those of any longer tree (a node is a function of its key
    range); a node straddling t is partial and merges the children that
    exist, as the trailing node of any tree does.  Returns
    (o, lse, key set, route records, tree).
    """
    n = position + 1
    tree = build_tree(np.asarray(K[:n]), ref, chunk, levels, g_dtype, n_tokens=n, keep_g=False,
                      leaf_dtype=leaf_dtype)
    if level_sizes(n, chunk, levels)[0] == 0:
        idx = attend_set(np.zeros(0, np.int64), n, chunk, sink, last_chunk)
        o, lse = attend(q, K, V, idx)
        return o, lse, idx, [], tree
    o, lse, idx, recs = route_and_attend(q, np.asarray(K[:n]), np.asarray(V[:n]), tree, ref, chunk, p, n,
                                         sink, last_chunk, top)
    return o, lse, idx, recs, tree
