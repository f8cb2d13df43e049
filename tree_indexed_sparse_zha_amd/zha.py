"""Thin ctypes binding of ``libzha.so`` (the ZHA C ABI in include/zha.h).

Argument marshalling only: every step of the path runs in the library's HIP
kernels.  PyTorch supplies device memory and the current HIP stream.  Loading
fails loudly when the library has not been built; there is no fallback.
"""
from __future__ import annotations

import ctypes as ct
import dataclasses
import math
import os
from typing import Dict, List, Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# ZHA_LIB_PATH selects another build of the library (the host-sanitizer
# build the CPU tests use); by default the in-tree one
LIB_PATH = os.environ.get("ZHA_LIB_PATH") or os.path.join(_HERE, "libzha.so")

ZHA_OK, ZHA_ERR_NULL, ZHA_ERR_ARG, ZHA_ERR_UNSUPPORTED, ZHA_ERR_CAPACITY, ZHA_ERR_ALIGN, ZHA_ERR_HIP = (
    0,
    -1,
    -2,
    -3,
    -4,
    -5,
    -6,
)
ZHA_F32, ZHA_BF16 = 0, 1
ZHA_SINK, ZHA_LAST_CHUNK, ZHA_ALL_KEYS, ZHA_CAUSAL = 1, 2, 4, 8
ZHA_LEAF_MEAN, ZHA_LEAF_WEIGHTS, ZHA_LEAF_WEIGHTS2 = 0, 1, 2
LEAF_FORMS = {"mean": ZHA_LEAF_MEAN, "weights": ZHA_LEAF_WEIGHTS, "weights2": ZHA_LEAF_WEIGHTS2}
ZHA_G_KV, ZHA_G_FP8, ZHA_G_FP4 = 0, 2, 4
G_DTYPES = {"kv": ZHA_G_KV, "fp8": ZHA_G_FP8, "fp4": ZHA_G_FP4}
MAX_LEVELS = 8
ZHA_NOALLOC_SCRATCH_BYTES = 32 << 20  # static scratch of zha_attend_noalloc (include/zha.h)


class ZhaError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"zha error {code}: {msg}")
        self.code = code


class Config(ct.Structure):
    _fields_ = [
        ("batch", ct.c_int32),
        ("n_kv_heads", ct.c_int32),
        ("q_per_kv", ct.c_int32),
        ("head_dim", ct.c_int32),
        ("n_ref", ct.c_int32),
        ("chunk", ct.c_int32),
        ("levels", ct.c_int32),
        ("kv_dtype", ct.c_int32),
        ("leaf_form", ct.c_int32),
        ("g_dtype", ct.c_int32),
        ("capacity_tokens", ct.c_int64),
    ]


class TreeLayout(ct.Structure):
    _fields_ = [
        ("levels", ct.c_int32),
        ("reserved", ct.c_int32),
        ("node_cap", ct.c_int64 * MAX_LEVELS),
        ("g_offset", ct.c_int64 * MAX_LEVELS),
        ("L_offset", ct.c_int64 * MAX_LEVELS),
        ("c_offset", ct.c_int64 * MAX_LEVELS),
        ("g_bytes", ct.c_int64 * MAX_LEVELS),
        ("total_bytes", ct.c_int64),
        ("s_offset", ct.c_int64 * MAX_LEVELS),
        ("scratch_offset", ct.c_int64),
        ("ref_offset", ct.c_int64),
    ]


class RouteLayout(ct.Structure):
    _fields_ = [
        ("levels", ct.c_int32),
        ("reserved", ct.c_int32),
        ("n_queries", ct.c_int64),
        ("words", ct.c_int64 * MAX_LEVELS),
        ("sel_offset", ct.c_int64 * MAX_LEVELS),
        ("score_offset", ct.c_int64 * MAX_LEVELS),
        ("score_stride", ct.c_int64 * MAX_LEVELS),
        ("stats_offset", ct.c_int64 * MAX_LEVELS),
        ("sel_words_total", ct.c_int64),
        ("score_floats_total", ct.c_int64),
        ("stats_total", ct.c_int64),
        ("workspace_bytes", ct.c_int64),
        ("logits_floats", ct.c_int64),
        ("workspace_min_bytes", ct.c_int64),
    ]


class SelectStats(ct.Structure):
    _fields_ = [
        ("max_score", ct.c_float),
        ("n_cand", ct.c_int32),
        ("n_kept", ct.c_int32),
        ("cut_key", ct.c_uint32),
        ("cut_id", ct.c_int32),
        ("shift", ct.c_int32),
        ("mass_total", ct.c_uint64),
        ("mass_kept", ct.c_uint64),
    ]


STATS_BYTES = ct.sizeof(SelectStats)
assert STATS_BYTES == 40

PROFILE_MAX = 32
K_BUILD, K_SCORE, K_SELECT, K_ATTEND, K_COMBINE, K_PROBE = 1, 2, 3, 4, 5, 6
KERNEL_NAMES = {K_BUILD: "build", K_SCORE: "score", K_SELECT: "select", K_ATTEND: "attend", K_COMBINE: "combine",
                K_PROBE: "probe"}
PROBE_MODES = {"read": 0, "read_nt": 1, "copy": 2, "copy_nt": 3, "mix": 4, "mix_nt": 5, "read_slab": 6,
               "read_slab_nt": 7, "tile_mix": 8}


class Profile(ct.Structure):
    _fields_ = [
        ("events", ct.c_void_p * (2 * PROFILE_MAX)),
        ("n_pairs", ct.c_int32),
        ("n_used", ct.c_int32),
        ("kernel", ct.c_int32 * PROFILE_MAX),
    ]


class HipEvents:
    """Raw hipEvent_t handles for zha_profile (created through libamdhip64)."""

    def __init__(self, n_pairs: int = PROFILE_MAX):
        self.hip = ct.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ct.POINTER(ct.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ct.POINTER(ct.c_float), ct.c_void_p, ct.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ct.c_void_p]
        self.prof = Profile()
        self.prof.n_pairs = n_pairs
        for i in range(2 * n_pairs):
            h = ct.c_void_p()
            if self.hip.hipEventCreate(ct.byref(h)) != 0:
                raise RuntimeError("hipEventCreate failed")
            self.prof.events[i] = h
        self.n_pairs = n_pairs

    def elapsed_ms(self):
        """[(kernel id, level, ms)] for the kernels timed by the last call (after a sync)."""
        out = []
        for k in range(min(self.prof.n_used, self.n_pairs)):
            ms = ct.c_float()
            rc = self.hip.hipEventElapsedTime(ct.byref(ms), self.prof.events[2 * k], self.prof.events[2 * k + 1])
            if rc != 0:
                raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
            code = self.prof.kernel[k]
            out.append((code // 16, code % 16, float(ms.value)))
        return out

    def __del__(self):
        try:
            for i in range(2 * self.n_pairs):
                self.hip.hipEventDestroy(self.prof.events[i])
        except Exception:
            pass

_lib: Optional[ct.CDLL] = None


def load(path: str = LIB_PATH) -> ct.CDLL:
    """Load libzha.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} not found: build it with `python -m tree_indexed_sparse_zha_amd.build_lib`")
    lib = ct.CDLL(path)
    P, I32, I64, F = ct.c_void_p, ct.c_int32, ct.c_int64, ct.c_float
    cfgp = ct.POINTER(Config)
    i64p = ct.POINTER(ct.c_int64)
    sig = {
        "zha_version": (ct.c_int, []),
        "zha_status_string": (ct.c_char_p, [ct.c_int]),
        "zha_last_error": (ct.c_char_p, []),
        "zha_get_tree_layout": (ct.c_int, [cfgp, ct.POINTER(TreeLayout)]),
        "zha_get_route_layout": (ct.c_int, [cfgp, I32, ct.POINTER(RouteLayout)]),
        "zha_attend_workspace_bytes": (I64, [cfgp, I32]),
        "zha_build": (ct.c_int, [cfgp, P, i64p, I64, P, P, P, P]),
        "zha_append": (ct.c_int, [cfgp, P, i64p, I64, I64, P, P, P, P]),
        "zha_route": (ct.c_int, [cfgp, P, I64, P, i64p, I32, F, P, i64p, P, P, P, P, P, I64, P, P]),
        "zha_route_levels": (ct.c_int, [cfgp, P, I64, P, i64p, I32, ct.POINTER(F), I32, P, i64p, P, P, P, P, P, I64, P, P]),
        "zha_spine_bytes": (I64, [cfgp, I32]),
        "zha_build_spine": (ct.c_int, [cfgp, P, i64p, I64, I32, P, P, P, P]),
        "zha_route_prefill": (ct.c_int, [cfgp, P, P, I64, P, i64p, I32, F, P, i64p, P, P, P, P, P, I64, P, P]),
        "zha_attend": (ct.c_int, [cfgp, P, i64p, I32, P, P, i64p, I64, P, I64, P, ct.c_uint32, P, P, P, I64, P, P]),
        "zha_dense_decode": (ct.c_int, [cfgp, P, i64p, I32, P, P, i64p, I64, P, P, P, I64, P, P]),
        "zha_attend_noalloc": (ct.c_int, [cfgp, P, i64p, I32, P, P, i64p, I64, P, I64, P, ct.c_uint32, P, P, P, P]),
        "zha_stream_probe": (ct.c_int, [I32, P, P, I64, I64, P, P]),
        "zha_selected_chunks": (ct.c_int, [P, I64, I64, I64, P, P, I64, P]),
        "zha_tree_bytes": (I64, [cfgp]),
        "zha_route_workspace_bytes": (I64, [cfgp, I32]),
        "zha_dense_workspace_bytes": (I64, [cfgp, I32]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(rc: int):
    if rc != ZHA_OK:
        raise ZhaError(rc, load().zha_last_error().decode())


def _i64(*vals) -> ct.Array:
    return (ct.c_int64 * len(vals))(*[int(v) for v in vals])


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ct.c_void_p(t.data_ptr())


def _stream(t: torch.Tensor):
    if t.is_cuda:
        return ct.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)
    return None


def _elem_strides(t: torch.Tensor, dims: int) -> List[int]:
    if t.stride(-1) != 1:
        raise ValueError("rows must be contiguous along the head dimension")
    return list(t.stride())[:dims]


@dataclasses.dataclass
class ZhaConfig:
    batch: int
    n_kv_heads: int
    q_per_kv: int
    head_dim: int
    n_ref: int
    chunk: int
    levels: int
    dtype: str  # "f32" | "bf16"
    capacity: int
    leaf_form: str = "mean"  # "mean" | "weights" (level 1 holds weights) | "weights2" (levels 1 and 2)
    g_dtype: str = "kv"  # "kv" (g in the KV dtype) | "fp8" (E4M3 with row scales) | "fp4" (OCP MXFP4)

    def c(self) -> Config:
        return Config(
            self.batch,
            self.n_kv_heads,
            self.q_per_kv,
            self.head_dim,
            self.n_ref,
            self.chunk,
            self.levels,
            ZHA_BF16 if self.dtype == "bf16" else ZHA_F32,
            LEAF_FORMS[self.leaf_form],
            G_DTYPES[self.g_dtype],
            self.capacity,
        )

    @property
    def n_caches(self) -> int:
        return self.batch * self.n_kv_heads

    @property
    def weights(self) -> bool:
        """Level 1 holds softmax weights (either weights form)."""
        return self.leaf_form in ("weights", "weights2")

    def weight_keys(self, level: int) -> int:
        """Keys per node of ``level`` when routing scores it from its keys
        (level 1 of the weights forms, level 2 of "weights2"), else 0."""
        if level == 1 and self.weights:
            return self.chunk
        if level == 2 and self.leaf_form == "weights2":
            return self.chunk * self.chunk
        return 0

    @property
    def esize(self) -> int:
        return 2 if self.dtype == "bf16" else 4

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32


def version() -> int:
    return load().zha_version()


def tree_layout(cfg: ZhaConfig) -> TreeLayout:
    out = TreeLayout()
    c = cfg.c()
    _check(load().zha_get_tree_layout(ct.byref(c), ct.byref(out)))
    return out


def route_layout(cfg: ZhaConfig, T: int) -> RouteLayout:
    out = RouteLayout()
    c = cfg.c()
    _check(load().zha_get_route_layout(ct.byref(c), int(T), ct.byref(out)))
    return out


def attend_workspace_bytes(cfg: ZhaConfig, T: int) -> int:
    c = cfg.c()
    n = load().zha_attend_workspace_bytes(ct.byref(c), int(T))
    if n < 0:
        _check(ZHA_ERR_ARG)
    return int(n)


def alloc_tree(cfg: ZhaConfig, device="cuda") -> torch.Tensor:
    tl = tree_layout(cfg)
    return torch.empty(int(tl.total_bytes), dtype=torch.uint8, device=device)


def _prof(ev: Optional["HipEvents"]):
    return None if ev is None else ct.byref(ev.prof)


def build(cfg: ZhaConfig, K: torch.Tensor, ref: torch.Tensor, tree: torch.Tensor, n_tokens: int, ev=None):
    c = cfg.c()
    ks = _i64(*_elem_strides(K, 3))
    _check(load().zha_build(ct.byref(c), _ptr(K), ks, int(n_tokens), _ptr(ref), _ptr(tree), _prof(ev), _stream(K)))


def append(cfg: ZhaConfig, K: torch.Tensor, ref: torch.Tensor, tree: torch.Tensor, n_old: int, n_new: int, ev=None):
    c = cfg.c()
    ks = _i64(*_elem_strides(K, 3))
    _check(
        load().zha_append(
            ct.byref(c), _ptr(K), ks, int(n_old), int(n_new), _ptr(ref), _ptr(tree), _prof(ev), _stream(K)
        )
    )


@dataclasses.dataclass
class RouteBuffers:
    sel: torch.Tensor  # int32 view of uint32 words
    score: torch.Tensor
    stats: torch.Tensor  # uint8 [n_records * 40]
    ws: torch.Tensor
    layout: RouteLayout
    logits: Optional[torch.Tensor] = None  # level-1 attention logits (weights form)


def alloc_route(cfg: ZhaConfig, T: int, device="cuda", logits: bool = False, split_select: bool = True) -> RouteBuffers:
    """Route outputs; ``logits`` also allocates the level-1 logits buffer
    (leaf-weights form) that zha_attend can read instead of the keys;
    ``split_select=False`` gives the smallest workspace, which keeps every
    level's selection at one workgroup per query."""
    rl = route_layout(cfg, T)
    ws_bytes = int(rl.workspace_bytes) if split_select else int(rl.workspace_min_bytes)
    lg = None
    if logits and int(rl.logits_floats) > 0:
        lg = torch.empty(int(rl.logits_floats), dtype=torch.float32, device=device)
    return RouteBuffers(
        sel=torch.zeros(int(rl.sel_words_total), dtype=torch.int32, device=device),
        score=torch.empty(int(rl.score_floats_total), dtype=torch.float32, device=device),
        stats=torch.zeros(max(1, int(rl.stats_total)) * STATS_BYTES, dtype=torch.uint8, device=device),
        ws=torch.empty(max(256, ws_bytes), dtype=torch.uint8, device=device),
        layout=rl,
        logits=lg,
    )


def route(cfg: ZhaConfig, tree: torch.Tensor, n_tokens: int, Q: torch.Tensor, T: int, p: float, buf: RouteBuffers,
          ev=None, K: Optional[torch.Tensor] = None):
    c = cfg.c()
    qs = _i64(*_elem_strides(Q, 4))
    ks = _i64(*_elem_strides(K, 3)) if K is not None else None
    _check(
        load().zha_route(
            ct.byref(c),
            _ptr(tree),
            int(n_tokens),
            _ptr(Q),
            qs,
            int(T),
            float(p),
            _ptr(K),
            ks,
            _ptr(buf.sel),
            _ptr(buf.score),
            _ptr(buf.stats),
            _ptr(buf.logits),
            _ptr(buf.ws),
            int(buf.ws.numel()),
            _prof(ev),
            _stream(Q),
        )
    )


def route_levels(cfg: ZhaConfig, tree: torch.Tensor, n_tokens: int, Q: torch.Tensor, T: int, p_levels,
                 buf: RouteBuffers, top_level: int = 0, ev=None, K: Optional[torch.Tensor] = None):
    """zha_route_levels: p_levels[l-1] is the fraction kept at level l;
    routing starts at top_level (0 = the tree's top)."""
    c = cfg.c()
    qs = _i64(*_elem_strides(Q, 4))
    ks = _i64(*_elem_strides(K, 3)) if K is not None else None
    pl = (ct.c_float * max(1, len(p_levels)))(*[float(x) for x in p_levels])
    _check(
        load().zha_route_levels(
            ct.byref(c), _ptr(tree), int(n_tokens), _ptr(Q), qs, int(T), pl, int(top_level), _ptr(K), ks,
            _ptr(buf.sel), _ptr(buf.score), _ptr(buf.stats), _ptr(buf.logits), _ptr(buf.ws), int(buf.ws.numel()),
            _prof(ev), _stream(Q),
        )
    )


def spine_bytes(cfg: ZhaConfig, T: int) -> int:
    c = cfg.c()
    n = load().zha_spine_bytes(ct.byref(c), int(T))
    if n < 0:
        _check(ZHA_ERR_ARG)
    return int(n)


def alloc_spine(cfg: ZhaConfig, T: int, device="cuda") -> torch.Tensor:
    return torch.empty(spine_bytes(cfg, T), dtype=torch.uint8, device=device)


def build_spine(cfg: ZhaConfig, K: torch.Tensor, ref: torch.Tensor, spine: torch.Tensor, n_tokens: int, T: int,
                ev=None):
    """zha_build_spine: partial nodes of the prefix trees of positions [n_tokens - T, n_tokens)."""
    c = cfg.c()
    ks = _i64(*_elem_strides(K, 3))
    _check(load().zha_build_spine(ct.byref(c), _ptr(K), ks, int(n_tokens), int(T), _ptr(ref), _ptr(spine),
                                  _prof(ev), _stream(K)))


def route_prefill(cfg: ZhaConfig, tree: torch.Tensor, spine: Optional[torch.Tensor], n_tokens: int, Q: torch.Tensor,
                  T: int, p: float, buf: RouteBuffers, ev=None, K: Optional[torch.Tensor] = None):
    """zha_route_prefill: query t of each head routes on its prefix of n_tokens - T + t + 1 tokens."""
    c = cfg.c()
    qs = _i64(*_elem_strides(Q, 4))
    ks = _i64(*_elem_strides(K, 3)) if K is not None else None
    _check(
        load().zha_route_prefill(
            ct.byref(c), _ptr(tree), _ptr(spine), int(n_tokens), _ptr(Q), qs, int(T), float(p), _ptr(K), ks,
            _ptr(buf.sel), _ptr(buf.score), _ptr(buf.stats), _ptr(buf.logits), _ptr(buf.ws), int(buf.ws.numel()),
            _prof(ev), _stream(Q),
        )
    )


def level1_sel(buf: RouteBuffers) -> torch.Tensor:
    """The level-1 bitsets [n_queries, words] (a view into buf.sel)."""
    rl = buf.layout
    nq, w = int(rl.n_queries), int(rl.words[0])
    off = int(rl.sel_offset[0])
    return buf.sel[off : off + nq * w].view(nq, w)


def attend(
    cfg: ZhaConfig,
    Q: torch.Tensor,
    T: int,
    K: torch.Tensor,
    V: torch.Tensor,
    n_tokens: int,
    sel1: Optional[torch.Tensor],
    flags: int,
    out: torch.Tensor,
    lse: Optional[torch.Tensor],
    ws: torch.Tensor,
    ev=None,
    logits: Optional[torch.Tensor] = None,
):
    c = cfg.c()
    qs = _i64(*_elem_strides(Q, 4))
    kvs = _i64(*_elem_strides(K, 3))
    if tuple(V.stride()[:3]) != tuple(K.stride()[:3]):
        raise ValueError("K and V must share strides")
    words = 0 if sel1 is None else int(sel1.shape[-1])
    _check(
        load().zha_attend(
            ct.byref(c),
            _ptr(Q),
            qs,
            int(T),
            _ptr(K),
            _ptr(V),
            kvs,
            int(n_tokens),
            _ptr(sel1),
            words,
            _ptr(logits),
            int(flags),
            _ptr(out),
            _ptr(lse),
            _ptr(ws),
            int(ws.numel()),
            _prof(ev),
            _stream(Q),
        )
    )


def attend_noalloc(cfg: ZhaConfig, Q: torch.Tensor, T: int, K: torch.Tensor, V: torch.Tensor, n_tokens: int,
                   sel1: Optional[torch.Tensor], flags: int, out: torch.Tensor, lse: Optional[torch.Tensor], ev=None,
                   logits: Optional[torch.Tensor] = None):
    """zha_attend_noalloc: zha_attend with the library's static per-GPU
    scratch instead of a caller workspace (allocates nothing; calls that
    overlap on one GPU race)."""
    c = cfg.c()
    qs = _i64(*_elem_strides(Q, 4))
    kvs = _i64(*_elem_strides(K, 3))
    if tuple(V.stride()[:3]) != tuple(K.stride()[:3]):
        raise ValueError("K and V must share strides")
    words = 0 if sel1 is None else int(sel1.shape[-1])
    _check(
        load().zha_attend_noalloc(
            ct.byref(c), _ptr(Q), qs, int(T), _ptr(K), _ptr(V), kvs, int(n_tokens), _ptr(sel1), words, _ptr(logits),
            int(flags), _ptr(out), _ptr(lse), _prof(ev), _stream(Q),
        )
    )


def selected_chunks(sel1: torch.Tensor, n_chunks: int, cap: int):
    """zha_selected_chunks: level-1 bitsets [n_queries, words] (int32 or
    uint32 words) -> (chunk_ids [n_queries, cap] int32, chunk_count
    [n_queries] int32); ids past a query's count are left at -1."""
    assert sel1.dim() == 2 and sel1.element_size() == 4 and sel1.is_contiguous()
    nq, words = sel1.shape
    ids = torch.full((nq, max(int(cap), 1)), -1, dtype=torch.int32, device=sel1.device)
    count = torch.empty(nq, dtype=torch.int32, device=sel1.device)
    _check(load().zha_selected_chunks(_ptr(sel1), int(words), int(nq), int(n_chunks), _ptr(ids), _ptr(count),
                                      int(cap), _stream(sel1)))
    return ids[:, : int(cap)], count


def stream_probe(mode: str, src: torch.Tensor, dst: torch.Tensor, n_bytes: int, ev=None):
    """zha_stream_probe: one launch of a plain streaming kernel (measurement only)."""
    _check(load().zha_stream_probe(PROBE_MODES[mode], _ptr(src), _ptr(dst), int(n_bytes),
                                   int(dst.numel() * dst.element_size()), _prof(ev), _stream(src)))


def dense_decode(cfg, Q, T, K, V, n_tokens, out, lse, ws, ev=None):
    c = cfg.c()
    qs = _i64(*_elem_strides(Q, 4))
    kvs = _i64(*_elem_strides(K, 3))
    _check(
        load().zha_dense_decode(
            ct.byref(c), _ptr(Q), qs, int(T), _ptr(K), _ptr(V), kvs, int(n_tokens), _ptr(out), _ptr(lse),
            _ptr(ws), int(ws.numel()), _prof(ev), _stream(Q)
        )
    )


# ---------------------------------------------------------------------------
# readout helpers (tests and reports): logical views of the library's buffers


def read_level(cfg: ZhaConfig, tree: torch.Tensor, level: int, n_nodes: Optional[int] = None) -> Dict[str, torch.Tensor]:
    """Level ``level`` (1 = chunks) as logical tensors on the tree's device.

    Returns g [caches, n, R, d] (storage dtype; fp8 levels: the decoded
    values times their row scale, fp32, plus "scale" [caches, n, R]), L and c
    [caches, n, R] fp32; level 1 in the weights forms returns w [caches, n,
    R, C] instead of g, and level 2 in "weights2" rho [caches, n, R, C], the
    children's mass shares exp(L(child) - L).
    """
    tl = tree_layout(cfg)
    i = level - 1
    cap = int(tl.node_cap[i])
    n = cap if n_nodes is None else n_nodes
    R, d, E = cfg.n_ref, cfg.head_dim, 16 // cfg.esize
    caches = cfg.n_caches
    gb = int(tl.g_offset[i])
    Lb, cb = int(tl.L_offset[i]), int(tl.c_offset[i])
    L = tree[Lb : Lb + caches * cap * R * 4].view(torch.float32).view(caches, cap, R)[:, :n]
    c = tree[cb : cb + caches * cap * R * 4].view(torch.float32).view(caches, cap, R)[:, :n]
    if level == 2 and cfg.leaf_form == "weights2":
        C = cfg.chunk  # rho [R][C]: each child's share exp(L(child) - L) of the node's mass
        rho = tree[gb : gb + caches * cap * R * C * 4].view(torch.float32).view(caches, cap, R, C)[:, :n]
        return {"rho": rho, "L": L, "c": c}
    wk = cfg.weight_keys(level)
    if wk:
        w = tree[gb : gb + caches * cap * R * wk * 4].view(torch.float32).view(caches, cap, R, wk)[:, :n]
        return {"w": w, "L": L, "c": c}
    sb = int(tl.s_offset[i])
    if sb >= 0 and cfg.g_dtype == "fp4":
        # E2M1 nibble (low first) of (j, e), step st = e // 32, k-group kg = (e % 32) // 8, in byte
        # (kg * R + j) * 16 + st * 4 + (e % 8) // 2; block scales [R][d / 32] as E8M0 bytes
        raw = tree[gb : gb + caches * cap * R * d // 2].view(caches, cap, -1)[:, :n].to(torch.int32)
        nib = torch.stack([raw & 15, raw >> 4], dim=-1).reshape(caches, n, 4, R, 4, 8)  # [kg][j][st][e % 8]
        table = torch.tensor([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], device=tree.device)
        vals = table[nib & 7] * torch.where(nib >= 8, -1.0, 1.0)
        vals = vals.permute(0, 1, 3, 4, 2, 5).reshape(caches, n, R, d)  # [j][st][kg][e % 8] -> d
        e8 = tree[sb : sb + caches * cap * R * (d // 32)].view(caches, cap, R, d // 32)[:, :n].to(torch.float32)
        scale = torch.where(e8 == 0, torch.tensor(2.0**-127, device=tree.device), torch.exp2(e8 - 127.0))
        return {"g": vals * scale.repeat_interleave(32, dim=-1), "scale": scale, "L": L, "c": c}
    if sb >= 0:
        # E4M3 byte of (j, e) with step s = e // 32, k-group kg = (e % 32) // 8 at
        # ((s // 2) * 4 * R + kg * R + j) * 16 + (s % 2) * 8 + e % 8
        raw = tree[gb : gb + caches * cap * R * d].view(torch.float8_e4m3fn).view(caches, cap, -1)[:, :n]
        vals = raw.float().reshape(caches, n, d // 64, 4, R, 2, 8).permute(0, 1, 4, 2, 5, 3, 6).reshape(caches, n, R, d)
        scale = tree[sb : sb + caches * cap * R * 4].view(torch.float32).view(caches, cap, R)[:, :n]
        return {"g": vals * scale.unsqueeze(-1), "scale": scale, "L": L, "c": c}
    graw = tree[gb : gb + caches * cap * R * d * cfg.esize].view(cfg.torch_dtype).view(caches, cap, -1)[:, :n]
    pieces = d // E
    # element offset ((k//4)*4*R + (k%4)*R + j)*E + e  ->  [k//4][k%4][j][e]
    g = graw.reshape(caches, n, pieces // 4, 4, R, E).permute(0, 1, 4, 2, 3, 5).reshape(caches, n, R, d)
    return {"g": g, "L": L, "c": c}


def unpack_bits(words: torch.Tensor, n: int) -> torch.Tensor:
    """[..., W] uint32 words (int32 storage) -> [..., n] bool."""
    w = words.to(torch.int64) & 0xFFFFFFFF
    bits = (w.unsqueeze(-1) >> torch.arange(32, device=w.device)) & 1
    return bits.reshape(*words.shape[:-1], -1)[..., :n].bool()


def pack_bits(mask: torch.Tensor, words: int) -> torch.Tensor:
    """[..., n] bool -> [..., words] int32 (uint32 bit patterns)."""
    n = mask.shape[-1]
    pad = words * 32 - n
    m = torch.nn.functional.pad(mask.to(torch.int64), (0, pad)).reshape(*mask.shape[:-1], words, 32)
    w = (m << torch.arange(32, device=m.device)).sum(-1)
    w = torch.where(w >= 2**31, w - 2**32, w)
    return w.to(torch.int32)


def level_scores(buf: RouteBuffers, level: int) -> torch.Tensor:
    """Score rows of a level, [n_queries, score_stride] (a view into buf.score)."""
    rl = buf.layout
    nq, st = int(rl.n_queries), int(rl.score_stride[level - 1])
    off = int(rl.score_offset[level - 1])
    return buf.score[off : off + nq * st].view(nq, st)


def stats_records(buf: RouteBuffers, level: int) -> List[SelectStats]:
    rl = buf.layout
    nq = int(rl.n_queries)
    off = int(rl.stats_offset[level - 1]) * STATS_BYTES
    raw = bytes(buf.stats[off : off + nq * STATS_BYTES].cpu().numpy().tobytes())
    return [SelectStats.from_buffer_copy(raw[i * STATS_BYTES : (i + 1) * STATS_BYTES]) for i in range(nq)]


def level_sizes(n_tokens: int, chunk: int, levels: int) -> List[int]:
    sizes = [n_tokens // chunk]
    for _ in range(1, levels):
        sizes.append(-(-sizes[-1] // chunk))
    return sizes
