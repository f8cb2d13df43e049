"""Seeded synthetic workloads for the ZHA decode path.

This module only draws random inputs.  It contains none of the method's
arithmetic (no logsumexp, no scores, no selection, no attention), so that the
HIP path and the CPU oracle can both be fed from it without sharing any code
that computes a result.

Workload shapes follow the two trees the ZHA explainer describes (MTP =
the article "Zyphra AI Introduces Zyphra Hierarchical Attention (ZHA): A Path
to True Subquadratic Attention", section "How does ZHA perform against dense
attention and MSA?": deep tree = chunk 4 with 6 levels, wide tree = chunk 256
with 1 level, 16 reference queries, p = 0.95).  The pages evaluate on public
long-context suites; none of their items is reproduced here.  Instead the keys
carry the structure those suites exercise:

* region structure: keys come in contiguous segments, each segment drawn
  around its own mean (``k = mu_s + 0.5 * eps``, ``mu_s ~ N(0, I)``);
* concentrated versus diffuse queries (MTP, "How does top-p routing pick
  tokens?": a single-fact lookup touches few branches, a many-fact query
  expands more): a planted needle key ``k = 2 q + sqrt(0.1) * eps`` makes the
  owning query's attention peak on it; diffuse queries own many needles.

Notation ``N(a, b)`` takes ``b`` as the variance.  Reference queries are drawn
``r ~ N(0, I/d)``; the pages learn them by distillation, which is out of scope.
For bf16 workloads every tensor is drawn in fp32 and rounded once
(round-to-nearest-even) to bf16; reference queries are returned as fp32 that
hold bf16-representable values.

All randomness is derived from ``(workload id, stream, sequence, kv head,
step)`` so that one cache can be regenerated on its own.  Generation runs on
whatever torch device is given; a test generates once and feeds both sides.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional, Tuple

import numpy as np
import torch

# random streams
S_SEG_MEAN = 1
S_KEY_NOISE = 2
S_VALUES = 3
S_REF = 4
S_QUERY = 5
S_NEEDLE = 6
S_APPEND = 7


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic decode workload (shapes, dtype, tree geometry, recipe)."""

    wid: int
    name: str
    batch: int
    n_kv_heads: int
    q_per_kv: int
    head_dim: int
    dtype: str  # "f32" or "bf16": K, V, Q and stored g
    n_tokens: int
    chunk: int
    levels: int
    n_ref: int
    p: Tuple[float, ...]
    queries_per_head: int  # T: decode queries per query head per step
    segment_len: int
    # needle plan: for query head g and query t, how many needles it owns
    needles_concentrated: int  # per concentrated query
    needles_diffuse: int  # per diffuse query
    append_tokens: int = 0  # tokens appended per decode step

    @property
    def n_caches(self) -> int:
        return self.batch * self.n_kv_heads

    @property
    def queries_per_cache(self) -> int:
        return self.q_per_kv * self.queries_per_head

    @property
    def n_queries(self) -> int:
        return self.n_caches * self.queries_per_cache

    @property
    def top_span(self) -> int:
        return self.chunk ** self.levels

    def needle_counts(self) -> np.ndarray:
        """Needles owned by each query of a cache, shape [G, T]."""
        G, T = self.q_per_kv, self.queries_per_head
        out = np.zeros((G, T), dtype=np.int64)
        if self.name == "tiny" or self.name == "deep32k":
            # queries t = 0..7 of every head own one needle, the rest none
            out[:, : min(8, T)] = self.needles_concentrated
        else:
            # heads in the first half concentrated, second half diffuse
            half = G // 2
            out[:half, :] = self.needles_concentrated
            out[half:, :] = self.needles_diffuse
        return out

    def with_tokens(self, n_tokens: int) -> "Workload":
        return dataclasses.replace(self, n_tokens=n_tokens)

    def with_batch(self, batch: int, n_kv_heads: Optional[int] = None) -> "Workload":
        return dataclasses.replace(
            self, batch=batch, n_kv_heads=self.n_kv_heads if n_kv_heads is None else n_kv_heads
        )


WORKLOADS: Dict[str, Workload] = {
    w.name: w
    for w in [
        Workload(0, "tiny", 1, 1, 1, 64, "f32", 4096, 4, 3, 4, (0.95,), 16, 256, 1, 0),
        Workload(1, "deep32k", 1, 8, 4, 128, "bf16", 32768, 4, 6, 16, (0.95,), 64, 512, 1, 0),
        Workload(2, "wide256k", 4, 8, 4, 128, "bf16", 262144, 256, 1, 16, (0.95,), 1, 4096, 1, 64),
        Workload(
            3, "deep1m", 8, 8, 4, 128, "bf16", 1048576, 4, 6, 16, (0.95, 0.9, 0.99), 1, 1024, 1, 127,
            append_tokens=4096,
        ),
        Workload(4, "deep10m", 2, 2, 4, 128, "bf16", 10485760, 4, 6, 16, (0.95,), 1, 10240, 1, 127),
        # The pages' lightweight speed-model geometry: 1 reference query, chunk 8.
        Workload(
            5, "light1m", 8, 8, 4, 128, "bf16", 1048576, 8, 4, 1, (0.75,), 1, 1024, 1, 127,
            append_tokens=4096,
        ),
    ]
}


def _seed(wid: int, stream: int, b: int, h: int, step: int = 0) -> int:
    ss = np.random.SeedSequence([1_000_003, wid, stream, b, h, step])
    return int(ss.generate_state(1, dtype=np.uint64)[0] & ((1 << 63) - 1))


def _gen(device, wid, stream, b, h, step=0) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(_seed(wid, stream, b, h, step))
    return g


def _round(x: torch.Tensor, dtype: str) -> torch.Tensor:
    if dtype == "bf16":
        return x.to(torch.bfloat16)
    return x.to(torch.float32)


def torch_dtype(dtype: str) -> torch.dtype:
    return torch.bfloat16 if dtype == "bf16" else torch.float32


@dataclasses.dataclass
class Batch:
    """Device tensors of one workload instance.

    K, V: [B, H, capacity, d] (dtype), Q: [B, H, G, T, d] (dtype),
    ref: [H, R, d] fp32, needle_pos: [B, H] lists of positions per query.
    """

    K: torch.Tensor
    V: torch.Tensor
    Q: torch.Tensor
    ref: torch.Tensor
    n_tokens: int
    capacity: int
    needles: List[List[np.ndarray]]  # [cache][query] -> positions


def make_ref(w: Workload, device="cpu") -> torch.Tensor:
    """Reference queries [H, R, d], r ~ N(0, I/d), bf16-representable for bf16."""
    out = torch.empty(w.n_kv_heads, w.n_ref, w.head_dim, dtype=torch.float32, device=device)
    for h in range(w.n_kv_heads):
        g = _gen(device, w.wid, S_REF, 0, h)
        r = torch.randn(w.n_ref, w.head_dim, generator=g, device=device) / math.sqrt(w.head_dim)
        out[h] = _round(r, w.dtype).to(torch.float32)
    return out


def make_queries(w: Workload, device="cpu", step: int = 0) -> torch.Tensor:
    """Decode queries [B, H, G, T, d], q ~ N(0, I)."""
    B, H, G, T, d = w.batch, w.n_kv_heads, w.q_per_kv, w.queries_per_head, w.head_dim
    out = torch.empty(B, H, G, T, d, dtype=torch_dtype(w.dtype), device=device)
    for b in range(B):
        for h in range(H):
            g = _gen(device, w.wid, S_QUERY, b, h, step)
            out[b, h] = _round(torch.randn(G, T, d, generator=g, device=device), w.dtype)
    return out


def _fill_segments(dst: torch.Tensor, n: int, seg: int, gen: torch.Generator, gen_noise: torch.Generator):
    """dst[:n] <- mu_{s(i)} + 0.5 eps, with contiguous segments of ``seg`` keys."""
    d = dst.shape[-1]
    device = dst.device
    n_seg = (n + seg - 1) // seg
    mu = torch.randn(n_seg, d, generator=gen, device=device)
    # work in slabs to bound temporary memory
    slab = max(seg, (1 << 22) // d // seg * seg)
    for s0 in range(0, n, slab):
        s1 = min(n, s0 + slab)
        eps = torch.randn(s1 - s0, d, generator=gen_noise, device=device)
        idx = torch.arange(s0, s1, device=device) // seg
        dst[s0:s1] = (mu[idx] + 0.5 * eps).to(dst.dtype)


def make_batch(
    w: Workload,
    device="cpu",
    capacity: Optional[int] = None,
    append_steps: int = 0,
    caches: Optional[List[Tuple[int, int]]] = None,
) -> Batch:
    """Generate K, V, Q, ref for workload ``w``.

    ``capacity`` sizes the token dimension of K/V (default ``n_tokens`` plus
    ``append_steps * append_tokens``).  Tokens past ``n_tokens`` are the
    appended ones: fresh segments of ``segment_len`` keys, no needles, drawn
    per step from their own stream so that step s does not depend on how many
    steps are generated.
    """
    B, H, d = w.batch, w.n_kv_heads, w.head_dim
    N = w.n_tokens
    if capacity is None:
        capacity = N + append_steps * w.append_tokens
    assert capacity >= N + append_steps * w.append_tokens
    dt = torch_dtype(w.dtype)
    K = torch.zeros(B, H, capacity, d, dtype=dt, device=device)
    V = torch.zeros(B, H, capacity, d, dtype=dt, device=device)
    Q = make_queries(w, device)
    ref = make_ref(w, device)
    counts = w.needle_counts()
    needles: List[List[np.ndarray]] = []
    all_caches = [(b, h) for b in range(B) for h in range(H)]
    want = set(all_caches if caches is None else caches)
    for b, h in all_caches:
        if (b, h) not in want:
            needles.append([])
            continue
        _fill_segments(K[b, h], N, w.segment_len, _gen(device, w.wid, S_SEG_MEAN, b, h), _gen(device, w.wid, S_KEY_NOISE, b, h))
        gv = _gen(device, w.wid, S_VALUES, b, h)
        for s0 in range(0, N, 1 << 20):
            s1 = min(N, s0 + (1 << 20))
            V[b, h, s0:s1] = torch.randn(s1 - s0, d, generator=gv, device=device).to(dt)
        # needles: distinct positions uniform in [C, N - C)
        gn = _gen(device, w.wid, S_NEEDLE, b, h)
        total = int(counts.sum())
        lo, hi = w.chunk, N - w.chunk
        pos = (torch.randperm(hi - lo, generator=gn, device=device)[:total] + lo).cpu().numpy()
        per_q: List[np.ndarray] = []
        k0 = 0
        G, T = w.q_per_kv, w.queries_per_head
        for gq in range(G):
            for t in range(T):
                c = int(counts[gq, t])
                pq = np.sort(pos[k0 : k0 + c])
                k0 += c
                per_q.append(pq)
                if c:
                    q32 = Q[b, h, gq, t].to(torch.float32)
                    eps = torch.randn(c, d, generator=gn, device=device)
                    nk = 2.0 * q32[None, :] + math.sqrt(0.1) * eps
                    K[b, h, torch.as_tensor(pq, device=device)] = nk.to(dt)
        needles.append(per_q)
        # appended tokens, step by step
        for s in range(append_steps):
            a0 = N + s * w.append_tokens
            a1 = a0 + w.append_tokens
            ga = _gen(device, w.wid, S_APPEND, b, h, s + 1)
            _fill_segments(K[b, h, a0:a1], a1 - a0, w.segment_len, ga, ga)
            V[b, h, a0:a1] = torch.randn(a1 - a0, d, generator=ga, device=device).to(dt)
    return Batch(K=K, V=V, Q=Q, ref=ref, n_tokens=N, capacity=capacity, needles=needles)


def random_cache(
    n_tokens: int,
    head_dim: int,
    n_ref: int,
    dtype: str = "f32",
    seed: int = 0,
    n_queries: int = 4,
    segment_len: int = 16,
    device="cpu",
):
    """Small single-cache input for unit tests: K, V [N, d]; ref [R, d]; Q [n, d]."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    d = head_dim
    n_seg = max(1, (n_tokens + segment_len - 1) // segment_len)
    mu = torch.randn(n_seg, d, generator=g, device=device)
    idx = torch.arange(n_tokens, device=device) // segment_len
    K = mu[idx] + 0.5 * torch.randn(n_tokens, d, generator=g, device=device)
    V = torch.randn(n_tokens, d, generator=g, device=device)
    ref = torch.randn(n_ref, d, generator=g, device=device) / math.sqrt(d)
    Q = torch.randn(n_queries, d, generator=g, device=device)
    dt = torch_dtype(dtype)
    return (
        K.to(dt),
        V.to(dt),
        _round(ref, dtype).to(torch.float32),
        Q.to(dt),
    )
