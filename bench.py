#!/usr/bin/env python3
"""Routed ZHA decode on one MI355X: queries/s and HBM roofline.

One step = one decode step of the whole hot path on the 1M-token deep-tree
workload (8 sequences x 8 KV heads x 4 query heads, d = 128, bf16 K/V,
chunk 4, 6 levels, 16 reference queries, p = 0.95):
  zha_append  (4,096 new tokens per sequence: new leaves + ancestors)
  zha_route   (256 decode queries, 6 levels of score + top-p select)
  zha_attend  (exact attention over the routed keys, sink, current chunk)
Inputs are seeded synthetic data already resident in HBM.  Prints one JSON
line (rank 0).  ``--gpus`` above 1 is refused: the library runs on one GPU.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import platform
import sys
import time

import numpy as np
import torch

from tree_indexed_sparse_zha_amd import workloads as W
from tree_indexed_sparse_zha_amd import zha

HBM_PEAK_GBS = 8000.0
FLAGS = zha.ZHA_SINK | zha.ZHA_LAST_CHUNK
ROOT = os.path.dirname(os.path.abspath(__file__))


def recorded_traffic(kernel: str, workload: str, leaf_form: str, p: float):
    """HBM bytes per launch of ``kernel`` measured by rocprofv3 counters
    (profiles/<workload>_traffic.json), or None when no record exists for
    this configuration or the kernel's source changed since it was taken."""
    import hashlib

    path = os.path.join(ROOT, "profiles", f"{workload}_traffic.json")
    if abs(p - 0.95) > 1e-9 or not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("leaf_form", "weights") != leaf_form:
        return None
    k = rec.get("kernels", {}).get(kernel)
    if not k:
        return None
    # the kernel's own source and the device headers every kernel includes
    for src in (k["source"], "zha_device.h", "zha_internal.h"):
        with open(os.path.join(ROOT, "tree_indexed_sparse_zha_amd", "csrc", src), "rb") as f:
            h = hashlib.sha256(f.read()).hexdigest()[:16]
        if h != rec["sources"].get(src):
            return None
    return k["bytes"]


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def cfg_of(w: W.Workload, capacity: int, leaf_form: str, g_dtype: str = "kv") -> zha.ZhaConfig:
    return zha.ZhaConfig(
        w.batch, w.n_kv_heads, w.q_per_kv, w.head_dim, w.n_ref, w.chunk, w.levels, w.dtype, capacity, leaf_form,
        g_dtype,
    )


def level_sizes(n, C, L):
    return zha.level_sizes(n, C, L)


def unpack_level(cfg, buf, lv, n_nodes):
    rl = buf.layout
    i = lv - 1
    nq, w = int(rl.n_queries), int(rl.words[i])
    off = int(rl.sel_offset[i])
    return zha.unpack_bits(buf.sel[off : off + nq * w].view(nq, w), n_nodes)


def selection_bytes(cfg: zha.ZhaConfig, buf, n_tokens: int, T: int, logits: bool = False, top: int = 0):
    """Algorithmic bytes of one route + attend from the selection it made.

    route, per cache and level: |union over the cache's queries of the
    candidates| x (R*d*2 bytes of g + 4R bytes of c; fp8 g: R*d + 8R with the
    row scales), or at level 1 in the weights forms x (C*d*2 bytes of keys +
    4RC of weights + 4R of c, plus 4*min(QC,16) bytes of logits written per
    key when they are kept); level 2 in "weights2" x (C*C*d*2 bytes of keys +
    C*4RC of its chunks' weights + 4RC of child shares + 4R of c), or with
    at most 4 queries per cache x (C*C*d*2 bytes of keys + 4R of its L +
    C*4R of its chunks' L read, the weights, shares and offsets recomputed;
    its chunks' level-1 scores (C*4*QC) and the logits of its keys
    (C*C*4*QC) written), while level 1 then reads or writes each score row
    entry once (4*QC bytes per chunk of the level);
    attend, per cache: |union over the cache's queries of the attended keys|
    x (d*2 bytes of V + d*2 bytes of K, or 4*min(QC,16) bytes of cached
    logits).  Also returns per-query selected share and per-level counts.
    """
    C, Lv, R, d = cfg.chunk, cfg.levels, cfg.n_ref, cfg.head_dim
    sizes = level_sizes(n_tokens, C, Lv)
    caches, QC = cfg.n_caches, cfg.q_per_kv * T
    gsize = 1 if cfg.g_dtype == "fp8" else cfg.esize  # bytes per stored g element
    node_bytes = R * d * gsize + 4 * R * (2 if cfg.g_dtype == "fp8" else 1)  # g, c (+ row scales)
    QW = min(QC, 16)  # useful logits per key (rows are padded to 4 in memory)
    top = top or Lv  # routing starts here; the levels above are not read
    fused = cfg.weight_keys(2) > 0 and QC <= 4 and top >= 2

    level_bytes = {lv: node_bytes for lv in range(1, Lv + 1)}
    if cfg.weights:  # level 1 from its keys and weights
        level_bytes[1] = C * d * cfg.esize + R * C * 4 + 4 * R + (C * QW * 4 if logits else 0)
    if cfg.weight_keys(2):
        if fused:  # its keys and the L of it and of its chunks; writes the level-1 scores (and logits)
            level_bytes[2] = C * C * d * cfg.esize + C * 4 * R + 4 * R + C * 4 * QC + (C * C * QW * 4 if logits else 0)
        else:  # its keys, its chunks' weights, its child shares and its c
            level_bytes[2] = C * C * d * cfg.esize + C * R * C * 4 + R * C * 4 + 4 * R
    per_level = {}
    kept_prev = None
    for lv in range(top, 0, -1):
        n = sizes[lv - 1]
        if lv == top:
            cand = torch.ones(caches * QC, n, dtype=torch.bool, device="cuda")
        else:
            cand = kept_prev.repeat_interleave(C, dim=1)[:, :n]
        kept = unpack_level(cfg, buf, lv, n)
        union = cand.view(caches, QC, n).any(dim=1).sum().item()
        per_level[lv] = dict(
            nodes=n,
            cand_per_query=float(cand.sum().item()) / (caches * QC),
            kept_per_query=float(kept.sum().item()) / (caches * QC),
            union_cand_per_cache=union / caches,
            alg_bytes=(caches * QC * n * 4) if (lv == 1 and fused) else union * level_bytes[lv],
        )
        kept_prev = kept
    # attended keys: kept chunks + sink + current chunk
    kept1 = kept_prev
    n1 = sizes[0]
    keys = kept1.repeat_interleave(C, dim=1)
    if keys.shape[1] < n_tokens:
        keys = torch.nn.functional.pad(keys, (0, n_tokens - keys.shape[1]))
    keys[:, 0] = True
    keys[:, C * ((n_tokens - 1) // C) : n_tokens] = True
    phi = keys.sum(dim=1).float() / n_tokens
    union_keys = keys.view(caches, QC, n_tokens).any(dim=1).sum().item()
    attend_bytes = union_keys * (d * cfg.esize + (QW * 4 if logits else d * cfg.esize))
    del keys
    return per_level, attend_bytes, phi.mean().item(), phi.min().item(), phi.max().item(), union_keys / caches


def cpu_baseline(w: W.Workload, batch, n0: int, p: float, T: int, cfg: zha.ZhaConfig, target_s: float = 10.0):
    """Time the CPU oracle on a bounded sample of the step: caches in order
    (sequence 0, KV head 0, then the next heads), each one decode step =
    build of the appended top span + route and attend of its G*T queries, on
    the oracle's tree of the same storage form, until about ``target_s``
    seconds of timed work.  Each cache's full tree build for the initial
    tokens is done first and not counted."""
    import oracle.zha_oracle as O

    try:
        from threadpoolctl import threadpool_info

        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas_threads = 1
    A = w.append_tokens
    n1 = n0 + A
    form = dict(leaf_dtype="f64" if cfg.weights else None, level2_dtype="f64" if cfg.weight_keys(2) else None)
    t_step = t_build_full = 0.0
    nq = n_caches = 0
    for cache in range(cfg.n_caches):
        b, h = divmod(cache, cfg.n_kv_heads)
        K = batch.K[b, h, :n1].to(torch.float64).cpu().numpy()
        V = batch.V[b, h, :n1].to(torch.float64).cpu().numpy()
        ref = batch.ref[h].to(torch.float64).cpu().numpy()
        Q = batch.Q[b, h].to(torch.float64).cpu().numpy()  # [G, T, d]
        t0 = time.time()
        tree = O.build_tree(K, ref, w.chunk, w.levels, w.dtype, n_tokens=n1, keep_g=False, **form)
        t_build_full += time.time() - t0
        # the step: the appended span's nodes, then route + attend of the cache's queries
        t0 = time.time()
        O.build_tree(K[n0:n1], ref, w.chunk, w.levels, w.dtype, keep_g=False, **form)
        for g in range(w.q_per_kv):
            for t in range(T):
                O.route_and_attend(Q[g, t], K, V, tree, ref, w.chunk, p, n1)
        t_step += time.time() - t0
        nq += w.q_per_kv * T
        n_caches += 1
        if t_step >= target_s:
            break
    return {
        "value": nq / t_step,
        "unit": "queries/s",
        "cores": int(blas_threads),
        "kind": "oracle",
        "sample": (
            f"{n_caches} of the workload's {cfg.n_caches} caches (sequence, KV head) at {n1} tokens, each: build of "
            f"the appended {A}-token top span + route and attend of its {w.q_per_kv * T} queries; {nq} queries, "
            f"fp64 numpy, {t_step:.1f} s timed (the oracle's initial full tree builds, {t_build_full:.1f} s, not "
            f"counted); BLAS threads {blas_threads}, other numpy work single-threaded; host "
            f"{platform.processor() or platform.machine()} with {len(os.sched_getaffinity(0))} usable cores"
        ),
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=8)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="deep1m")
    ap.add_argument("--p", type=float, default=None, help="top-p (default: the workload's first p)")
    ap.add_argument("--tokens", type=int, default=None, help="override the context length (sweeps)")
    ap.add_argument("--leaf-form", default="auto", choices=["auto", "weights", "weights2", "mean"],
                    help="storage of the bottom levels: level 1 as softmax weights scored from raw keys "
                         "(weights), levels 1 and 2 as weights (weights2; chunk 4), or mean keys; auto (default) "
                         "takes weights2 where level 1 can read level 2's logits (<= 4 queries per cache), "
                         "else weights where the chunk allows it, else mean")
    ap.add_argument("--p-levels", default=None,
                    help="depth-aware schedule: comma-separated p per level, level 1 first (overrides --p)")
    ap.add_argument("--top-level", type=int, default=0, help="level routing starts from (0 = the tree's top)")
    ap.add_argument("--g-dtype", default="kv", choices=["kv", "fp8"],
                    help="storage of the mean keys g: the KV dtype (default) or FP8 E4M3 with row scales")
    ap.add_argument("--no-logits", action="store_true",
                    help="attention recomputes every logit from K instead of reading the route's level-1 logits")
    ap.add_argument("--prefill", type=int, default=0,
                    help="chunked-prefill mode: each step appends a block of this many positions per sequence and "
                         "routes + attends all of them causally (prints its own JSON line)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(
            "bench.py measures the single-GPU path only; --gpus above 1 is not supported "
            "(the per-GPU share at real shape is what one GPU can show).",
            file=sys.stderr,
        )
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a ROCm GPU", file=sys.stderr)
        sys.exit(2)
    zha.load()
    w = W.WORKLOADS[args.workload]
    if args.tokens:
        w = w.with_tokens(args.tokens)
    if args.prefill:
        return prefill_main(args, w)
    p = args.p if args.p is not None else w.p[0]
    p_levels = [float(x) for x in args.p_levels.split(",")] if args.p_levels else None
    T = w.queries_per_head
    A = w.append_tokens
    n_steps = args.warmup + args.steps
    N0 = w.n_tokens
    capacity = N0 + n_steps * A
    if args.leaf_form == "auto":
        args.leaf_form = "weights2" if w.q_per_kv * T <= 4 and not args.no_logits else "weights"
    if args.leaf_form == "weights2" and (w.chunk != 4 or w.levels < 3 or args.g_dtype != "kv"):
        args.leaf_form = "weights"
    if args.leaf_form == "weights" and w.chunk not in (4, 8, 16):
        args.leaf_form = "mean"
    cfg = cfg_of(w, capacity, args.leaf_form, args.g_dtype)
    torch.cuda.set_device(0)
    log(f"workload {w.name}: N={N0} caches={cfg.n_caches} p={p} capacity={capacity}")

    t0 = time.time()
    batch = W.make_batch(w, device="cuda", capacity=capacity, append_steps=n_steps)
    torch.cuda.synchronize()
    log(f"generated inputs in {time.time() - t0:.1f}s")
    K, V, Q, ref = batch.K, batch.V, batch.Q, batch.ref
    tree = zha.alloc_tree(cfg)
    buf = zha.alloc_route(cfg, T, logits=not args.no_logits)
    nq = int(buf.layout.n_queries)
    out = torch.empty(nq, cfg.head_dim, device="cuda")
    lse = torch.empty(nq, device="cuda")
    ws = torch.empty(zha.attend_workspace_bytes(cfg, T), dtype=torch.uint8, device="cuda")
    log(
        f"tree {tree.numel() / 1e9:.1f} GB, K+V {2 * K.numel() * K.element_size() / 1e9:.1f} GB, "
        f"scores {buf.score.numel() * 4 / 1e9:.2f} GB"
    )

    # tree build over the initial context (reported separately)
    ev_build = zha.HipEvents(1)
    zha.build(cfg, K, ref, tree, N0, ev=ev_build)
    torch.cuda.synchronize()
    zha.build(cfg, K, ref, tree, N0, ev=ev_build)
    torch.cuda.synchronize()
    build_ms = ev_build.elapsed_ms()[0][2]
    log(f"build {build_ms:.2f} ms")

    ev_app = [zha.HipEvents(2) for _ in range(n_steps)]  # the split append launches two kernels
    ev_route = [zha.HipEvents(2 * cfg.levels) for _ in range(n_steps)]
    ev_att = [zha.HipEvents(2) for _ in range(n_steps)]

    def step(s):
        n_old = N0 + s * A
        zha.append(cfg, K, ref, tree, n_old, A, ev=ev_app[s])
        n = n_old + A
        if p_levels is not None or args.top_level:
            zha.route_levels(cfg, tree, n, Q, T, p_levels or [p] * cfg.levels, buf, top_level=args.top_level,
                             ev=ev_route[s], K=K)
        else:
            zha.route(cfg, tree, n, Q, T, p, buf, ev=ev_route[s], K=K)
        zha.attend(cfg, Q, T, K, V, n, zha.level1_sel(buf), FLAGS, out, lse, ws, ev=ev_att[s], logits=buf.logits)
        return n

    for s in range(args.warmup):
        step(s)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for s in range(args.warmup, n_steps):
        n_final = step(s)
    end.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    ms_per_step = total_ms / args.steps
    value = nq / (ms_per_step / 1e3)
    log(f"{ms_per_step:.3f} ms/step -> {value:.1f} queries/s")

    # per-kernel times over the timed steps
    kt = {}
    for s in range(args.warmup, n_steps):
        per_step = {}  # a stage may launch several kernels (the split append launches two)
        for evs in (ev_app[s], ev_route[s], ev_att[s]):
            for kid, lvl, ms in evs.elapsed_ms():
                key = f"{zha.KERNEL_NAMES[kid]}" + (f"_L{lvl}" if lvl else "")
                per_step[key] = per_step.get(key, 0.0) + ms
        for key, ms in per_step.items():
            kt.setdefault(key, []).append(ms)
    kmean = {k: float(np.mean(v)) for k, v in kt.items()}
    route_ms = sum(v for k, v in kmean.items() if k.startswith(("score", "select")))
    attend_ms = kmean.get("attend", 0.0) + kmean.get("combine", 0.0)
    append_ms = kmean.get("build", 0.0)

    # algorithmic bytes from the last step's selection
    per_level, attend_bytes, phi, phi_min, phi_max, ukeys = selection_bytes(
        cfg, buf, n_final, T, logits=buf.logits is not None, top=args.top_level
    )
    route_bytes = sum(v["alg_bytes"] for v in per_level.values())
    g8 = cfg.g_dtype == "fp8"
    mean_node = cfg.n_ref * (cfg.head_dim * (1 if g8 else cfg.esize) + (12 if g8 else 8))  # g, L, c (+ scales)
    # node bytes: weights [R][C] or child shares [R][C] (4RC) + L, c (8R); else the mean-key node
    tree_bytes_per_token = sum(
        (cfg.n_ref * (4 * cfg.chunk + 8) if cfg.weight_keys(l) else mean_node) / (cfg.chunk**l)
        for l in range(1, cfg.levels + 1)
    )
    append_bytes = cfg.n_caches * A * (cfg.head_dim * cfg.esize + tree_bytes_per_token)
    alg = {"attend": attend_bytes, "build": append_bytes}
    for lv, v in per_level.items():
        alg[f"score_L{lv}"] = v["alg_bytes"]
        alg[f"select_L{lv}"] = nq * v["nodes"] * 4  # one read of the score row per query
    dom = max(kmean, key=kmean.get)
    dom_bytes = alg.get(dom)
    roofline = {
        "kernel": dom,
        "bound": "hbm",
        "achieved": round(dom_bytes / (kmean[dom] / 1e3) / 1e9, 1) if dom_bytes else None,
        "peak": HBM_PEAK_GBS,
        "unit": "GB/s",
        "frac": round(dom_bytes / (kmean[dom] / 1e3) / 1e9 / HBM_PEAK_GBS, 4) if dom_bytes else None,
        "traffic": recorded_traffic(dom, w.name, cfg.leaf_form, p)
        if (p_levels is None and not args.top_level and cfg.g_dtype == "kv" and not args.tokens) else None,
        "alg_bytes_per_launch": dom_bytes,
        "avg_launch_ms": round(kmean[dom], 4),
    }
    ra_ms = route_ms + attend_ms
    ra_gbs = (route_bytes + attend_bytes) / (ra_ms / 1e3) / 1e9 if ra_ms > 0 else None

    dense = None
    if not args.no_dense:
        ev_d = zha.HipEvents(2)
        times = []
        for r in range(4):
            zha.dense_decode(cfg, Q, T, K, V, n_final, out, lse, ev=ev_d, ws=ws)
            torch.cuda.synchronize()
            if r:
                times.append(sum(ms for _, _, ms in ev_d.elapsed_ms()))
        dms = float(np.mean(times))
        dbytes = cfg.n_caches * n_final * 2 * cfg.head_dim * cfg.esize
        dense = {
            "ms": round(dms, 4),
            "queries_per_s": round(nq / (dms / 1e3), 1),
            "GB_s": round(dbytes / (dms / 1e3) / 1e9, 1),
            "frac_of_peak": round(dbytes / (dms / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
            "route_plus_attend_over_dense": round(ra_ms / dms, 3),
        }
        log(f"dense {dms:.3f} ms")

    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        cpu = cpu_baseline(w, batch, n_final - A, p, T, cfg)
        log(f"cpu baseline {cpu['value']:.3f} queries/s")

    res = {
        "metric": "routed decode queries/s + HBM GB/s (% of peak) at 1M ctx, deep tree",
        "value": round(value, 2),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": w.name,
            "n_tokens": N0,
            "batch": w.batch,
            "kv_heads": w.n_kv_heads,
            "q_per_kv": w.q_per_kv,
            "head_dim": w.head_dim,
            "chunk": w.chunk,
            "levels": w.levels,
            "n_ref": w.n_ref,
            "p": p_levels if p_levels is not None else p,
            "top_level": args.top_level or w.levels,
            "append_tokens_per_step": A,
            "leaf_form": cfg.leaf_form,
            "g_dtype": cfg.g_dtype,
            "cached_logits": buf.logits is not None,
            "queries_per_step": nq,
        },
        "roofline": roofline,
        "cpu_baseline": cpu,
        "route_attend": {
            "ms": round(ra_ms, 4),
            "alg_GB": round((route_bytes + attend_bytes) / 1e9, 3),
            "GB_s": round(ra_gbs, 1) if ra_gbs else None,
            "frac_of_peak": round(ra_gbs / HBM_PEAK_GBS, 4) if ra_gbs else None,
        },
        "append_ms": round(append_ms, 4),
        "kernel_ms": {k: round(v, 4) for k, v in sorted(kmean.items())},
        "alg_bytes": {k: int(v) for k, v in alg.items()},
        "selected_share": {"mean": round(phi, 4), "min": round(phi_min, 4), "max": round(phi_max, 4)},
        "levels": {str(k): {kk: round(vv, 2) for kk, vv in v.items()} for k, v in sorted(per_level.items())},
        "build": {
            "ms": round(build_ms, 3),
            "tokens_per_s": round(w.batch * N0 / (build_ms / 1e3), 1),
            "token_heads_per_s": round(cfg.n_caches * N0 / (build_ms / 1e3), 1),
            "GB_s": round(cfg.n_caches * N0 * (cfg.head_dim * cfg.esize + tree_bytes_per_token) / (build_ms / 1e3) / 1e9, 1),
        },
        "dense": dense,
    }
    print(json.dumps(res), flush=True)


def prefill_main(args, w):
    """Chunked prefill: per step, append a block of P positions to every
    sequence, build the block's spine, route all its queries on their prefix
    trees and attend causally; against the same-GPU dense causal attention of
    the block."""
    P = args.prefill
    p = args.p if args.p is not None else w.p[0]
    n_steps = args.warmup + args.steps
    N0 = w.n_tokens
    # the appended positions hold the workload's appended segments (zeros when it has none)
    app = -(-n_steps * P // w.append_tokens) if w.append_tokens else 0
    capacity = N0 + max(n_steps * P, app * w.append_tokens)
    # the prefill spine takes mean keys above level 1: level-2 weights fall back to the weights form
    leaf_form = "weights" if args.leaf_form in ("auto", "weights2") else args.leaf_form
    leaf_form = leaf_form if w.chunk in (4, 8, 16) else "mean"
    cfg = cfg_of(w, capacity, leaf_form, args.g_dtype)
    if cfg.q_per_kv * P > 1024:
        print("--prefill: q_per_kv * block must be <= 1024", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    log(f"prefill {w.name}: N0={N0} block={P} caches={cfg.n_caches} p={p}")
    batch = W.make_batch(w, device="cuda", capacity=capacity, append_steps=app)
    K, V, ref = batch.K, batch.V, batch.ref
    # the block's queries: synthetic, seeded; K/V of the appended positions stay those of the generator
    gq = torch.Generator(device="cuda")
    gq.manual_seed(12345)
    Q = torch.randn(cfg.batch, cfg.n_kv_heads, cfg.q_per_kv, P, cfg.head_dim, generator=gq, device="cuda").to(
        cfg.torch_dtype)
    tree = zha.alloc_tree(cfg)
    spine = zha.alloc_spine(cfg, P)
    # the cached level-1 logits grow with queries x context: keep them only while they stay small
    keep_logits = cfg.leaf_form == "weights" and zha.route_layout(cfg, P).logits_floats * 4 <= (8 << 30)
    buf = zha.alloc_route(cfg, P, logits=keep_logits)
    nq = int(buf.layout.n_queries)
    out = torch.empty(nq, cfg.head_dim, device="cuda")
    lse = torch.empty(nq, device="cuda")
    ws = torch.empty(zha.attend_workspace_bytes(cfg, P), dtype=torch.uint8, device="cuda")
    zha.build(cfg, K, ref, tree, N0)
    torch.cuda.synchronize()
    flags = FLAGS | zha.ZHA_CAUSAL
    ev = [[zha.HipEvents(2 * cfg.levels + 4) for _ in range(4)] for _ in range(n_steps)]

    def step(s):
        n_old = N0 + s * P
        n = n_old + P
        zha.append(cfg, K, ref, tree, n_old, P, ev=ev[s][0])
        zha.build_spine(cfg, K, ref, spine, n, P, ev=ev[s][1])
        zha.route_prefill(cfg, tree, spine, n, Q, P, p, buf, ev=ev[s][2], K=K)
        zha.attend(cfg, Q, P, K, V, n, zha.level1_sel(buf), flags, out, lse, ws, ev=ev[s][3], logits=buf.logits)
        return n

    for s in range(args.warmup):
        step(s)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for s in range(args.warmup, n_steps):
        n_final = step(s)
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    parts = {}
    for s in range(args.warmup, n_steps):
        for name, e in zip(("append", "spine", "route", "attend"), ev[s]):
            parts.setdefault(name, []).append(sum(x[2] for x in e.elapsed_ms()))
    parts = {k: round(float(np.mean(v)), 4) for k, v in parts.items()}
    dense_ms = None
    if not args.no_dense:
        ev_d = zha.HipEvents(2)
        times = []
        for r in range(4):
            zha.attend(cfg, Q, P, K, V, n_final, None, zha.ZHA_ALL_KEYS | zha.ZHA_CAUSAL, out, lse, ws, ev=ev_d)
            torch.cuda.synchronize()
            if r:
                times.append(sum(x[2] for x in ev_d.elapsed_ms()))
        dense_ms = round(float(np.mean(times)), 4)
    tokens = cfg.batch * P
    res = {
        "metric": "chunked prefill tokens/s (routed, causal)",
        "value": round(tokens / (ms / 1e3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {
            "workload": w.name + "-prefill",
            "context_at_block_end": n_final,
            "block_positions": P,
            "batch": w.batch,
            "kv_heads": w.n_kv_heads,
            "q_per_kv": w.q_per_kv,
            "chunk": w.chunk,
            "levels": w.levels,
            "n_ref": w.n_ref,
            "p": p,
            "leaf_form": cfg.leaf_form,
            "g_dtype": cfg.g_dtype,
            "cached_logits": keep_logits,
        },
        "stage_ms": parts,
        "dense_causal_attend_ms": dense_ms,
        "routed_over_dense": round((parts["spine"] + parts["route"] + parts["attend"]) / dense_ms, 3) if dense_ms else None,
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
