"""zha_attend_noalloc (the static-scratch variant of zha_attend, for callers
that cannot allocate) against zha_attend through the C ABI: two calls in a
row on the same GPU, the second with a smaller input, each bit-identical to
zha_attend with a caller workspace (the same kernels in the same launch
configuration), and within the bf16 tolerance of the oracle on sampled
queries."""
import math
import sys

import numpy as np
import pytest
import torch

import oracle.zha_oracle as O
from tests import parity as PAR
from tree_indexed_sparse_zha_amd import zha

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[no-alloc] {msg}", flush=True)
    sys.stdout.flush()


def _case(cfg, T, N, seed, logits):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    B, H, G, d, cap = cfg.batch, cfg.n_kv_heads, cfg.q_per_kv, cfg.head_dim, cfg.capacity
    K = torch.randn(B, H, cap, d, generator=g, device="cuda").to(torch.bfloat16)
    V = torch.randn(B, H, cap, d, generator=g, device="cuda").to(torch.bfloat16)
    Q = torch.randn(B, H, G, T, d, generator=g, device="cuda").to(torch.bfloat16)
    ref = (torch.randn(H, cfg.n_ref, d, generator=g, device="cuda") / math.sqrt(d)).to(torch.bfloat16).float()
    tree = zha.alloc_tree(cfg)
    zha.build(cfg, K, ref, tree, N)
    buf = zha.alloc_route(cfg, T, logits=logits)
    zha.route(cfg, tree, N, Q, T, 0.9, buf, K=K)
    return K, V, Q, buf


def _both(cfg, T, N, K, V, Q, buf, flags):
    nq = int(buf.layout.n_queries)
    ws = torch.empty(zha.attend_workspace_bytes(cfg, T), dtype=torch.uint8, device="cuda")
    assert ws.numel() <= zha.ZHA_NOALLOC_SCRATCH_BYTES
    o1, l1 = torch.full((nq, cfg.head_dim), float("nan"), device="cuda"), torch.full((nq,), float("nan"), device="cuda")
    o2, l2 = torch.full_like(o1, float("nan")), torch.full_like(l1, float("nan"))
    zha.attend(cfg, Q, T, K, V, N, zha.level1_sel(buf), flags, o1, l1, ws, logits=buf.logits)
    zha.attend_noalloc(cfg, Q, T, K, V, N, zha.level1_sel(buf), flags, o2, l2, logits=buf.logits)
    torch.cuda.synchronize()
    return (o1, l1), (o2, l2)


def test_noalloc_matches_attend_twice_second_smaller():
    torch.cuda.set_device(0)
    zha.load()
    flags = zha.ZHA_SINK | zha.ZHA_LAST_CHUNK
    # first call: 2 x 4 caches, 4 queries each, 300K tokens (many key tiles, cached logits)
    cfg_a = zha.ZhaConfig(2, 4, 4, 128, 16, 4, 6, "bf16", 300_000, "weights2")
    # second call: a smaller input on the same GPU (fewer caches, tokens and tiles; no cached logits)
    cfg_b = zha.ZhaConfig(1, 2, 4, 128, 16, 4, 5, "bf16", 20_000, "weights")
    for name, cfg, T, N, logits, seed in (("large", cfg_a, 1, 299_993, True, 1), ("small", cfg_b, 2, 17_001, False, 2)):
        _say(f"{name}: caches {cfg.n_caches}, T {T}, N {N}, scratch "
             f"{zha.attend_workspace_bytes(cfg, T)} of {zha.ZHA_NOALLOC_SCRATCH_BYTES} bytes")
        K, V, Q, buf = _case(cfg, T, N, seed, logits)
        (o1, l1), (o2, l2) = _both(cfg, T, N, K, V, Q, buf, flags)
        assert torch.isfinite(o1).all() and torch.isfinite(l1).all()
        assert torch.equal(o1, o2), f"{name}: outputs differ by {float((o1 - o2).abs().max())}"
        assert torch.equal(l1, l2), f"{name}: lse differ by {float((l1 - l2).abs().max())}"
        # and the oracle on two sampled queries
        QC = cfg.q_per_kv * T
        sizes = O.level_sizes(N, cfg.chunk, cfg.levels)
        rl = buf.layout
        for qi in (0, int(rl.n_queries) - 1):
            cache, ql = divmod(qi, QC)
            b, h = divmod(cache, cfg.n_kv_heads)
            w = int(rl.words[0])
            bits = zha.unpack_bits(buf.sel[int(rl.sel_offset[0]) + qi * w: int(rl.sel_offset[0]) + (qi + 1) * w].cpu(),
                                   sizes[0]).numpy()
            idx = O.attend_set(np.nonzero(bits)[0], N, cfg.chunk, True, True)
            o, l = O.attend(Q[b, h, ql // T, ql % T].double().cpu().numpy(), K[b, h, :N].double().cpu().numpy(),
                            V[b, h, :N].double().cpu().numpy(), idx)
            np.testing.assert_allclose(o2[qi].cpu().numpy(), o, rtol=0, atol=PAR.OUT_TOL["bf16"])
            np.testing.assert_allclose(float(l2[qi]), l, rtol=0, atol=PAR.OUT_TOL["bf16"])
        _say(f"{name}: bit-identical to zha_attend, oracle ok")
        del K, V, Q, buf
