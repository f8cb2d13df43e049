"""The measurement probes (zha_stream_probe) write what their header says:
a copy is the source, and the tile mix writes, per 256 bytes read, the xor
of the 16 pieces one lane loaded (64 KiB tiles, rows of 256 bytes, lane
(wave w, q = lane % 16, k = lane / 16) reading row 64w + 16i + q, piece
4s + k, for i, s < 4), including a ragged last tile."""
import pytest
import torch

from tree_indexed_sparse_zha_amd import zha

pytestmark = pytest.mark.gpu


def _tile_mix_expected(src_i32: torch.Tensor, n_bytes: int) -> torch.Tensor:
    n16 = n_bytes // 16
    pieces = src_i32[: n16 * 4].view(n16, 4)
    tiles = (n16 + 4095) // 4096
    pad = torch.zeros(tiles * 4096, 4, dtype=torch.int32, device=src_i32.device)
    pad[:n16] = pieces
    t = torch.arange(256, device=src_i32.device)
    w, lane = t // 64, t % 64
    q, k = lane % 16, lane // 16
    idx = torch.stack([(64 * w + 16 * i + q) * 16 + 4 * s + k for i in range(4) for s in range(4)], dim=1)  # [256, 16]
    out = []
    for b in range(tiles):
        v = pad[b * 4096 + idx]  # [256, 16, 4]
        x = v[:, 0]
        for j in range(1, 16):
            x = torch.bitwise_xor(x, v[:, j])
        out.append(x)
    full = torch.cat(out)  # [tiles * 256, 4]
    n_out = (n16 + 15) // 16
    return full[:n_out]


@pytest.mark.parametrize("n_bytes", [3 * 65536, 2 * 65536 + 4096 + 192])
def test_tile_mix_and_copy_write_what_they_read(n_bytes):
    torch.manual_seed(7)
    src = torch.randint(-(2**31), 2**31 - 1, (n_bytes // 4,), dtype=torch.int32, device="cuda")
    n_out = (n_bytes // 16 + 15) // 16
    dst = torch.full((n_out * 4 + 64,), 12345, dtype=torch.int32, device="cuda")
    zha.stream_probe("tile_mix", src, dst, n_bytes)
    torch.cuda.synchronize()
    exp = _tile_mix_expected(src, n_bytes)
    assert torch.equal(dst[: n_out * 4].view(n_out, 4), exp)
    assert bool((dst[n_out * 4 :] == 12345).all())  # nothing past n_bytes / 16
    cp = torch.zeros(n_bytes // 4, dtype=torch.int32, device="cuda")
    zha.stream_probe("copy", src, cp, n_bytes)
    torch.cuda.synchronize()
    assert torch.equal(cp, src)
