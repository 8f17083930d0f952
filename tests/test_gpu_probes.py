"""The HBM ceiling probes (snac_hbm_probe) move what they claim to, at launch
shapes the benchmark uses and sizes with whole tiles, a short last tile and
fewer tiles than workgroups: the copy probe copies every byte, the write
probe writes its word everywhere and nowhere else, and the read probe's
first lane reads exactly its words (its sink is written only when the XOR
of what it read equals `magic`, which the test computes on the host)."""
from __future__ import annotations

import numpy as np
import pytest

import copy_reduce_snac_amd as snac
from copy_reduce_snac_amd import workloads as wl
from gpu_helpers import CANARY, DevBuf, gpu_available

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

SHAPES = [(64, 4096, 2), (64, 4096, 5), (64, 16384, 3), (256, 16384, 1), (256, 4096, 4)]
# whole tiles, a short last tile, and fewer tiles than workgroups
SIZES = [16, 4096 * 7 + 48, 16384 * 300, (1 << 22) + 16 * 5]


def sync():
    import torch

    torch.cuda.synchronize()


@pytest.mark.parametrize("threads,tile,wgs", SHAPES)
@pytest.mark.parametrize("nbytes", SIZES)
def test_probe_copy_write_read(threads, tile, wgs, nbytes):
    data = wl.raw_bytes(nbytes, wl.CFG_TEST, 3, seed=nbytes % 1000)
    src = DevBuf(nbytes, data=data)
    dst = DevBuf(nbytes)
    snac.snac_hbm_probe("copy", dst.ptr, src.ptr, nbytes, threads, tile, wgs)
    sync()
    assert dst.guards_ok(), "copy probe wrote outside its range"
    assert np.array_equal(dst.download(), data), "copy probe output differs from its input"

    magic = 0x5A5AA5A5
    snac.snac_hbm_probe("write", dst.ptr, None, nbytes, threads, tile, wgs, magic)
    sync()
    assert dst.guards_ok(), "write probe wrote outside its range"
    assert np.all(dst.download(np.uint32) == magic)

    # the read probe folds, per lane, every word it reads; lane 0 of
    # workgroup 0 reads unit u of tiles 0, grid, 2 grid, ... at byte
    # t * tile + u * threads * 16 (words past the end read as zero).  Its fold,
    # computed here, is the magic: the sink is then written only if that
    # lane read exactly those words.
    import torch

    cus = torch.cuda.get_device_properties(0).multi_processor_count
    tiles = -(-nbytes // tile)
    grid = min(cus * wgs, tiles)
    words = data.view(np.uint32)
    fold = 0
    for t in range(0, tiles, grid):
        for u in range(tile // (threads * 16)):
            off = t * tile + u * threads * 16
            if off < nbytes and off < t * tile + tile:
                fold ^= int(np.bitwise_xor.reduce(words[off // 4:off // 4 + 4]))
    sink = DevBuf(4)
    sink.upload(np.array([~fold & 0xFFFFFFFF], dtype=np.uint32))
    snac.snac_hbm_probe("read", sink.ptr, src.ptr, nbytes, threads, tile, wgs, fold)
    sync()
    assert sink.guards_ok()
    assert int(sink.download(np.uint32)[0]) == fold, "lane 0 of workgroup 0 did not read exactly its words"


@pytest.mark.parametrize("threads,tile,wgs", [(256, 16384, 1), (64, 16384, 2), (256, 16384, 2)])
@pytest.mark.parametrize("nbytes", [16384 * 300, (1 << 22) + 16 * 5, 16384 * 4096 + 48])
def test_ordered_probes_copy_and_write(threads, tile, wgs, nbytes):
    """With tiles handed out in order from the probes' counters, the copy
    probe still copies every byte once and the write probe writes its word
    everywhere, twice in a row (the counters are left at zero for the next
    launch)."""
    data = wl.raw_bytes(nbytes, wl.CFG_TEST, 5, seed=nbytes % 997)
    src = DevBuf(nbytes, data=data)
    for rep in range(2):
        dst = DevBuf(nbytes)
        snac.snac_hbm_probe("copy_ordered", dst.ptr, src.ptr, nbytes, threads, tile, wgs)
        sync()
        assert dst.guards_ok(), f"ordered copy probe wrote outside its range (call {rep})"
        assert np.array_equal(dst.download(), data), f"ordered copy probe output differs (call {rep})"
        magic = 0x3C3CC3C3 + rep
        snac.snac_hbm_probe("write_ordered", dst.ptr, None, nbytes, threads, tile, wgs, magic)
        sync()
        assert dst.guards_ok()
        assert np.all(dst.download(np.uint32) == magic), f"ordered write probe missed words (call {rep})"
    sink = DevBuf(4)
    snac.snac_hbm_probe("read_ordered", sink.ptr, src.ptr, nbytes, threads, tile, wgs, 0)
    sync()
    assert sink.guards_ok()
