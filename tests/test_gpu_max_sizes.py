"""Sizes past the 32-bit boundaries: a copy of more than 4 GiB, an AllReduce
with more than 2^30 elements per rank, an AllToAll whose chunks are 2 GiB
and a SNAC pipeline call of 5 GiB per rank.  Byte offsets, element indices,
tile and unit numbers must not wrap.

The copy is compared whole on the GPU (a copy equals its source byte for
byte, at any size).  The AllReduce and the pipeline are checked by the
oracle on sampled positions (both are elementwise across ranks), the AllToAll by its definition (chunk s of output d is
chunk d of input s) on sampled positions: the first and last 4096 elements
of every output, positions around each 2^31 and 2^32 byte boundary, and
2^16 random positions.  The inputs are drawn by torch on the GPU."""
from __future__ import annotations

import numpy as np
import pytest

import copy_reduce_snac_amd as snac
import oracle
from gpu_helpers import assert_same, gpu_available

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

GiB = 1 << 30


@pytest.fixture(scope="module")
def torch():
    import torch

    torch.cuda.set_device(0)
    return torch


def sample_idx(m: int, esize: int, seed: int) -> np.ndarray:
    g = np.random.default_rng(seed)
    parts = [np.arange(min(4096, m)), np.arange(max(0, m - 4096), m), g.integers(0, m, size=1 << 16)]
    for b in (1 << 31, 1 << 32):
        e = b // esize
        parts.append(np.arange(max(0, e - 64), min(m, e + 64)))
    return np.unique(np.concatenate(parts))


def gather(torch, t, idx: np.ndarray):
    return t[torch.from_numpy(idx.astype(np.int64)).cuda()].cpu()


def random_bf16(torch, m: int, seed: int):
    """m finite bf16 values, made on the GPU in pieces (normal draws)."""
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    out = torch.empty(m, dtype=torch.bfloat16, device="cuda")
    step = 1 << 28
    for lo in range(0, m, step):
        hi = min(m, lo + step)
        out[lo:hi] = torch.randn(hi - lo, generator=g, device="cuda").to(torch.bfloat16)
    return out


def test_copy_past_4_gib(torch):
    n = 4 * GiB + 4099
    src = torch.empty(n + 16, dtype=torch.uint8, device="cuda")
    src.random_(0, 256)
    dst = torch.full((n + 32,), 0xA5, dtype=torch.uint8, device="cuda")
    snac.snac_copy(dst[8:].data_ptr(), src[3:].data_ptr(), n)
    torch.cuda.synchronize()
    assert torch.equal(dst[8:8 + n], src[3:3 + n])
    assert bool((dst[:8] == 0xA5).all()) and bool((dst[8 + n:] == 0xA5).all())
    del src, dst
    torch.cuda.empty_cache()


def test_all_reduce_past_2_30_elements(torch):
    n = 2
    m = (1 << 30) + (1 << 28) + 5  # bf16 elements per rank: 2.5 GiB
    xs = [random_bf16(torch, m, seed=40 + r) for r in range(n)]
    outs = [torch.empty_like(xs[0]) for _ in range(n)]
    ctx = snac.snac_init(n, 0)
    try:
        snac.snac_all_reduce(ctx, xs, outs, m * 2, "bf16")
        torch.cuda.synchronize()
        snac.snac_check(ctx)
    finally:
        snac.snac_finalize(ctx)
    idx = sample_idx(m, 2, seed=41)
    ins = [gather(torch, x, idx).view(torch.int16).numpy().view(np.uint16) for x in xs]
    want = oracle.reduce_n(ins, "bf16")
    for r in range(n):
        got = gather(torch, outs[r], idx).view(torch.int16).numpy().view(np.uint16)
        assert_same(got, want, "bf16", f"AllReduce dst[{r}] past 2^30 elements")
    del xs, outs
    torch.cuda.empty_cache()


def test_all_to_all_with_2_gib_chunks(torch):
    n = 2
    per_rank = 4 * GiB + 32  # two chunks of 2 GiB + 16 bytes
    e = per_rank // 4
    xs = []
    for r in range(n):
        t = torch.empty(e, dtype=torch.int32, device="cuda")
        t.random_(-(1 << 31), 1 << 31)
        xs.append(t)
    outs = [torch.empty(e, dtype=torch.int32, device="cuda") for _ in range(n)]
    ctx = snac.snac_init(n, 0)
    try:
        snac.snac_all_to_all(ctx, xs, outs, per_rank, "u32")
        torch.cuda.synchronize()
        snac.snac_check(ctx)
    finally:
        snac.snac_finalize(ctx)
    mc = e // n
    for d in range(n):
        idx = sample_idx(e, 4, seed=50 + d)
        got = gather(torch, outs[d], idx).numpy().view(np.uint32)
        # out[d] chunk s (elements s*mc ..) is in[s] chunk d: the exchange's
        # definition applied to the sampled elements
        s_of = idx // mc
        i_of = idx % mc
        want = np.empty(len(idx), dtype=np.uint32)
        for s in range(n):
            sel = s_of == s
            src_idx = d * mc + i_of[sel]
            want[sel] = gather(torch, xs[s], src_idx).numpy().view(np.uint32)
        assert np.array_equal(got, want), f"AllToAll dst[{d}] with 2 GiB chunks"
    del xs, outs
    torch.cuda.empty_cache()


def test_pipeline_past_4_gib(torch):
    n = 2
    m = (1 << 31) + (1 << 29) + 7  # bf16 elements per rank: 5 GiB + 14 bytes
    xs = [random_bf16(torch, m, seed=60 + r) for r in range(n)]
    out = torch.empty_like(xs[0])
    ctx = snac.snac_init(n, 0)
    try:
        snac.snac_pipeline_scale_reduce(ctx, xs, out, m, "bf16")
        torch.cuda.synchronize()
        snac.snac_check(ctx)
    finally:
        snac.snac_finalize(ctx)
    idx = sample_idx(m, 2, seed=61)
    ins = [gather(torch, x, idx).view(torch.int16).numpy().view(np.uint16) for x in xs]
    want = oracle.pipeline_scale_reduce(ins, "bf16")
    got = gather(torch, out, idx).view(torch.int16).numpy().view(np.uint16)
    assert_same(got, want, "bf16", "pipeline past 4 GiB per rank")
    del xs, out
    torch.cuda.empty_cache()
