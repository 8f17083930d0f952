"""Stress of the SNAC protocol on the GPU: producers skewed by an injected
delay while staging slots are reused many times, and a thousand
back-to-back pipeline calls whose every output is checked.  The results
must equal the oracle bit for bit and no wait may time out."""
from __future__ import annotations

import numpy as np
import pytest

import copy_reduce_snac_amd as snac
import oracle
from copy_reduce_snac_amd import workloads as wl
from gpu_helpers import gpu_available

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

N = 8


def up(torch, a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.uint8).copy()).to("cuda")


@pytest.fixture()
def restore_tuning():
    saved = snac.snac_get_tuning()
    yield
    snac.snac_set_tuning(**saved)


@pytest.mark.parametrize("lookahead,wpc", [(0, 0), (1, 4), (3, 2), (0, 1)])
def test_skewed_producers_with_slot_reuse(restore_tuning, lookahead, wpc):
    import torch

    count = 1 << 20  # 2 MiB per rank bf16: 32 tiles of 64 KiB over a 4-slot ring
    xs = [wl.normal_bf16(count, wl.CFG_PIPELINE_N8, r, seed=lookahead * 7 + wpc) for r in range(N)]
    want = oracle.pipeline_scale_reduce(xs, "bf16")
    snac.snac_set_tuning(pipeline_tile_bytes=65536, pipeline_lookahead=lookahead, wgs_per_cu=wpc,
                         debug_producer_delay=20)
    ctx = snac.snac_init(N, 4 * 65536)
    try:
        src = [up(torch, x) for x in xs]
        out = torch.empty(count * 2, dtype=torch.uint8, device="cuda")
        for rep in range(3):
            out.fill_(0)
            snac.snac_pipeline_scale_reduce(ctx, src, out, count, "bf16")
            snac.snac_check(ctx)  # synchronises; raises on a timeout
            got = out.cpu().numpy().view(np.uint16)
            assert np.array_equal(got, want), f"lookahead={lookahead} wpc={wpc} rep {rep}"
    finally:
        snac.snac_finalize(ctx)


def test_thousand_back_to_back_calls(restore_tuning):
    import torch

    count = 32 << 10  # 64 KiB per rank bf16
    sets = []
    for k in range(2):
        xs = [wl.normal_bf16(count, wl.CFG_PIPELINE_N8, r, seed=100 + k) for r in range(N)]
        sets.append(([up(torch, x) for x in xs], oracle.pipeline_scale_reduce(xs, "bf16")))
    calls = 1000
    results = torch.empty((calls, count * 2), dtype=torch.uint8, device="cuda")
    ctx = snac.snac_init(N, 1 << 20)
    try:
        out = torch.empty(count * 2, dtype=torch.uint8, device="cuda")
        for i in range(calls):
            snac.snac_pipeline_scale_reduce(ctx, sets[i % 2][0], out, count, "bf16")
            results[i].copy_(out)
        snac.snac_check(ctx)
        res = results.cpu().numpy().view(np.uint16)
        for i in range(calls):
            assert np.array_equal(res[i], sets[i % 2][1]), f"call {i}"
    finally:
        snac.snac_finalize(ctx)
