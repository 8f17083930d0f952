"""The tensor-level calls (copy_reduce_snac_amd.tensors) against the oracle:
every collective through torch tensors of several dtypes, with argument
checks.  The calls only marshal; the kernels are the library's."""
from __future__ import annotations

import numpy as np
import pytest

import copy_reduce_snac_amd as snac
import oracle
from copy_reduce_snac_amd import tensors as T
from copy_reduce_snac_amd import workloads as wl
from gpu_helpers import assert_same, gpu_available

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

N = 4


@pytest.fixture(scope="module")
def torch():
    import torch

    torch.cuda.set_device(0)
    return torch


@pytest.fixture(scope="module")
def handle(torch):
    h = snac.snac_init(N, 0)
    yield h
    snac.snac_finalize(h)


def dev(torch, a: np.ndarray, dtype):
    t = torch.from_numpy(np.ascontiguousarray(a).view(np.uint8).copy()).cuda()
    return t.view(dtype)


def host(t, np_dtype):
    import torch

    return t.cpu().contiguous().view(-1).view(torch.uint8).numpy().view(np_dtype)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_all_reduce_and_reduce_scatter(torch, handle, dtype):
    m = N * 3001
    xs_h = [wl.normal_bf16(m, wl.CFG_TEST, r, seed=31) if dtype == "bf16" else wl.normal_f32(m, wl.CFG_TEST, r, seed=31)
            for r in range(N)]
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    npd = np.uint16 if dtype == "bf16" else np.float32
    xs = [dev(torch, h, tdt) for h in xs_h]
    outs = [torch.empty_like(x) for x in xs]
    T.all_reduce(xs, outs, handle)
    rs = [torch.empty(m // N, dtype=tdt, device="cuda") for _ in range(N)]
    T.reduce_scatter(xs, rs, handle)
    torch.cuda.synchronize()
    want = oracle.all_reduce(xs_h, dtype)
    for r in range(N):
        assert_same(host(outs[r], npd), want[r], dtype, f"all_reduce out[{r}]")
    want_rs = oracle.reduce_scatter(xs_h, dtype)
    for r in range(N):
        assert_same(host(rs[r], npd), want_rs[r], dtype, f"reduce_scatter out[{r}]")


@pytest.mark.parametrize("tdt_name", ["int32", "int16", "uint8", "float32"])
def test_copy_collectives_any_dtype(torch, handle, tdt_name):
    tdt = getattr(torch, tdt_name)
    e = torch.empty(0, dtype=tdt).element_size()
    m = N * 1237
    words = [wl.raw_u32((m * e + 3) // 4, wl.CFG_TEST, r, seed=32).view(np.uint8)[: m * e] for r in range(N)]
    xs = [dev(torch, w, tdt) for w in words]
    ag = [torch.empty(N * m, dtype=tdt, device="cuda") for _ in range(N)]
    T.all_gather(xs, ag, handle)
    a2a = [torch.empty(m, dtype=tdt, device="cuda") for _ in range(N)]
    T.all_to_all(xs, a2a, handle)
    torch.cuda.synchronize()
    chunks = [w.reshape(N, -1) for w in words]  # rank s's N chunks of m/N elements (as bytes)
    for r in range(N):
        assert np.array_equal(host(ag[r], np.uint8), np.concatenate(words)), f"all_gather out[{r}]"
        want = np.concatenate([chunks[s][r] for s in range(N)])
        assert np.array_equal(host(a2a[r], np.uint8), want), f"all_to_all out[{r}]"


def test_v_collectives(torch, handle):
    c = wl.v_counts(N, 4000, N, cfg=wl.CFG_TEST, seed=33)
    words = [wl.raw_u32(int(c[s].sum()), wl.CFG_TEST, s, seed=34) for s in range(N)]
    xs = [dev(torch, w, torch.int32) for w in words]
    outs = [torch.empty(int(c[:, d].sum()), dtype=torch.int32, device="cuda") for d in range(N)]
    T.all_to_all_v(xs, outs, c.tolist(), handle)
    row = [int(v) for v in c[0]]
    parts = [wl.raw_u32(row[r], wl.CFG_TEST, r, seed=35) for r in range(N)]
    pin = [dev(torch, p, torch.int32) if p.size else torch.empty(0, dtype=torch.int32, device="cuda") for p in parts]
    agv = [torch.empty(sum(row), dtype=torch.int32, device="cuda") for _ in range(N)]
    T.all_gather_v(pin, agv, handle)
    fl = [wl.normal_f32(sum(row), wl.CFG_TEST, r, seed=36) for r in range(N)]
    rsv = [torch.empty(row[r], dtype=torch.float32, device="cuda") for r in range(N)]
    T.reduce_scatter_v([dev(torch, f, torch.float32) for f in fl], rsv, handle)
    torch.cuda.synchronize()
    want = oracle.all_to_all_v(words, c)
    for d in range(N):
        assert np.array_equal(host(outs[d], np.uint32), want[d]), f"all_to_all_v out[{d}]"
    want_agv = oracle.all_gather_v(parts, row)
    for r in range(N):
        assert np.array_equal(host(agv[r], np.uint32), want_agv[r]), f"all_gather_v out[{r}]"
    want_rsv = oracle.reduce_scatter_v(fl, row, "f32")
    for r in range(N):
        if row[r]:
            assert_same(host(rsv[r], np.float32), want_rsv[r], "f32", f"reduce_scatter_v out[{r}]")


def test_argument_checks(torch, handle):
    x = [torch.zeros(64, dtype=torch.float32, device="cuda") for _ in range(N)]
    with pytest.raises(ValueError):
        T.all_reduce(x[:3], x[:3], handle)
    with pytest.raises(TypeError):
        T.all_reduce([t.to(torch.int32) for t in x], [t.to(torch.int32) for t in x], handle)
    with pytest.raises(ValueError):
        T.reduce_scatter(x, [torch.zeros(15, device="cuda") for _ in range(N)], handle)
    with pytest.raises(ValueError):
        T.all_gather(x, [torch.zeros(64, device="cuda") for _ in range(N)], handle)
    with pytest.raises(ValueError):
        T.all_reduce([torch.zeros(8, 8, device="cuda").t() for _ in range(N)], x, handle)
    with pytest.raises(ValueError):
        T.all_reduce([t.cpu() for t in x], x, handle)
