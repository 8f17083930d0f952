"""The seeded input generators: reproducible, prefix-stable, and the count
matrix has the structure the variable-length workloads ask for."""
import numpy as np
import pytest

from copy_reduce_snac_amd import workloads as wl


def test_streams_are_reproducible_and_prefix_stable():
    a = wl.normal_bf16(3 * wl.CHUNK + 17, wl.CFG_TEST, 2)
    b = wl.normal_bf16(3 * wl.CHUNK + 17, wl.CFG_TEST, 2, threads=1)
    assert np.array_equal(a, b)
    c = wl.normal_bf16(wl.CHUNK + 5, wl.CFG_TEST, 2)
    assert np.array_equal(a[: wl.CHUNK + 5], c)
    assert not np.array_equal(a[:1000], wl.normal_bf16(1000, wl.CFG_TEST, 3))


def test_distributions():
    x = wl.normal_f32(1 << 20, wl.CFG_TEST, 0)
    assert abs(float(x.mean())) < 0.01 and abs(float(x.std()) - 1.0) < 0.01
    u = wl.uniform_f32(1 << 20, wl.CFG_TEST, 0)
    assert u.min() >= -1.0 and u.max() < 1.0
    b = wl.normal_bf16(1 << 16, wl.CFG_TEST, 0)
    f = (b.astype(np.uint32) << 16).view(np.float32)
    assert abs(float(f.std()) - 1.0) < 0.02
    w = wl.raw_u32(1 << 20, wl.CFG_TEST, 0)
    assert w.max() > 0xF0000000 and w.min() < 0x10000000


@pytest.mark.parametrize("rows", [1, 8])
def test_v_counts(rows):
    total = 33_554_432
    m = wl.v_counts(8, total, rows, cfg=wl.CFG_A2A_N8)
    assert m.shape == (rows, 8)
    assert np.all(m.sum(axis=1) == total)
    assert (m == 0).any()
    assert (m % 4 != 0).any()
    assert np.all(m >= 0)
    assert np.array_equal(m, wl.v_counts(8, total, rows, cfg=wl.CFG_A2A_N8))


def test_v_counts_zero_fraction():
    m = np.concatenate([wl.v_counts(8, 10_000, 8, cfg=c) for c in range(200)])
    frac = float((m == 0).mean())
    assert 0.06 < frac < 0.16
