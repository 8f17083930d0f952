"""Pins: the CPU oracle checked against what the pages and the mathematics fix.

Each pin compares the oracle with something other than itself: a value the
pages print, a closed form, an invariant of the collectives, an independent
scalar implementation on tiny inputs, or a library routine for a special case.
``test_planted_mistakes_are_caught`` plants plausible mistakes in the oracle
(on the CPU) and checks that at least one pin fails for each.
"""
from __future__ import annotations

import json
import os
import struct
from fractions import Fraction

import numpy as np
import pytest

import oracle
import oracle.bf16 as obf
import oracle.collectives as oc
from copy_reduce_snac_amd import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- helpers
def f32_scalar(x: float) -> float:
    """Round a Python float (binary64) to binary32, ties to even (C cast)."""
    try:
        return struct.unpack("<f", struct.pack("<f", x))[0]
    except OverflowError:
        return float("inf") if x > 0 else float("-inf")


def f32_bits(x: float) -> int:
    return struct.unpack("<I", struct.pack("<f", x))[0]


def bf16_scalar_from_f32(x: float) -> int:
    """Round a binary32 value to bfloat16 from the definition, with exact
    rationals: pick the nearer of the two neighbouring bfloat16 values, the
    even one on a tie.  Returns the 16-bit pattern.  NaN is not handled."""
    bits = f32_bits(x)
    sign = bits >> 31
    if x == 0.0:
        return sign << 15
    if x in (float("inf"), float("-inf")):
        return (sign << 15) | 0x7F80
    v = abs(Fraction(x))
    e = v.numerator.bit_length() - v.denominator.bit_length()
    if Fraction(2) ** e > v:
        e -= 1
    e = max(e, -126)  # subnormal range shares the minimum exponent
    ulp = Fraction(2) ** (e - 7)
    q = v / ulp
    n = q.numerator // q.denominator
    rem = q - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    r = n * ulp
    if r >= Fraction(2) ** 128:
        return (sign << 15) | 0x7F80
    rb = f32_bits(float(r))  # r is a bfloat16 value, exact in binary32
    assert rb & 0xFFFF == 0
    return (sign << 15) | (rb >> 16)


def bf16_value(b: int) -> float:
    return struct.unpack("<f", struct.pack("<I", (b & 0xFFFF) << 16))[0]


def scalar_reduce(vals: list[float], dtype: str):
    """Sequential binary32 sum in rank order, independent of NumPy: each step
    is a binary64 add of two binary32 values rounded once to binary32 (the
    binary64 sum rounds correctly to binary32 since 53 >= 2*24 + 2)."""
    acc = vals[0]
    for v in vals[1:]:
        acc = f32_scalar(acc + v)
    if dtype == "bf16":
        return bf16_scalar_from_f32(acc)
    return f32_bits(acc)


def as_bits(a: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32).view(np.uint32)
    return np.asarray(a)


def rand_inputs(n: int, m: int, dtype: str, seed: int) -> list[np.ndarray]:
    if dtype == "f32":
        return [wl.uniform_f32(m, wl.CFG_TEST, r, seed=seed) for r in range(n)]
    if dtype == "bf16":
        return [wl.normal_bf16(m, wl.CFG_TEST, r, seed=seed) for r in range(n)]
    return [wl.raw_bytes(m, wl.CFG_TEST, r, seed=seed) for r in range(n)]


# ---------------------------------------------------------------- pins
def pin_worked_example():
    with open(os.path.join(GOLDEN, "nki_allreduce_worked_example.json")) as f:
        g = json.load(f)
    srcs = [np.asarray(x, dtype=np.float32).reshape(-1) for x in g["inputs"]]
    outs = oc.all_reduce(srcs, "f32")
    for o, e in zip(outs, g["expected"]):
        assert np.array_equal(o.reshape(g["shape"]), np.asarray(e, dtype=np.float32))


def pin_closed_form_small_integers():
    # in_k[i] = (k+1)*(i mod 7): the sum is N(N+1)/2 * (i mod 7), exact in
    # binary32 and (for N <= 16, values <= 816) exact in bfloat16 only when
    # representable; use N <= 8 for bf16 (max 216 = 0b11011000, 5 bits).
    for dtype in ("f32", "bf16"):
        for n in (1, 2, 3, 5, 8) + ((16,) if dtype == "f32" else ()):
            i = np.arange(300)
            base = (i % 7).astype(np.float32)
            srcs = []
            for k in range(n):
                v = base * np.float32(k + 1)
                srcs.append(v if dtype == "f32" else (v.view(np.uint32) >> 16).astype(np.uint16))
            expect = base * np.float32(n * (n + 1) // 2)
            got = oc.reduce_n(srcs, dtype)
            if dtype == "bf16":
                got = obf.bf16_to_f32(got)
            assert np.array_equal(got, expect), (dtype, n)
    # constant inputs c_k sum to sum(c_k)
    cs = [0.5, -2.0, 3.25, 8.0]
    srcs = [np.full(10, c, dtype=np.float32) for c in cs]
    assert np.all(oc.reduce_n(srcs, "f32") == np.float32(sum(cs)))


def pin_rank_order():
    # 2^24 + 1 rounds back to 2^24 (tie to even), so the fixed order
    # ((a + b) + c) gives 0 while any order that adds b last gives 1.
    a, b, c = np.float32(2.0 ** 24), np.float32(1.0), np.float32(-(2.0 ** 24))
    srcs = [np.array([a]), np.array([b]), np.array([c])]
    assert oc.reduce_n(srcs, "f32")[0] == 0.0
    assert oc.reduce_n([srcs[0], srcs[2], srcs[1]], "f32")[0] == 1.0
    # a one-sided version in bf16 units: 256 + 1 + 1 is 256 in bf16 steps
    # only if rounding happens per step; one final rounding keeps 258.
    one = np.array([0x3F80], dtype=np.uint16)       # 1.0
    big = np.array([0x4380], dtype=np.uint16)       # 256.0
    got = oc.reduce_n([big, one, one], "bf16")
    assert bf16_value(int(got[0])) == 258.0


def pin_negative_zero_start():
    nz = np.array([0x8000], dtype=np.uint16)
    assert int(oc.reduce_n([nz, nz, nz], "bf16")[0]) == 0x8000
    f = np.array([-0.0], dtype=np.float32)
    assert f32_bits(float(oc.reduce_n([f, f], "f32")[0])) == 0x80000000
    pz = np.array([0.0], dtype=np.float32)
    assert f32_bits(float(oc.reduce_n([f, pz], "f32")[0])) == 0


def pin_bf16_hand_cases():
    cases = {
        0x3F808000: 0x3F80,  # tie, even below
        0x3F818000: 0x3F82,  # tie, odd below -> up
        0x3F808001: 0x3F81,  # just above the tie
        0x3F807FFF: 0x3F80,  # just below the tie
        0x7F7FFFFF: 0x7F80,  # largest finite rounds to +inf
        0xFF7FFFFF: 0xFF80,  # and to -inf
        0x7F7F7FFF: 0x7F7F,  # stays finite
        0x00008000: 0x0000,  # smallest subnormal tie -> even (zero)
        0x00018000: 0x0002,  # subnormal tie, odd -> up
        0x007FFFFF: 0x0080,  # largest subnormal rounds to smallest normal
        0x80000000: 0x8000,  # -0
        0x7F800000: 0x7F80,  # +inf
    }
    u = np.array(list(cases.keys()), dtype=np.uint32)
    got = obf.f32_to_bf16(u.view(np.float32))
    assert [int(x) for x in got] == list(cases.values())
    # NaN stays NaN (quiet), keeping its sign
    nans = np.array([0x7F800001, 0xFFC00000, 0x7FFFFFFF, 0xFF800001], dtype=np.uint32)
    out = obf.f32_to_bf16(nans.view(np.float32)).astype(np.uint32)
    assert np.all((out & 0x7F80) == 0x7F80) and np.all((out & 0x7F) != 0)
    assert list(out >> 15) == [0, 1, 0, 1]
    # widening is exact: every non-NaN bf16 pattern round-trips
    allb = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    keep = (allb.astype(np.uint32) & 0x7FFF) <= 0x7F80
    assert np.array_equal(obf.f32_to_bf16(obf.bf16_to_f32(allb[keep])), allb[keep])


def pin_bf16_scalar_definition():
    # the vectorised narrowing against the exact-rational definition on a
    # spread of patterns (all exponents, boundary fraction bits)
    g = np.random.default_rng(7)
    pats = list(g.integers(0, 1 << 32, size=3000, dtype=np.uint64))
    for e in range(0, 255):
        for low in (0x0000, 0x7FFF, 0x8000, 0x8001, 0xFFFF):
            for lsb in (0, 1):
                pats.append((e << 23) | (lsb << 16) | low | (0x55 << 17))
    pats = np.array(pats, dtype=np.uint64).astype(np.uint32)
    f = pats.view(np.float32)
    fin = np.isfinite(f)
    got = obf.f32_to_bf16(f[fin])
    ref = [bf16_scalar_from_f32(float(x)) for x in f[fin]]
    assert [int(x) for x in got] == ref


def pin_bruteforce_tiny():
    # vectorised oracle == scalar definitions written straight from the
    # element-index formulas, N in {1,2,3,4,8}, tiny sizes, counts with zeros
    for n in (1, 2, 3, 4, 8):
        for dtype in ("f32", "bf16"):
            for m in (0, 1, n, 3 * n, 5 * n + (0 if n > 1 else 1)):
                srcs = rand_inputs(n, m, dtype, seed=11 + n + m)
                vals = [[float(v) for v in (s if dtype == "f32" else obf.bf16_to_f32(s))] for s in srcs]
                # reduce / all_reduce
                ar = oc.all_reduce(srcs, dtype)
                for i in range(m):
                    want = scalar_reduce([vals[k][i] for k in range(n)], dtype)
                    for r in range(n):
                        assert int(as_bits(ar[r], dtype)[i]) == want, (n, m, dtype, i)
                # reduce_scatter
                if m % n == 0:
                    rs = oc.reduce_scatter(srcs, dtype)
                    mc = m // n
                    for r in range(n):
                        assert len(rs[r]) == mc
                        for i in range(mc):
                            want = scalar_reduce([vals[k][r * mc + i] for k in range(n)], dtype)
                            assert int(as_bits(rs[r], dtype)[i]) == want
        # copy-only collectives on bytes
        for m in (0, 1, 2 * n, 4 * n + (1 if n > 1 else 0)):
            srcs = rand_inputs(n, m, "byte", seed=5 + n + m)
            ag = oc.all_gather(srcs)
            for r in range(n):
                assert len(ag[r]) == n * m
                for k in range(n):
                    for i in range(m):
                        assert ag[r][k * m + i] == srcs[k][i]
            if m % n == 0:
                a2a = oc.all_to_all(srcs)
                mc = m // n
                for d in range(n):
                    for s in range(n):
                        for i in range(mc):
                            assert a2a[d][s * mc + i] == srcs[s][d * mc + i]
        # V variants with zero counts
        g = np.random.default_rng(100 + n)
        for trial in range(4):
            c = g.integers(0, 5, size=n)
            if trial == 0:
                c[0] = 0
            tot = int(c.sum())
            srcs = rand_inputs(n, max(tot, 1) + 2, "f32", seed=31 + trial)
            agv = oc.all_gather_v(srcs, list(c))
            for r in range(n):
                pos = 0
                for k in range(n):
                    for i in range(int(c[k])):
                        assert agv[r][pos] == srcs[k][i]
                        pos += 1
                assert pos == len(agv[r])
            rsv = oc.reduce_scatter_v(srcs, list(c), "f32")
            vals = [[float(v) for v in s] for s in srcs]
            pos = 0
            for r in range(n):
                assert len(rsv[r]) == c[r]
                for i in range(int(c[r])):
                    assert int(as_bits(rsv[r], "f32")[i]) == scalar_reduce([vals[k][pos + i] for k in range(n)], "f32")
                pos += int(c[r])
            cm = g.integers(0, 4, size=(n, n))
            cm[0, n - 1] = 0
            srcs = [rand_inputs(1, int(cm[s].sum()) + 1, "byte", seed=60 + s + trial)[0] for s in range(n)]
            a2av = oc.all_to_all_v(srcs, cm)
            for d in range(n):
                pos = 0
                for s in range(n):
                    off = 0
                    for j in range(d):
                        off += int(cm[s, j])
                    for i in range(int(cm[s, d])):
                        assert a2av[d][pos] == srcs[s][off + i]
                        pos += 1
                assert pos == len(a2av[d])


def pin_invariants():
    n = 8
    m = n * 96
    for dtype in ("f32", "bf16"):
        srcs = rand_inputs(n, m, dtype, seed=3)
        ar = oc.all_reduce(srcs, dtype)
        rs = oc.reduce_scatter(srcs, dtype)
        agrs = oc.all_gather(rs)
        for r in range(n):
            assert np.array_equal(as_bits(agrs[r], dtype), as_bits(ar[r], dtype))
            assert np.array_equal(as_bits(rs[r], dtype), as_bits(ar[0], dtype)[r * (m // n):(r + 1) * (m // n)])
    # N = 1: every collective is a copy
    x = rand_inputs(1, 50, "f32", seed=4)
    for out in (oc.all_reduce(x, "f32"), oc.reduce_scatter(x, "f32"), oc.all_gather(x), oc.all_to_all(x)):
        assert np.array_equal(out[0], x[0])
    # AllGather with one nonzero rank replicates that rank's data
    z = [np.zeros(64, dtype=np.float32) for _ in range(n)]
    z[5] = rand_inputs(1, 64, "f32", seed=9)[0]
    ag = oc.all_gather(z)
    assert np.array_equal(ag[2][5 * 64:6 * 64], z[5]) and not ag[2][:5 * 64].any()
    # AllToAll twice is the identity for equal chunks; output is a permutation
    srcs = rand_inputs(n, n * 40, "byte", seed=8)
    once = oc.all_to_all(srcs)
    twice = oc.all_to_all(once)
    for r in range(n):
        assert np.array_equal(twice[r], srcs[r])
    assert np.array_equal(np.sort(np.concatenate(once)), np.sort(np.concatenate(srcs)))
    # V variants at equal counts equal the fixed-size collectives
    mc = 40
    srcs = rand_inputs(n, n * mc, "f32", seed=12)
    assert all(np.array_equal(a, b) for a, b in zip(oc.all_to_all_v(srcs, np.full((n, n), mc)), oc.all_to_all(srcs)))
    assert all(np.array_equal(as_bits(a, "f32"), as_bits(b, "f32"))
               for a, b in zip(oc.reduce_scatter_v(srcs, [mc] * n, "f32"), oc.reduce_scatter(srcs, "f32")))
    short = [s[:mc] for s in srcs]
    assert all(np.array_equal(a, b) for a, b in zip(oc.all_gather_v(short, [mc] * n), oc.all_gather(short)))
    # AllToAllV with C then with C transposed returns every rank's buffer
    cm = wl.v_counts(n, 1000, n, cfg=wl.CFG_TEST)
    srcs = [rand_inputs(1, 1000, "byte", seed=20 + s)[0] for s in range(n)]
    fwd = oc.all_to_all_v(srcs, cm)
    back = oc.all_to_all_v(fwd, cm.T)
    for r in range(n):
        assert np.array_equal(back[r], srcs[r])


def pin_pipeline_closed_form():
    n = 8
    for dtype in ("f32", "bf16"):
        zero = [np.zeros(100, dtype=np.float32 if dtype == "f32" else np.uint16) for _ in range(n)]
        out = oc.pipeline_scale_reduce(zero, dtype)
        val = out if dtype == "f32" else obf.bf16_to_f32(out)
        assert np.all(val == 28.0)
        # x == c: sum over r of (c/2 + r), exact for small c
        c = np.float32(3.0)
        xs = [np.full(10, c, dtype=np.float32) for _ in range(n)]
        if dtype == "bf16":
            xs = [np.full(10, 0x4040, dtype=np.uint16) for _ in range(n)]  # 3.0
        out = oc.pipeline_scale_reduce(xs, dtype)
        val = out if dtype == "f32" else obf.bf16_to_f32(out)
        assert np.all(val == np.float32(n * 1.5 + 28.0))
    # the staged value is rounded to bf16 before the reduce.  N = 3, x = 2^-7:
    # rank 0 stages 2^-8 exactly, rank 1 stages bf16(1 + 2^-8) = 1.0 (tie to
    # even), rank 2 stages bf16(2 + 2^-8) = 2.0; the sum 3 + 2^-8 rounds to
    # 3.0.  Without the staging rounding the sum would be 3 + 3*2^-8, which
    # rounds to 3 + 2^-6.
    xs = [np.array([0x3C00], dtype=np.uint16) for _ in range(3)]
    out = oc.pipeline_scale_reduce(xs, "bf16")
    assert bf16_value(int(out[0])) == 3.0


def pin_copy():
    """The copy Atom moves bytes, not values: every binary32 bit pattern
    survives, signalling NaNs, payloads, infinities and -0 included; the
    length and element type are kept; the result is a buffer of its own.
    Checked against Python ``bytes`` built from the integer values, a path
    that shares nothing with NumPy's array copy."""
    pats = [0x7F800001, 0xFF800001, 0x7FBFFFFF, 0x7FC00000, 0xFFC00001, 0xFFFFFFFF, 0x7F800000, 0xFF800000,
            0x80000000, 0x00000000, 0x00000001, 0x807FFFFF, 0x3F800000]
    words = np.array(pats, dtype=np.uint32)
    f = words.view(np.float32)
    out = oc.copy(f)
    assert out.dtype == np.float32 and out.shape == f.shape
    assert out.tobytes() == b"".join(struct.pack("<I", p) for p in pats)
    # bf16 NaN and infinity patterns as 16-bit words
    h = np.array([0x7F81, 0xFF81, 0x7FC1, 0x7F80, 0xFF80, 0x8000, 0x0001], dtype=np.uint16)
    assert oc.copy(h).tobytes() == b"".join(struct.pack("<H", int(p)) for p in h.tolist())
    # raw random bytes of ragged lengths, 0 included
    for n in (0, 1, 3, 15, 4099):
        b = wl.raw_bytes(n, wl.CFG_TEST, 7)
        o = oc.copy(b)
        assert o.dtype == b.dtype and len(o) == n
        assert o.tobytes() == bytes(int(v) for v in b.tolist())
    # a separate buffer: writing the copy leaves the source alone
    b = wl.raw_bytes(64, wl.CFG_TEST, 8)
    keep = bytes(int(v) for v in b.tolist())
    o = oc.copy(b)
    o[:] ^= 0xFF
    assert b.tobytes() == keep


PINS = [
    pin_copy,
    pin_worked_example,
    pin_closed_form_small_integers,
    pin_rank_order,
    pin_negative_zero_start,
    pin_bf16_hand_cases,
    pin_bf16_scalar_definition,
    pin_bruteforce_tiny,
    pin_invariants,
    pin_pipeline_closed_form,
]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin()


@pytest.mark.slow
def test_bf16_narrowing_exhaustive_vs_torch():
    """Every non-NaN binary32 pattern against torch's CPU bfloat16 cast (a
    library routine, used here only as an independent reference)."""
    torch = pytest.importorskip("torch")
    from concurrent.futures import ThreadPoolExecutor

    step = 1 << 22

    def chunk(lo):
        u = np.arange(lo, lo + step, dtype=np.uint64).astype(np.uint32)
        f = u.view(np.float32)
        ours = obf.f32_to_bf16(f)
        ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        nan = np.isnan(f)
        ok = bool(np.array_equal(ours[~nan], ref[~nan]))
        ok_nan = bool(np.all((ours[nan] & 0x7F80) == 0x7F80) and np.all((ours[nan] & 0x7F) != 0))
        return lo, ok, ok_nan

    # the chunks are independent and NumPy and torch release the GIL inside
    # their loops, so threads share the 2^32 patterns
    workers = max(1, min(8, len(os.sched_getaffinity(0))))
    with ThreadPoolExecutor(max_workers=workers) as pool:
        for lo, ok, ok_nan in pool.map(chunk, range(0, 1 << 32, step)):
            assert ok, hex(lo)
            assert ok_nan, hex(lo)


# ---------------------------------------------------------------- mutations
def _mut_drop_last(srcs, dtype):
    return _orig["reduce_n"](list(srcs)[:-1] if len(srcs) > 1 else srcs, dtype)


def _mut_reverse(srcs, dtype):
    return _orig["reduce_n"](list(srcs)[::-1], dtype)


def _mut_pairwise(srcs, dtype):
    ws = [oc._widen(s, dtype) for s in srcs]
    while len(ws) > 1:
        nxt = [np.add(ws[i], ws[i + 1], dtype=np.float32) for i in range(0, len(ws) - 1, 2)]
        if len(ws) % 2:
            nxt.append(ws[-1])
        ws = nxt
    return oc._narrow(ws[0], dtype)


def _mut_zero_start(srcs, dtype):
    acc = np.zeros(len(srcs[0]), dtype=np.float32)
    for s in srcs:
        acc = np.add(acc, oc._widen(s, dtype), dtype=np.float32)
    return oc._narrow(acc, dtype)


def _mut_truncate_bf16(f):
    return (np.ascontiguousarray(f, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _mut_half_up_bf16(f):
    return ((np.ascontiguousarray(f, dtype=np.float32).view(np.uint32) + 0x8000) >> 16).astype(np.uint16)


def _mut_a2a_transposed(srcs):
    n = len(srcs)
    mc = len(srcs[0]) // n
    return [np.concatenate([srcs[d][s * mc:(s + 1) * mc] for s in range(n)]) for d in range(n)]


def _mut_rs_shift(srcs, dtype):
    out = _orig["reduce_scatter"](srcs, dtype)
    return out[1:] + out[:1]


def _mut_ag_reverse(srcs):
    return _orig["all_gather"](list(srcs)[::-1])


def _mut_a2av_wrong_offset(srcs, counts):
    n = len(srcs)
    c = np.asarray(counts, dtype=np.int64).reshape(n, n)
    outs = []
    for d in range(n):
        parts = []
        for s in range(n):
            sd = int(c[:s, d].sum())  # receive displacement used as send offset
            parts.append(np.asarray(srcs[s])[sd:sd + int(c[s, d])])
        outs.append(np.concatenate(parts))
    return outs


def _mut_agv_offset(srcs, counts):
    out = _orig["all_gather_v"](srcs, list(counts))
    return [np.roll(o, 1) for o in out]


def _mut_pipeline_sign(xs, dtype):
    staged = []
    for r, x in enumerate(xs):
        xf = oc._widen(x, dtype)
        y = np.subtract(np.multiply(xf, np.float32(0.5), dtype=np.float32), np.float32(r), dtype=np.float32)
        staged.append(oc._narrow(y, dtype))
    return oc.reduce_n(staged, dtype)


def _mut_pipeline_unrounded(xs, dtype):
    staged = []
    for r, x in enumerate(xs):
        xf = oc._widen(x, dtype)
        staged.append(np.add(np.multiply(xf, np.float32(0.5), dtype=np.float32), np.float32(r), dtype=np.float32))
    acc = staged[0].copy()
    for s in staged[1:]:
        acc = np.add(acc, s, dtype=np.float32)
    return oc._narrow(acc, dtype)


def _mut_copy_through_f64(src):
    # a value copy: widening quiets signalling NaNs
    a = np.asarray(src)
    if a.dtype == np.float32:
        with np.errstate(invalid="ignore"):
            return a.astype(np.float64).astype(np.float32)
    return np.array(a, copy=True)


def _mut_copy_short(src):
    return np.array(src, copy=True)[:-1] if len(src) else np.array(src, copy=True)


def _mut_copy_alias(src):
    return src


_orig = {
    "reduce_n": oc.reduce_n,
    "reduce_scatter": oc.reduce_scatter,
    "all_gather": oc.all_gather,
    "all_gather_v": oc.all_gather_v,
}

MUTATIONS = {
    "copy through float64": (oc, "copy", _mut_copy_through_f64),
    "copy drops last element": (oc, "copy", _mut_copy_short),
    "copy aliases its source": (oc, "copy", _mut_copy_alias),
    "reduce drops last rank": (oc, "reduce_n", _mut_drop_last),
    "reduce in reverse order": (oc, "reduce_n", _mut_reverse),
    "reduce in pairwise order": (oc, "reduce_n", _mut_pairwise),
    "reduce starts from +0": (oc, "reduce_n", _mut_zero_start),
    "bf16 truncation": (oc, "f32_to_bf16", _mut_truncate_bf16),
    "bf16 round half up": (oc, "f32_to_bf16", _mut_half_up_bf16),
    "all_to_all transposed": (oc, "all_to_all", _mut_a2a_transposed),
    "reduce_scatter chunk shift": (oc, "reduce_scatter", _mut_rs_shift),
    "all_gather reversed ranks": (oc, "all_gather", _mut_ag_reverse),
    "all_to_all_v wrong send offset": (oc, "all_to_all_v", _mut_a2av_wrong_offset),
    "all_gather_v off by one": (oc, "all_gather_v", _mut_agv_offset),
    "pipeline subtracts rank": (oc, "pipeline_scale_reduce", _mut_pipeline_sign),
    "pipeline skips staging rounding": (oc, "pipeline_scale_reduce", _mut_pipeline_unrounded),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistakes_are_caught(name, monkeypatch):
    mod, attr, fn = MUTATIONS[name]
    monkeypatch.setattr(mod, attr, fn)
    if attr == "f32_to_bf16":
        monkeypatch.setattr(obf, attr, fn)
    failed = []
    for pin in PINS:
        try:
            pin()
        except (AssertionError, ValueError, IndexError):
            failed.append(pin.__name__)
    assert failed, f"no pin catches: {name}"
