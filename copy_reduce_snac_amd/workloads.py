"""Seeded synthetic inputs for the collectives.

This module only draws random numbers and lays them out; it performs none of
the collective arithmetic (no sums, no output rounding, no layout maps).  The
CPU oracle and the HIP path both take their inputs from here, so both sides
see the same bits.

Recipes (all streams are PCG64 seeded from ``SeedSequence([seed, cfg, rank,
chunk])`` so that a buffer's contents do not depend on how many threads drew
it or on which prefix of it is used):

* ``normal_bf16``  N(0,1) drawn in float32, then quantised to bfloat16 bit
  patterns by adding 0x8000 to the float32 bits and keeping the high half.
  This quantisation is only a way to produce bf16-valued inputs; it is not
  the output rounding of the reduction (which is round-to-nearest-even).
* ``normal_f32``   N(0,1) float32.
* ``uniform_f32``  U[-1, 1) float32 (drawn as U[0,1) float32, times 2, minus 1).
* ``raw_u32``      uniform 32-bit words: every bit pattern, including the NaN
  and infinity encodings when viewed as float32.
* ``v_counts``     per-(src, dst) element counts for the variable-length
  collectives: each row holds ``n`` counts summing to ``total``; about 10 % of
  entries are zero (at least one per matrix), the nonzero entries are a
  Dirichlet(0.5) split rounded to whole elements (largest remainder, ties to
  the lower index), and at least one count is not a multiple of 4 elements
  (so some chunk ends 4 bytes short of a 16-byte boundary).
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

SEED = 0
CHUNK = 1 << 20  # elements per independently seeded chunk

# configuration ids used in the seed sequence
CFG_AR_F32_N2 = 1
CFG_AR_BF16_N8 = 2
CFG_RS_AG_BF16_N8 = 3
CFG_A2A_N8 = 4
CFG_PIPELINE_N8 = 5
CFG_TEST = 100  # small parity cases


def _rng(seed: int, cfg: int, rank: int, chunk: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, cfg, rank, chunk])))


def _draw(kind: str, n: int, cfg: int, rank: int, seed: int, threads: int | None) -> np.ndarray:
    """Draw ``n`` values of ``kind`` for (cfg, rank), chunk by chunk."""
    if kind in ("normal_f32", "uniform_f32"):
        out = np.empty(n, dtype=np.float32)
    else:
        out = np.empty(n, dtype=np.uint32)
    nchunks = (n + CHUNK - 1) // CHUNK

    def fill(c: int) -> None:
        lo = c * CHUNK
        hi = min(n, lo + CHUNK)
        g = _rng(seed, cfg, rank, c)
        m = hi - lo
        if kind == "normal_f32":
            out[lo:hi] = g.standard_normal(CHUNK, dtype=np.float32)[:m]
        elif kind == "uniform_f32":
            u = g.random(CHUNK, dtype=np.float32)[:m]
            out[lo:hi] = u * np.float32(2.0) - np.float32(1.0)
        elif kind == "raw_u32":
            out[lo:hi] = g.integers(0, 1 << 32, size=CHUNK, dtype=np.uint32)[:m]
        else:
            raise ValueError(kind)

    if threads is None:
        threads = min(16, len(os.sched_getaffinity(0)))
    if nchunks <= 1 or threads <= 1:
        for c in range(nchunks):
            fill(c)
    else:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(fill, range(nchunks)))
    return out


def normal_bf16(n: int, cfg: int, rank: int, seed: int = SEED, threads: int | None = None) -> np.ndarray:
    """N(0,1) values quantised to bfloat16; returned as uint16 bit patterns."""
    f = _draw("normal_f32", n, cfg, rank, seed, threads)
    bits = f.view(np.uint32)
    return ((bits + np.uint32(0x8000)) >> np.uint32(16)).astype(np.uint16)


def normal_f32(n: int, cfg: int, rank: int, seed: int = SEED, threads: int | None = None) -> np.ndarray:
    return _draw("normal_f32", n, cfg, rank, seed, threads)


def uniform_f32(n: int, cfg: int, rank: int, seed: int = SEED, threads: int | None = None) -> np.ndarray:
    return _draw("uniform_f32", n, cfg, rank, seed, threads)


def raw_u32(n: int, cfg: int, rank: int, seed: int = SEED, threads: int | None = None) -> np.ndarray:
    return _draw("raw_u32", n, cfg, rank, seed, threads)


def raw_bytes(n: int, cfg: int, rank: int, seed: int = SEED) -> np.ndarray:
    """``n`` uniform random bytes (a prefix of the raw_u32 stream)."""
    w = raw_u32((n + 3) // 4, cfg, rank, seed)
    return w.view(np.uint8)[:n].copy()


def _split_row(g: np.random.Generator, n: int, total: int, zero_frac: float) -> np.ndarray:
    zero = g.random(n) < zero_frac
    if zero.all():
        zero[int(g.integers(0, n))] = False
    nz = np.flatnonzero(~zero)
    p = g.dirichlet([0.5] * len(nz))
    raw = p * total
    c = np.floor(raw).astype(np.int64)
    rem = total - int(c.sum())
    frac = raw - c
    # largest fractional parts get the remainder; ties go to the lower index
    order = sorted(range(len(nz)), key=lambda i: (-frac[i], i))
    for i in order[:rem]:
        c[i] += 1
    row = np.zeros(n, dtype=np.int64)
    row[nz] = c
    return row


def v_counts(n: int, total: int, rows: int, cfg: int, seed: int = SEED, zero_frac: float = 0.10) -> np.ndarray:
    """Count matrix of shape (rows, n); each row sums to ``total`` elements."""
    g = _rng(seed, cfg, 1000, 0)
    m = np.stack([_split_row(g, n, total, zero_frac) for _ in range(rows)])
    # at least one zero-length chunk somewhere (needs a row with >= 2 entries)
    if n >= 2 and not (m == 0).any():
        r = 0
        lo = int(np.argmin(m[r]))
        hi = int(np.argmax(m[r]))
        if lo == hi:
            hi = (lo + 1) % n
        m[r, hi] += m[r, lo]
        m[r, lo] = 0
    # at least one count that is not a multiple of 4 elements
    if total % 4 != 0 or n < 2:
        return m
    if not (m % 4 != 0).any():
        r = 0
        order = np.argsort(-m[r], kind="stable")
        a, b = int(order[0]), int(order[1])
        if m[r, a] > 0:
            m[r, a] -= 1
            m[r, b] += 1
    return m
