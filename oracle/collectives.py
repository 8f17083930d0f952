"""Plain definitions of the collectives (test infrastructure only).

Notation: N ranks, rank buffers ``srcs[0..N-1]`` (1-D NumPy arrays), element
index i, ``D(c)`` the exclusive prefix sum of a count vector.

Data types (``dtype`` argument):

* ``"f32"``  float32 arrays;
* ``"bf16"`` uint16 arrays of bfloat16 bit patterns;
* ``"byte"`` uint8 (or any other) arrays, copy-only collectives.

Readings taken where the pages are silent or disagree (each one is listed
with its reason in the design notes of the repository):

1. Summation order is rank order 0..N-1 in binary32 with a single final
   rounding.  The Purlin pages promise only "repeatable" results in
   deterministic mode; a fixed order is the plainest way to get them.
2. The accumulator starts from the rank-0 value, not from +0.0 (differs only
   when every input is -0.0: the result is then -0.0).
3. AllReduce writes the full result to every rank (the NKI worked example
   shows both ranks holding it).
4. ReduceScatter and AllToAll split dim 0 into N equal contiguous chunks,
   chunk r going to rank r (NKI reduce_scatter and all_to_all entries);
   sizes not divisible by N are rejected here and go through the V variants.
5. The variable-length variants take counts in elements, pack the chunks
   back to back, and place chunk k at the exclusive prefix sum of the counts
   before it; AllToAllV counts are a row-major [src][dst] matrix.
6. The device-side producer step of the SNAC pipeline computes
   ``y = 0.5 * x + rank`` in binary32 and stores y in the run's data type
   before the N-to-1 reduce.
"""
from __future__ import annotations

from typing import Sequence

import numpy as np

from .bf16 import bf16_to_f32, f32_to_bf16

DTYPES = ("f32", "bf16", "byte")


def _widen(a: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32)
    if dtype == "bf16":
        return bf16_to_f32(a)
    raise ValueError(f"reduction needs f32 or bf16, got {dtype!r}")


def _narrow(acc: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return acc.astype(np.float32, copy=True)
    if dtype == "bf16":
        return f32_to_bf16(acc)
    raise ValueError(dtype)


def exclusive_prefix(counts: Sequence[int]) -> list[int]:
    """D(c)[k] = sum of c[j] for j < k."""
    out, run = [], 0
    for c in counts:
        out.append(run)
        run += int(c)
    return out


def copy(src: np.ndarray) -> np.ndarray:
    """Copy Atom: dst = src, byte for byte.

    Follows Purlin 0.6.5, "Samples" (an Atom copies a slice from src to dst).
    """
    return np.array(src, copy=True)


def reduce_n(srcs: Sequence[np.ndarray], dtype: str) -> np.ndarray:
    """N-to-1 reduce: out[i] = R(f32(in_0[i]) + f32(in_1[i]) + ... ), in order.

    Follows Purlin 0.6.4, "# Purlin" (the N-to-1 reduce primitive combines
    several input buffers into one output) with readings 1 and 2 above.  Each
    ``+`` is one binary32 addition with round-to-nearest-even (NumPy float32
    add; no fused multiply-add is involved).
    """
    if len(srcs) == 0:
        raise ValueError("reduce_n needs at least one input")
    n = len(srcs[0])
    for s in srcs:
        if len(s) != n:
            raise ValueError("reduce_n inputs differ in length")
    acc = _widen(srcs[0], dtype).copy()
    for k in range(1, len(srcs)):
        acc = np.add(acc, _widen(srcs[k], dtype), dtype=np.float32)
    return _narrow(acc, dtype)


def all_reduce(srcs: Sequence[np.ndarray], dtype: str) -> list[np.ndarray]:
    """AllReduce(sum): every rank receives reduce_n over all ranks' buffers.

    Follows NKI Collective Communication Kernels API, all_reduce_hbm_kernel
    ("sum tensors across all ranks") and its worked example (both ranks end
    with the sum); Purlin 0.6.5 "Host-side" (allReduce from src to dst).
    """
    out = reduce_n(srcs, dtype)
    return [out.copy() for _ in srcs]


def reduce_scatter(srcs: Sequence[np.ndarray], dtype: str) -> list[np.ndarray]:
    """ReduceScatter: rank r receives the reduction of chunk r of every rank.

    Follows NKI Collective Communication Kernels API, reduce_scatter_hbm_kernel
    (sum, then scatter along dim 0 split into num_ranks chunks) and Iris
    Device Context, reduce_scatter (a rank keeps its contiguous block).
    """
    n = len(srcs)
    m = len(srcs[0])
    if m % n:
        raise ValueError("reduce_scatter needs a length divisible by the rank count")
    mc = m // n
    return [reduce_n([s[r * mc:(r + 1) * mc] for s in srcs], dtype) for r in range(n)]


def all_gather(srcs: Sequence[np.ndarray]) -> list[np.ndarray]:
    """AllGather: every rank receives all ranks' buffers concatenated in rank order.

    Follows NKI Collective Communication Kernels API, all_gather_hbm_kernel
    (gather along dim 0); Purlin 0.6.5 "Understanding totalBytes" (the output
    is N times the per-rank input).
    """
    out = np.concatenate([np.asarray(s) for s in srcs])
    return [out.copy() for _ in srcs]


def all_to_all(srcs: Sequence[np.ndarray]) -> list[np.ndarray]:
    """AllToAll: rank d receives chunk d of every rank s, placed at chunk s.

    Follows NKI Collective Communication Kernels API, all_to_all_hbm_kernel
    (rank sends input[i, :] to rank i; dim-0 chunks).  Iris's column-wise
    description is the same exchange on a transposed view.
    """
    n = len(srcs)
    m = len(srcs[0])
    if m % n:
        raise ValueError("all_to_all needs a length divisible by the rank count")
    mc = m // n
    return [np.concatenate([srcs[s][d * mc:(d + 1) * mc] for s in range(n)]) for d in range(n)]


def all_gather_v(srcs: Sequence[np.ndarray], counts: Sequence[int]) -> list[np.ndarray]:
    """AllGatherV: rank k contributes counts[k] elements, packed at D(counts)[k].

    Purlin 0.6.4 "# Purlin" names the variable-length variants; the packed
    layout is reading 5.
    """
    n = len(srcs)
    if len(counts) != n:
        raise ValueError("one count per rank")
    parts = []
    for k in range(n):
        if len(srcs[k]) < counts[k]:
            raise ValueError("source shorter than its count")
        parts.append(np.asarray(srcs[k])[: int(counts[k])])
    out = np.concatenate(parts) if parts else np.empty(0)
    return [out.copy() for _ in range(n)]


def reduce_scatter_v(srcs: Sequence[np.ndarray], counts: Sequence[int], dtype: str) -> list[np.ndarray]:
    """ReduceScatterV: rank r receives the reduction of elements
    [D(counts)[r], D(counts)[r] + counts[r]) of every rank.  Reading 5."""
    n = len(srcs)
    if len(counts) != n:
        raise ValueError("one count per rank")
    disp = exclusive_prefix(counts)
    total = disp[-1] + int(counts[-1])
    for s in srcs:
        if len(s) < total:
            raise ValueError("source shorter than the sum of counts")
    return [reduce_n([s[disp[r]:disp[r] + int(counts[r])] for s in srcs], dtype) for r in range(n)]


def all_to_all_v(srcs: Sequence[np.ndarray], counts: np.ndarray) -> list[np.ndarray]:
    """AllToAllV with a row-major count matrix C[s][d] (elements).

    Rank s sends elements [SD[s][d], SD[s][d] + C[s][d]) of its buffer to rank
    d, where SD[s][d] = sum_{j<d} C[s][j]; rank d stores them at RD[d][s] =
    sum_{j<s} C[j][d].  Rank d's output holds sum_s C[s][d] elements.
    Reading 5.
    """
    n = len(srcs)
    c = np.asarray(counts, dtype=np.int64).reshape(n, n)
    outs = []
    for d in range(n):
        parts = []
        for s in range(n):
            sd = int(c[s, :d].sum())
            parts.append(np.asarray(srcs[s])[sd:sd + int(c[s, d])])
        outs.append(np.concatenate(parts))
    return outs


def pipeline_scale_reduce(xs: Sequence[np.ndarray], dtype: str) -> np.ndarray:
    """Device-side SNAC pipeline: producers stage y_r = 0.5 * x_r + r, the
    consumers N-to-1 reduce the staged tiles into one output (reading 6).

    The producer/consumer structure follows Purlin 0.6.5 "Samples" (a
    collective called from inside a kernel between other work) and Purlin
    0.6.4 "Key Idea" (Stage, Notify, And Consume).  0.5 * x is exact in
    binary32 (or rounds the same way a fused multiply-add would, for
    subnormal x), then one binary32 addition of the rank index; y is rounded
    to the run's data type (identity for f32) when it is staged.
    """
    staged = []
    for r, x in enumerate(xs):
        xf = _widen(x, dtype)
        y = np.add(np.multiply(xf, np.float32(0.5), dtype=np.float32), np.float32(r), dtype=np.float32)
        staged.append(_narrow(y, dtype))
    return reduce_n(staged, dtype)
