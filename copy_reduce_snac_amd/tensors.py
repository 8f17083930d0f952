"""Tensor-level collectives over the C ABI, shaped like the PyTorch call of
Purlin 0.6.5 ("Host-side", the torch example: a contiguous CUDA tensor ``x``,
an output tensor the caller creates, ``all_reduce(x, out, handle, stream)``
between initialize and finalize).  The handle is the context from
``snac_init``.

All N logical ranks live in one GPU's HBM, so ``x`` and ``out`` are
sequences of N tensors, one per rank.  This module only checks shapes,
dtypes and devices and hands pointers and sizes to the library; every byte
is moved by its kernels.  ``stream`` defaults to torch's current stream.

Reductions take bfloat16 or float32 tensors.  Copy collectives take tensors
of any dtype and move their bytes.
"""
from __future__ import annotations

from typing import Sequence

from . import (snac_all_gather, snac_all_gather_v, snac_all_reduce_ex, snac_all_to_all, snac_all_to_all_v,
               snac_ctx_nranks, snac_reduce_scatter, snac_reduce_scatter_v)


def _torch():
    import torch

    return torch


def _reduce_dtype(t) -> str:
    torch = _torch()
    names = {torch.bfloat16: "bf16", torch.float32: "f32"}
    if t.dtype not in names:
        raise TypeError(f"reductions take bfloat16 or float32 tensors, not {t.dtype}")
    return names[t.dtype]


def _stream(stream):
    return stream if stream is not None else _torch().cuda.current_stream()


def _check(handle, xs: Sequence, outs: Sequence, what: str, same_numel: bool = True):
    n = snac_ctx_nranks(handle)
    if n <= 0:
        raise ValueError(f"{what}: invalid handle")
    xs, outs = list(xs), list(outs)
    if len(xs) != n or len(outs) != n:
        raise ValueError(f"{what}: need {n} inputs and {n} outputs, got {len(xs)} and {len(outs)}")
    dev = xs[0].device
    for t in xs + outs:
        if not t.is_cuda or t.device != dev:
            raise ValueError(f"{what}: every tensor must be on {dev}")
        if not t.is_contiguous():
            raise ValueError(f"{what}: tensors must be contiguous")
        if t.dtype != xs[0].dtype:
            raise TypeError(f"{what}: every tensor must have dtype {xs[0].dtype}")
    if same_numel and any(x.numel() != xs[0].numel() for x in xs):
        raise ValueError(f"{what}: every input must have the same number of elements")
    return n, xs, outs


def all_reduce(x: Sequence, out: Sequence, handle: int, stream=None, mode: str = "deterministic") -> None:
    """out[r] = sum over ranks k of x[k], for every rank r.  ``mode`` is
    "deterministic" (fixed rank order, binary32 accumulation, one rounding)
    or "atomic" (float atomics; order and last bits may vary)."""
    n, xs, outs = _check(handle, x, out, "all_reduce")
    dt = _reduce_dtype(xs[0])
    if any(o.numel() != xs[0].numel() for o in outs):
        raise ValueError("all_reduce: every output must have the inputs' number of elements")
    nbytes = xs[0].numel() * xs[0].element_size()
    snac_all_reduce_ex(handle, xs, outs, nbytes, dt, mode, _stream(stream))


def reduce_scatter(x: Sequence, out: Sequence, handle: int, stream=None) -> None:
    """out[r] = sum over ranks k of chunk r of x[k] (dim-0 chunks of equal size)."""
    n, xs, outs = _check(handle, x, out, "reduce_scatter")
    dt = _reduce_dtype(xs[0])
    m = xs[0].numel()
    if m % n or any(o.numel() != m // n for o in outs):
        raise ValueError(f"reduce_scatter: inputs of {m} elements need outputs of {m} / {n} elements")
    snac_reduce_scatter(handle, xs, outs, m * xs[0].element_size(), dt, _stream(stream))


def all_gather(x: Sequence, out: Sequence, handle: int, stream=None) -> None:
    """out[r] = x[0], x[1], ..., x[N-1] concatenated, for every rank r."""
    n, xs, outs = _check(handle, x, out, "all_gather")
    m = xs[0].numel()
    if any(o.numel() != n * m for o in outs):
        raise ValueError(f"all_gather: outputs need {n} * {m} elements")
    snac_all_gather(handle, xs, outs, m * xs[0].element_size(), "byte", _stream(stream))


def all_to_all(x: Sequence, out: Sequence, handle: int, stream=None) -> None:
    """Chunk d of x[s] goes to chunk s of out[d] (dim-0 chunks of equal size)."""
    n, xs, outs = _check(handle, x, out, "all_to_all")
    m = xs[0].numel()
    if m % n or any(o.numel() != m for o in outs):
        raise ValueError(f"all_to_all: inputs and outputs need the same element count, a multiple of {n}")
    e = xs[0].element_size()
    snac_all_to_all(handle, xs, outs, m * e, "u32" if e == 4 else "byte", _stream(stream))


def all_gather_v(x: Sequence, out: Sequence, handle: int, stream=None) -> None:
    """out[r] = x[0], ..., x[N-1] concatenated; the inputs may differ in length."""
    n, xs, outs = _check(handle, x, out, "all_gather_v", same_numel=False)
    counts = [t.numel() * t.element_size() for t in xs]
    if any(o.numel() * o.element_size() != sum(counts) for o in outs):
        raise ValueError("all_gather_v: every output needs the sum of the inputs' elements")
    snac_all_gather_v(handle, xs, outs, counts, "byte", _stream(stream))


def reduce_scatter_v(x: Sequence, out: Sequence, handle: int, stream=None) -> None:
    """out[r] = sum over ranks k of the r-th piece of x[k], the pieces sized
    by the outputs in rank order."""
    n, xs, outs = _check(handle, x, out, "reduce_scatter_v", same_numel=False)
    dt = _reduce_dtype(xs[0])
    counts = [o.numel() for o in outs]
    if any(t.numel() != sum(counts) for t in xs):
        raise ValueError("reduce_scatter_v: every input needs the sum of the outputs' elements")
    snac_reduce_scatter_v(handle, xs, outs, counts, dt, _stream(stream))


def all_to_all_v(x: Sequence, out: Sequence, counts, handle: int, stream=None) -> None:
    """counts[s][d] elements go from rank s to rank d, packed in rank order on
    both sides (send and receive offsets are prefix sums)."""
    n, xs, outs = _check(handle, x, out, "all_to_all_v", same_numel=False)
    c = [[int(v) for v in row] for row in counts]
    if len(c) != n or any(len(row) != n for row in c):
        raise ValueError(f"all_to_all_v: counts must be {n} x {n}")
    for s in range(n):
        if xs[s].numel() < sum(c[s]):
            raise ValueError(f"all_to_all_v: input {s} holds fewer than its {sum(c[s])} elements to send")
    for d in range(n):
        if outs[d].numel() < sum(c[s][d] for s in range(n)):
            raise ValueError(f"all_to_all_v: output {d} is too small for what it receives")
    e = xs[0].element_size()
    flat = [v * e for row in c for v in row]
    snac_all_to_all_v(handle, xs, outs, flat, "byte", _stream(stream))
