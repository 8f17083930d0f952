"""Python binding of libsnac.so, the C-ABI copy / N-to-1 reduce collective
library for MI355X (declared in include/snac.h).

Argument marshalling only: every function here has the name of the C entry
point it calls and does nothing but convert Python arguments (ints, torch
tensors, streams) into the C types and turn a non-OK status into SnacError.
All data movement and arithmetic happens in the library's HIP kernels.
There is no fallback: if libsnac.so is missing, every call raises.

Pointer arguments accept ints or any object with ``data_ptr()`` (a torch
tensor).  ``stream`` accepts an int (a hipStream_t), an object with a
``cuda_stream`` attribute (a torch stream), or None (the null stream).
``dtype`` accepts the SNAC_* constants or "byte", "u32", "f32", "bf16".
"""
from __future__ import annotations

import ctypes
import os
from typing import Iterable, Sequence

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libsnac.so")

SNAC_OK, SNAC_E_ARG, SNAC_E_UNSUPPORTED, SNAC_E_NOMEM, SNAC_E_HIP, SNAC_E_TIMEOUT, SNAC_E_STATE, SNAC_E_ABORTED = range(8)
SNAC_BYTE, SNAC_U32, SNAC_F32, SNAC_BF16 = range(4)
(SNAC_COLL_ALL_REDUCE, SNAC_COLL_REDUCE_SCATTER, SNAC_COLL_ALL_GATHER, SNAC_COLL_ALL_TO_ALL,
 SNAC_COLL_ALL_GATHER_V, SNAC_COLL_REDUCE_SCATTER_V, SNAC_COLL_ALL_TO_ALL_V) = range(7)
SNAC_MAX_RANKS = 16
SNAC_MAX_BYTES = 1 << 40  # largest buffer extent (bytes) or V count (elements) a call accepts

_DTYPES = {"byte": SNAC_BYTE, "u8": SNAC_BYTE, "u32": SNAC_U32, "f32": SNAC_F32, "bf16": SNAC_BF16}
ESIZE = {SNAC_BYTE: 1, SNAC_U32: 4, SNAC_F32: 4, SNAC_BF16: 2}


class SnacError(RuntimeError):
    def __init__(self, status: int, func: str, detail: str):
        self.status = status
        super().__init__(f"{func}: status {status} ({_status_name(status)}): {detail}")


class snac_job(ctypes.Structure):
    _fields_ = [
        ("src_off", ctypes.c_uint64),
        ("dst_off", ctypes.c_uint64),
        ("bytes", ctypes.c_uint64),
        ("src_rank", ctypes.c_int32),
        ("dst_rank", ctypes.c_int32),
    ]


class snac_tuning(ctypes.Structure):
    _fields_ = [
        ("wgs_per_cu", ctypes.c_int32),
        ("cache_policy", ctypes.c_int32),
        ("pipeline_tile_bytes", ctypes.c_int32),
        ("pipeline_lookahead", ctypes.c_int32),
        ("spin_limit_log2", ctypes.c_int32),
        ("debug_drop_notify", ctypes.c_int32),
        ("copy_multicast", ctypes.c_int32),
        ("debug_producer_delay", ctypes.c_int32),
        ("tile_schedule", ctypes.c_int32),
    ]


SNAC_RULE_ANY, SNAC_RULE_ANY_REDUCE, SNAC_RULE_ANY_COPY = -1, -2, -3
SNAC_RULE_ATOM_COPY, SNAC_RULE_ATOM_REDUCE, SNAC_RULE_PIPELINE = 100, 101, 200
SNAC_MAX_TUNING_RULES = 256
SNAC_MAX_COUNTS = SNAC_MAX_RANKS * SNAC_MAX_RANKS


class snac_tuning_rule(ctypes.Structure):
    _fields_ = [
        ("coll", ctypes.c_int32),
        ("min_ranks", ctypes.c_int32),
        ("max_ranks", ctypes.c_int32),
        ("esize", ctypes.c_int32),
        ("min_bytes", ctypes.c_uint64),
        ("max_bytes", ctypes.c_uint64),
        ("wgs_per_cu", ctypes.c_int32),
        ("cache_policy", ctypes.c_int32),
    ]
SNAC_DESC_ALIGNED = 1
SNAC_FLAG_STRIDE = 16


class snac_dev_ctx(ctypes.Structure):
    _fields_ = [
        ("nranks", ctypes.c_int32),
        ("spin_limit_log2", ctypes.c_uint32),
        ("status", ctypes.c_void_p),
        ("abort_word", ctypes.c_void_p),
        ("barrier", ctypes.c_void_p),
        ("flags", ctypes.c_void_p),
        ("nflags", ctypes.c_uint32),
        ("reserved", ctypes.c_uint32),
        ("staging", ctypes.c_void_p),
        ("staging_bytes", ctypes.c_uint64),
    ]


class snac_coll_desc(ctypes.Structure):
    _fields_ = [
        ("coll", ctypes.c_int32),
        ("nsrc", ctypes.c_int32),
        ("ndst", ctypes.c_int32),
        ("esize", ctypes.c_int32),
        ("split_multicast", ctypes.c_int32),
        ("flags", ctypes.c_int32),
        ("bytes", ctypes.c_uint64),
        ("src", ctypes.c_void_p * SNAC_MAX_RANKS),
        ("dst", ctypes.c_void_p * SNAC_MAX_RANKS),
        ("counts", ctypes.c_uint64 * SNAC_MAX_COUNTS),
    ]


_lib = None
_VP = ctypes.c_void_p
_SZ = ctypes.c_size_t
_I = ctypes.c_int

# name -> (restype, argtypes)
_SIGS = {
    "snac_abi_version": (_I, []),
    "snac_status_str": (ctypes.c_char_p, [_I]),
    "snac_last_error": (ctypes.c_char_p, []),
    "snac_init": (_I, [_I, _SZ, _VP, ctypes.POINTER(_VP)]),
    "snac_finalize": (_I, [_VP, _VP]),
    "snac_check": (_I, [_VP, _VP]),
    "snac_ctx_nranks": (_I, [_VP]),
    "snac_abort": (_I, [_VP]),
    "snac_copy": (_I, [_VP, _VP, _SZ, _VP]),
    "snac_hbm_probe": (_I, [_I, _VP, _VP, _SZ, _I, _I, _I, ctypes.c_uint32, _VP]),
    "snac_reduce_n": (_I, [ctypes.POINTER(_VP), _I, ctypes.POINTER(_VP), _I, _SZ, _I, _VP]),
    "snac_all_reduce": (_I, [_VP, ctypes.POINTER(_VP), ctypes.POINTER(_VP), _SZ, _I, _VP]),
    "snac_all_reduce_ex": (_I, [_VP, ctypes.POINTER(_VP), ctypes.POINTER(_VP), _SZ, _I, _I, _VP]),
    "snac_all_reduce_atomic_static": (_I, [_I, ctypes.POINTER(_VP), ctypes.POINTER(_VP), _SZ, _I, _VP]),
    "snac_reduce_scatter": (_I, [_VP, ctypes.POINTER(_VP), ctypes.POINTER(_VP), _SZ, _I, _VP]),
    "snac_all_gather": (_I, [_VP, ctypes.POINTER(_VP), ctypes.POINTER(_VP), _SZ, _I, _VP]),
    "snac_all_to_all": (_I, [_VP, ctypes.POINTER(_VP), ctypes.POINTER(_VP), _SZ, _I, _VP]),
    "snac_all_gather_v": (_I, [_VP, ctypes.POINTER(_VP), ctypes.POINTER(_VP), ctypes.POINTER(_SZ), _I, _VP]),
    "snac_reduce_scatter_v": (_I, [_VP, ctypes.POINTER(_VP), ctypes.POINTER(_VP), ctypes.POINTER(_SZ), _I, _VP]),
    "snac_all_to_all_v": (_I, [_VP, ctypes.POINTER(_VP), ctypes.POINTER(_VP), ctypes.POINTER(_SZ), _I, _VP]),
    "snac_pipeline_scale_reduce": (_I, [_VP, ctypes.POINTER(_VP), _VP, _SZ, _I, _VP]),
    "snac_plan": (_I, [_I, _I, _I, _SZ, ctypes.POINTER(_SZ), ctypes.POINTER(snac_job), _I, ctypes.POINTER(_I)]),
    "snac_get_device_context": (_I, [_VP, ctypes.POINTER(snac_dev_ctx)]),
    "snac_describe": (_I, [_VP, _I, ctypes.POINTER(_VP), ctypes.POINTER(_VP), _SZ, ctypes.POINTER(_SZ), _I,
                           ctypes.POINTER(snac_coll_desc)]),
    "snac_set_tuning_rules": (_I, [ctypes.POINTER(snac_tuning_rule), _I]),
    "snac_get_tuning_rules": (_I, [ctypes.POINTER(snac_tuning_rule), _I, ctypes.POINTER(_I)]),
    "snac_tuning_lookup": (_I, [ctypes.c_int32, _I, _I, _SZ, ctypes.POINTER(snac_tuning)]),
    "snac_get_tuning": (_I, [ctypes.POINTER(snac_tuning)]),
    "snac_set_tuning": (_I, [ctypes.POINTER(snac_tuning)]),
}


def lib() -> ctypes.CDLL:
    """Load libsnac.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m copy_reduce_snac_amd.build` "
                "(there is no CPU fallback)"
            )
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(l, name)
            f.restype = res
            f.argtypes = args
        _lib = l
    return _lib


def _status_name(s: int) -> str:
    try:
        return lib().snac_status_str(s).decode()
    except Exception:  # library not loadable while formatting an error
        return "?"


def _check(status: int, func: str) -> None:
    if status != SNAC_OK:
        raise SnacError(status, func, lib().snac_last_error().decode())


def _ptr(x) -> int:
    if x is None:
        return 0
    if isinstance(x, int):
        return x
    if hasattr(x, "data_ptr"):
        return int(x.data_ptr())
    raise TypeError(f"cannot take a device pointer from {type(x).__name__}")


def _stream(s) -> int:
    if s is None:
        return 0
    if isinstance(s, int):
        return s
    if hasattr(s, "cuda_stream"):
        return int(s.cuda_stream)
    raise TypeError(f"cannot take a stream from {type(s).__name__}")


def _dtype(t) -> int:
    if isinstance(t, str):
        return _DTYPES[t]
    return int(t)


def _ptrs(xs: Iterable) -> ctypes.Array:
    vals = [_ptr(x) for x in xs]
    return (_VP * max(1, len(vals)))(*vals)


def _sizes(xs: Iterable[int]) -> ctypes.Array:
    vals = [int(x) for x in xs]
    return (_SZ * max(1, len(vals)))(*vals)


# ------------------------------------------------------------------ info
def snac_abi_version() -> int:
    return lib().snac_abi_version()


def snac_status_str(status: int) -> str:
    return lib().snac_status_str(status).decode()


def snac_last_error() -> str:
    return lib().snac_last_error().decode()


# --------------------------------------------------------------- context
def snac_init(nranks: int, staging_bytes_per_rank: int = 0, stream=None) -> int:
    out = _VP()
    _check(lib().snac_init(nranks, staging_bytes_per_rank, _stream(stream), ctypes.byref(out)), "snac_init")
    return out.value


def snac_finalize(ctx: int, stream=None) -> None:
    _check(lib().snac_finalize(ctx, _stream(stream)), "snac_finalize")


def snac_check(ctx: int, stream=None) -> None:
    _check(lib().snac_check(ctx, _stream(stream)), "snac_check")


def snac_ctx_nranks(ctx: int) -> int:
    return lib().snac_ctx_nranks(ctx)


def snac_abort(ctx: int) -> None:
    _check(lib().snac_abort(ctx), "snac_abort")


# ----------------------------------------------------------------- Atoms
def snac_copy(dst, src, nbytes: int, stream=None) -> None:
    _check(lib().snac_copy(_ptr(dst), _ptr(src), nbytes, _stream(stream)), "snac_copy")


SNAC_PROBE_READ, SNAC_PROBE_WRITE, SNAC_PROBE_COPY = range(3)
SNAC_PROBE_ORDERED = 8
_PROBES = {"read": SNAC_PROBE_READ, "write": SNAC_PROBE_WRITE, "copy": SNAC_PROBE_COPY}
_PROBES.update({k + "_ordered": v | SNAC_PROBE_ORDERED for k, v in list(_PROBES.items())})


def snac_hbm_probe(kind, dst, src, nbytes: int, threads: int = 64, tile_bytes: int = 4096, wgs_per_cu: int = 4,
                   magic: int = 0x9E3779B9, stream=None) -> None:
    """HBM ceiling probe (measurement helper): kind "read", "write" or "copy", or the same with "_ordered"
    (tiles handed out in order from counters after 8 grid-stride rounds)."""
    k = _PROBES[kind] if isinstance(kind, str) else int(kind)
    _check(lib().snac_hbm_probe(k, _ptr(dst), _ptr(src) if src is not None else None, nbytes, threads, tile_bytes,
                                wgs_per_cu, magic & 0xFFFFFFFF, _stream(stream)), "snac_hbm_probe")


def snac_reduce_n(dsts: Sequence, srcs: Sequence, count: int, dtype, stream=None) -> None:
    _check(lib().snac_reduce_n(_ptrs(dsts), len(dsts), _ptrs(srcs), len(srcs), count, _dtype(dtype), _stream(stream)),
           "snac_reduce_n")


# ----------------------------------------------------------- collectives
def _ctx_ranks(ctx: int) -> int:
    return snac_ctx_nranks(ctx) if ctx else 0


def _rank_ptrs(ctx: int, xs: Sequence, what: str) -> ctypes.Array:
    """Pointer array of a per-rank argument.  The library reads exactly
    snac_ctx_nranks(ctx) entries, so a list of another length is refused here
    rather than read past its end."""
    xs = list(xs)
    n = _ctx_ranks(ctx)
    if n and len(xs) != n:
        raise ValueError(f"{what}: {len(xs)} buffers for a context of {n} ranks")
    return _ptrs(xs)


def _rank_sizes(ctx: int, counts: Iterable[int], per_pair: bool, what: str) -> ctypes.Array:
    """Count array of a V collective: N entries, or N * N for AllToAllV."""
    counts = [int(c) for c in counts]
    n = _ctx_ranks(ctx)
    want = n * n if per_pair else n
    if n and len(counts) != want:
        raise ValueError(f"{what}: {len(counts)} counts for a context of {n} ranks (need {want})")
    return _sizes(counts)


def _fixed(name: str, ctx: int, srcs: Sequence, dsts: Sequence, nbytes: int, dtype, stream) -> None:
    f = getattr(lib(), name)
    _check(f(ctx, _rank_ptrs(ctx, srcs, name + " srcs"), _rank_ptrs(ctx, dsts, name + " dsts"), nbytes, _dtype(dtype),
             _stream(stream)), name)


def _vary(name: str, ctx: int, srcs: Sequence, dsts: Sequence, counts: Iterable[int], dtype, stream) -> None:
    f = getattr(lib(), name)
    cnt = _rank_sizes(ctx, counts, name == "snac_all_to_all_v", name + " counts")
    _check(f(ctx, _rank_ptrs(ctx, srcs, name + " srcs"), _rank_ptrs(ctx, dsts, name + " dsts"), cnt, _dtype(dtype),
             _stream(stream)), name)


def snac_all_reduce(ctx, srcs, dsts, nbytes, dtype, stream=None):
    _fixed("snac_all_reduce", ctx, srcs, dsts, nbytes, dtype, stream)


SNAC_REDUCE_DETERMINISTIC, SNAC_REDUCE_ATOMIC = 0, 1
_MODES = {"deterministic": SNAC_REDUCE_DETERMINISTIC, "atomic": SNAC_REDUCE_ATOMIC}


def snac_all_reduce_ex(ctx, srcs, dsts, nbytes, dtype, mode, stream=None):
    m = _MODES[mode] if isinstance(mode, str) else int(mode)
    _check(lib().snac_all_reduce_ex(ctx, _rank_ptrs(ctx, srcs, "snac_all_reduce_ex srcs"),
                                    _rank_ptrs(ctx, dsts, "snac_all_reduce_ex dsts"), nbytes, _dtype(dtype), m,
                                    _stream(stream)),
           "snac_all_reduce_ex")


def snac_all_reduce_atomic_static(srcs, dsts, nbytes, dtype, stream=None):
    """The context-free, allocation-free atomic AllReduce over len(srcs) ranks."""
    srcs, dsts = list(srcs), list(dsts)
    if len(srcs) != len(dsts):
        raise ValueError(f"snac_all_reduce_atomic_static: {len(srcs)} sources but {len(dsts)} destinations")
    _check(lib().snac_all_reduce_atomic_static(len(srcs), _ptrs(srcs), _ptrs(dsts), nbytes, _dtype(dtype),
                                               _stream(stream)),
           "snac_all_reduce_atomic_static")


def snac_reduce_scatter(ctx, srcs, dsts, nbytes, dtype, stream=None):
    _fixed("snac_reduce_scatter", ctx, srcs, dsts, nbytes, dtype, stream)


def snac_all_gather(ctx, srcs, dsts, nbytes, dtype, stream=None):
    _fixed("snac_all_gather", ctx, srcs, dsts, nbytes, dtype, stream)


def snac_all_to_all(ctx, srcs, dsts, nbytes, dtype, stream=None):
    _fixed("snac_all_to_all", ctx, srcs, dsts, nbytes, dtype, stream)


def snac_all_gather_v(ctx, srcs, dsts, counts, dtype, stream=None):
    _vary("snac_all_gather_v", ctx, srcs, dsts, counts, dtype, stream)


def snac_reduce_scatter_v(ctx, srcs, dsts, counts, dtype, stream=None):
    _vary("snac_reduce_scatter_v", ctx, srcs, dsts, counts, dtype, stream)


def snac_all_to_all_v(ctx, srcs, dsts, counts, dtype, stream=None):
    _vary("snac_all_to_all_v", ctx, srcs, dsts, counts, dtype, stream)


def snac_pipeline_scale_reduce(ctx, xs, out, count, dtype, stream=None):
    _check(lib().snac_pipeline_scale_reduce(ctx, _rank_ptrs(ctx, xs, "snac_pipeline_scale_reduce xs"), _ptr(out), count,
                                            _dtype(dtype), _stream(stream)),
           "snac_pipeline_scale_reduce")


# -------------------------------------------------------- device-side API
def snac_get_device_context(ctx: int) -> snac_dev_ctx:
    """The device view of a context, for kernels using include/snac_device.hpp."""
    out = snac_dev_ctx()
    _check(lib().snac_get_device_context(ctx, ctypes.byref(out)), "snac_get_device_context")
    return out


def snac_describe(ctx: int, coll: int, srcs: Sequence, dsts: Sequence, nbytes: int = 0,
                  counts: Iterable[int] | None = None, dtype="byte") -> snac_coll_desc:
    """A validated, laid-out collective for snac::collective() in a user kernel."""
    out = snac_coll_desc()
    cnt = None
    if coll in (SNAC_COLL_ALL_GATHER_V, SNAC_COLL_REDUCE_SCATTER_V, SNAC_COLL_ALL_TO_ALL_V):
        cnt = _rank_sizes(ctx, counts if counts is not None else [], coll == SNAC_COLL_ALL_TO_ALL_V,
                          "snac_describe counts")
    elif counts is not None:
        cnt = _sizes(counts)
    _check(lib().snac_describe(ctx, coll, _rank_ptrs(ctx, srcs, "snac_describe srcs"),
                               _rank_ptrs(ctx, dsts, "snac_describe dsts"), nbytes, cnt, _dtype(dtype),
                               ctypes.byref(out)),
           "snac_describe")
    return out


# ---------------------------------------------------------- layout, tuning
def snac_plan(coll: int, nranks: int, dtype, nbytes: int = 0, counts: Iterable[int] | None = None,
              max_jobs: int = SNAC_MAX_RANKS * SNAC_MAX_RANKS) -> list[tuple[int, int, int, int, int]]:
    """Jobs of a collective as (src_off, dst_off, bytes, src_rank, dst_rank)."""
    jobs = (snac_job * max_jobs)()
    nj = _I()
    cnt = _sizes(counts) if counts is not None else None
    _check(lib().snac_plan(coll, nranks, _dtype(dtype), nbytes, cnt, jobs, max_jobs, ctypes.byref(nj)), "snac_plan")
    return [(j.src_off, j.dst_off, j.bytes, j.src_rank, j.dst_rank) for j in jobs[: nj.value]]


def snac_get_tuning() -> dict:
    t = snac_tuning()
    _check(lib().snac_get_tuning(ctypes.byref(t)), "snac_get_tuning")
    return {name: getattr(t, name) for name, _ in snac_tuning._fields_}


def snac_set_tuning(**kw) -> None:
    cur = snac_get_tuning()
    cur.update(kw)
    t = snac_tuning(**{k: int(v) for k, v in cur.items()})
    _check(lib().snac_set_tuning(ctypes.byref(t)), "snac_set_tuning")


_RULE_FIELDS = [n for n, _ in snac_tuning_rule._fields_]


def snac_set_tuning_rules(rules: Sequence[dict] | None) -> None:
    """Install a rule table (dicts with the snac_tuning_rule field names);
    None or [] restores the built-in table."""
    rules = list(rules or [])
    arr = (snac_tuning_rule * max(1, len(rules)))()
    for i, r in enumerate(rules):
        for k, v in r.items():
            if k not in _RULE_FIELDS:
                raise KeyError(f"unknown rule field {k}")
            setattr(arr[i], k, int(v))
    _check(lib().snac_set_tuning_rules(arr if rules else None, len(rules)), "snac_set_tuning_rules")


def snac_get_tuning_rules() -> list[dict]:
    # one call into room for the largest table: the table may be replaced
    # from another thread between a size query and a copy
    n = _I()
    arr = (snac_tuning_rule * SNAC_MAX_TUNING_RULES)()
    _check(lib().snac_get_tuning_rules(arr, SNAC_MAX_TUNING_RULES, ctypes.byref(n)), "snac_get_tuning_rules")
    return [{k: getattr(arr[i], k) for k in _RULE_FIELDS} for i in range(n.value)]


def snac_tuning_lookup(coll: int, nranks: int, esize: int, nbytes: int) -> dict:
    t = snac_tuning()
    _check(lib().snac_tuning_lookup(coll, nranks, esize, nbytes, ctypes.byref(t)), "snac_tuning_lookup")
    return {name: getattr(t, name) for name, _ in snac_tuning._fields_}
