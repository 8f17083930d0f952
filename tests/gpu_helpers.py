"""Device-buffer helpers for the GPU parity tests: canary-guarded buffers at
chosen byte offsets, upload and download of NumPy arrays.  Torch is used only
to hold device memory."""
from __future__ import annotations

import numpy as np

CANARY = 0xA5
GUARD = 256


def torch_mod():
    import torch

    return torch


def gpu_available() -> bool:
    try:
        torch = torch_mod()
    except Exception:
        return False
    return torch.cuda.is_available()


class DevBuf:
    """``nbytes`` device bytes at ``offset`` past a 256-byte-aligned base,
    with GUARD canary bytes (0xA5) on both sides."""

    def __init__(self, nbytes: int, offset: int = 0, data: np.ndarray | None = None):
        torch = torch_mod()
        self.nbytes = int(nbytes)
        self.offset = int(offset)
        total = GUARD + self.offset + self.nbytes + GUARD
        self.t = torch.full((total,), CANARY, dtype=torch.uint8, device="cuda")
        self.lo = GUARD + self.offset
        if data is not None:
            self.upload(data)

    @property
    def ptr(self) -> int:
        return int(self.t.data_ptr()) + self.lo

    def upload(self, a: np.ndarray) -> None:
        torch = torch_mod()
        b = np.ascontiguousarray(a).view(np.uint8).reshape(-1)
        assert b.size == self.nbytes, (b.size, self.nbytes)
        if b.size:
            self.t[self.lo:self.lo + self.nbytes].copy_(torch.from_numpy(b.copy()))

    def download(self, dtype=np.uint8) -> np.ndarray:
        b = self.t[self.lo:self.lo + self.nbytes].cpu().numpy()
        return b.view(dtype)

    def guards_ok(self) -> bool:
        full = self.t.cpu().numpy()
        return bool(np.all(full[:self.lo] == CANARY) and np.all(full[self.lo + self.nbytes:] == CANARY))


def np_dtype(dtype: str):
    return {"f32": np.float32, "bf16": np.uint16, "byte": np.uint8, "u32": np.uint32}[dtype]


def bits(a: np.ndarray, dtype: str) -> np.ndarray:
    """Integer view for bitwise comparison."""
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32).view(np.uint32)
    return np.asarray(a)


def assert_same(got: np.ndarray, want: np.ndarray, dtype: str, what: str = "") -> None:
    """Bitwise equality; a NaN output matches a NaN oracle output."""
    g = bits(got, dtype)
    w = bits(want, dtype)
    assert g.shape == w.shape, (what, g.shape, w.shape)
    if dtype in ("f32", "bf16"):
        if dtype == "f32":
            gn = np.isnan(got.view(np.float32))
            wn = np.isnan(want.view(np.float32))
        else:
            gn = (g & 0x7FFF) > 0x7F80
            wn = (w & 0x7FFF) > 0x7F80
        bad = (g != w) & ~(gn & wn)
    else:
        bad = g != w
    if bad.any():
        idx = np.flatnonzero(bad)
        i = int(idx[0])
        raise AssertionError(f"{what}: {idx.size} mismatches; first at {i}: got {g[i]:#x} want {w[i]:#x}")
