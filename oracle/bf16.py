"""bfloat16 <-> binary32 conversions for the oracle (test infrastructure only).

bfloat16 is the upper half of a binary32 word: 1 sign bit, 8 exponent bits,
7 fraction bits.  Widening is therefore exact (append 16 zero bits).
Narrowing rounds to nearest, ties to even, as IEEE 754 defines it for a
format with the same exponent range:

* the discarded low 16 bits are compared with half an ulp (0x8000); above
  rounds up, below truncates, exactly half rounds to the even neighbour.
  Adding ``0x7FFF + lsb`` and truncating does all three cases at once; the
  carry may ripple into the exponent, which is the correct result (rounding
  up to the next binade, or to infinity from the largest finite value);
* subnormals go through the same rule (no flush to zero);
* a NaN input keeps its sign and its high payload bits and is made quiet
  (fraction MSB 0x0040 set) so it cannot round into an infinity.

Reading (pages silent): the pages fix neither the output rounding nor NaN
handling; round-to-nearest-even is the IEEE default and what every reduction
test here assumes.  Any NaN output counts as matching a NaN oracle output.
"""
from __future__ import annotations

import numpy as np


def bf16_to_f32(u16: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns (uint16) to float32."""
    u = np.asarray(u16, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32)


def f32_to_bf16(f: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); uint16 out."""
    u = np.ascontiguousarray(f, dtype=np.float32).view(np.uint32)
    is_nan = (u & np.uint32(0x7FFFFFFF)) > np.uint32(0x7F800000)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    rounded = (u + (np.uint32(0x7FFF) + lsb)) >> np.uint32(16)
    quiet = (u >> np.uint32(16)) | np.uint32(0x0040)
    return np.where(is_nan, quiet, rounded).astype(np.uint16)
