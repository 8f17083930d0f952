"""CPU oracle for the copy / N-to-1 reduce collectives.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this package: only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library (no kernels, headers, helpers, tables or constants); the only common
module is the seeded input generator, which holds none of the arithmetic.

The oracle is the plain definition of each collective, written out with NumPy
on the host:

* copies are exact byte copies;
* reductions widen every input to binary32, add them one at a time in rank
  order 0, 1, ..., N-1 starting from the rank-0 value (never ``np.sum``,
  whose blocking order is not the contract), and round once to the output
  type (identity for float32, round-to-nearest-even for bfloat16).

bfloat16 data is carried as ``uint16`` bit patterns; the oracle does its own
widening and narrowing in ``oracle.bf16``.

Every function names the passage of the pages it follows.  Readings taken
where the pages are silent are listed in the module docstrings.  Pins (tests
that check the oracle against something other than itself) live in
``tests/test_oracle_pins.py``; no function here is parity-unpinned.
"""
from .bf16 import bf16_to_f32, f32_to_bf16
from .collectives import (
    DTYPES,
    all_gather,
    all_gather_v,
    all_reduce,
    all_to_all,
    all_to_all_v,
    copy,
    exclusive_prefix,
    pipeline_scale_reduce,
    reduce_n,
    reduce_scatter,
    reduce_scatter_v,
)

__all__ = [
    "DTYPES",
    "bf16_to_f32",
    "f32_to_bf16",
    "all_gather",
    "all_gather_v",
    "all_reduce",
    "all_to_all",
    "all_to_all_v",
    "copy",
    "exclusive_prefix",
    "pipeline_scale_reduce",
    "reduce_n",
    "reduce_scatter",
    "reduce_scatter_v",
]
