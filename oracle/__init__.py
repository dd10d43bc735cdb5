"""CPU oracle for block-paged KV attention.

TEST INFRASTRUCTURE ONLY. Nothing in the product path (the HIP library and its
Python binding) may import, call or execute anything under ``oracle/``. Only
the test suite, the smoke check in ``__graft_entry__`` and the CPU-baseline leg
of ``bench.py`` use it.

The oracle is a plain, slow, obviously correct restatement of what the hot path
computes, written from the mlx-node paged-cache and perf documentation pages
(see each function's docstring for the passage it follows):

* ``attention`` -- slot-mapped KV write, block-table gather, decode attention
  and chunked-prefill attention, in float64 after materialising each
  request's contiguous K/V from its block table.
* ``fp8`` -- the FP8 (E4M3) KV cache encoding: encode, decode and the
  per-layer-scale quantization a write applies.
* ``allocator`` -- ``RefAllocator``, the host block allocator (refcounts,
  prefix table, LRU eviction, null sentinel), written from the written policy,
  not from the C++ library.

Every function here is pinned by the ``-m "not gpu"`` tests in
``tests/test_oracle_pins.py`` and ``tests/test_ref_allocator.py`` against
closed forms, hand-worked fixtures in ``tests/golden/`` and invariants, and
``fp8`` by ``tests/test_oracle_fp8.py``.
Nothing here is "parity unpinned".
"""

from . import attention, allocator, fp8  # noqa: F401
from .attention import (  # noqa: F401
    kv_write,
    gather_positions,
    attend_one,
    decode,
    prefill_chunk,
    decode_attended_range,
    prefill_attended_range,
)
from .allocator import RefAllocator, AllocError  # noqa: F401
