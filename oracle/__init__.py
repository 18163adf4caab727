"""CPU oracle for the paged-attention hot path.  TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import anything from this package.  The library never calls it, and it never
calls the library: the two share no code.  The only thing both sides consume
is the seeded input recipe in ``workloads``.

Contents
--------
layout        the element order inside one (block, kv-head) tile of the pools
attention     cache write, block copy, gather through the block table, and
              plain fp64 decode / chunked-prefill attention
block_manager a plain Python model of the block manager (free list,
              reference counts, copy-on-write)

Every function is the plain definition of what it computes: no blocking,
partitioning or online softmax.  The pins that tie it to the pages and to
mathematics live in ``tests/test_oracle_*.py``.  Parity of every function is
pinned; none is left unpinned.
"""

from . import attention, block_manager, layout  # noqa: F401
