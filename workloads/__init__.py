"""Seeded synthetic inputs for the paged-attention hot path.

This package builds the inputs that both the GPU library and the CPU oracle
consume: shapes, context lengths, the sharing structure of sequences, the
initial free-block order, and the random q/K/V values.  It holds none of the
method's arithmetic: no slot computation, no tile layout, no attention.  Block
tables and slots are produced from the program it emits by a block manager
(the library's, or the oracle's).
"""

from .configs import (  # noqa: F401
    WORKLOADS,
    Workload,
    make_workload,
    run_program,
    to_storage,
    storage_dtype,
)
