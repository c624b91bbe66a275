"""Seeded synthetic inputs for paged KV attention.

This package is shared by the HIP path's callers (tests, bench) and by the CPU
oracle.  It holds input *generation* only: random values, request lengths,
block allocation and the packing of requests into a varlen batch.  It performs
none of the method's arithmetic (no slot computation, no scatter, no attention).
"""

from .gen import (  # noqa: F401
    Workload,
    CONFIG_NAMES,
    make_workload,
    bf16_bits_from_f32,
    f16_bits_from_f32,
    storage_dtype,
    element_size,
)
