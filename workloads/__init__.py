"""Seeded synthetic inputs for the resolver and the sparse-MLA decode step.

This package generates inputs only (top-k traces, sequence lengths, host
row placement, block tables, row bytes, admission state).  It holds none of
the method's arithmetic, so both the HIP path and the CPU oracle can take
their inputs from it.
"""
from .gen import (  # noqa: F401
    Workload,
    synth,
    config1_tiny,
    config2_dsa_decode,
    config3_mixed_residency,
    config4_indexshare_1m,
    admission,
    decode_writes,
    fill_host_rows_uniform,
    fill_host_rows_mla,
    make_queries,
    ROW_BYTES,
)
