"""CPU oracle of the HiSparse swap-in resolver (test infrastructure only).

Only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path never does.
"""
from .oracle import (  # noqa: F401
    build_oracle,
    load_oracle,
    OracleState,
    oracle_resolve,
    oracle_sparse_mla_decode,
    oracle_mirror_rows,
    oracle_invalidate_tokens,
    oracle_invalidate_host_rows,
    e4m3_to_double,
    bf16_to_double,
)
