"""HiSparse swap-in resolver for AMD Instinct MI355X (gfx950).

Thin Python binding of ``libhisparse.so`` (C ABI in ``include/hisparse.h``).
Every step of the resolver and of the sparse-MLA decode runs in the HIP
kernels of that library; this package only marshals arguments (torch tensors
for device memory, torch streams) and checks shapes and dtypes so that a
wrong tensor is rejected on the host instead of being read out of bounds on
the GPU.  There is no fallback: if the library is missing, importing the
binding raises.  With HISPARSE_LIBRARY=diag set before the import, the
binding loads ``libhisparse_diag.so`` instead: the same entry points with the
plan kernel's phase trace compiled in, plus the diagnostic ones of
``include/hisparse_diag.h`` (phase trace, floor kernels).
"""
from ._binding import (  # noqa: F401
    EXCHANGE_ROW_INTS,
    HisparseError,
    HostBuffer,
    PoolConfig,
    STAT_NAMES,
    hisparse_decode_layers_overlapped,
    hisparse_destroy_pool,
    hisparse_diag_exchange,
    hisparse_diag_floor,
    hisparse_diag_hit_detection,
    hisparse_diag_phase_clear,
    hisparse_diag_phase_read,
    hisparse_gather_copy,
    hisparse_gather_copy_step,
    hisparse_host_alloc,
    hisparse_host_free,
    hisparse_init_pool,
    hisparse_invalidate_host_rows,
    hisparse_invalidate_tokens,
    hisparse_last_error,
    hisparse_mirror_rows,
    hisparse_resolve,
    hisparse_resolve_plan,
    hisparse_resolve_steps,
    hisparse_sparse_mla_decode,
    hisparse_sparse_mla_decode_noalloc,
    is_diag_library,
    library_path,
    load_library,
)
