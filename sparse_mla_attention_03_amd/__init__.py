"""libsparsemla: sparse MLA attention forward on AMD MI355X (gfx950).

The compute lives in the HIP shared library ``csrc/libsparsemla.so`` behind a
C ABI (``include/sparse_mla.h``).  This package is a thin ctypes binding over
it (argument marshalling only) plus the seeded synthetic-input generator.
"""
from .binding import (  # noqa: F401
    KV_BF16, KV_FP8_E4M3, SparseMLAError, load_library, sparse_mla_fwd,
    sparse_mla_fwd_ex, sparse_mla_workspace_bytes, sparse_mla_num_splits,
    sparse_mla_quantize_q_fp8, sparse_mla_status_string, sparse_mla_last_error,
)
