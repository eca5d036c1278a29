"""Chunked prefill (and the single-token decode step) of delta-rule linear
attention (GDN, KDA) on MI355X.

Python binding of the C ABI in ``include/drla.h`` (``libdrla.so``): argument
marshalling only.  PyTorch provides device memory and the current stream;
every step of the computation runs in the library's HIP kernels.  If the
library is not built the calls raise; there is no other code path.
"""
from ._lib import (  # noqa: F401
    KEEP_INTERMEDIATES,
    DECAY_ONLY,
    SERIAL,
    HEAD_SCAN,
    COLUMN_SCAN,
    NOALLOC_SCRATCH_BYTES,
    DrlaError,
    PreparedPrefill,
    decay_decode,
    decay_prefill,
    gdn_decode,
    gdn_prefill,
    kda_decode,
    kda_prefill,
    lib_path,
    load_library,
    prefill_noalloc,
    prepare_prefill,
    workspace_bytes,
    workspace_layout,
)

__all__ = ["gdn_prefill", "kda_prefill", "gdn_decode", "kda_decode", "decay_prefill",
           "decay_decode", "DECAY_ONLY", "workspace_bytes", "workspace_layout",
           "load_library", "lib_path", "prefill_noalloc", "DrlaError", "KEEP_INTERMEDIATES", "SERIAL", "HEAD_SCAN",
           "COLUMN_SCAN",
           "NOALLOC_SCRATCH_BYTES", "prepare_prefill", "PreparedPrefill"]
