"""MI355X (gfx950) MLA latent-cache decode.

The decode runs in hand-written HIP kernels behind the C ABI of
include/mla_decode.h (libmla_decode.so, built in-tree by
``python -m mla_latent_cache_decode_amd.build``).  This package is the thin
ctypes binding; PyTorch supplies device memory and the stream.
"""

from ._lib import (  # noqa: F401
    MlaDecode,
    MlaError,
    load_library,
    kv_row_bytes,
    kv_row_stride,
    status_string,
    EXPORTED_SYMBOLS,
    LIB_PATH,
    MLA_OK,
    MLA_ERR_INVALID_ARGUMENT,
    MLA_ERR_UNSUPPORTED,
    MLA_ERR_WORKSPACE_TOO_SMALL,
    MLA_ERR_HIP,
    MLA_ERR_OUT_OF_MEMORY,
    MLA_FLAG_KV_WITHIN_4GIB,
    KV_WINDOW_BYTES,
    NOALLOC_SCRATCH_BYTES,
)
