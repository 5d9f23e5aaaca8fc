"""Paged KV-cache decode attention for AMD MI355X (gfx950).

The compute lives in ``libpagedkv.so`` (C ABI in ``include/pagedkv.h``):
a C++ block-table manager and hand-written HIP kernels.  This package is the
ctypes binding (same names as the C entry points) plus ``TorchKVPool``, which
only allocates the device buffers with torch.  Importing it fails if the
library has not been built; there is no fallback path.
"""
from ._binding import *  # noqa: F401,F403
from ._binding import (EXPORTED, PagedKVError, PagedKVOOM, DTYPE_CODE, ELEM_BYTES,  # noqa: F401
                       kv_pool_desc, paged_decode_args, kv_block_copy, make_desc, make_decode_args)
from .torch_pool import TorchKVPool  # noqa: F401
