"""Attention over a paged KV cache on MI355X (gfx950).

The product is the C-ABI library ``lib/libpa.so`` (include/pa.h) built from
``csrc/`` by ``paged_kv_cache_103_amd.build``; ``_lib`` is its ctypes binding
and ``workloads`` makes seeded synthetic inputs.
"""

from . import _lib as pa  # noqa: F401
from ._lib import (  # noqa: F401
    PAError,
    abi_version,
    decode,
    decode_workspace_bytes,
    prefill_chunk,
    prefill_workspace_bytes,
    reshape_and_cache,
)
