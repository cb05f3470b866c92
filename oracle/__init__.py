"""CPU oracle for attention over a paged KV cache — TEST INFRASTRUCTURE ONLY.

This package is a slow, plain, float64 NumPy statement of what the paged-KV
hot path computes. It exists so that the HIP kernels can be checked against
something written independently of them. Only the test suite, the smoke check
in ``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` may import
it; the product path (``paged_kv_cache_103_amd``) never does, and this package
imports nothing from the product path.

Modules
-------
formats    exact decoding of stored element bits (fp32, bf16, OCP e4m3fn) to
           float64, plus the e4m3fn encoder used by the quantising write.
paging     block arithmetic and the KV write (``reshape_and_cache``): slot =
           physical block * block_size + offset, byte-exact scatter.
attention  gather through the block table and exact softmax attention with
           causal / sliding-window masks; sparse decode over chosen blocks;
           partial-softmax merge.
mla        decode over a paged latent (MLA) cache: one shared row per token,
           absorbed queries, values from the row's first dv elements;
           imported on its own as ``oracle.mla``.
blocks     plain model of the block manager's policy (refcounts, prefix reuse
           over full blocks, LRU free queue, fork and copy-on-write), imported
           on its own as ``oracle.blocks``.

Every function names the page passage it follows in its docstring. Pins
(page facts, closed forms, brute force) live in ``tests/test_oracle_*.py``.
"""

from . import formats, paging, attention  # noqa: F401
from .formats import to_f64, bf16_bits_to_f64, e4m3fn_bits_to_f64, e4m3fn_encode  # noqa: F401
from .paging import (  # noqa: F401
    blocks_needed,
    block_bytes,
    kv_cache_bytes,
    tokens_in_budget,
    max_concurrency,
    slot_of,
    reshape_and_cache,
    reshape_and_cache_fp8,
)
from .attention import (  # noqa: F401
    gather_kv,
    paged_attention,
    attend_sequence,
    attend_selected_blocks,
    selected_positions,
    partial_softmax,
    merge_partials,
    normalized_partial,
    merge_normalized,
)
