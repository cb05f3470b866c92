"""Decode attention over a paged latent (MLA) cache — oracle side (test
infrastructure; only tests/, the smoke check and bench.py's CPU baseline use
it).

Multi-head latent attention keeps one compressed vector c per token for all
heads instead of a K and a V per head; a head reads its K and V back through
its own up-projection of c, and because those projections are fixed after
training they are folded into the query side ("matrix absorption"), so each
head takes the inner product of its absorbed query q' directly with c and c
is never expanded ("宣稱省下 106 倍成本…", "MLA(Multi-head Latent Attention)是
什麼、為什麼讓 TP 沒效率" and its two Q&As: how the heads are compressed into
one and restored, and where MLA saves work). The value side is folded the
same way: the attention-weighted sum of the c_j is formed in latent space
and each head's up-projection is applied to that sum afterwards, outside
attention.

So per head h, with scale s and the cached rows c_j of the sequence:

    score_hj = s * <q'_h, c_j>,   out_h = sum_j softmax_j(score_h) * c_j[:dv]

Readings where the pages are silent: a cached row may carry dk >= dv
elements, of which the first dv are the latent c (the value side) and all dk
take part in the score (dk = dv is the pages' plain case, K = V = c; the
extra dk - dv elements model a positional part kept beside the latent); one
row per token in 16-token blocks [num_blocks][16][dk]; the query of a
decode step attends to every cached token, itself included.
"""

from __future__ import annotations

import numpy as np

from .formats import to_f64


def latent_rows(pool, cache_dtype: str, block_table_row, positions, block_size: int = 16):
    """Cached latent rows (float64 [n][dk]) at logical ``positions``."""
    positions = np.asarray(positions, dtype=np.int64)
    blk = np.asarray(block_table_row, dtype=np.int64)[positions // block_size]
    return to_f64(pool[blk, positions % block_size, :], cache_dtype)


def mla_decode_sequence(q_f64, pool, cache_dtype: str, block_table_row, ctx: int, scale: float, dv: int,
                        block_size: int = 16):
    """Output [H][dv] (float64) of one decode query q_f64 [H][dk] (absorbed
    queries, one per head) over the sequence's ctx cached rows."""
    C = latent_rows(pool, cache_dtype, block_table_row, np.arange(ctx), block_size)  # [ctx][dk]
    s = scale * (q_f64 @ C.T)                    # [H][ctx]
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    return (p @ C[:, :dv]) / p.sum(axis=1, keepdims=True)


def mla_decode(query, q_dtype: str, pool, cache_dtype: str, block_table, context_lens, scale: float, dv: int,
               block_size: int = 16, seqs=None):
    """Batch decode: query raw [S][H][dk] -> out float64 [S][H][dv]; rows of
    sequences not in ``seqs`` are NaN."""
    q = to_f64(query, q_dtype)
    S, H, _ = q.shape
    out = np.full((S, H, dv), np.nan)
    for s in (range(S) if seqs is None else seqs):
        out[s] = mla_decode_sequence(q[s], pool, cache_dtype, block_table[s], int(context_lens[s]), scale, dv,
                                     block_size)
    return out


def mla_cache_bytes(positions: int, latent_dim: int, dtype_bytes: int) -> int:
    """Bytes of one layer's latent cache read for ``positions`` tokens: one
    shared row per position, whatever the head count (the pages' worked
    comparison)."""
    return positions * latent_dim * dtype_bytes


def per_head_key_bytes(heads: int, head_dim: int, positions: int, dtype_bytes: int) -> int:
    """Bytes of per-head keys for the same positions, as the comparison counts
    them (keys only)."""
    return heads * positions * head_dim * dtype_bytes
