"""Exact attention over a paged KV cache — oracle side (test infrastructure).

Paging changes where K and V live, not what attention computes: the block
table only maps logical order onto arbitrary physical blocks ("从静态批处理到
状态化推理集群", "PagedAttention：把逻辑连续与物理连续分开"; the kernel reads
K/V through the block table). So the oracle is the textbook definition,
evaluated in float64 on values gathered through the block table:

    s_j = scale * <q_h, K_j>,    out_h = sum_j exp(s_j - max s) V_j / sum_j exp(s_j - max s)

(the output formula in "宣稱省下 106 倍成本…", "中：Kimi K3 的 DCP 選擇與 DEP 轉折",
the online-softmax Q&A: output = sum exp(score) * value / sum exp(score), with
the local maximum subtracted before exponentiating).

Readings where the pages are silent (each is also listed in the design notes):
* the new token's K/V is written before attention and the query attends to
  itself: a decode query at position ctx-1 sees ctx keys (the prefill/decode
  example of the agentic-serving page: step 2 "looks at 7 tokens" = the 6
  prompt tokens plus the one just generated);
* causal: key j is visible to the query at position p iff j <= p;
* query row r of a sequence with q_len query tokens and ctx cached tokens
  (this chunk included) sits at position p = ctx - q_len + r;
* sliding window W > 0: keys [max(0, p - W + 1), p] (W keys including
  itself; the DeepSeek-V4.1 write-up rebuilds the window [H-128, H));
* grouped-query attention: query head h reads KV head h // (Hq / Hkv);
* fp8 caches carry one fp32 scale per physical block for K and one for V:
  stored value = e4m3fn_decode(byte) * scale[block].
"""

from __future__ import annotations

import numpy as np

from .formats import FP8, to_f64


def gather_kv(k_pool, v_pool, cache_dtype: str, k_scale, v_scale, block_table_row,
              kv_head: int, positions, block_size: int = 16):
    """K, V rows (float64, [n][head_size]) of one KV head at logical ``positions``.

    Physical block of position j = block_table_row[j // block_size], slot
    offset j % block_size; K pool is [NB][Hkv][B][D], V pool [NB][Hkv][D][B].
    """
    positions = np.asarray(positions, dtype=np.int64)
    blk = np.asarray(block_table_row, dtype=np.int64)[positions // block_size]
    off = positions % block_size
    k_raw = k_pool[blk, kv_head, off, :]                   # [n][D]
    v_raw = v_pool[:, kv_head].transpose(0, 2, 1)[blk, off, :]  # [NB][B][D] -> [n][D]
    K = to_f64(k_raw, cache_dtype)
    V = to_f64(v_raw, cache_dtype)
    if cache_dtype == FP8:
        ks = np.asarray(k_scale, dtype=np.float32).astype(np.float64)[blk]
        vs = np.asarray(v_scale, dtype=np.float32).astype(np.float64)[blk]
        K = K * ks[:, None]
        V = V * vs[:, None]
    return K, V


def _visible(q_pos: np.ndarray, k_pos: np.ndarray, window: int) -> np.ndarray:
    """mask[r, j]: key position k_pos[j] is visible to the query at q_pos[r]."""
    vis = k_pos[None, :] <= q_pos[:, None]
    if window > 0:
        vis &= k_pos[None, :] >= (q_pos[:, None] - window + 1)
    return vis


def attend_sequence(q_f64, k_pool, v_pool, cache_dtype: str, k_scale, v_scale,
                    block_table_row, ctx: int, num_kv_heads: int, scale: float,
                    sliding_window: int = 0, block_size: int = 16, heads=None, rows=None):
    """Attention output of one sequence, float64.

    q_f64: [q_len][Hq][D] queries of this sequence (already float64), the
    last q_len positions of a context of ``ctx`` tokens. Returns
    [q_len][Hq][D]; heads not listed in ``heads`` and query rows not listed
    in ``rows`` are left NaN (each row's result depends on that row alone,
    so leaving rows out changes nothing for the others).
    """
    q_len, Hq, D = q_f64.shape
    assert 1 <= q_len <= ctx, "a sequence attends to at least itself"
    G = Hq // num_kv_heads
    rows = np.arange(q_len, dtype=np.int64) if rows is None else np.asarray(sorted(set(rows)), dtype=np.int64)
    q_pos_all = np.arange(ctx - q_len, ctx, dtype=np.int64)
    lo = 0 if sliding_window <= 0 else max(0, int(q_pos_all[rows[0]]) - sliding_window + 1)
    k_pos = np.arange(lo, ctx, dtype=np.int64)
    out = np.full((q_len, Hq, D), np.nan)
    heads = range(Hq) if heads is None else heads
    for g in sorted({h // G for h in heads}):
        K, V = gather_kv(k_pool, v_pool, cache_dtype, k_scale, v_scale, block_table_row,
                         g, k_pos, block_size)
        for r0 in range(0, len(rows), 256):  # bounded memory for long chunks
            rr = rows[r0:r0 + 256]
            vis = _visible(q_pos_all[rr], k_pos, sliding_window)
            for h in [h for h in heads if h // G == g]:
                s = scale * (q_f64[rr, h, :] @ K.T)               # [rows][n]
                s = np.where(vis, s, -np.inf)
                m = s.max(axis=1, keepdims=True)
                p = np.exp(s - m)
                out[rr, h, :] = (p @ V) / p.sum(axis=1, keepdims=True)
    return out


def paged_attention(query, q_dtype: str, k_pool, v_pool, cache_dtype: str, k_scale, v_scale,
                    block_table, cu_seqlens, context_lens, num_kv_heads: int, scale: float,
                    sliding_window: int = 0, block_size: int = 16, seqs=None):
    """Whole flattened varlen batch: out[num_q_tokens][Hq][D] in float64.

    query: raw storage [num_q_tokens][Hq][D]; sequence s owns query rows
    cu_seqlens[s] .. cu_seqlens[s+1]-1 and has context_lens[s] cached tokens
    (this call's tokens included). Decode is the case q_len == 1.
    Rows of sequences not in ``seqs`` are left NaN.
    """
    q = to_f64(query, q_dtype)
    out = np.full(q.shape, np.nan)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    ctx = np.asarray(context_lens, dtype=np.int64)
    S = len(ctx)
    for s in (range(S) if seqs is None else seqs):
        r0, r1 = int(cu[s]), int(cu[s + 1])
        out[r0:r1] = attend_sequence(q[r0:r1], k_pool, v_pool, cache_dtype, k_scale, v_scale,
                                     block_table[s], int(ctx[s]), num_kv_heads, scale,
                                     sliding_window, block_size)
    return out


def selected_positions(ctx: int, selected, block_size: int = 16) -> np.ndarray:
    """Key positions a sparse decode query reads: every position < ctx inside
    the chosen logical blocks, in ascending order.

    Sparse attention looks only at the top-k positions an indexer picks out
    of the history ("宣稱省下 106 倍成本…", "下：DeepSeek V4 的挑戰與 PCP/DEP 方案",
    "背景：什麼是稀疏注意力"); the candidates here are whole blocks (reading).
    Readings: an entry outside [0, newest block) is ignored, order and
    repeats do not matter, and the block holding the newest token is always
    read, so the query always sees itself.
    """
    nbk = -(-ctx // block_size)
    keep = {int(e) for e in np.asarray(selected, dtype=np.int64).ravel() if 0 <= int(e) < nbk - 1}
    keep.add(nbk - 1)
    pos = [b * block_size + o for b in sorted(keep) for o in range(block_size) if b * block_size + o < ctx]
    return np.asarray(pos, dtype=np.int64)


def attend_selected_blocks(q_f64, k_pool, v_pool, cache_dtype: str, k_scale, v_scale,
                           block_table_row, ctx: int, selected, num_kv_heads: int, scale: float,
                           block_size: int = 16):
    """Sparse decode of one sequence, float64: the query of its newest token
    (position ctx - 1, q_f64 [1][Hq][D]) attends to the keys at
    ``selected_positions(ctx, selected)`` only, with the same softmax as
    ``attend_sequence`` (all of them precede the query, so none is masked).
    The selection is one list for the whole sequence, shared by every head:
    the indexer hands over one global top-k list ("三個讓 TP 更不划算的原因",
    second reason), and fetching the chosen entries is the work that stays
    ("真正貴的部分…", third reason; the DeepSeek-V4.1 write-up,
    "三、第二招：把能合的内核全合成一个", sparse MQA logits: only candidates
    are scored, so the cost stops growing with the context).
    """
    assert q_f64.shape[0] == 1 and ctx >= 1
    Hq = q_f64.shape[1]
    G = Hq // num_kv_heads
    k_pos = selected_positions(ctx, selected, block_size)
    out = np.full(q_f64.shape, np.nan)
    for g in range(num_kv_heads):
        K, V = gather_kv(k_pool, v_pool, cache_dtype, k_scale, v_scale, block_table_row, g, k_pos,
                         block_size)
        for h in range(g * G, (g + 1) * G):
            s = scale * (K @ q_f64[0, h, :])
            p = np.exp(s - s.max())
            out[0, h, :] = (p @ V) / p.sum()
    return out


def partial_softmax(scores, values):
    """Summary of one key range: (m, l, o) = (max s, sum e^(s-m), sum e^(s-m) v).

    The per-range state each worker hands over in the distributed
    weighted-average Q&A ("local weighted sum" and "local weight sum", with the
    local maximum subtracted before exponentiating).
    """
    s = np.asarray(scores, dtype=np.float64)
    v = np.asarray(values, dtype=np.float64)
    m = s.max()
    w = np.exp(s - m)
    return m, w.sum(), w @ v


def normalized_partial(scores, values):
    """One key range's result in the form a context-parallel rank hands over:
    (o, lse) = (sum e^s v / sum e^s, ln sum e^s), computed as
    o = o_i / l_i and lse = m_i + ln l_i from ``partial_softmax``.

    Decode context parallelism splits a sequence's cached positions into
    contiguous ranges, one per GPU; each attends over its own range and the
    ranges' results are combined by the online-softmax correction
    ("宣稱省下 106 倍成本…", "DCP 的切法：照「序列位置」切，不照「頭」切" and the
    online-softmax Q&A of "中：Kimi K3 的 DCP 選擇與 DEP 轉折").
    """
    m, l, o = partial_softmax(scores, values)
    return np.asarray(o, dtype=np.float64) / l, m + np.log(l)


def merge_normalized(parts):
    """Exact result from per-range (o_r, lse_r): with M = max_r lse_r,
    out = sum_r e^(lse_r - M) o_r / sum_r e^(lse_r - M). A range with no keys
    (lse = -inf) weighs nothing."""
    M = max(p[1] for p in parts)
    w = [np.exp(p[1] - M) for p in parts]
    return sum(wi * np.asarray(p[0], dtype=np.float64) for wi, p in zip(w, parts)) / sum(w)


def merge_partials(parts):
    """Exact softmax output from per-range summaries (m_i, l_i, o_i).

    M = max_i m_i, L = sum_i l_i e^(m_i - M), out = sum_i o_i e^(m_i - M) / L:
    each range's sums are brought to the common maximum by the correction
    factor e^(m_i - M), then added and divided once.
    """
    M = max(p[0] for p in parts)
    L = sum(p[1] * np.exp(p[0] - M) for p in parts)
    O = sum(np.asarray(p[2], dtype=np.float64) * np.exp(p[0] - M) for p in parts)
    return O / L
