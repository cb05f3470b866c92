"""Block arithmetic and the KV write — oracle side (test infrastructure).

Sources (page titles as printed at the top of each page):

* "宣稱省下 106 倍成本：vLLM 怎麼把 Serving 系統校準給 Agentic Workload",
  section "vLLM 的解法：統一分頁 + 共用池": a sequence's logical blocks map
  through a block table onto physical blocks that need not be contiguous
  (the diagram: 10 tokens, 4 tokens per block, physical blocks 37, 12, 58);
  one shared pool; prefix blocks shared by reference counting.
* the vLLM architecture summary (ai.youdonthavefriends.com), "第一部分：LLM
  引擎核心": bytes of one block of one layer = 2 * block_size(16) *
  num_kv_heads * head_size * dtype_bytes; ``allocate_slots`` needs
  ceil(new_tokens / 16) blocks (17 tokens -> 2 blocks); the forward pass
  builds ``slot_mapping`` while preparing inputs.
* "从静态批处理到状态化推理集群", section "KV Cache：动态批处理把显存变成主资源":
  M_KV = 2 * L * b * H_kv * d_h * sum_i T_i; section "PagedAttention：把逻辑连续
  与物理连续分开": (sequence, logical block) -> physical block, and the waste of
  a sequence is below one block (fewer than P_b slots, all in its last block).
* "大模型推理优化学习笔记", section "KV Cache": the startup log that converts the
  KV budget into a token count (643,232 tokens; 15.70x concurrency at 40,960
  tokens per request; 21,840 tokens in a 256 MiB budget).

Pool layout (the boundary's contract; the pages fix only the byte count):
    k_pool[num_blocks][num_kv_heads][block_size][head_size]   (key row-major)
    v_pool[num_blocks][num_kv_heads][head_size][block_size]   (value transposed
                                                               inside the block)
"""

from __future__ import annotations

import numpy as np

from .formats import e4m3fn_encode


def blocks_needed(num_tokens: int, block_size: int = 16) -> int:
    """ceil(tokens / block_size): physical blocks that hold ``num_tokens``."""
    return -(-int(num_tokens) // int(block_size))


def block_bytes(block_size: int, num_kv_heads: int, head_size: int, dtype_bytes: int) -> int:
    """Bytes of one physical block of one layer: K and V for block_size tokens."""
    return 2 * block_size * num_kv_heads * head_size * dtype_bytes


def kv_cache_bytes(num_layers: int, dtype_bytes: int, num_kv_heads: int, head_size: int,
                   seq_lens) -> int:
    """M_KV = 2 L b H_kv d_h sum_i T_i (token-exact, before block rounding)."""
    return 2 * num_layers * dtype_bytes * num_kv_heads * head_size * int(sum(seq_lens))


def tokens_in_budget(budget_bytes: int, bytes_per_token_per_layer_block: int,
                     block_size: int = 16) -> int:
    """Tokens a fixed KV budget holds when memory is handed out in whole blocks.

    ``bytes_per_token_per_layer_block`` is the size of one block across all
    layers; the budget holds floor(budget / that) blocks of block_size tokens.
    """
    return (int(budget_bytes) // int(bytes_per_token_per_layer_block)) * int(block_size)


def max_concurrency(cache_tokens: int, tokens_per_request: int) -> float:
    """Requests that fit at once if every request uses its full length."""
    return cache_tokens / tokens_per_request


def slot_of(block_table_row, position: int, block_size: int = 16) -> int:
    """Flat cache slot of the token at logical ``position`` of one sequence.

    The logical block is position // block_size, the block table gives its
    physical block, and the slot inside it is position % block_size.
    """
    return int(block_table_row[position // block_size]) * block_size + position % block_size


def reshape_and_cache(k_pool: np.ndarray, v_pool: np.ndarray, key: np.ndarray,
                      value: np.ndarray, slot_mapping, block_size: int = 16) -> None:
    """Scatter new K/V rows into the pool, in place, byte for byte.

    key/value: raw storage [num_tokens][num_kv_heads][head_size];
    slot_mapping[t] = physical_block * block_size + offset, negative = skip.
    Every pool element that no slot names is left untouched.
    """
    for t, slot in enumerate(np.asarray(slot_mapping).tolist()):
        if slot < 0:
            continue
        blk, off = divmod(int(slot), block_size)
        k_pool[blk, :, off, :] = key[t]
        v_pool[blk, :, :, off] = value[t]


def reshape_and_cache_fp8(k_pool: np.ndarray, v_pool: np.ndarray, key_f32: np.ndarray,
                          value_f32: np.ndarray, k_scale, v_scale, slot_mapping,
                          block_size: int = 16) -> None:
    """Quantising write into an e4m3fn pool with one fp32 scale per block.

    byte = e4m3fn_encode(x / scale[block]), round to nearest even, saturating.
    The quotient decides an integer code, so it is taken in the precision the
    kernel uses: an IEEE float32 division (correctly rounded), then encoded
    exactly. The scale of the destination block is an input (the pages do
    not say how it is chosen).
    """
    for t, slot in enumerate(np.asarray(slot_mapping).tolist()):
        if slot < 0:
            continue
        blk, off = divmod(int(slot), block_size)
        kq = np.asarray(key_f32[t], dtype=np.float32) / np.float32(k_scale[blk])
        vq = np.asarray(value_f32[t], dtype=np.float32) / np.float32(v_scale[blk])
        k_pool[blk, :, off, :] = e4m3fn_encode(kq.astype(np.float64))
        v_pool[blk, :, :, off] = e4m3fn_encode(vq.astype(np.float64))
