"""Pins for the oracle's block arithmetic and KV write (CPU only).

Page facts (tests/golden/*.json, each with its citation): the block-table
diagram of the agentic-serving page, allocate_slots' ceil(17/16) = 2, the
block-bytes formula, the KV-budget log lines, M_KV. Invariants: the write
touches exactly the named slots and nothing else; waste is below one block.
"""

import numpy as np
import pytest

import oracle
from oracle import formats as F


def test_block_table_diagram(golden):
    g = golden("block_table_diagram.json")
    B = g["block_size"]
    row = g["block_table"]
    slots = [oracle.slot_of(row, p, B) for p in range(g["num_tokens"])]
    assert slots == g["expected_slots_by_position"]
    assert oracle.blocks_needed(g["num_tokens"], B) == len(row)
    assert oracle.blocks_needed(g["num_tokens"], B) * B - g["num_tokens"] == g["expected_last_block_free_slots"]


def test_block_table_diagram_write_then_gather(golden):
    """Writing the 10 tokens through their slots lands them in blocks 37, 12, 58
    in that order, and gathering through the table returns them in logical order."""
    g = golden("block_table_diagram.json")
    B, row, n = g["block_size"], g["block_table"], g["num_tokens"]
    NB, H, D = 64, 1, 3
    k_pool = np.full((NB, H, B, D), -1.0, dtype=np.float32)
    v_pool = np.full((NB, H, D, B), -1.0, dtype=np.float32)
    key = np.arange(n * D, dtype=np.float32).reshape(n, H, D) + 1.0
    val = -key
    slots = g["expected_slots_by_position"]
    oracle.reshape_and_cache(k_pool, v_pool, key, val, slots, B)
    # token t (position) sits in physical block row[t // B], offset t % B
    for t in range(n):
        assert (k_pool[row[t // B], 0, t % B, :] == key[t, 0]).all()
        assert (v_pool[row[t // B], 0, :, t % B] == val[t, 0]).all()
    K, V = oracle.gather_kv(k_pool, v_pool, F.F32, None, None, row, 0, np.arange(n), B)
    assert (K == key[:, 0].astype(np.float64)).all()
    assert (V == val[:, 0].astype(np.float64)).all()
    # everything else untouched
    touched = np.zeros((NB, B), dtype=bool)
    for s in slots:
        touched[s // B, s % B] = True
    assert (k_pool.transpose(0, 2, 1, 3)[~touched] == -1.0).all()
    assert (v_pool.transpose(0, 3, 1, 2)[~touched] == -1.0).all()


def test_write_skips_negative_slots_and_is_bytewise():
    rng = np.random.default_rng(0)
    NB, H, B, D, T = 8, 2, 16, 8, 20
    k_pool = rng.integers(0, 2 ** 16, (NB, H, B, D)).astype(np.uint16)
    v_pool = rng.integers(0, 2 ** 16, (NB, H, D, B)).astype(np.uint16)
    k0, v0 = k_pool.copy(), v_pool.copy()
    key = rng.integers(0, 2 ** 16, (T, H, D)).astype(np.uint16)
    val = rng.integers(0, 2 ** 16, (T, H, D)).astype(np.uint16)
    slots = rng.permutation(NB * B)[:T].astype(np.int64)
    slots[::5] = -1
    oracle.reshape_and_cache(k_pool, v_pool, key, val, slots, B)
    for t, s in enumerate(slots):
        if s < 0:
            continue
        assert (k_pool[s // B, :, s % B, :] == key[t]).all()
        assert (v_pool[s // B, :, :, s % B] == val[t]).all()
    mask = np.ones((NB, B), dtype=bool)
    for s in slots:
        if s >= 0:
            mask[s // B, s % B] = False
    assert (k_pool.transpose(0, 2, 1, 3)[mask] == k0.transpose(0, 2, 1, 3)[mask]).all()
    assert (v_pool.transpose(0, 3, 1, 2)[mask] == v0.transpose(0, 3, 1, 2)[mask]).all()


def test_allocate_slots(golden):
    g = golden("capacity_facts.json")["allocate_slots"]
    assert oracle.blocks_needed(g["new_tokens"], g["block_size"]) == g["expected_blocks"]


def test_block_bytes_formula(golden):
    for B, H, D, b, expect in golden("capacity_facts.json")["block_bytes_formula"]["cases"]:
        assert oracle.block_bytes(B, H, D, b) == expect


def test_kv_budget_log(golden):
    g = golden("capacity_facts.json")["kv_budget_log"]
    assert round(oracle.max_concurrency(g["cache_tokens"], g["tokens_per_request"]), 2) == g["expected_concurrency_2dp"]
    assert g["cache_tokens"] % 16 == 0  # the pool is handed out in whole 16-token blocks


def test_qwen_256mib_budget(golden):
    g = golden("capacity_facts.json")["qwen_256mib"]
    per_block_all_layers = g["num_layers"] * oracle.block_bytes(g["block_size"], g["num_kv_heads"],
                                                                g["head_size"], g["dtype_bytes"])
    assert oracle.tokens_in_budget(g["budget_bytes"], per_block_all_layers, g["block_size"]) == g["expected_tokens"]


def test_pd_transfer_whole_block(golden):
    g = golden("capacity_facts.json")["pd_transfer_15_tokens"]
    nblk = oracle.blocks_needed(g["prompt_tokens"], g["block_size"])
    nbytes = nblk * g["num_layers"] * oracle.block_bytes(g["block_size"], g["num_kv_heads"],
                                                         g["head_size"], g["dtype_bytes"])
    assert round(nbytes / 2 ** 20, 3) == g["expected_mib_3dp"]


def test_mkv_formula(golden):
    e = golden("capacity_facts.json")["mkv_formula"]["example"]
    assert oracle.kv_cache_bytes(e["num_layers"], e["dtype_bytes"], e["num_kv_heads"], e["head_size"],
                                 e["seq_lens"]) == e["expected_bytes"]
    # M_KV for one layer equals the block formula when lengths fill whole blocks
    assert oracle.kv_cache_bytes(1, 2, 8, 128, [64]) == 4 * oracle.block_bytes(16, 8, 128, 2)


@pytest.mark.parametrize("n", [1, 15, 16, 17, 31, 32, 33, 1000, 142000])
def test_waste_below_one_block(n):
    B = 16
    waste = oracle.blocks_needed(n, B) * B - n
    assert 0 <= waste < B


def test_fp8_quantising_write_round_trip():
    """Values that are exact e4m3 multiples of the block scale come back exactly."""
    rng = np.random.default_rng(11)
    NB, H, B, D, T = 4, 2, 16, 8, 10
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    k_scale = np.float32([0.5, 2.0, 0.125, 4.0])
    v_scale = np.float32([1.0, 0.25, 8.0, 0.5])
    slots = rng.permutation(NB * B)[:T]
    kc = rng.choice(codes, (T, H, D))
    vc = rng.choice(codes, (T, H, D))
    kx = np.stack([F.e4m3fn_bits_to_f64(kc[t]) * k_scale[s // B] for t, s in enumerate(slots)]).astype(np.float32)
    vx = np.stack([F.e4m3fn_bits_to_f64(vc[t]) * v_scale[s // B] for t, s in enumerate(slots)]).astype(np.float32)
    k_pool = np.zeros((NB, H, B, D), np.uint8)
    v_pool = np.zeros((NB, H, D, B), np.uint8)
    oracle.reshape_and_cache_fp8(k_pool, v_pool, kx, vx, k_scale, v_scale, slots, B)
    for t, s in enumerate(slots):
        got_k = k_pool[s // B, :, s % B, :]
        got_v = v_pool[s // B, :, :, s % B]
        # +0 and -0 both decode to zero; compare values, not just codes
        assert (F.e4m3fn_bits_to_f64(got_k) == F.e4m3fn_bits_to_f64(kc[t])).all()
        assert (F.e4m3fn_bits_to_f64(got_v) == F.e4m3fn_bits_to_f64(vc[t])).all()
