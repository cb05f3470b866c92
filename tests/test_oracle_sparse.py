"""Pins for the oracle's sparse decode over chosen blocks (CPU only).

* brute force: pure-Python softmax over the keys of the chosen blocks, on
  K/V placed into a shuffled pool by loops written here, agrees to 1e-12;
* choosing every block is exactly the dense decode;
* choosing nothing leaves the newest block: with one token in it the output
  is that token's V exactly;
* order, repeats and out-of-range entries of the list change nothing, and
  keys outside the chosen blocks (NaN-poisoned) are never read.
"""

import math

import numpy as np
import pytest

import oracle
from oracle import formats as F
from tests.test_oracle_attention import brute_attention, place_in_pool


def _setup(rng, ctxs, Hkv, D, B, fill=np.nan):
    seq_K = [rng.normal(size=(Hkv, c, D)).astype(np.float32) for c in ctxs]
    seq_V = [rng.normal(size=(Hkv, c, D)).astype(np.float32) for c in ctxs]
    NB = sum(-(-c // B) for c in ctxs) + 2
    k_pool, v_pool, table = place_in_pool(seq_K, seq_V, B, NB, rng.permutation(NB), Hkv, D, fill)
    return seq_K, seq_V, k_pool, v_pool, table


@pytest.mark.parametrize("ctx,sel,Hq,Hkv", [
    (17, [0, 2], 4, 2),             # block 2 is before the newest (4)
    (23, [5, 1, 1, 9, -3], 2, 1),   # newest block 5 listed; 9 and -3 out of range; 1 twice
    (40, [], 4, 4),                 # newest block only
    (8, [0, 1], 3, 1),              # the newest block is 1: 0 only
    (33, [7, 6, 5, 4, 3, 2, 1, 0], 6, 2),  # every block, reversed
])
def test_sparse_matches_brute_force(ctx, sel, Hq, Hkv):
    rng = np.random.default_rng(ctx + len(sel))
    B, D = 4, 5
    G = Hq // Hkv
    seq_K, seq_V, k_pool, v_pool, table = _setup(rng, [ctx], Hkv, D, B)
    q = rng.normal(size=(1, Hq, D)).astype(np.float32)
    scale = 1.0 / math.sqrt(D)
    got = oracle.attend_selected_blocks(F.to_f64(q, F.F32), k_pool, v_pool, F.F32, None, None, table[0], ctx, sel,
                                        Hkv, scale, B)
    newest = (ctx - 1) // B
    chosen = [newest]
    for e in sel:
        if 0 <= e < newest and e not in chosen:
            chosen.append(e)
    keys = [j for j in range(ctx) if j // B in chosen]
    for h in range(Hq):
        g = h // G
        Krows = [[float(x) for x in seq_K[0][g, j]] for j in keys]
        Vrows = [[float(x) for x in seq_V[0][g, j]] for j in keys]
        ref = brute_attention([[float(x) for x in q[0, h]]], Krows, Vrows, scale, [len(keys) - 1], 0)
        np.testing.assert_allclose(got[0, h], np.array(ref[0]), rtol=0, atol=1e-12)


def test_every_block_chosen_is_dense_decode():
    rng = np.random.default_rng(3)
    ctx, Hq, Hkv, D = 77, 8, 2, 16
    _, _, k_pool, v_pool, table = _setup(rng, [ctx], Hkv, D, 16)
    q = rng.normal(size=(1, Hq, D)).astype(np.float32)
    dense = oracle.paged_attention(q, F.F32, k_pool, v_pool, F.F32, None, None, table, [0, 1], [ctx], Hkv, 0.25)
    sparse = oracle.attend_selected_blocks(F.to_f64(q, F.F32), k_pool, v_pool, F.F32, None, None, table[0], ctx,
                                           list(range(5)), Hkv, 0.25)
    np.testing.assert_allclose(sparse, dense, rtol=0, atol=1e-13)


def test_nothing_chosen_with_one_token_in_the_newest_block_returns_its_v():
    rng = np.random.default_rng(4)
    ctx = 49  # newest block 3 holds token 48 only
    seq_K, seq_V, k_pool, v_pool, table = _setup(rng, [ctx], 2, 8, 16)
    q = rng.normal(size=(1, 4, 8)).astype(np.float32)
    out = oracle.attend_selected_blocks(F.to_f64(q, F.F32), k_pool, v_pool, F.F32, None, None, table[0], ctx, [],
                                        2, 0.3)
    for h in range(4):
        assert (out[0, h] == seq_V[0][h // 2, 48].astype(np.float64)).all()


def test_list_order_repeats_and_range_do_not_matter():
    rng = np.random.default_rng(5)
    ctx, Hq, Hkv, D = 200, 4, 2, 8
    _, _, k_pool, v_pool, table = _setup(rng, [ctx], Hkv, D, 16)
    q = F.to_f64(rng.normal(size=(1, Hq, D)).astype(np.float32), F.F32)
    a = oracle.attend_selected_blocks(q, k_pool, v_pool, F.F32, None, None, table[0], ctx, [2, 5, 9], Hkv, 0.3)
    b = oracle.attend_selected_blocks(q, k_pool, v_pool, F.F32, None, None, table[0], ctx,
                                      [9, 12, 5, 2, 2, 40, -1, 9, 13], Hkv, 0.3)
    assert np.array_equal(a, b)
    assert oracle.selected_positions(ctx, [9, 12, 5, 2, 2, 40, -1]).tolist() == (
        list(range(32, 48)) + list(range(80, 96)) + list(range(144, 160)) + list(range(192, 200)))


def test_unchosen_blocks_are_never_read():
    """Blocks outside the choice are overwritten with NaN: the result stays."""
    rng = np.random.default_rng(6)
    ctx, Hq, Hkv, D = 90, 4, 1, 8
    _, _, k_pool, v_pool, table = _setup(rng, [ctx], Hkv, D, 16)
    q = F.to_f64(rng.normal(size=(1, Hq, D)).astype(np.float32), F.F32)
    ref = oracle.attend_selected_blocks(q, k_pool, v_pool, F.F32, None, None, table[0], ctx, [1, 3], Hkv, 0.3)
    for lb in (0, 2, 4):
        k_pool[table[0, lb]] = np.nan
        v_pool[table[0, lb]] = np.nan
    got = oracle.attend_selected_blocks(q, k_pool, v_pool, F.F32, None, None, table[0], ctx, [1, 3], Hkv, 0.3)
    assert np.array_equal(got, ref) and np.isfinite(got).all()
