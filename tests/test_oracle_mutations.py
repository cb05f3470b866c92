"""The oracle's pins catch plausible mistakes (CPU only).

Each case plants one mistake in a copy of an oracle function (monkeypatched
for the duration of the test, on the CPU) and checks that at least one pin
fails. This shows the pins are not vacuous: a dropped term, a wrong index or a
transposed operand in the oracle would not go unnoticed.
"""

import numpy as np
import pytest

import oracle
from oracle import attention as A
from oracle import formats as F
from tests import test_oracle_attention as TA
from tests import test_oracle_formats as TF


def _expect_failure(fn, *args):
    with pytest.raises(AssertionError):
        fn(*args)


BRUTE_CASES = [
    (4, 2, 4, 0, [1, 1, 1], [1, 5, 17]),
    (8, 2, 2, 7, [6, 2, 1], [6, 30, 16]),
    (2, 2, 5, 4, [5, 1], [9, 12]),
]


def _brute_pins_fail():
    failures = 0
    for case in BRUTE_CASES:
        try:
            TA.test_oracle_matches_brute_force(*case)
        except AssertionError:
            failures += 1
    assert failures > 0, "the planted mistake passed every brute-force pin"


def test_wrong_group_mapping_is_caught(monkeypatch):
    orig = A.attend_sequence

    def mutant(q_f64, k_pool, v_pool, cache_dtype, k_scale, v_scale, row, ctx, num_kv_heads, scale,
               sliding_window=0, block_size=16, heads=None):
        # interleaved groups (h % Hkv) instead of contiguous ones (h // G)
        q_len, Hq, D = q_f64.shape
        perm = [(h % num_kv_heads) * (Hq // num_kv_heads) + h // num_kv_heads for h in range(Hq)]
        out = orig(q_f64[:, perm, :], k_pool, v_pool, cache_dtype, k_scale, v_scale, row, ctx,
                   num_kv_heads, scale, sliding_window, block_size)
        res = np.empty_like(out)
        res[:, perm, :] = out
        return res

    monkeypatch.setattr(A, "attend_sequence", mutant)
    _brute_pins_fail()


def test_causal_off_by_one_is_caught(monkeypatch):
    def mutant(q_pos, k_pos, window):
        vis = k_pos[None, :] < q_pos[:, None]  # excludes the query itself
        vis[:, 0] = True
        if window > 0:
            vis &= k_pos[None, :] >= (q_pos[:, None] - window + 1)
        return vis

    monkeypatch.setattr(A, "_visible", mutant)
    _brute_pins_fail()


def test_window_off_by_one_is_caught(monkeypatch):
    def mutant(q_pos, k_pos, window):
        vis = k_pos[None, :] <= q_pos[:, None]
        if window > 0:
            vis &= k_pos[None, :] >= (q_pos[:, None] - window)  # W + 1 keys
        return vis

    monkeypatch.setattr(A, "_visible", mutant)
    _brute_pins_fail()


def test_untransposed_value_layout_is_caught(monkeypatch):
    def mutant(k_pool, v_pool, cache_dtype, k_scale, v_scale, row, kv_head, positions, block_size=16):
        positions = np.asarray(positions, dtype=np.int64)
        blk = np.asarray(row, dtype=np.int64)[positions // block_size]
        off = positions % block_size
        K = F.to_f64(k_pool[blk, kv_head, off, :], cache_dtype)
        # reads V as if it were [NB][H][B][D]
        flat = v_pool[:, kv_head].reshape(v_pool.shape[0], block_size, -1)
        V = F.to_f64(flat[blk, off, :], cache_dtype)
        return K, V

    monkeypatch.setattr(A, "gather_kv", mutant)
    _brute_pins_fail()


def test_dropped_scale_is_caught(monkeypatch):
    orig = A.attend_sequence

    def mutant(q_f64, k_pool, v_pool, cache_dtype, k_scale, v_scale, row, ctx, num_kv_heads, scale,
               sliding_window=0, block_size=16, heads=None):
        return orig(q_f64, k_pool, v_pool, cache_dtype, k_scale, v_scale, row, ctx, num_kv_heads, 1.0,
                    sliding_window, block_size, heads)

    monkeypatch.setattr(A, "attend_sequence", mutant)
    _brute_pins_fail()


def test_merge_without_correction_factor_is_caught(monkeypatch, golden):
    def mutant(parts):
        L = sum(p[1] for p in parts)
        O = sum(np.asarray(p[2], dtype=np.float64) for p in parts)
        return O / L

    monkeypatch.setattr(oracle, "merge_partials", mutant)
    _expect_failure(TA.test_weighted_average_example, golden)


def test_wrong_e4m3_bias_is_caught(monkeypatch):
    def mutant(codes):
        c = np.asarray(codes).view(np.uint8).astype(np.int64)
        sign = np.where((c & 0x80) != 0, -1.0, 1.0)
        e = (c >> 3) & 0xF
        m = (c & 0x7).astype(np.float64)
        normal = sign * (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 8.0)
        sub = sign * (m / 8.0) * 2.0 ** -7
        out = np.where(e == 0, sub, normal)
        return np.where((c & 0x7F) == 0x7F, np.nan, out)

    monkeypatch.setattr(F, "e4m3fn_bits_to_f64", mutant)
    _expect_failure(TF.test_e4m3_defining_points)
    _expect_failure(TF.test_e4m3_decode_matches_torch_on_all_codes)


def test_slot_math_mistake_is_caught(monkeypatch, golden):
    from oracle import paging as P
    from tests import test_oracle_paging as TP

    # offset taken from the logical block instead of the position
    monkeypatch.setattr(oracle, "slot_of", lambda row, p, B=16: int(row[p // B]) * B + (p // B) % B)
    _expect_failure(TP.test_block_table_diagram, golden)
    monkeypatch.undo()
    monkeypatch.setattr(oracle, "blocks_needed", lambda n, B=16: n // B)
    _expect_failure(TP.test_allocate_slots, golden)


# ---------------------------------------------------------------------------
# sparse decode over chosen blocks
# ---------------------------------------------------------------------------
from tests import test_oracle_sparse as TS  # noqa: E402

SPARSE_CASES = [
    (17, [0, 2], 4, 2),
    (23, [5, 1, 1, 9, -3], 2, 1),
    (40, [], 4, 4),
    (8, [0, 1], 3, 1),
]


def _sparse_pins_fail():
    failures = 0
    for case in SPARSE_CASES:
        try:
            TS.test_sparse_matches_brute_force(*case)
        except AssertionError:
            failures += 1
    for fn in (TS.test_nothing_chosen_with_one_token_in_the_newest_block_returns_its_v,
               TS.test_every_block_chosen_is_dense_decode):
        try:
            fn()
        except (AssertionError, IndexError, ValueError):
            failures += 1
    assert failures > 0, "the planted mistake passed every sparse pin"


def _positions(keep, ctx, B):
    return np.asarray([b * B + o for b in sorted(keep) for o in range(B) if b * B + o < ctx], dtype=np.int64)


def test_sparse_without_the_newest_block_is_caught(monkeypatch):
    def mutant(ctx, selected, block_size=16):
        nbk = -(-ctx // block_size)
        keep = {int(e) for e in np.asarray(selected).ravel() if 0 <= int(e) < nbk}
        return _positions(keep or {nbk - 1}, ctx, block_size)

    monkeypatch.setattr(A, "selected_positions", mutant)
    _sparse_pins_fail()


def test_sparse_reading_past_the_context_is_caught(monkeypatch):
    def mutant(ctx, selected, block_size=16):
        nbk = -(-ctx // block_size)
        keep = {int(e) for e in np.asarray(selected).ravel() if 0 <= int(e) < nbk - 1} | {nbk - 1}
        return np.asarray([b * block_size + o for b in sorted(keep) for o in range(block_size)], dtype=np.int64)

    monkeypatch.setattr(A, "selected_positions", mutant)
    _sparse_pins_fail()


def test_sparse_newest_block_off_by_one_is_caught(monkeypatch):
    def mutant(ctx, selected, block_size=16):
        nbk = ctx // block_size  # should round up
        keep = {int(e) for e in np.asarray(selected).ravel() if 0 <= int(e) < nbk - 1} | {max(nbk - 1, 0)}
        return _positions(keep, ctx, block_size)

    monkeypatch.setattr(A, "selected_positions", mutant)
    _sparse_pins_fail()


def test_lse_merge_without_correction_is_caught(monkeypatch):
    from tests import test_oracle_dcp as TD

    def mutant(parts):  # plain average of the ranges' results
        return sum(np.asarray(p[0], dtype=np.float64) for p in parts) / len(parts)

    monkeypatch.setattr(oracle, "merge_normalized", mutant)
    import json
    import os
    with open(os.path.join(os.path.dirname(__file__), "golden", "weighted_average_merge.json")) as f:
        g = json.load(f)
    _expect_failure(TD.test_weighted_average_example_in_normalized_form, lambda name: g)


# ---------------------------------------------------------------------------
# latent-cache (MLA) decode
# ---------------------------------------------------------------------------
def _mla_pins_fail():
    from tests import test_oracle_mla as TM

    failures = 0
    for case in [(1, 1, 6, 4), (20, 3, 10, 8), (33, 2, 7, 7)]:
        try:
            TM.test_brute_force_with_positional_part(*case)
        except AssertionError:
            failures += 1
    try:
        TM.test_equals_gqa_oracle_with_one_kv_head()
    except AssertionError:
        failures += 1
    assert failures > 0, "the planted mistake passed every latent-decode pin"


def test_mla_values_from_the_wrong_end_are_caught(monkeypatch):
    from oracle import mla as M

    def mutant(q_f64, pool, cache_dtype, row, ctx, scale, dv, block_size=16):
        C = M.latent_rows(pool, cache_dtype, row, np.arange(ctx), block_size)
        s = scale * (q_f64 @ C.T)
        p = np.exp(s - s.max(axis=1, keepdims=True))
        return (p @ C[:, C.shape[1] - dv:]) / p.sum(axis=1, keepdims=True)

    monkeypatch.setattr(M, "mla_decode_sequence", mutant)
    _mla_pins_fail()


def test_mla_scores_without_the_positional_part_are_caught(monkeypatch):
    from oracle import mla as M

    def mutant(q_f64, pool, cache_dtype, row, ctx, scale, dv, block_size=16):
        C = M.latent_rows(pool, cache_dtype, row, np.arange(ctx), block_size)
        s = scale * (q_f64[:, :dv] @ C[:, :dv].T)
        p = np.exp(s - s.max(axis=1, keepdims=True))
        return (p @ C[:, :dv]) / p.sum(axis=1, keepdims=True)

    monkeypatch.setattr(M, "mla_decode_sequence", mutant)
    _mla_pins_fail()
