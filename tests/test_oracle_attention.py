"""Pins for the oracle's attention (CPU only).

* brute force: a pure-Python loop implementation of softmax attention over
  contiguous K/V (no pool, no block table, no NumPy) on tiny inputs, with K/V
  placed into a shuffled pool by index code written here, agrees to 1e-12;
* the weighted-average worked example (= 29), both as attention and through
  the partial-summary merge;
* closed forms: one key gives V_0 exactly; equal scores give the mean of V;
* paging invariants: permuted physical blocks, shared vs copied prefix
  blocks, one chunk vs several chunks, W >= ctx vs full attention;
* the decode-step example: step k of a 6-token prompt sees 6 + k - 1 keys.
"""

import math

import numpy as np
import pytest

import oracle
from oracle import formats as F


# ----------------------------------------------------------------------------
# independent brute force (pure Python)
# ----------------------------------------------------------------------------
def brute_attention(q_rows, K_rows, V_rows, scale, q_positions, window):
    """q_rows: list of query vectors; K_rows/V_rows: per key position 0..n-1."""
    out = []
    for q, p in zip(q_rows, q_positions):
        keys = [j for j in range(len(K_rows)) if j <= p and (window <= 0 or j > p - window)]
        scores = [scale * sum(a * b for a, b in zip(q, K_rows[j])) for j in keys]
        mx = max(scores)
        w = [math.exp(s - mx) for s in scores]
        tot = sum(w)
        out.append([sum(w[i] * V_rows[j][d] for i, j in enumerate(keys)) / tot
                    for d in range(len(V_rows[0]))])
    return out


def place_in_pool(seq_K, seq_V, B, NB, perm, H, D, fill=np.nan):
    """Put each sequence's contiguous K/V ([Hkv][n][D]) into a float32 pool via
    explicit loops; block tables come from ``perm``. Returns pools, table."""
    k_pool = np.full((NB, H, B, D), fill, dtype=np.float32)
    v_pool = np.full((NB, H, D, B), fill, dtype=np.float32)
    nblk = [-(-K.shape[1] // B) for K in seq_K]
    stride = max(nblk)
    table = np.zeros((len(seq_K), stride), dtype=np.int32)
    nxt = 0
    for s, (K, V) in enumerate(zip(seq_K, seq_V)):
        for lb in range(nblk[s]):
            table[s, lb] = perm[nxt]
            nxt += 1
        for j in range(K.shape[1]):
            pb = table[s, j // B]
            for h in range(H):
                for d in range(D):
                    k_pool[pb, h, j % B, d] = K[h, j, d]
                    v_pool[pb, h, d, j % B] = V[h, j, d]
    return k_pool, v_pool, table


@pytest.mark.parametrize("Hq,Hkv,D,window,q_lens,ctxs", [
    (4, 2, 4, 0, [1, 1, 1], [1, 5, 17]),
    (4, 1, 3, 0, [3, 1], [20, 33]),
    (2, 2, 5, 4, [5, 1], [9, 12]),
    (8, 2, 2, 7, [6, 2, 1], [6, 30, 16]),
    (3, 3, 4, 1, [2, 1], [4, 3]),
])
def test_oracle_matches_brute_force(Hq, Hkv, D, window, q_lens, ctxs):
    rng = np.random.default_rng(42 + Hq + D + window)
    B = 4
    G = Hq // Hkv
    seq_K = [rng.normal(size=(Hkv, c, D)).astype(np.float32) for c in ctxs]
    seq_V = [rng.normal(size=(Hkv, c, D)).astype(np.float32) for c in ctxs]
    NB = sum(-(-c // B) for c in ctxs) + 3
    perm = rng.permutation(NB)
    k_pool, v_pool, table = place_in_pool(seq_K, seq_V, B, NB, perm, Hkv, D)
    cu = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    q = rng.normal(size=(int(cu[-1]), Hq, D)).astype(np.float32)
    scale = 1.0 / math.sqrt(D)
    got = oracle.paged_attention(q, F.F32, k_pool, v_pool, F.F32, None, None, table, cu,
                                 np.array(ctxs, np.int32), Hkv, scale, window, B)
    for s, (ql, c) in enumerate(zip(q_lens, ctxs)):
        for h in range(Hq):
            g = h // G  # grouped-query reading: contiguous groups
            qrows = [[float(x) for x in q[cu[s] + r, h]] for r in range(ql)]
            Krows = [[float(x) for x in seq_K[s][g, j]] for j in range(c)]
            Vrows = [[float(x) for x in seq_V[s][g, j]] for j in range(c)]
            ref = brute_attention(qrows, Krows, Vrows, scale, list(range(c - ql, c)), window)
            np.testing.assert_allclose(got[cu[s]:cu[s + 1], h, :], np.array(ref), rtol=0, atol=1e-12)


@pytest.mark.parametrize("window", [0, 40])
def test_sampled_rows_and_heads_match_brute_force(window):
    """attend_sequence(rows=, heads=) evaluates only the listed query rows and
    heads (more than 256 rows: evaluated in bounded batches) and each equals
    the pure-Python brute force; the rest stays NaN."""
    rng = np.random.default_rng(7 + window)
    B, Hq, Hkv, D, ctx, ql = 4, 4, 2, 3, 320, 300
    K = [rng.normal(size=(Hkv, ctx, D)).astype(np.float32)]
    V = [rng.normal(size=(Hkv, ctx, D)).astype(np.float32)]
    NB = -(-ctx // B) + 2
    k_pool, v_pool, table = place_in_pool(K, V, B, NB, rng.permutation(NB), Hkv, D)
    q = rng.normal(size=(ql, Hq, D)).astype(np.float64)
    rows, heads = [299, 0, 7, 255, 256, 257], [1, 2]
    scale = 0.5
    got = oracle.attend_sequence(q, k_pool, v_pool, F.F32, None, None, table[0], ctx, Hkv, scale, window, B,
                                 heads=heads, rows=rows)
    for h in range(Hq):
        for r in range(ql):
            if h not in heads or r not in rows:
                assert np.isnan(got[r, h]).all()
                continue
            g = h // (Hq // Hkv)
            ref = brute_attention([[float(x) for x in q[r, h]]], [[float(x) for x in K[0][g, j]] for j in range(ctx)],
                                  [[float(x) for x in V[0][g, j]] for j in range(ctx)], scale, [ctx - ql + r], window)
            np.testing.assert_allclose(got[r, h], np.array(ref[0]), rtol=0, atol=1e-12)


def test_weighted_average_example(golden):
    g = golden("weighted_average_merge.json")
    wa, wb = g["worker_a"], g["worker_b"]
    # each worker's own sums as printed
    assert sum(w * v for w, v in zip(wa["weights"], wa["values"])) == wa["weighted_sum"]
    assert sum(wb["weights"]) == wb["weight_sum"]
    weights = wa["weights"] + wb["weights"]
    values = wa["values"] + wb["values"]
    scores = np.log(np.array(weights, dtype=np.float64))
    # (1) as attention: d = 1, q = 1, K_j = ln(w_j), V_j = value_j, scale 1
    n = len(weights)
    k_pool = np.zeros((1, 1, n, 1), np.float64).astype(np.float32)
    v_pool = np.zeros((1, 1, 1, n), np.float32)
    k_pool[0, 0, :, 0] = scores
    v_pool[0, 0, 0, :] = values
    out = oracle.attend_sequence(np.ones((1, 1, 1)), k_pool, v_pool, F.F32, None, None, [0], n, 1, 1.0,
                                 0, block_size=n)
    assert out[0, 0, 0] == pytest.approx(g["expected_output"], abs=1e-6)  # K stored as float32
    # (2) through per-worker summaries merged by the correction factor
    pa = oracle.partial_softmax(scores[:2], np.array(values[:2], np.float64)[:, None])
    pb = oracle.partial_softmax(scores[2:], np.array(values[2:], np.float64)[:, None])
    # the summaries are the page's sums, scaled by e^(-local max)
    assert pa[1] * math.exp(pa[0]) == pytest.approx(wa["weight_sum"], rel=1e-12)
    assert pa[2][0] * math.exp(pa[0]) == pytest.approx(wa["weighted_sum"], rel=1e-12)
    assert pb[2][0] * math.exp(pb[0]) == pytest.approx(wb["weighted_sum"], rel=1e-12)
    merged = oracle.merge_partials([pa, pb])
    assert merged[0] == pytest.approx(g["expected_output"], rel=1e-14)
    # any split of the four positions merges to the same value
    for cut in (1, 3):
        parts = [oracle.partial_softmax(scores[:cut], np.array(values[:cut], np.float64)[:, None]),
                 oracle.partial_softmax(scores[cut:], np.array(values[cut:], np.float64)[:, None])]
        assert oracle.merge_partials(parts)[0] == pytest.approx(29.0, rel=1e-14)


def _random_setup(rng, ctxs, Hq=4, Hkv=2, D=8, B=16, extra_blocks=2):
    seq_K = [rng.normal(size=(Hkv, c, D)).astype(np.float32) for c in ctxs]
    seq_V = [rng.normal(size=(Hkv, c, D)).astype(np.float32) for c in ctxs]
    NB = sum(-(-c // B) for c in ctxs) + extra_blocks
    return seq_K, seq_V, NB


def test_single_key_returns_v0_exactly():
    rng = np.random.default_rng(1)
    seq_K, seq_V, NB = _random_setup(rng, [1])
    k_pool, v_pool, table = place_in_pool(seq_K, seq_V, 16, NB, np.arange(NB), 2, 8)
    q = rng.normal(size=(1, 4, 8)).astype(np.float32)
    out = oracle.paged_attention(q, F.F32, k_pool, v_pool, F.F32, None, None, table, [0, 1], [1], 2, 0.3)
    for h in range(4):
        assert (out[0, h] == seq_V[0][h // 2, 0].astype(np.float64)).all()


def test_equal_scores_give_mean():
    rng = np.random.default_rng(2)
    c = 37
    seq_K = [np.ones((1, c, 4), np.float32)]
    seq_V = [rng.normal(size=(1, c, 4)).astype(np.float32)]
    k_pool, v_pool, table = place_in_pool(seq_K, seq_V, 16, 5, np.arange(5), 1, 4)
    q = np.full((1, 1, 4), 0.5, np.float32)
    out = oracle.paged_attention(q, F.F32, k_pool, v_pool, F.F32, None, None, table, [0, 1], [c], 1, 1.0)
    np.testing.assert_allclose(out[0, 0], seq_V[0][0].astype(np.float64).mean(axis=0), rtol=0, atol=1e-14)


def test_decode_step_key_counts(golden):
    g = golden("capacity_facts.json")["decode_step_keys"]
    rng = np.random.default_rng(5)
    for step, seen in enumerate(g["keys_seen_by_step"], start=1):
        ctx = g["prompt_tokens"] + step - 1
        assert ctx == seen
        # equal scores: the output is the mean over exactly the keys seen
        V = rng.normal(size=(1, ctx, 2)).astype(np.float32)
        k_pool, v_pool, table = place_in_pool([np.zeros((1, ctx, 2), np.float32)], [V], 16, 2,
                                              np.arange(2), 1, 2)
        out = oracle.paged_attention(np.zeros((1, 1, 2), np.float32), F.F32, k_pool, v_pool, F.F32,
                                     None, None, table, [0, 1], [ctx], 1, 1.0)
        np.testing.assert_allclose(out[0, 0], V[0].astype(np.float64).mean(axis=0), atol=1e-14)


def test_block_permutation_invariance():
    rng = np.random.default_rng(3)
    ctxs = [50, 17, 100]
    seq_K, seq_V, NB = _random_setup(rng, ctxs, extra_blocks=5)
    q = rng.normal(size=(3, 4, 8)).astype(np.float32)
    outs = []
    for seed in range(3):
        perm = np.random.default_rng(100 + seed).permutation(NB)
        k_pool, v_pool, table = place_in_pool(seq_K, seq_V, 16, NB, perm, 2, 8)
        outs.append(oracle.paged_attention(q, F.F32, k_pool, v_pool, F.F32, None, None, table,
                                           [0, 1, 2, 3], ctxs, 2, 0.35))
    assert (outs[0] == outs[1]).all() and (outs[0] == outs[2]).all()


def test_shared_prefix_equals_copied_prefix():
    """Four sequences whose first full blocks point at the same physical blocks
    give the same result as four sequences with private copies."""
    rng = np.random.default_rng(4)
    B, H, D = 16, 2, 8
    prefix = 64  # 4 full blocks shared
    tails = [5, 16, 1, 30]
    Kp = rng.normal(size=(H, prefix, D)).astype(np.float32)
    Vp = rng.normal(size=(H, prefix, D)).astype(np.float32)
    seq_K = [np.concatenate([Kp, rng.normal(size=(H, t, D)).astype(np.float32)], axis=1) for t in tails]
    seq_V = [np.concatenate([Vp, rng.normal(size=(H, t, D)).astype(np.float32)], axis=1) for t in tails]
    ctxs = [prefix + t for t in tails]
    q = rng.normal(size=(4, 4, D)).astype(np.float32)
    NB = 40
    k_copy, v_copy, t_copy = place_in_pool(seq_K, seq_V, B, NB, rng.permutation(NB), H, D)
    copied = oracle.paged_attention(q, F.F32, k_copy, v_copy, F.F32, None, None, t_copy,
                                    [0, 1, 2, 3, 4], ctxs, H, 0.3)
    # shared: move sequences 1..3's prefix blocks onto sequence 0's blocks and
    # poison the now-unused copies
    t_shared = t_copy.copy()
    for s in (1, 2, 3):
        for lb in range(prefix // B):
            k_copy[t_shared[s, lb]] = np.nan
            v_copy[t_shared[s, lb]] = np.nan
            t_shared[s, lb] = t_copy[0, lb]
    shared = oracle.paged_attention(q, F.F32, k_copy, v_copy, F.F32, None, None, t_shared,
                                    [0, 1, 2, 3, 4], ctxs, H, 0.3)
    assert (shared == copied).all()


def test_chunking_changes_nothing():
    """Prefill of a prompt in one chunk vs several chunks: every token's output
    is the same (chunking only changes scheduling)."""
    rng = np.random.default_rng(6)
    c = 45
    seq_K, seq_V, NB = _random_setup(rng, [c])
    k_pool, v_pool, table = place_in_pool(seq_K, seq_V, 16, NB, rng.permutation(NB), 2, 8)
    q = rng.normal(size=(c, 4, 8)).astype(np.float32)
    whole = oracle.paged_attention(q, F.F32, k_pool, v_pool, F.F32, None, None, table, [0, c], [c], 2, 0.4)
    pieces = []
    done = 0
    for chunk in (16, 3, 20, 6):
        done += chunk
        pieces.append(oracle.paged_attention(q[done - chunk:done], F.F32, k_pool, v_pool, F.F32, None,
                                             None, table, [0, chunk], [done], 2, 0.4))
    np.testing.assert_allclose(np.concatenate(pieces), whole, rtol=0, atol=1e-14)


def test_window_at_least_context_is_full_attention():
    rng = np.random.default_rng(8)
    ctxs = [20, 33]
    seq_K, seq_V, NB = _random_setup(rng, ctxs)
    k_pool, v_pool, table = place_in_pool(seq_K, seq_V, 16, NB, rng.permutation(NB), 2, 8)
    q = rng.normal(size=(4, 4, 8)).astype(np.float32)
    cu = [0, 3, 4]
    full = oracle.paged_attention(q, F.F32, k_pool, v_pool, F.F32, None, None, table, cu, ctxs, 2, 0.3, 0)
    win = oracle.paged_attention(q, F.F32, k_pool, v_pool, F.F32, None, None, table, cu, ctxs, 2, 0.3, 33)
    assert (full == win).all()
    narrow = oracle.paged_attention(q, F.F32, k_pool, v_pool, F.F32, None, None, table, cu, ctxs, 2, 0.3, 1)
    # W = 1: each query sees only itself, so the output is its own V row
    for r, p in zip(range(3), range(17, 20)):
        for h in range(4):
            assert (narrow[r, h] == seq_V[0][h // 2, p].astype(np.float64)).all()


def test_fp8_gather_applies_block_scales():
    rng = np.random.default_rng(9)
    NB, H, B, D = 3, 1, 16, 4
    k_pool = rng.integers(0, 0x7E, (NB, H, B, D)).astype(np.uint8)
    v_pool = rng.integers(0, 0x7E, (NB, H, D, B)).astype(np.uint8)
    ks = np.float32([0.5, 3.0, 0.0078125])
    vs = np.float32([2.0, 0.25, 10.0])
    table = [2, 0, 1]
    pos = np.arange(40)
    K, V = oracle.gather_kv(k_pool, v_pool, F.FP8, ks, vs, table, 0, pos, B)
    for j in pos:
        pb = table[j // B]
        assert (K[j] == F.e4m3fn_bits_to_f64(k_pool[pb, 0, j % B]) * np.float64(ks[pb])).all()
        assert (V[j] == F.e4m3fn_bits_to_f64(v_pool[pb, 0, :, j % B]) * np.float64(vs[pb])).all()
