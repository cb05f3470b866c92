"""Pins for the oracle's context-parallel pieces (CPU only): a range's
normalised result (o, lse) and the merge of several ranges.

* the pages' worked example in this form: worker A hands over (70/4, ln 4),
  worker B (220/6, ln 6), and the merge gives 29;
* closed forms: one key gives lse = its score, n equal scores s give
  s + ln n; an empty range (lse = -inf) weighs nothing;
* any split of a sequence's keys into contiguous ranges, empty ones
  included, merges to the dense oracle's result to 1e-12.
"""

import math

import numpy as np
import pytest

import oracle
from oracle import formats as F


def test_weighted_average_example_in_normalized_form(golden):
    g = golden("weighted_average_merge.json")
    parts = []
    for w in (g["worker_a"], g["worker_b"]):
        scores = np.log(np.array(w["weights"], dtype=np.float64))
        o, lse = oracle.normalized_partial(scores, np.array(w["values"], np.float64)[:, None])
        assert o[0] == pytest.approx(w["weighted_sum"] / w["weight_sum"], rel=1e-14)
        assert lse == pytest.approx(math.log(w["weight_sum"]), rel=1e-14)
        parts.append((o, lse))
    assert oracle.merge_normalized(parts)[0] == pytest.approx(g["expected_output"], rel=1e-14)
    assert oracle.merge_normalized(parts[::-1])[0] == pytest.approx(g["expected_output"], rel=1e-14)


def test_lse_closed_forms():
    o, lse = oracle.normalized_partial(np.array([0.7]), np.array([[3.0, -1.0]]))
    assert lse == 0.7 and o.tolist() == [3.0, -1.0]
    o, lse = oracle.normalized_partial(np.full(5, -2.5), np.arange(10.0).reshape(5, 2))
    assert lse == pytest.approx(-2.5 + math.log(5), rel=1e-15)
    assert o.tolist() == pytest.approx([4.0, 5.0], rel=1e-15)
    merged = oracle.merge_normalized([(np.array([1.0, 2.0]), 0.3), (np.array([7.0, 7.0]), -np.inf)])
    assert merged.tolist() == [1.0, 2.0]


@pytest.mark.parametrize("ctx,cuts", [(50, [25]), (97, [0, 30, 30, 64]), (16, [1, 2, 3]), (300, [100, 200, 299])])
def test_any_split_merges_to_dense(ctx, cuts):
    rng = np.random.default_rng(ctx)
    Hq, Hkv, D = 4, 2, 8
    G = Hq // Hkv
    K = rng.normal(size=(Hkv, ctx, D))
    V = rng.normal(size=(Hkv, ctx, D))
    q = rng.normal(size=(1, Hq, D))
    scale = 1 / math.sqrt(D)
    # dense oracle through a contiguous pool
    nb = -(-ctx // 16)
    kp = np.full((nb, Hkv, 16, D), np.nan, np.float32)
    vp = np.full((nb, Hkv, D, 16), np.nan, np.float32)
    oracle.reshape_and_cache(kp, vp, K.transpose(1, 0, 2).astype(np.float32), V.transpose(1, 0, 2).astype(np.float32),
                             np.arange(ctx), 16)
    dense = oracle.paged_attention(q.astype(np.float32), F.F32, kp, vp, F.F32, None, None, [np.arange(nb)], [0, 1],
                                   [ctx], Hkv, scale)
    Kf = F.to_f64(K.astype(np.float32), F.F32)
    Vf = F.to_f64(V.astype(np.float32), F.F32)
    qf = F.to_f64(q.astype(np.float32), F.F32)
    bounds = [0] + cuts + [ctx]
    for h in range(Hq):
        g = h // G
        parts = []
        for a, b in zip(bounds[:-1], bounds[1:]):
            if b == a:
                parts.append((np.zeros(D), -np.inf))
                continue
            parts.append(oracle.normalized_partial(scale * (Kf[g, a:b] @ qf[0, h]), Vf[g, a:b]))
        np.testing.assert_allclose(oracle.merge_normalized(parts), dense[0, h], rtol=0, atol=1e-12)
