"""Pins for the oracle's latent-cache (MLA) decode (CPU only).

* the pages' byte comparison: 8 heads x 16-dim keys over 1000 positions move
  256,000 bytes, one shared 32-dim c moves 64,000 (4x less);
* matrix absorption: attention of raw queries over per-head keys and values
  expanded from c (K_h = W_k,h c, V_h = W_v,h c) equals the latent decode of
  the absorbed queries W_k,h^T q_h with W_v,h applied to its output, to 1e-12;
* with dk = dv it is the paged GQA oracle with one KV head whose K and V are
  both c;
* pure-Python brute force with a positional part (dk > dv).
"""

import math

import numpy as np
import pytest

import oracle
from oracle import formats as F
from oracle import mla


def _pool(rng, ctx, dk, nb_extra=2, fill=np.nan):
    nb = -(-ctx // 16) + nb_extra
    perm = rng.permutation(nb)
    pool = np.full((nb, 16, dk), fill, dtype=np.float32)
    C = rng.normal(size=(ctx, dk)).astype(np.float32)
    row = perm[: -(-ctx // 16)]
    for j in range(ctx):
        pool[row[j // 16], j % 16] = C[j]
    return pool, row, C


def test_byte_comparison_example(golden):
    g = golden("mla_bytes_example.json")
    a = mla.per_head_key_bytes(g["heads"], g["head_dim"], g["positions"], g["dtype_bytes"])
    b = mla.mla_cache_bytes(g["positions"], g["latent_dim"], g["dtype_bytes"])
    assert a == g["expected_per_head_key_bytes"] and b == g["expected_latent_bytes"]
    assert a // b == g["expected_ratio"]


@pytest.mark.parametrize("ctx,H,dh,L", [(1, 2, 3, 5), (37, 4, 8, 16), (100, 3, 4, 12)])
def test_matrix_absorption(ctx, H, dh, L):
    rng = np.random.default_rng(ctx + H)
    pool, row, C = _pool(rng, ctx, L)
    Wk = rng.normal(size=(H, dh, L))
    Wv = rng.normal(size=(H, dh, L))
    q = rng.normal(size=(H, dh))
    scale = 1 / math.sqrt(dh)
    Cf = C.astype(np.float64)
    # standard attention with every head's K and V expanded from c
    ref = np.zeros((H, dh))
    for h in range(H):
        K = Cf @ Wk[h].T          # [ctx][dh]
        V = Cf @ Wv[h].T
        s = scale * (K @ q[h])
        p = np.exp(s - s.max())
        ref[h] = p @ V / p.sum()
    # latent decode of the absorbed queries, then each head's value projection
    qa = np.stack([Wk[h].T @ q[h] for h in range(H)])      # [H][L]
    lat = mla.mla_decode_sequence(qa, pool, F.F32, row, ctx, scale, L)
    got = np.stack([Wv[h] @ lat[h] for h in range(H)])
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_equals_gqa_oracle_with_one_kv_head():
    rng = np.random.default_rng(9)
    ctx, H, D = 70, 8, 16
    pool, row, C = _pool(rng, ctx, D)
    kp = pool[:, None, :, :].copy()                       # [NB][1][16][D]
    vp = np.ascontiguousarray(pool.transpose(0, 2, 1))[:, None, :, :]  # [NB][1][D][16]
    q = rng.normal(size=(1, H, D)).astype(np.float32)
    ref = oracle.paged_attention(q, F.F32, kp, vp, F.F32, None, None, [row], [0, 1], [ctx], 1, 0.3)
    got = mla.mla_decode(q, F.F32, pool, F.F32, [row], [ctx], 0.3, D)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-13)


@pytest.mark.parametrize("ctx,H,dk,dv", [(1, 1, 6, 4), (20, 3, 10, 8), (33, 2, 7, 7)])
def test_brute_force_with_positional_part(ctx, H, dk, dv):
    rng = np.random.default_rng(ctx * 7 + dk)
    pool, row, C = _pool(rng, ctx, dk)
    q = rng.normal(size=(1, H, dk)).astype(np.float32)
    scale = 0.37
    got = mla.mla_decode(q, F.F32, pool, F.F32, [row], [ctx], scale, dv)
    for h in range(H):
        sc = [scale * sum(float(q[0, h, d]) * float(C[j, d]) for d in range(dk)) for j in range(ctx)]
        mx = max(sc)
        w = [math.exp(x - mx) for x in sc]
        ref = [sum(w[j] * float(C[j, d]) for j in range(ctx)) / sum(w) for d in range(dv)]
        np.testing.assert_allclose(got[0, h], ref, rtol=0, atol=1e-12)
