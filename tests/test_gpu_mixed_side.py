"""GPU parity of mixed batches whose one-token rows run beside the prefill.

pa_prefill_chunk decodes the one-token rows of a batch that also holds
longer chunks on a second stream, next to the prefill kernel, when the
shapes allow it (bf16 queries, bf16 or fp8 e4m3 cache, head size 128, 1, 2,
4 or 8 query heads per KV head, contexts long enough for the split plan, LDS
for the sequence count):
"从静态批处理到状态化推理集群", "Chunked prefill：在共置引擎里治理阶段干扰" (a
step mixes decode rows and prefill chunks). Every row is compared with the
oracle at the usual bar; the split plan the side kernel leaves in the
workspace (its chunk size, for the merge) shows that it ran.
"""

import numpy as np
import pytest
import torch

from paged_kv_cache_103_amd import _lib as pa
from paged_kv_cache_103_amd import workloads as W
from tests.helpers import assert_close, oracle_rows, out_f64

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _log(msg):
    print(msg, flush=True)


def run_prefill(b):
    m = b.meta(DEV)
    out = torch.empty_like(b.query)
    n = pa.prefill_workspace_bytes(b.num_seqs, b.num_q_tokens, b.max_q_len, b.max_context_len, b.num_heads,
                                   b.num_kv_heads, b.head_size, b.cache_dtype, b.sliding_window)
    ws = torch.zeros(max(n, 4), dtype=torch.uint8, device=DEV)
    pa.prefill_chunk(out, b.query, b.k_cache, b.v_cache, m["block_table"], m["cu_seqlens"], m["context_lens"],
                     b.max_q_len, b.max_context_len, b.scale, b.k_scale, b.v_scale, b.sliding_window, ws)
    return out, ws


def split_chunk(b, waves):
    """Blocks per wave of the even split over `waves` waves (at least 8, even)
    for the batch's one-token rows: the plan the decode kernels share."""
    total = 0
    for s in range(b.num_seqs):
        if b.q_lens[s] != 1:
            continue
        ctx = int(b.context_lens[s])
        lo = max(0, ctx - b.sliding_window) if b.sliding_window > 0 else 0
        total += ((ctx - 1) >> 4) - (lo >> 4) + 1
    total *= b.num_kv_heads
    c = max((total + waves - 1) // waves, 8)
    return (c + 1) & ~1


def check_all(b, out, what, atol=2e-3, seqs=None):
    seqs = range(b.num_seqs) if seqs is None else seqs
    ref = oracle_rows(b, seqs)
    got = out_f64(out)
    cu = b.cu_seqlens
    worst = (0.0, 0.0)
    for s in seqs:
        ma, mr = assert_close(got[cu[s]:cu[s + 1]], ref[s], f"{what} seq {s}", atol=atol)
        worst = (max(worst[0], ma), max(worst[1], mr))
    _log(f"{what}: {len(seqs)} sequences, max abs {worst[0]:.2e}, max rel {worst[1]:.2e}")


CASES = [
    # (contexts, query lengths, sliding window): partial last blocks, one-block
    # rows, streams split over several waves, chunks of 1..3 tiles
    ([17, 300, 1000, 4097, 20000, 2100, 31000, 16], [1, 1, 1, 1, 1, 100, 1, 1], 0),
    ([5000, 12345, 700, 3000, 64, 8191, 24001], [1, 1, 1, 37, 1, 1, 1], 1000),   # window start mid-block
    ([9000, 16, 33, 2049, 18000, 6000], [1, 1, 1, 512, 1, 1], 0),
]


# (case, query heads, KV heads, cache dtype): the group sizes and cache types
# the side kernel serves
SHAPES = [(0, 32, 8, "bf16"), (1, 32, 8, "bf16"), (2, 32, 8, "bf16"), (0, 32, 8, "fp8_e4m3"),
          (1, 32, 8, "fp8_e4m3"), (2, 16, 8, "bf16"), (0, 8, 8, "fp8_e4m3"), (1, 16, 16, "bf16"),
          (2, 16, 8, "fp8_e4m3"), (0, 64, 8, "fp8_e4m3"), (1, 64, 8, "bf16")]


@pytest.mark.parametrize("case,hq,hkv,cache", SHAPES)
def test_mixed_batch_rows_beside_prefill(case, hq, hkv, cache):
    ctx, ql, win = CASES[case]
    b = W.make_batch(f"side{case}_{hq}_{hkv}_{cache}", 980 + case + hq + 7 * hkv, ctx, ql, hq, hkv, 128, "bf16", cache,
                     sliding_window=win, device=DEV, extra_blocks=2)
    out, ws = run_prefill(b)
    torch.cuda.synchronize()
    check_all(b, out, f"mixed batch {case} ({hq}/{hkv} heads, {cache}, window {win})")
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    c = int(ws[:4].view(torch.int32).item())
    # the side kernel splits over 4 waves per CU, the stand-alone decode over
    # 8 (the two plans differ unless both hit the 8-block minimum)
    assert c == split_chunk(b, 4 * cus), (c, split_chunk(b, 4 * cus), split_chunk(b, 8 * cus))
    if split_chunk(b, 4 * cus) != split_chunk(b, 8 * cus):
        assert c != split_chunk(b, 8 * cus)
    _log(f"mixed batch {case}: rows decoded beside the prefill (chunk {c} blocks per wave)")


def test_mixed_batch_large_values_beside_prefill():
    """bf16 values times 2^100 on a batch that takes the side path: the side
    kernel's value product is bf16 x (bf16 hi + lo) in fp32, exact in range."""
    ctx, ql = [3000, 17000, 900, 12000, 400], [1, 1, 200, 1, 1]
    b = W.make_batch("side_big", 990, ctx, ql, 32, 8, 128, "bf16", "bf16", device=DEV, extra_blocks=2)
    f = 2.0 ** 100
    b.v_cache.mul_(f)
    out, _ = run_prefill(b)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
    check_all(b, out, "side path, values x 2^100", atol=2e-3 * f)


def test_mixed_batch_many_rows_falls_back():
    """2000 one-token rows and a chunk: the side kernel's LDS (sequence prefix
    sums beside the ring) would not leave room for a prefill workgroup, so
    the rows take the stand-alone decode kernel first; a sample of rows."""
    rng = np.random.default_rng(991)
    n = 2000
    ctx = [int(x) for x in rng.integers(257, 700, size=n)] + [1500]
    ql = [1] * n + [300]
    b = W.make_batch("side_many", 991, ctx, ql, 32, 8, 128, "bf16", "bf16", device=DEV, extra_blocks=2)
    out, ws = run_prefill(b)
    torch.cuda.synchronize()
    check_all(b, out, "2000 rows + chunk", seqs=list(range(0, n, 97)) + [n - 1, n])
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert int(ws[:4].view(torch.int32).item()) == split_chunk(b, 8 * cus)
