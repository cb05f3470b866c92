"""GPU parity of the sparse decode (pa_decode_sparse) against the oracle.

Every logical block a sequence did not choose points at one shared block of
NaN, so reading any of them shows in the output. Cases: ragged contexts
(1 token to several thousand), GQA groups 1..16, d 64/128, bf16 and fp8
caches, lists with repeats, out-of-range ids, the newest block itself, and a
tail past num_selected naming unchosen blocks; the empty choice; every
block chosen (bitwise equal to pa_decode); batches of many streams, which
one launch serves; and the benchmark's long-context batch on sampled
sequences.
"""

import numpy as np
import pytest
import torch

import oracle
from paged_kv_cache_103_amd import _lib as pa
from paged_kv_cache_103_amd import workloads as W
from tests.helpers import ORACLE_DTYPE, assert_close, out_f64, raw

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _log(msg):
    print(msg, flush=True)


def run_sparse(b, choice, max_ctx=None, out=None):
    m = b.meta(DEV)
    c = choice.device(DEV)
    out = torch.empty_like(b.query) if out is None else out
    ms = choice.selected.shape[1]
    ws = torch.empty(max(pa.decode_sparse_workspace_bytes(b.num_seqs, ms, b.num_heads, b.num_kv_heads, b.head_size,
                                                          b.cache_dtype), 1), dtype=torch.uint8, device=DEV)
    pa.decode_sparse(out, b.query, b.k_cache, b.v_cache, m["block_table"], m["context_lens"],
                     b.max_context_len if max_ctx is None else max_ctx, c["selected"], c["num_selected"], b.scale,
                     b.k_scale, b.v_scale, ws)
    return out


def oracle_sparse_rows(b, choice, seqs):
    """Oracle rows of ``seqs``: only the blocks each one reads are copied."""
    q = raw(b.query)
    dt = ORACLE_DTYPE[b.cache_dtype]
    qd = ORACLE_DTYPE[b.q_dtype]
    res = {}
    for s in seqs:
        ctx = int(b.context_lens[s])
        nbk = -(-ctx // 16)
        blks = choice.chosen[s]
        phys = torch.tensor([int(b.block_table[s, x]) for x in blks], dtype=torch.int64, device=DEV)
        kp, vp = raw(b.k_cache.index_select(0, phys)), raw(b.v_cache.index_select(0, phys))
        ks = vs = None
        if b.k_scale is not None:
            ks, vs = raw(b.k_scale.index_select(0, phys)), raw(b.v_scale.index_select(0, phys))
        row = np.zeros(nbk, dtype=np.int64)
        row[blks] = np.arange(len(blks))
        n = int(choice.num_selected[s])
        qf = oracle.formats.to_f64(q[s:s + 1], qd)
        res[s] = oracle.attend_selected_blocks(qf, kp, vp, dt, ks, vs, row, ctx, choice.selected[s, :n],
                                               b.num_kv_heads, b.scale)
    return res


def check(b, choice, out, seqs, what):
    ref = oracle_sparse_rows(b, choice, seqs)
    got = out_f64(out)
    worst = (0.0, 0.0)
    for s in seqs:
        ma, mr = assert_close(got[s:s + 1], ref[s], f"{what} seq {s}")
        worst = (max(worst[0], ma), max(worst[1], mr))
    _log(f"{what}: {len(seqs)} sequences, max abs {worst[0]:.2e}, max rel {worst[1]:.2e}")


CASES = [
    # (ctx lens, k blocks, Hq, Hkv, D, cache dtype)
    ([1, 16, 17, 33, 300, 1000, 4097], 8, 32, 8, 128, "bf16"),
    ([5000, 2500, 17, 40], 64, 16, 16, 64, "bf16"),     # G = 1
    ([3000, 700, 129], 20, 64, 4, 128, "bf16"),         # G = 16
    ([2048, 999, 16, 65], 5, 16, 2, 64, "fp8_e4m3"),
    ([6000, 1], 300, 32, 8, 128, "fp8_e4m3"),           # k beyond a short context
    ([160, 161, 175, 176, 177], 1, 8, 1, 128, "bf16"),  # G = 8
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_sparse_small(case):
    ctx, k, Hq, Hkv, D, cd = CASES[case]
    _log(f"sparse case {case}: ctx {ctx}, k {k}, {Hq}/{Hkv} d{D} {cd}")
    b, choice = W.make_sparse_batch(f"sparse{case}", 700 + case, ctx, k, Hq, Hkv, D, "bf16", cd, device=DEV,
                                    noise=True)
    out = run_sparse(b, choice)
    torch.cuda.synchronize()
    check(b, choice, out, range(b.num_seqs), f"sparse case {case}")


def test_sparse_empty_choice_reads_the_newest_block_only():
    b, choice = W.make_sparse_batch("sparse_empty", 730, [40, 17, 1, 1000], 0, 16, 4, 128, device=DEV)
    assert choice.selected.shape[1] == 1 and (choice.num_selected == 0).all()
    out = run_sparse(b, choice)
    torch.cuda.synchronize()
    check(b, choice, out, range(b.num_seqs), "sparse empty choice")


def test_sparse_every_block_is_dense_decode_bitwise():
    """Choosing every block compacts to the same table and context: the same
    kernels on the same streams, so the same bits as pa_decode."""
    b = W.make_batch("sparse_all", 731, [1, 100, 2049, 7000, 333], [1] * 5, 32, 8, 128, "bf16", "bf16",
                     device=DEV, extra_blocks=5)
    nbk = [-(-int(c) // 16) for c in b.context_lens]
    width = max(nbk)
    sel = np.full((b.num_seqs, width), -1, dtype=np.int32)
    for s, n in enumerate(nbk):
        sel[s, :n] = np.random.default_rng(s).permutation(n)
    choice = W.SparseChoice(sel, np.asarray(nbk, dtype=np.int32), [list(range(n)) for n in nbk])
    out = run_sparse(b, choice)
    m = b.meta(DEV)
    dense = torch.empty_like(b.query)
    ws = torch.empty(max(pa.decode_workspace_bytes(b.num_seqs, b.max_context_len, 32, 8, 128), 1), dtype=torch.uint8,
                     device=DEV)
    pa.decode(dense, b.query, b.k_cache, b.v_cache, m["block_table"], m["context_lens"], b.max_context_len, b.scale,
              workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), dense.view(torch.int16))
    check(b, choice, out, [0, 3], "sparse every block")


FUSED_CASES = [
    # (sequences, context range, k blocks, Hq, Hkv, D, cache dtype): at least
    # two (sequence, KV head) streams per CU, so one launch serves the call
    (64, (1, 6000), 40, 32, 8, 128, "bf16"),
    (128, (1, 3000), 25, 8, 4, 64, "fp8_e4m3"),
    (512, (1, 1200), 10, 16, 1, 128, "bf16"),         # G = 16
    (256, (100, 4000), 60, 16, 2, 128, "fp8_e4m3"),   # G = 8
    (600, (1, 400), 3, 1, 1, 64, "bf16"),             # G = 1, ragged grid
    (64, (20000, 40000), 300, 32, 8, 128, "bf16"),    # long lists (parts of ~80 blocks)
    (512, (1, 3000), 0, 8, 1, 128, "bf16"),           # nothing chosen: the newest block (and noise) only
]


@pytest.mark.parametrize("case", range(len(FUSED_CASES)))
def test_sparse_one_launch(case):
    """Batches with many streams take the one-launch kernel (selection,
    decode and merge in a workgroup per stream), which leaves the workspace
    untouched: checked, then every sequence against the oracle."""
    S, (c0, c1), k, Hq, Hkv, D, cd = FUSED_CASES[case]
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    if S * Hkv < 2 * cus:
        pytest.skip(f"{S * Hkv} streams are fewer than two per CU on this device ({cus} CUs)")
    rng = np.random.default_rng(2600 + case)
    ctx = rng.integers(c0, c1 + 1, S).tolist()
    _log(f"sparse one-launch case {case}: {S} seqs, ctx {c0}..{c1}, k {k}, {Hq}/{Hkv} d{D} {cd}")
    b, choice = W.make_sparse_batch(f"sparse_fused{case}", 2600 + case, ctx, k, Hq, Hkv, D, "bf16", cd, device=DEV,
                                    noise=True)
    m = b.meta(DEV)
    c = choice.device(DEV)
    ms = choice.selected.shape[1]
    ws = torch.full((pa.decode_sparse_workspace_bytes(S, ms, Hq, Hkv, D, b.cache_dtype),), 0xA5, dtype=torch.uint8,
                    device=DEV)
    out = torch.empty_like(b.query)
    pa.decode_sparse(out, b.query, b.k_cache, b.v_cache, m["block_table"], m["context_lens"], b.max_context_len,
                     c["selected"], c["num_selected"], b.scale, b.k_scale, b.v_scale, ws)
    torch.cuda.synchronize()
    assert bool((ws == 0xA5).all()), "the one-launch path writes no workspace"
    check(b, choice, out, range(S), f"sparse one-launch case {case}")


def test_sparse_many_streams_long_lists_take_three_launches():
    """Lists of 1024 entries or more are not served in one launch even with
    many streams: the selection kernel writes its tables to the workspace
    (checked) and the result still matches the oracle."""
    S = 64
    rng = np.random.default_rng(2700)
    ctx = rng.integers(20000, 30000, S).tolist()
    b, choice = W.make_sparse_batch("sparse_long_lists", 2700, ctx, 1100, 32, 8, 128, "bf16", "bf16", device=DEV,
                                    noise=True)
    ms = choice.selected.shape[1]
    assert ms >= 1024
    _log(f"sparse long lists: {S} seqs, max_selected {ms}")
    m = b.meta(DEV)
    c = choice.device(DEV)
    ws = torch.full((pa.decode_sparse_workspace_bytes(S, ms, 32, 8, 128, b.cache_dtype),), 0xA5, dtype=torch.uint8,
                    device=DEV)
    out = torch.empty_like(b.query)
    pa.decode_sparse(out, b.query, b.k_cache, b.v_cache, m["block_table"], m["context_lens"], b.max_context_len,
                     c["selected"], c["num_selected"], b.scale, b.k_scale, b.v_scale, ws)
    torch.cuda.synchronize()
    assert not bool((ws == 0xA5).all()), "the three-launch path keeps its tables in the workspace"
    check(b, choice, out, [0, 21, 42, 63], "sparse long lists")


def test_sparse_more_than_16000_sequences_three_launches():
    """16,100 sequences whose lists are padded to 1030 entries (so the
    three-launch path serves them): the selection covers every sequence and
    the decode over the compacted tables runs as groups of 16000."""
    S = 16100
    rng = np.random.default_rng(2800)
    ctx = rng.integers(1, 300, S).tolist()
    b, choice = W.make_sparse_batch("sparse_16100", 2800, ctx, 3, 8, 2, 64, "bf16", "bf16", device=DEV, noise=True)
    sel = np.full((S, 1030), -1, dtype=np.int32)
    sel[:, :choice.selected.shape[1]] = choice.selected
    choice = W.SparseChoice(sel, choice.num_selected, choice.chosen)
    _log(f"sparse {S} sequences, lists padded to 1030 entries")
    out = run_sparse(b, choice)
    torch.cuda.synchronize()
    check(b, choice, out, [0, 1, 15999, 16000, 16099], f"sparse {S} sequences")


def test_sparse_long_context_sampled():
    """The benchmark's batch: 64 sequences, contexts U{32768..524288}, 128
    chosen blocks each, 32/8 heads, d 128, bf16."""
    b, choice = W.make_sparse_config(device=DEV)
    out = run_sparse(b, choice)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
    check(b, choice, out, [0, 17, 40, 63], "sparse long context")


def test_sparse_random_shapes():
    """Seeded random sparse batches: head size, group size, KV heads, cache
    dtype, contexts and the number of chosen blocks (also beyond a short
    context's earlier blocks)."""
    rng = np.random.default_rng(1400)
    for it in range(24):
        D = int(rng.choice([64, 128]))
        G = int(rng.choice([1, 2, 4, 8, 16]))
        Hkv = int(rng.choice([1, 2, 4, 8]))
        cd = str(rng.choice(["bf16", "bf16", "fp8_e4m3"]))
        S = int(rng.integers(1, 7))
        ctx = rng.integers(1, 8000, S).tolist()
        k = int(rng.integers(0, 300))
        _log(f"sparse random {it}: ctx {ctx}, k {k}, {G * Hkv}/{Hkv} d{D} {cd}")
        b, choice = W.make_sparse_batch(f"sparse_rand{it}", 1500 + it, ctx, k, G * Hkv, Hkv, D, "bf16", cd,
                                        device=DEV, noise=True)
        out = run_sparse(b, choice)
        torch.cuda.synchronize()
        check(b, choice, out, range(S), f"sparse random {it}")
