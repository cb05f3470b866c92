"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

KV write: bit-exact over the whole pool (including slots no token names).
Attention: element-wise |gpu - oracle| <= 2e-3 + 1e-2 |oracle| (bf16/fp8
inputs, fp32 accumulation), on the named configurations at their full sizes
(all sequences where the oracle is cheap, sampled sequences otherwise) and on
small ragged batches that span several tiles and a ragged tail.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle import formats as F
from paged_kv_cache_103_amd import _lib as pa
from paged_kv_cache_103_amd import workloads as W
from tests.helpers import ORACLE_DTYPE, assert_close, oracle_rows, out_f64, raw

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _log(msg):
    print(msg, flush=True)


def run_decode(b, out=None, **kw):
    m = b.meta(DEV)
    out = torch.empty_like(b.query) if out is None else out
    ws_bytes = pa.decode_workspace_bytes(b.num_seqs, b.max_context_len, b.num_heads, b.num_kv_heads,
                                         b.head_size, b.cache_dtype, b.sliding_window)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=DEV)
    pa.decode(out, b.query, b.k_cache, b.v_cache, m["block_table"], m["context_lens"],
              b.max_context_len, b.scale, b.k_scale, b.v_scale, b.sliding_window, ws, **kw)
    return out


def run_prefill(b, out=None):
    m = b.meta(DEV)
    out = torch.empty_like(b.query) if out is None else out
    ws_bytes = pa.prefill_workspace_bytes(b.num_seqs, b.num_q_tokens, b.max_q_len, b.max_context_len,
                                          b.num_heads, b.num_kv_heads, b.head_size, b.cache_dtype, b.sliding_window)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=DEV)
    pa.prefill_chunk(out, b.query, b.k_cache, b.v_cache, m["block_table"], m["cu_seqlens"],
                     m["context_lens"], b.max_q_len, b.max_context_len, b.scale, b.k_scale, b.v_scale,
                     b.sliding_window, ws)
    return out


def check_rows(b, out, seqs, what):
    ref = oracle_rows(b, seqs)
    got = out_f64(out)
    cu = b.cu_seqlens
    worst = (0.0, 0.0)
    for s in seqs:
        ma, mr = assert_close(got[cu[s]:cu[s + 1]], ref[s], f"{what} seq {s}")
        worst = (max(worst[0], ma), max(worst[1], mr))
    _log(f"{what}: {len(seqs)} sequences, max abs {worst[0]:.2e}, max rel {worst[1]:.2e}")


@pytest.fixture(autouse=True)
def _free():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


# ----------------------------------------------------------------------------
# KV write
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("cfg", ["tiny_decode", "small_bf16", "small_prefill"])
def test_reshape_and_cache_bit_exact(cfg):
    if cfg == "small_bf16":
        b = W.make_batch(cfg, 11, [1, 16, 17, 300, 1023], [1] * 5, 16, 4, 128, "bf16", "bf16",
                         device=DEV, extra_blocks=7)
    elif cfg == "small_prefill":
        b = W.make_batch(cfg, 12, [64, 100, 33], [64, 37, 1], 8, 8, 64, "bf16", "bf16", device=DEV,
                         extra_blocks=3)
    else:
        b = W.make_config(cfg, device=DEV)
    m = b.meta(DEV)
    # scribble over the destination slots so the write has something to change
    st = m["slot_mapping"]
    blk, off = st // 16, st % 16
    kc, vc = b.k_cache.clone(), b.v_cache.clone()
    fill = -3.0 if kc.dtype != torch.uint8 else 0x33
    kc[blk, :, off, :] = fill
    vc[blk, :, :, off] = fill
    k_host, v_host = raw(kc), raw(vc)
    pa.reshape_and_cache(b.new_key, b.new_value, kc, vc, st)
    torch.cuda.synchronize()
    oracle.reshape_and_cache(k_host, v_host, raw(b.new_key), raw(b.new_value), b.slot_mapping)
    assert np.array_equal(raw(kc).view(np.uint8), k_host.view(np.uint8))
    assert np.array_equal(raw(vc).view(np.uint8), v_host.view(np.uint8))
    # the write restores exactly what the generator put there
    assert torch.equal(kc.view(torch.uint8), b.k_cache.view(torch.uint8))
    assert torch.equal(vc.view(torch.uint8), b.v_cache.view(torch.uint8))


def test_reshape_and_cache_skips_negative_slots():
    b = W.make_batch("neg", 13, [40, 70], [20, 30], 4, 2, 64, "bf16", "bf16", device=DEV, extra_blocks=2)
    m = b.meta(DEV)
    st = m["slot_mapping"].clone()
    st[::3] = -1
    kc, vc = b.k_cache.clone(), b.v_cache.clone()
    k_host, v_host = raw(kc), raw(vc)
    key = torch.randn_like(b.new_key, dtype=torch.float32).to(torch.bfloat16)
    val = torch.randn_like(b.new_value, dtype=torch.float32).to(torch.bfloat16)
    pa.reshape_and_cache(key, val, kc, vc, st)
    torch.cuda.synchronize()
    oracle.reshape_and_cache(k_host, v_host, raw(key), raw(val), st.cpu().numpy())
    assert np.array_equal(raw(kc), k_host)
    assert np.array_equal(raw(vc), v_host)


@pytest.mark.parametrize("src", ["bf16", "f32"])
def test_reshape_and_cache_fp8_quantising_bit_exact(src):
    """Quantising write into an e4m3fn pool: every byte equals the oracle's
    round-to-nearest-even, saturating encode of x / scale[block]."""
    gen = torch.Generator(device=DEV)
    gen.manual_seed(21)
    NB, H, D, T = 40, 4, 128, 300
    kc = torch.zeros((NB, H, 16, D), dtype=torch.uint8, device=DEV)
    vc = torch.zeros((NB, H, D, 16), dtype=torch.uint8, device=DEV)
    ks = torch.rand(NB, generator=gen, device=DEV) * 0.05 + 1e-3
    vs = torch.rand(NB, generator=gen, device=DEV) * 0.05 + 1e-3
    # values spanning subnormals, normal range and saturation
    key = torch.randn((T, H, D), generator=gen, device=DEV) * torch.logspace(-4, 1.5, D, device=DEV)
    val = torch.randn((T, H, D), generator=gen, device=DEV) * torch.logspace(1.5, -4, D, device=DEV)
    key, val = key.to(getattr(torch, {"bf16": "bfloat16", "f32": "float32"}[src])), \
        val.to(getattr(torch, {"bf16": "bfloat16", "f32": "float32"}[src]))
    slots = torch.randperm(NB * 16, generator=gen, device=DEV)[:T].to(torch.int64)
    k_host, v_host = raw(kc), raw(vc)
    pa.reshape_and_cache(key, val, kc, vc, slots, ks, vs)
    torch.cuda.synchronize()
    kf = key.float().cpu().numpy()
    vf = val.float().cpu().numpy()
    oracle.reshape_and_cache_fp8(k_host, v_host, kf, vf, ks.cpu().numpy(), vs.cpu().numpy(),
                                 slots.cpu().numpy())
    gk, gv = raw(kc), raw(vc)
    # +0 / -0 are the same value; compare codes after mapping -0 to +0
    def canon(a):
        a = a.copy()
        a[a == 0x80] = 0
        return a
    assert np.array_equal(canon(gk), canon(k_host)), f"{int((canon(gk) != canon(k_host)).sum())} K bytes differ"
    assert np.array_equal(canon(gv), canon(v_host)), f"{int((canon(gv) != canon(v_host)).sum())} V bytes differ"


# ----------------------------------------------------------------------------
# decode on the named configurations
# ----------------------------------------------------------------------------
def test_decode_tiny():
    b = W.make_config("tiny_decode", device=DEV)
    out = run_decode(b)
    torch.cuda.synchronize()
    check_rows(b, out, range(b.num_seqs), "tiny_decode")


def test_decode_llama8b_full():
    b = W.make_config("llama8b_decode", device=DEV)
    out = run_decode(b)
    torch.cuda.synchronize()
    check_rows(b, out, range(b.num_seqs), "llama8b_decode")


@pytest.mark.parametrize("cd", ["bf16", "fp8_e4m3"])
def test_decode_more_than_16000_sequences(cd):
    """Beyond 16000 sequences pa_decode runs groups of 16000 on the
    matrix-core kernel, one workspace (a group's) for all: sequences on both
    sides of the group boundary and across the batch against the oracle,
    and pa_decode_partial's outputs equal to pa_decode's bit for bit."""
    S = 16500
    rng = np.random.default_rng(4200)
    ctx = rng.integers(1, 300, S).tolist()
    _log(f"decode {S} sequences, ctx 1..299, 8/2 heads d64 {cd}")
    b = W.make_batch(f"decode_{S}_{cd}", 4200, ctx, [1] * S, 8, 2, 64, "bf16", cd, device=DEV)
    one_group = pa.decode_workspace_bytes(16000, b.max_context_len, 8, 2, 64, b.cache_dtype, 0)
    assert one_group > 0  # (the split plan: some stream has more than 16 blocks)
    assert pa.decode_workspace_bytes(S, b.max_context_len, 8, 2, 64, b.cache_dtype, 0) == one_group
    out = run_decode(b)
    torch.cuda.synchronize()
    check_rows(b, out, [0, 1, 7999, 15998, 15999, 16000, 16001, 16499], f"decode {S} seqs {cd}")
    m = b.meta(DEV)
    part = torch.empty_like(b.query)
    lse = torch.empty((S, 8), dtype=torch.float32, device=DEV)
    ws = torch.empty(one_group, dtype=torch.uint8, device=DEV)
    pa.decode_partial(part, lse, b.query, b.k_cache, b.v_cache, m["block_table"], m["context_lens"],
                      b.max_context_len, b.scale, b.k_scale, b.v_scale, ws)
    torch.cuda.synchronize()
    assert torch.equal(part.view(torch.int16), out.view(torch.int16))
    assert bool(torch.isfinite(lse).all())


def test_mixed_batch_more_than_16000_rows():
    """A mixed batch of 16,099 one-token rows and a 64-token chunk: the rows
    run as groups of 16000 (addressed through cu_seqlens), the chunk on the
    prefill kernel; the workspace is what pa_prefill_workspace_bytes says."""
    S = 16100
    rng = np.random.default_rng(4300)
    ctx = rng.integers(1, 300, S).tolist()
    ctx[-1] = 500
    ql = [1] * (S - 1) + [64]
    _log(f"mixed batch: {S - 1} one-token rows + a 64-token chunk, 8/2 heads d64")
    b = W.make_batch("mixed_16100", 4300, ctx, ql, 8, 2, 64, "bf16", "bf16", device=DEV)
    out = run_prefill(b)
    torch.cuda.synchronize()
    check_rows(b, out, [0, 15999, 16000, 16098, 16099], f"mixed batch of {S} sequences")


def test_decode_agentic_sampled():
    b = W.make_config("agentic_decode", device=DEV)
    out = run_decode(b)
    torch.cuda.synchronize()
    # one member of every group (a different position in each group)
    check_rows(b, out, [grp[i % len(grp)] for i, grp in enumerate(b.shared_groups)], "agentic_decode")
    # members of a group share their prefix blocks but not their tails;
    # equal context lengths within a group
    for grp in b.shared_groups:
        assert len({int(b.context_lens[s]) for s in grp}) == 1


def run_decode_shared(b, out=None):
    m = b.meta(DEV)
    gm = b.group_meta(DEV)
    out = torch.empty_like(b.query) if out is None else out
    ng = gm["group_prefix_len"].numel()
    ws_bytes = pa.decode_shared_prefix_workspace_bytes(b.num_seqs, ng, b.max_context_len, b.num_heads,
                                                       b.num_kv_heads, b.head_size, b.cache_dtype,
                                                       b.sliding_window)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=DEV)
    pa.decode_shared_prefix(out, b.query, b.k_cache, b.v_cache, m["block_table"], m["context_lens"],
                            b.max_context_len, gm["cu_groups"], gm["group_prefix_len"], b.scale, b.k_scale,
                            b.v_scale, b.sliding_window, ws)
    return out


def test_decode_shared_prefix_agentic():
    """The agentic batch through the shared-prefix decode (each group's
    prefix blocks read once for its four members): the oracle on one member
    of every group, and the plain decode's result within the same bar."""
    b = W.make_config("agentic_decode", device=DEV)
    out = run_decode_shared(b)
    ref_plain = out_f64(run_decode(b))
    torch.cuda.synchronize()
    check_rows(b, out, [grp[i % len(grp)] for i, grp in enumerate(b.shared_groups)], "agentic shared-prefix")
    got = out_f64(out)
    ma, mr = assert_close(got, ref_plain, "agentic shared-prefix vs plain decode")
    _log(f"agentic shared-prefix vs plain decode: max abs {ma:.2e}, max rel {mr:.2e}")


SHARED_CASES = [
    # (ctx lens, groups [(first, size, prefix tokens)], Hq, Hkv, D, cache dtype)
    ([40, 40, 40, 40, 100, 7, 33, 33], [(0, 4, 32), (4, 1, 64), (6, 2, 32)], 16, 4, 128, "bf16"),
    ([300, 310, 290, 305, 320, 299], [(0, 6, 288)], 32, 8, 128, "bf16"),         # 6 members > 16/G = 2
    ([1000, 1017, 1001], [(0, 3, 1000)], 8, 8, 64, "bf16"),                      # G = 1: 16 members per chunk
    ([5000, 4990, 17, 4999], [(0, 2, 4096), (3, 1, 4000)], 64, 4, 128, "bf16"),  # G = 16: one member per chunk
    ([700, 650, 800, 720, 20], [(0, 4, 640), (4, 1, 0)], 16, 2, 64, "fp8_e4m3"),
    ([129, 129, 129], [(0, 3, 4096)], 8, 2, 128, "bf16"),                         # prefix clamped to ctx - 1
    ([64, 80, 96, 112, 128, 144, 160, 176, 192], [(1, 8, 48)], 32, 8, 128, "fp8_e4m3"),
]


@pytest.mark.parametrize("case", range(len(SHARED_CASES)))
def test_decode_shared_prefix_small(case):
    ctx, groups, Hq, Hkv, D, cd = SHARED_CASES[case]
    sg = [list(range(f, f + n)) for f, n, _ in groups]
    sp = {gi: p for gi, (_, _, p) in enumerate(groups)}
    # blocks really shared only up to what every member can hold
    sp_blocks = {gi: min(p, min(ctx[s] for s in sg[gi]) - 1) // 16 * 16 for gi, p in sp.items()}
    b = W.make_batch(f"shared{case}", 500 + case, ctx, [1] * len(ctx), Hq, Hkv, D, "bf16", cd,
                     shared_groups=sg, shared_prefix=sp_blocks, device=DEV, extra_blocks=3)
    b.shared_prefix = sp  # the call gets the unclamped lengths
    out = run_decode_shared(b)
    torch.cuda.synchronize()
    check_rows(b, out, range(b.num_seqs), f"shared-prefix case {case}")


def test_decode_shared_prefix_random():
    """Seeded random shared-prefix batches: groups of consecutive sequences
    (singletons too), prefix lengths up to and beyond what every member
    holds, head and group sizes, bf16/fp8 caches."""
    rng = np.random.default_rng(779)
    for it in range(32):
        D = int(rng.choice([64, 128]))
        G = int(rng.choice([1, 2, 4, 8, 16]))
        Hkv = int(rng.choice([1, 2, 4, 8]))
        cd = str(rng.choice(["bf16", "bf16", "fp8_e4m3"]))
        S = int(rng.integers(1, 13))
        base = int(rng.integers(1, 4000))
        ctx = [max(1, base + int(rng.integers(-40, 200))) for _ in range(S)]
        sg, s0 = [], 0
        while s0 < S:
            n = int(rng.integers(1, S - s0 + 1))
            sg.append(list(range(s0, s0 + n)))
            s0 += n
        sp = {gi: int(rng.integers(0, base + 100)) for gi in range(len(sg))}
        sp_blocks = {gi: max(0, min(p, min(ctx[s] for s in sg[gi]) - 1)) // 16 * 16 for gi, p in sp.items()}
        _log(f"shared random {it}: D {D} G {G} Hkv {Hkv} {cd} ctx {ctx} groups {sg} prefix {sp}")
        b = W.make_batch(f"shr{it}", 800 + it, ctx, [1] * S, G * Hkv, Hkv, D, "bf16", cd,
                         shared_groups=sg, shared_prefix=sp_blocks, device=DEV, extra_blocks=2)
        b.shared_prefix = sp  # the call gets the unclamped lengths
        out = run_decode_shared(b)
        torch.cuda.synchronize()
        check_rows(b, out, range(S), f"shared random {it}")


def test_decode_fp8_sampled():
    b = W.make_config("fp8_decode", device=DEV)
    out = run_decode(b)
    torch.cuda.synchronize()
    # 16 sequences spread over the context range, shortest and longest included
    order = np.argsort(b.context_lens)
    check_rows(b, out, sorted({int(order[i]) for i in np.linspace(0, len(order) - 1, 16).astype(int)}),
               "fp8_decode")


def test_decode_fp8_swa128_full():
    b = W.make_config("fp8_swa128", device=DEV)
    out = run_decode(b)
    torch.cuda.synchronize()
    check_rows(b, out, range(b.num_seqs), "fp8_swa128")


def test_mixed_step_sampled():
    """Write all 2240 new tokens, then the flattened varlen batch (192 decode
    rows + one 2048-row chunk on a 65536-token prefix), as the benchmark's
    step runs it. The write is compared byte for byte with the oracle's over
    every block it touches (the destination slots scribbled over first);
    the chunk on the first and last row of each of its 32 query tiles (every
    head) plus every row for the query heads of one KV head; decode rows on
    a spread of sequences."""
    b = W.make_config("mixed_step", device=DEV)
    m = b.meta(DEV)
    st = m["slot_mapping"]
    blk, off = st // 16, st % 16
    touched = torch.unique(blk)
    b.k_cache[blk, :, off, :] = -3.0
    b.v_cache[blk, :, :, off] = -3.0
    k_before, v_before = raw(b.k_cache[touched]), raw(b.v_cache[touched])
    pa.reshape_and_cache(b.new_key, b.new_value, b.k_cache, b.v_cache, st)
    out = run_prefill(b)
    torch.cuda.synchronize()
    remap = {int(x): i for i, x in enumerate(touched.tolist())}
    local = np.array([remap[int(s) // 16] * 16 + int(s) % 16 for s in b.slot_mapping], dtype=np.int64)
    oracle.reshape_and_cache(k_before, v_before, raw(b.new_key), raw(b.new_value), local)
    assert np.array_equal(raw(b.k_cache[touched]).view(np.uint8), k_before.view(np.uint8))
    assert np.array_equal(raw(b.v_cache[touched]).view(np.uint8), v_before.view(np.uint8))
    _log(f"mixed_step write: {b.num_q_tokens} tokens into {len(touched)} blocks, byte-exact")
    # decode rows: a spread of sequences
    check_rows(b, out, list(range(0, 192, 12)) + [191], "mixed_step decode rows")
    s = 192
    cu = b.cu_seqlens
    got = out_f64(out)[cu[s]:cu[s + 1]]
    tq = 256 // (b.num_heads // b.num_kv_heads)  # query tokens per tile
    rows = sorted({r for t in range(2048 // tq) for r in (t * tq, t * tq + tq - 1)} | {1, 31, 32, 1000})
    ref = oracle_rows(b, [s], rows=rows)[s]
    ma, mr = assert_close(got[rows], ref[rows], "mixed_step chunk rows")
    _log(f"mixed_step chunk: {len(rows)} rows over all {2048 // tq} tiles, max abs {ma:.2e}, max rel {mr:.2e}")
    heads = list(range(b.num_heads // b.num_kv_heads))  # the query heads of KV head 0
    ref = oracle_rows(b, [s], heads=heads)[s]
    ma, mr = assert_close(got[:, heads], ref[:, heads], "mixed_step chunk, KV head 0")
    _log(f"mixed_step chunk: all 2048 rows of heads {heads}, max abs {ma:.2e}, max rel {mr:.2e}")


def test_prefill_fp8_chunk_sampled():
    """The 2048-token chunk on a 65,536-token prefix over an fp8 e4m3 cache
    with per-block scales: the batch and launch the fp8 chunk timing uses,
    sampled rows across the tiles (first and last tile, a tile edge)."""
    b = W.make_batch("mixed_step_chunk_fp8", 4, [65536 + 2048], [2048], 32, 8, 128, "bf16", "fp8_e4m3",
                     device=DEV)
    out = run_prefill(b)
    torch.cuda.synchronize()
    ref = oracle_rows(b, [0])[0]
    got = out_f64(out)
    rows = [0, 1, 63, 64, 1000, 1983, 2046, 2047]
    ma, mr = assert_close(got[rows], ref[rows], "fp8 chunk rows")
    _log(f"fp8 chunk: rows {rows}, max abs {ma:.2e}, max rel {mr:.2e}")


# ----------------------------------------------------------------------------
# small ragged batches: decode and chunked prefill
# ----------------------------------------------------------------------------
DECODE_CASES = [
    # (ctx lens, Hq, Hkv, D, q dtype, cache dtype, window)
    ([1, 2, 15, 16, 17, 31, 32, 33, 1000], 8, 2, 128, "bf16", "bf16", 0),
    ([1, 5, 16, 300, 4097], 4, 4, 64, "bf16", "bf16", 0),
    ([7, 100, 2049, 9000], 16, 1, 128, "bf16", "bf16", 0),
    ([3, 40, 517, 12000], 32, 2, 128, "bf16", "fp8_e4m3", 0),
    ([1, 50, 129, 700], 8, 8, 64, "bf16", "fp8_e4m3", 0),
    ([1, 100, 128, 129, 5000], 8, 1, 128, "bf16", "bf16", 128),
    ([20, 300, 3000], 16, 2, 64, "f32", "f32", 37),
    # every stream at most 16 blocks: one wave per (sequence, KV head), no merge
    ([1, 2, 15, 16, 17, 100, 255, 256], 8, 2, 128, "bf16", "bf16", 0),
    ([1, 30, 200, 256], 16, 4, 64, "bf16", "fp8_e4m3", 0),
    ([3000, 40000, 5, 241], 32, 8, 128, "bf16", "fp8_e4m3", 240),
    ([1, 33, 800], 4, 1, 128, "f32", "f32", 0),
]


@pytest.mark.parametrize("case", range(len(DECODE_CASES)))
def test_decode_small(case):
    ctx, Hq, Hkv, D, qd, cd, w = DECODE_CASES[case]
    b = W.make_batch(f"dec{case}", 100 + case, ctx, [1] * len(ctx), Hq, Hkv, D, qd, cd,
                     sliding_window=w, device=DEV, extra_blocks=5)
    out = run_decode(b)
    torch.cuda.synchronize()
    check_rows(b, out, range(b.num_seqs), f"decode case {case}")


@pytest.mark.parametrize("case", [0, 1, 3, 4, 5, 9])
def test_decode_valu_small(case):
    """pa_decode_valu (the vector-ALU kernel, kept for side-by-side
    measurement) on the bf16 and fp8 decode cases."""
    ctx, Hq, Hkv, D, qd, cd, w = DECODE_CASES[case]
    b = W.make_batch(f"valu{case}", 150 + case, ctx, [1] * len(ctx), Hq, Hkv, D, qd, cd,
                     sliding_window=w, device=DEV, extra_blocks=5)
    m = b.meta(DEV)
    out = torch.empty_like(b.query)
    n = pa.decode_valu_workspace_bytes(b.num_seqs, b.max_context_len, b.num_heads, b.num_kv_heads, b.head_size,
                                       b.cache_dtype, b.sliding_window)
    ws = torch.empty(max(n, 1), dtype=torch.uint8, device=DEV)
    pa.decode_valu(out, b.query, b.k_cache, b.v_cache, m["block_table"], m["context_lens"], b.max_context_len,
                   b.scale, b.k_scale, b.v_scale, b.sliding_window, ws)
    torch.cuda.synchronize()
    check_rows(b, out, range(b.num_seqs), f"valu decode case {case}")


PREFILL_CASES = [
    # (ctx lens, q lens, Hq, Hkv, D, cache dtype, window)
    ([37, 50, 1000, 17, 2100], [37, 1, 130, 1, 300], 32, 8, 128, "bf16", 0),
    ([64, 65, 129], [64, 65, 2], 8, 8, 64, "bf16", 0),
    ([300, 4000], [300, 257], 8, 1, 128, "bf16", 0),
    ([500, 20, 1500], [129, 20, 33], 16, 1, 64, "bf16", 0),
    ([700, 90], [200, 90], 4, 2, 128, "fp8_e4m3", 0),
    ([1000, 260], [300, 260], 8, 2, 128, "bf16", 100),
    ([2000, 33], [64, 1], 16, 8, 128, "bf16", 1),
    ([5000], [1], 8, 2, 128, "bf16", 0),
    ([1500, 300], [700, 300], 64, 4, 128, "fp8_e4m3", 0),    # fp8, G = 16
    ([900, 2000], [128, 513], 16, 4, 64, "fp8_e4m3", 200),  # fp8, head 64 (half the waves copy), window
]


@pytest.mark.parametrize("case", range(len(PREFILL_CASES)))
def test_prefill_small(case):
    ctx, ql, Hq, Hkv, D, cd, w = PREFILL_CASES[case]
    b = W.make_batch(f"pre{case}", 200 + case, ctx, ql, Hq, Hkv, D, "bf16", cd, sliding_window=w,
                     device=DEV, extra_blocks=4)
    out = run_prefill(b)
    torch.cuda.synchronize()
    check_rows(b, out, range(b.num_seqs), f"prefill case {case}")


@pytest.mark.parametrize("log2_scale", [13, -20])
def test_prefill_values_across_fp16_range(log2_scale):
    """The bf16-cache prefill kernel takes the values into its PV product as
    fp16: exact for magnitudes in fp16's normal range, 2^-24 of absolute
    resolution below it. Values scaled by 2^13 (up to ~4e4, inside the range)
    must keep the bar scaled by the same factor; values scaled by 2^-20 (fp16
    subnormals) must stay within 2^-24 absolute."""
    ctx, ql = [700, 3000, 48], [300, 129, 48]
    b = W.make_batch(f"vrange{log2_scale}", 400 + log2_scale, ctx, ql, 16, 4, 128, "bf16", "bf16",
                     device=DEV, extra_blocks=3)
    f = 2.0 ** log2_scale
    b.v_cache.mul_(f)  # exact in bf16 (a power of two; NaN poison stays NaN)
    assert torch.isfinite(b.v_cache[b.v_cache == b.v_cache]).all()
    out = run_prefill(b)
    torch.cuda.synchronize()
    ref = oracle_rows(b, range(b.num_seqs))
    got = out_f64(out)
    cu = b.cu_seqlens
    atol = 2e-3 * f if log2_scale > 0 else 2.0 ** -24
    for s in range(b.num_seqs):
        ma, mr = assert_close(got[cu[s]:cu[s + 1]], ref[s], f"values x 2^{log2_scale} seq {s}", atol=atol)
        _log(f"values x 2^{log2_scale} seq {s}: max abs {ma:.3e} (bar {atol:.3e}), max rel {mr:.3e}")


def test_random_shapes():
    """Seeded random small shapes over head size, group size, dtypes, context,
    chunk length and window (decode and prefill)."""
    rng = np.random.default_rng(777)
    for it in range(64):
        D = int(rng.choice([64, 128]))
        G = int(rng.choice([1, 2, 4, 8, 16]))
        Hkv = int(rng.choice([1, 2, 4]))
        cd = str(rng.choice(["bf16", "bf16", "fp8_e4m3"]))
        S = int(rng.integers(1, 5))
        ctx = rng.integers(1, 5000, S)
        ql = np.minimum(ctx, rng.integers(1, 300, S))
        ql[rng.random(S) < 0.4] = 1
        w = int(rng.choice([0, 0, int(rng.integers(1, 200))]))
        b = W.make_batch(f"rand{it}", 300 + it, ctx.tolist(), ql.tolist(), G * Hkv, Hkv, D, "bf16", cd,
                         sliding_window=w, device=DEV, extra_blocks=int(rng.integers(0, 5)))
        _log(f"random case {it}: D {D} G {G} Hkv {Hkv} cache {cd} ctx {ctx.tolist()} q {ql.tolist()} W {w}")
        out = run_prefill(b)
        torch.cuda.synchronize()
        check_rows(b, out, range(S), f"random case {it}")


def test_random_decode_shapes():
    """Seeded random decode batches through pa_decode: head size, group size,
    KV heads, bf16/fp8/fp32 caches, contexts long (split work, merged) and
    short (a wave per stream), sliding windows."""
    rng = np.random.default_rng(778)
    for it in range(64):
        D = int(rng.choice([64, 128]))
        G = int(rng.choice([1, 2, 4, 8, 16]))
        Hkv = int(rng.choice([1, 2, 4, 8]))
        cd = str(rng.choice(["bf16", "bf16", "fp8_e4m3", "f32"]))
        qd = "f32" if cd == "f32" else "bf16"
        S = int(rng.integers(1, 9))
        ctx = rng.integers(1, 300 if rng.random() < 0.3 else 6000, S)
        w = int(rng.choice([0, 0, int(rng.integers(1, 300))]))
        b = W.make_batch(f"rdec{it}", 500 + it, ctx.tolist(), [1] * S, G * Hkv, Hkv, D, qd, cd,
                         sliding_window=w, device=DEV, extra_blocks=int(rng.integers(0, 5)))
        _log(f"random decode {it}: D {D} G {G} Hkv {Hkv} {qd}/{cd} ctx {ctx.tolist()} W {w}")
        out = run_decode(b)
        torch.cuda.synchronize()
        check_rows(b, out, range(S), f"random decode {it}")


# ----------------------------------------------------------------------------
# invariances (bitwise on the GPU)
# ----------------------------------------------------------------------------
def _permuted(b, seed):
    """Same batch with the physical blocks permuted and the table remapped."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    perm = torch.randperm(b.num_blocks, generator=g)           # new id of old block i
    inv = torch.empty_like(perm)
    inv[perm] = torch.arange(b.num_blocks)
    import copy
    c = copy.copy(b)
    c.device_meta = {}
    c.k_cache = b.k_cache[inv.to(DEV)].contiguous()
    c.v_cache = b.v_cache[inv.to(DEV)].contiguous()
    if b.k_scale is not None:
        c.k_scale = b.k_scale[inv.to(DEV)].contiguous()
        c.v_scale = b.v_scale[inv.to(DEV)].contiguous()
    c.block_table = perm.numpy()[b.block_table].astype(np.int32)
    return c


@pytest.mark.parametrize("cd", ["bf16", "fp8_e4m3"])
def test_block_permutation_is_bitwise_invariant(cd):
    b = W.make_batch("perm", 31, [17, 500, 3000, 64], [1, 1, 40, 1], 16, 4, 128, "bf16", cd,
                     device=DEV, extra_blocks=10)
    o1 = run_prefill(b)
    o2 = run_prefill(_permuted(b, 5))
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


def test_shared_prefix_equals_copied_blocks_bitwise():
    kw = dict(ctx_lens=[1000, 1000, 1000, 1000], q_lens=[1] * 4, num_heads=32, num_kv_heads=8,
              head_size=128)
    b = W.make_batch("shared", 41, shared_groups=[[0, 1, 2, 3]], shared_prefix={0: 960}, device=DEV,
                     extra_blocks=0, **kw)
    o_shared = run_decode(b)
    # copy the shared blocks into private blocks for members 1..3
    import copy
    c = copy.copy(b)
    c.device_meta = {}
    ns = 960 // 16
    extra = []
    table = b.block_table.copy()
    nxt = b.num_blocks
    for s in (1, 2, 3):
        for lb in range(ns):
            extra.append(int(b.block_table[0, lb]))
            table[s, lb] = nxt
            nxt += 1
    idx = torch.tensor(extra, device=DEV, dtype=torch.int64)
    c.k_cache = torch.cat([b.k_cache, b.k_cache[idx]]).contiguous()
    c.v_cache = torch.cat([b.v_cache, b.v_cache[idx]]).contiguous()
    c.block_table = table
    c.num_blocks = nxt
    o_copied = run_decode(c)
    torch.cuda.synchronize()
    assert torch.equal(o_shared.view(torch.int16), o_copied.view(torch.int16))
    check_rows(b, o_shared, range(4), "shared prefix")


def test_decode_equals_prefill_with_one_token():
    b = W.make_batch("d_eq_p", 51, [1, 90, 4000, 33, 17000], [1] * 5, 32, 8, 128, device=DEV)
    o1 = run_decode(b)
    o2 = run_prefill(b)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


def test_repeatable_bitwise():
    b = W.make_batch("rep", 61, [5000, 70000, 12], [1, 300, 1], 32, 8, 128, device=DEV)
    o1 = run_prefill(b)
    o2 = run_prefill(b)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


def test_chunking_matches_whole_prompt():
    """A 600-token prompt attended in one chunk vs four chunks (each chunk's
    context = tokens so far): same outputs within tolerance."""
    b = W.make_batch("chunks", 71, [600], [600], 16, 4, 128, device=DEV)
    whole = out_f64(run_prefill(b))
    import copy
    pieces = []
    done = 0
    for chunk in (100, 1, 300, 199):
        done += chunk
        c = copy.copy(b)
        c.device_meta = {}
        c.context_lens = np.array([done], np.int32)
        c.q_lens = np.array([chunk], np.int32)
        c.query = b.query[done - chunk:done].contiguous()
        pieces.append(out_f64(run_prefill(c)))
    torch.cuda.synchronize()
    assert_close(np.concatenate(pieces), whole, "chunked vs whole", atol=2e-3, rtol=1e-2)


def test_nan_poison_never_leaks():
    """Every slot outside the contexts holds NaN; no output is NaN."""
    for cd in ("bf16", "fp8_e4m3"):
        b = W.make_batch("poison", 81, [1, 17, 31, 257, 1025], [1, 17, 2, 100, 1], 16, 2, 128, "bf16", cd,
                         device=DEV, extra_blocks=20)
        out = run_prefill(b)
        torch.cuda.synchronize()
        assert torch.isfinite(out.float()).all()


def test_fp8_all_codes_decode_exactly():
    """A single-key decode returns V_0 exactly (up to the output's bf16
    rounding); with the 254 finite e4m3fn codes spread over V rows this checks
    the hardware conversion against the oracle's closed form."""
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    D = 128
    S = 2  # 254 codes over 2 sequences x 128 dims (two duplicates)
    b = W.make_batch("codes", 91, [1] * S, [1] * S, 8, 8, D, "bf16", "fp8_e4m3", device=DEV, extra_blocks=0)
    vals = np.resize(codes, S * D).reshape(S, D)
    for s in range(S):
        blk = int(b.block_table[s, 0])
        b.v_cache[blk, :, :, 0] = torch.from_numpy(vals[s]).to(DEV)[None, :]
        b.v_scale[blk] = 1.0
    out = run_decode(b)
    torch.cuda.synchronize()
    got = out_f64(out)
    ref = F.e4m3fn_bits_to_f64(vals)
    ref_bf16 = torch.from_numpy(ref).to(torch.bfloat16).to(torch.float64).numpy()
    for s in range(S):
        assert np.array_equal(got[s, :, :], np.broadcast_to(ref_bf16[s], (8, D)))


def test_peak_probes_run():
    """The achievable-peak probes bench.py reports beside the path launch and
    write their sinks (a small gather and a short MFMA loop)."""
    from paged_kv_cache_103_amd import peaks

    buf = torch.ones(64 * 4096, dtype=torch.uint8, device=DEV)
    ids = torch.randperm(64, device="cpu").to(torch.int32).to(DEV)
    sink = torch.full((256 * 8,), -1.0, dtype=torch.float32, device=DEV)
    for mode in (0, 1):
        peaks.read_tiles(buf, ids, mode, 8, sink)
    # the global->LDS gather reads the right bytes: each workgroup's thread 0
    # leaves the XOR of the first 16 bytes of every 1 KiB of its wave's tiles
    # (wave 0 of workgroup b takes tiles [4 b C, 4 b C + C), C = 64 / 32)
    words = torch.randint(-2**31, 2**31 - 1, (64 * 1024,), dtype=torch.int32)
    buf2 = words.to(DEV).view(torch.uint8)
    sink2 = torch.zeros(8, dtype=torch.int32, device=DEV)
    peaks.read_tiles(buf2, ids, 2, 8, sink2)
    torch.cuda.synchronize()
    w = words.view(64, 4, 256)[:, :, :4]  # tile, 1 KiB chunk, first 4 words
    idl = ids.cpu().long()
    for b in range(8):
        want = 0
        for t in idl[8 * b:8 * b + 2]:
            for x in w[t].reshape(-1).tolist():
                want ^= x
        assert int(sink2[b].item()) == want, (b, int(sink2[b].item()), want)
    flops = peaks.mfma(0, 10, 8, sink)
    peaks.mfma(1, 10, 8, sink)
    torch.cuda.synchronize()
    assert flops == 4.0 * 32768 * 10 * 8 * 4
    assert torch.isfinite(sink).all()
