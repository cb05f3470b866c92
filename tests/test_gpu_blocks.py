"""GPU: the copy-on-write block copy, and the block manager driving the KV
write and the decode end to end (through the C ABI).

pa_copy_blocks must reproduce the pool byte for byte: destination blocks
become their sources (every head's K and V tile and, for fp8, the block
scales), every other byte stays. The end-to-end case admits a prompt, forks
it into branches that each decode past the shared partial block (so copies
happen), admits a second request that hits the prefix cache, writes every
new token's K/V through the manager's slots, and decodes all branches; the
oracle attends over each branch's own K/V history laid out contiguously,
with no sharing at all.
"""

import numpy as np
import pytest
import torch

import oracle
from oracle import formats as F
from paged_kv_cache_103_amd import _lib as pa
from paged_kv_cache_103_amd import blocks
from tests.helpers import assert_close, out_f64, raw

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _log(msg):
    print(msg, flush=True)


def _pool(gen, NB, H, D, dtype):
    shape_k, shape_v = (NB, H, 16, D), (NB, H, D, 16)
    if dtype == "f32":
        return (torch.randn(shape_k, generator=gen), torch.randn(shape_v, generator=gen))
    if dtype == "bf16":
        return (torch.randn(shape_k, generator=gen).to(torch.bfloat16),
                torch.randn(shape_v, generator=gen).to(torch.bfloat16))
    k = torch.randint(0, 256, shape_k, generator=gen, dtype=torch.uint8).view(torch.float8_e4m3fn)
    v = torch.randint(0, 256, shape_v, generator=gen, dtype=torch.uint8).view(torch.float8_e4m3fn)
    return k, v


@pytest.mark.parametrize("dtype,H,D", [("bf16", 8, 128), ("bf16", 3, 64), ("f32", 2, 128), ("fp8", 8, 128),
                                       ("fp8", 1, 64)])
def test_copy_blocks_bit_exact(dtype, H, D):
    _log(f"copy_blocks {dtype} H={H} D={D}")
    gen = torch.Generator().manual_seed({"bf16": 1, "f32": 2, "fp8": 3}[dtype] * 1000 + H * 10 + D)
    NB = 300
    k, v = _pool(gen, NB, H, D, dtype)
    ks = vs = None
    if dtype == "fp8":
        ks, vs = torch.rand(NB, generator=gen) + 0.5, torch.rand(NB, generator=gen) + 0.5
    perm = torch.randperm(NB, generator=gen).tolist()
    src, dst = perm[:60], perm[60:120]
    pairs = [[s, d] for s, d in zip(src, dst)] + [[NB, perm[200]], [perm[201], -1]]  # last two skipped
    want_k, want_v = raw(k).copy(), raw(v).copy()
    want_ks = None if ks is None else ks.numpy().copy()
    want_vs = None if vs is None else vs.numpy().copy()
    for s, d in zip(src, dst):
        want_k[d] = want_k[s]
        want_v[d] = want_v[s]
        if ks is not None:
            want_ks[d], want_vs[d] = want_ks[s], want_vs[s]
    kd, vd = k.to(DEV), v.to(DEV)
    ksd = None if ks is None else ks.to(DEV)
    vsd = None if vs is None else vs.to(DEV)
    blocks.copy_blocks(kd, vd, torch.tensor(pairs, dtype=torch.int32, device=DEV), ksd, vsd)
    torch.cuda.synchronize()
    assert np.array_equal(raw(kd), want_k)
    assert np.array_equal(raw(vd), want_v)
    if ks is not None:
        assert np.array_equal(ksd.cpu().numpy(), want_ks)
        assert np.array_equal(vsd.cpu().numpy(), want_vs)
    # no pairs: nothing changes
    blocks.copy_blocks(kd, vd, torch.zeros((0, 2), dtype=torch.int32, device=DEV), ksd, vsd)
    torch.cuda.synchronize()
    assert np.array_equal(raw(kd), want_k)


def test_fork_copy_on_write_decode_against_oracle():
    """Prompt of 37 tokens, four branches decoding 1..21 tokens each (the
    first three appends to the shared partial block copy it), and a second
    request whose prompt shares the first 32 tokens (a prefix-cache hit)."""
    Hq, Hkv, D, NB = 16, 4, 128, 64
    gen = torch.Generator().manual_seed(77)
    bm = blocks.BlockManager(NB)
    kc = torch.full((NB, Hkv, 16, D), float("nan"), dtype=torch.bfloat16, device=DEV)
    vc = torch.full((NB, Hkv, D, 16), float("nan"), dtype=torch.bfloat16, device=DEV)
    hist = {}  # request -> (token ids, K rows, V rows), each row [Hkv][D] bf16

    def new_kv(n):
        return (torch.randn((n, Hkv, D), generator=gen).to(torch.bfloat16),
                torch.randn((n, Hkv, D), generator=gen).to(torch.bfloat16))

    def write(req, tok, K, V):
        slots, cow = bm.append(req, tok)
        if cow is not None:
            blocks.copy_blocks(kc, vc, torch.tensor([cow], dtype=torch.int32, device=DEV))
        pa.reshape_and_cache(K.to(DEV), V.to(DEV), kc, vc, torch.from_numpy(slots).to(DEV))
        t0, k0, v0 = hist[req]
        hist[req] = (t0 + list(tok), torch.cat([k0, K]), torch.cat([v0, V]))
        return cow

    prompt = list(range(500, 537))
    assert bm.add_request(0, prompt) == 0
    hist[0] = ([], torch.empty((0, Hkv, D), dtype=torch.bfloat16), torch.empty((0, Hkv, D), dtype=torch.bfloat16))
    write(0, prompt, *new_kv(37))
    for c in (1, 2, 3):
        bm.fork(0, c)
        hist[c] = hist[0]
    steps = {0: 21, 1: 1, 2: 12, 3: 5}
    cows = 0
    for i in range(max(steps.values())):
        for r in (1, 2, 0, 3):
            if i < steps[r]:
                cows += write(r, [1000 + 10 * r + i], *new_kv(1)) is not None
    assert cows == 3
    # a new request with the same first 32 tokens: two blocks from the cache
    p2 = prompt[:32] + [7, 8, 9]
    assert bm.add_request(9, p2) == 32
    hist[9] = (p2[:32], hist[0][1][:32], hist[0][2][:32])
    write(9, p2[32:], *new_kv(3))
    reqs = [0, 1, 2, 3, 9]
    tables = [bm.info(r)[1] for r in reqs]
    assert all(t[:2] == tables[0][:2] for t in tables)  # the shared full blocks
    assert len({t[2] for t in tables}) == 5  # every branch owns its third block
    ctx = [bm.info(r)[0] for r in reqs]
    assert ctx == [58, 38, 49, 42, 35]
    stride = max(len(t) for t in tables)
    bt = torch.tensor([t + [0] * (stride - len(t)) for t in tables], dtype=torch.int32, device=DEV)
    cl = torch.tensor(ctx, dtype=torch.int32, device=DEV)
    q = torch.randn((len(reqs), Hq, D), generator=gen).to(torch.bfloat16).to(DEV)
    scale = D ** -0.5
    out = torch.empty_like(q)
    ws = torch.empty(max(pa.decode_workspace_bytes(len(reqs), max(ctx), Hq, Hkv, D), 1), dtype=torch.uint8,
                     device=DEV)
    pa.decode(out, q, kc, vc, bt, cl, max(ctx), scale, workspace=ws)
    out_sp = torch.empty_like(q)
    cu_groups = torch.tensor([0, len(reqs)], dtype=torch.int32, device=DEV)
    gpl = torch.tensor([32], dtype=torch.int32, device=DEV)
    ws2 = torch.empty(max(pa.decode_shared_prefix_workspace_bytes(len(reqs), 1, max(ctx), Hq, Hkv, D), 1),
                      dtype=torch.uint8, device=DEV)
    pa.decode_shared_prefix(out_sp, q, kc, vc, bt, cl, max(ctx), cu_groups, gpl, scale, workspace=ws2)
    torch.cuda.synchronize()
    qh = F.to_f64(raw(q), F.BF16)
    got, got_sp = out_f64(out), out_f64(out_sp)
    for i, r in enumerate(reqs):
        toks, K, V = hist[r]
        n = len(toks)
        assert n == ctx[i]
        nblk = (n + 15) // 16
        kp = np.zeros((nblk, Hkv, 16, D), dtype=np.uint16)
        vp = np.zeros((nblk, Hkv, D, 16), dtype=np.uint16)
        oracle.reshape_and_cache(kp, vp, raw(K), raw(V), np.arange(n), 16)
        ref = oracle.attend_sequence(qh[i:i + 1], kp, vp, F.BF16, None, None, np.arange(nblk), n, Hkv, scale)
        assert_close(got[i:i + 1], ref, f"request {r} decode")
        assert_close(got_sp[i:i + 1], ref, f"request {r} shared-prefix decode")
    _log(f"fork/copy-on-write decode: {len(reqs)} requests, contexts {ctx}, {cows} block copies")
    for r in reqs:
        bm.free(r)
    assert bm.num_free == NB
