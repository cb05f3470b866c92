"""Seeded synthetic inputs shaped like the pages' workloads.

This module only draws random numbers and lays out metadata (which physical
block holds which logical block, which slot each new token goes to); it holds
none of the attention arithmetic. Both the HIP path and the CPU oracle read
the tensors it makes.

Recipe (per named configuration, seed fixed per configuration):
  * metadata from numpy.random.default_rng(seed): context lengths, the
    physical pool as a random permutation of block ids, shared prefixes;
  * values from a torch.Generator on the target device seeded with the same
    seed: K, V and queries ~ N(0, 1) in fp32, rounded to nearest even into the
    stored type; an fp8 pool takes one fp32 scale per block for K and one for
    V, amax(|drawn block values|) / 448, and codes = e4m3fn(x / scale) via
    PyTorch's float8_e4m3fn cast;
  * every pool slot no sequence owns (the tail of a last block, unassigned
    blocks) is poisoned with NaN so that a read outside the context shows;
  * the new tokens of a step are the last q_len positions of each sequence;
    their slot_mapping is block_table[s][p // 16] * 16 + p % 16 and the
    key/value rows handed to the write equal what the pool holds there (for an
    fp8 pool: the dequantised value rounded to bf16), so a write is
    idempotent and a step can be repeated.

The named configurations stand in for the pages' agentic traces (input median
142K tokens, >96% prefix reuse, subagent forks of about 4), which are not
available here.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence

import numpy as np
import torch

BLOCK = 16
FP8_MAX = 448.0

DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8_e4m3": torch.uint8}
ELEM_BYTES = {"f32": 4, "bf16": 2, "fp8_e4m3": 1}


@dataclass
class Batch:
    name: str
    seed: int
    num_heads: int
    num_kv_heads: int
    head_size: int
    q_dtype: str
    cache_dtype: str
    scale: float
    sliding_window: int
    context_lens: np.ndarray          # int32 [S]
    q_lens: np.ndarray                # int32 [S]
    block_table: np.ndarray           # int32 [S][stride]
    num_blocks: int
    slot_mapping: np.ndarray          # int64 [sum q_lens]
    query: torch.Tensor               # [Nq][Hq][D]
    k_cache: torch.Tensor             # [NB][Hkv][16][D]
    v_cache: torch.Tensor             # [NB][Hkv][D][16]
    k_scale: Optional[torch.Tensor]   # fp32 [NB] (fp8 only)
    v_scale: Optional[torch.Tensor]
    new_key: torch.Tensor             # [T][Hkv][D] (q dtype for fp8 pools, else cache dtype)
    new_value: torch.Tensor
    shared_groups: List[List[int]] = field(default_factory=list)
    shared_prefix: Dict[int, int] = field(default_factory=dict)   # group index -> shared tokens
    device_meta: Dict[str, torch.Tensor] = field(default_factory=dict)

    # ---- derived sizes ----
    @property
    def num_seqs(self) -> int:
        return int(len(self.context_lens))

    @property
    def cu_seqlens(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.q_lens)]).astype(np.int32)

    @property
    def num_q_tokens(self) -> int:
        return int(self.q_lens.sum())

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max())

    @property
    def max_q_len(self) -> int:
        return int(self.q_lens.max())

    def meta(self, device) -> Dict[str, torch.Tensor]:
        """block_table, context_lens, cu_seqlens, slot_mapping as device tensors (cached)."""
        key = str(device)
        if key not in self.device_meta:
            self.device_meta[key] = {
                "block_table": torch.from_numpy(self.block_table).to(device),
                "context_lens": torch.from_numpy(self.context_lens).to(device),
                "cu_seqlens": torch.from_numpy(self.cu_seqlens).to(device),
                "slot_mapping": torch.from_numpy(self.slot_mapping).to(device),
            }
        return self.device_meta[key]

    def group_meta(self, device) -> Dict[str, torch.Tensor]:
        """cu_groups int32 [G+1] and group_prefix_len int32 [G] of the shared
        groups as the shared-prefix decode takes them: each group a run of
        consecutive sequences, runs in order; sequences between runs are
        given as runs of one with no shared prefix."""
        key = "groups:" + str(device)
        if key not in self.device_meta:
            groups = sorted((sorted(g), self.shared_prefix.get(gi, 0)) for gi, g in enumerate(self.shared_groups))
            cu, pl = [], []
            nxt = groups[0][0][0] if groups else 0
            for members, p in groups:
                assert members == list(range(members[0], members[0] + len(members))), "groups must be runs"
                while nxt < members[0]:
                    cu.append(nxt)
                    pl.append(0)
                    nxt += 1
                cu.append(members[0])
                pl.append(p)
                nxt = members[-1] + 1
            cu.append(nxt)
            self.device_meta[key] = {
                "cu_groups": torch.tensor(cu, dtype=torch.int32).to(device),
                "group_prefix_len": torch.tensor(pl, dtype=torch.int32).to(device),
            }
        return self.device_meta[key]

    def kv_bytes_read(self) -> int:
        """Algorithmic K+V bytes one attention pass reads: every key each
        sequence attends to (window applied), times Hkv*D*2*elem, plus the fp8
        per-block scales of the blocks touched."""
        e = ELEM_BYTES[self.cache_dtype]
        total = 0
        blocks = 0
        for ctx, ql in zip(self.context_lens.tolist(), self.q_lens.tolist()):
            lo = 0 if self.sliding_window <= 0 else max(0, ctx - ql + 1 - self.sliding_window)
            total += ctx - lo
            blocks += (ctx - 1) // BLOCK - lo // BLOCK + 1
        b = total * self.num_kv_heads * self.head_size * 2 * e
        if self.cache_dtype == "fp8_e4m3":
            b += blocks * 8
        return b

    def unique_kv_bytes_read(self) -> int:
        """As kv_bytes_read, counting each physical block once (shared prefixes)."""
        e = ELEM_BYTES[self.cache_dtype]
        seen = {}
        for s, (ctx, ql) in enumerate(zip(self.context_lens.tolist(), self.q_lens.tolist())):
            lo = 0 if self.sliding_window <= 0 else max(0, ctx - ql + 1 - self.sliding_window)
            for b in range(lo // BLOCK, (ctx - 1) // BLOCK + 1):
                phys = int(self.block_table[s, b])
                k0 = max(lo, b * BLOCK) - b * BLOCK
                k1 = min(ctx, (b + 1) * BLOCK) - b * BLOCK
                prev = seen.get(phys, (BLOCK, 0))
                seen[phys] = (min(prev[0], k0), max(prev[1], k1))
        toks = sum(k1 - k0 for k0, k1 in seen.values())
        b = toks * self.num_kv_heads * self.head_size * 2 * e
        if self.cache_dtype == "fp8_e4m3":
            b += len(seen) * 8
        return b


def _nan_bits(dtype: str):
    return {"f32": float("nan"), "bf16": float("nan"), "fp8_e4m3": 0x7F}[dtype]


def _assign_blocks(rng, ctx_lens: Sequence[int], shared_groups: Sequence[Sequence[int]],
                   shared_prefix: Dict[int, int], extra_blocks: int, pool_blocks: Optional[int]):
    """Physical block ids for every sequence's logical blocks.

    Sequences of a shared group point their first shared_prefix[group] // 16
    logical blocks at the same physical blocks (a refcounted prefix); all other
    blocks are private. Ids come from a random permutation of the pool.
    """
    need = []
    owner_of_prefix = {}
    for gi, grp in enumerate(shared_groups):
        owner_of_prefix[gi] = grp[0]
    seq_group = {s: gi for gi, grp in enumerate(shared_groups) for s in grp}
    total = 0
    for s, c in enumerate(ctx_lens):
        nb = -(-c // BLOCK)
        if s in seq_group and owner_of_prefix[seq_group[s]] != s:
            total += nb - shared_prefix[seq_group[s]] // BLOCK
        else:
            total += nb
        need.append(nb)
    NB = pool_blocks if pool_blocks is not None else total + extra_blocks
    assert NB >= total, "pool too small"
    perm = rng.permutation(NB).astype(np.int32)
    stride = max(need)
    table = np.zeros((len(ctx_lens), stride), dtype=np.int32)
    nxt = 0
    for s, nb in enumerate(need):
        start = 0
        if s in seq_group and owner_of_prefix[seq_group[s]] != s:
            ns = shared_prefix[seq_group[s]] // BLOCK
            table[s, :ns] = table[owner_of_prefix[seq_group[s]], :ns]
            start = ns
        for lb in range(start, nb):
            table[s, lb] = perm[nxt]
            nxt += 1
    used = perm[:nxt]
    return table, NB, used


def make_batch(name: str, seed: int, ctx_lens: Sequence[int], q_lens: Sequence[int], num_heads: int,
               num_kv_heads: int, head_size: int, q_dtype: str = "bf16", cache_dtype: str = "bf16",
               sliding_window: int = 0, scale: Optional[float] = None, device="cpu",
               shared_groups: Sequence[Sequence[int]] = (), shared_prefix: Optional[Dict[int, int]] = None,
               extra_blocks: int = 0, pool_blocks: Optional[int] = None, rng=None,
               chunk_blocks: int = 16384) -> Batch:
    """Generic seeded batch. ``rng`` (numpy Generator) defaults to default_rng(seed)."""
    rng = np.random.default_rng(seed) if rng is None else rng
    ctx_lens = [int(c) for c in ctx_lens]
    q_lens = [int(q) for q in q_lens]
    assert all(1 <= q <= c for q, c in zip(q_lens, ctx_lens))
    table, NB, used = _assign_blocks(rng, ctx_lens, shared_groups, shared_prefix or {}, extra_blocks,
                                     pool_blocks)
    return _finish_batch(name, seed, ctx_lens, q_lens, num_heads, num_kv_heads, head_size, q_dtype, cache_dtype,
                         sliding_window, scale, device, table, NB, used, chunk_blocks, shared_groups,
                         shared_prefix)


def _finish_batch(name, seed, ctx_lens, q_lens, num_heads, num_kv_heads, head_size, q_dtype, cache_dtype,
                  sliding_window, scale, device, table, NB, used, chunk_blocks, shared_groups=(),
                  shared_prefix=None) -> Batch:
    """Draws the pool, poisons what no sequence owns, draws the queries and
    the new tokens' rows, for a given block assignment."""
    H, D = num_kv_heads, head_size
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    is_fp8 = cache_dtype == "fp8_e4m3"
    store = DTYPES[cache_dtype]
    k_cache = torch.empty((NB, H, BLOCK, D), dtype=store, device=device)
    v_cache = torch.empty((NB, H, D, BLOCK), dtype=store, device=device)
    k_scale = torch.empty(NB, dtype=torch.float32, device=device) if is_fp8 else None
    v_scale = torch.empty(NB, dtype=torch.float32, device=device) if is_fp8 else None
    for b0 in range(0, NB, chunk_blocks):
        b1 = min(NB, b0 + chunk_blocks)
        for cache, sc in ((k_cache, k_scale), (v_cache, v_scale)):
            x = torch.randn((b1 - b0,) + tuple(cache.shape[1:]), generator=gen, device=device,
                            dtype=torch.float32)
            if is_fp8:
                amax = x.abs().amax(dim=(1, 2, 3)).clamp_min(1e-30)
                s = amax / FP8_MAX
                sc[b0:b1] = s
                cache[b0:b1] = (x / s[:, None, None, None]).to(torch.float8_e4m3fn).view(torch.uint8)
            else:
                cache[b0:b1] = x.to(store)
            del x
    # poison everything no sequence owns
    owned = torch.zeros((NB, BLOCK), dtype=torch.bool)
    used_t = torch.from_numpy(np.asarray(used, dtype=np.int64))
    owned[used_t] = True
    for s, c in enumerate(ctx_lens):
        if c % BLOCK:
            owned[int(table[s, (c - 1) // BLOCK]), c % BLOCK:] = False
    owned = owned.to(device)
    poison = _nan_bits(cache_dtype)
    k_cache.masked_fill_(~owned[:, None, :, None], poison)
    v_cache.masked_fill_(~owned[:, None, None, :], poison)

    # queries
    S = len(ctx_lens)
    Nq = sum(q_lens)
    query = torch.randn((Nq, num_heads, D), generator=gen, device=device, dtype=torch.float32)
    query = query.to(DTYPES[q_dtype])

    # new tokens: the last q_len positions of every sequence
    slots = []
    for s, (c, q) in enumerate(zip(ctx_lens, q_lens)):
        for p in range(c - q, c):
            slots.append(int(table[s, p // BLOCK]) * BLOCK + p % BLOCK)
    slot_mapping = np.asarray(slots, dtype=np.int64)
    st = torch.from_numpy(slot_mapping).to(device)
    blk, off = st // BLOCK, st % BLOCK
    nk = k_cache[blk, :, off, :]                                   # [T][H][D]
    nv = v_cache[blk].gather(3, off.view(-1, 1, 1, 1).expand(-1, H, D, 1)).squeeze(3)  # [T][H][D]
    if is_fp8:
        f8k = nk.view(torch.float8_e4m3fn).to(torch.float32) * k_scale[blk][:, None, None]
        f8v = nv.view(torch.float8_e4m3fn).to(torch.float32) * v_scale[blk][:, None, None]
        new_key = f8k.to(DTYPES[q_dtype]).contiguous()
        new_value = f8v.to(DTYPES[q_dtype]).contiguous()
    else:
        new_key, new_value = nk.contiguous(), nv.contiguous()

    if scale is None:
        scale = 1.0 / math.sqrt(D)
    return Batch(name=name, seed=seed, num_heads=num_heads, num_kv_heads=num_kv_heads, head_size=D,
                 q_dtype=q_dtype, cache_dtype=cache_dtype, scale=float(scale),
                 sliding_window=int(sliding_window),
                 context_lens=np.asarray(ctx_lens, dtype=np.int32),
                 q_lens=np.asarray(q_lens, dtype=np.int32), block_table=table, num_blocks=NB,
                 slot_mapping=slot_mapping, query=query, k_cache=k_cache, v_cache=v_cache,
                 k_scale=k_scale, v_scale=v_scale, new_key=new_key, new_value=new_value,
                 shared_groups=[list(g) for g in shared_groups],
                 shared_prefix=dict(shared_prefix or {}))


@dataclass
class SparseChoice:
    """Chosen logical blocks per sequence as pa_decode_sparse takes them."""
    selected: np.ndarray      # int32 [S][width] (entries past num_selected are -1)
    num_selected: np.ndarray  # int32 [S]
    chosen: List[List[int]]   # per sequence: the distinct valid blocks, ascending, newest last

    def device(self, device) -> Dict[str, torch.Tensor]:
        return {"selected": torch.from_numpy(self.selected).to(device),
                "num_selected": torch.from_numpy(self.num_selected).to(device)}


def make_sparse_batch(name: str, seed: int, ctx_lens: Sequence[int], k_blocks: int, num_heads: int,
                      num_kv_heads: int, head_size: int, q_dtype: str = "bf16", cache_dtype: str = "bf16",
                      device="cpu", noise: bool = False, chunk_blocks: int = 16384):
    """A decode batch where each sequence's indexer picked k_blocks of its
    earlier blocks (distinct, uniform over [0, newest block), listed in a
    random order). Only the chosen blocks and the newest block own physical
    blocks with data; every other logical block points at one shared block
    of NaN, so a read of an unchosen block shows in the output. With
    ``noise`` the lists also carry repeats, the newest block, ids past it
    and negative ids (to be ignored), and a tail past num_selected that names
    unchosen blocks (never to be read). Returns (Batch, SparseChoice)."""
    rng = np.random.default_rng(seed)
    ctx_lens = [int(c) for c in ctx_lens]
    S = len(ctx_lens)
    lists, chosen = [], []
    for c in ctx_lens:
        nbk = -(-c // BLOCK)
        k = min(k_blocks, nbk - 1)
        pick = rng.choice(nbk - 1, size=k, replace=False).astype(np.int64) if k > 0 else np.zeros(0, np.int64)
        lst = pick.tolist()
        if noise:
            lst += [int(x) for x in rng.choice(pick, size=min(3, k))] if k else []
            lst += [nbk - 1, nbk, nbk + 7, -1, -5]
        rng.shuffle(lst)
        lists.append(lst)
        chosen.append(sorted(int(x) for x in pick) + [nbk - 1])
    tail = 2 if noise else 0
    width = max(1, max(len(x) for x in lists) + tail)
    selected = np.full((S, width), -1, dtype=np.int32)
    num_selected = np.zeros(S, dtype=np.int32)
    for s, lst in enumerate(lists):
        selected[s, :len(lst)] = lst
        num_selected[s] = len(lst)
        nbk = -(-ctx_lens[s] // BLOCK)
        unchosen = sorted(set(range(nbk - 1)) - set(chosen[s]))
        for t in range(tail):
            if unchosen:
                selected[s, len(lst) + t] = unchosen[t % len(unchosen)]
    total = sum(len(x) for x in chosen)
    NB = total + 1
    perm = rng.permutation(NB).astype(np.int32)
    poison_block = int(perm[-1])
    stride = max(-(-c // BLOCK) for c in ctx_lens)
    table = np.full((S, stride), poison_block, dtype=np.int32)
    nxt = 0
    for s, blks in enumerate(chosen):
        for b in blks:
            table[s, b] = perm[nxt]
            nxt += 1
    used = perm[:nxt]
    batch = _finish_batch(name, seed, ctx_lens, [1] * S, num_heads, num_kv_heads, head_size, q_dtype, cache_dtype,
                          0, None, device, table, NB, used, chunk_blocks)
    return batch, SparseChoice(selected, num_selected, chosen)


@dataclass
class MlaBatch:
    """Decode batch over a paged latent (MLA) cache."""
    name: str
    num_heads: int
    head_dim_k: int
    scale: float
    context_lens: np.ndarray   # int32 [S]
    block_table: np.ndarray    # int32 [S][stride]
    query: torch.Tensor        # bf16 [S][H][dk]
    cache: torch.Tensor        # bf16 [NB][16][dk]

    @property
    def num_seqs(self) -> int:
        return int(len(self.context_lens))

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max())

    def latent_bytes_read(self) -> int:
        """Algorithmic bytes one decode reads: every cached row once (shared by
        all heads), plus the queries."""
        return int(self.context_lens.sum()) * self.head_dim_k * 2 + self.query.numel() * 2


def make_mla_batch(name: str, seed: int, ctx_lens: Sequence[int], num_heads: int, head_dim_k: int,
                   device="cpu", extra_blocks: int = 0, scale: Optional[float] = None,
                   chunk_blocks: int = 16384) -> MlaBatch:
    """Latent rows and absorbed queries ~ N(0, 1) rounded to bf16; block ids a
    seeded permutation of the pool; every slot no sequence owns is NaN."""
    rng = np.random.default_rng(seed)
    ctx_lens = [int(c) for c in ctx_lens]
    table, NB, used = _assign_blocks(rng, ctx_lens, (), {}, extra_blocks, None)
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    cache = torch.empty((NB, BLOCK, head_dim_k), dtype=torch.bfloat16, device=device)
    for b0 in range(0, NB, chunk_blocks):
        b1 = min(NB, b0 + chunk_blocks)
        cache[b0:b1] = torch.randn((b1 - b0, BLOCK, head_dim_k), generator=gen, device=device).to(torch.bfloat16)
    owned = torch.zeros((NB, BLOCK), dtype=torch.bool)
    owned[torch.from_numpy(np.asarray(used, dtype=np.int64))] = True
    for s, c in enumerate(ctx_lens):
        if c % BLOCK:
            owned[int(table[s, (c - 1) // BLOCK]), c % BLOCK:] = False
    cache.masked_fill_(~owned.to(device)[:, :, None], float("nan"))
    query = torch.randn((len(ctx_lens), num_heads, head_dim_k), generator=gen, device=device).to(torch.bfloat16)
    if scale is None:
        scale = 1.0 / math.sqrt(head_dim_k)
    return MlaBatch(name, num_heads, head_dim_k, float(scale), np.asarray(ctx_lens, dtype=np.int32), table, query,
                    cache)


def make_mla_config(device="cpu") -> MlaBatch:
    """Latent-cache decode shaped like the pages' MLA models: 64 sequences,
    contexts U{4096..32768}, 128 heads, rows of 576 (512 latent + 64), bf16."""
    rng = np.random.default_rng(7)
    ctx = rng.integers(4096, 32769, 64).tolist()
    return make_mla_batch("mla_decode", 7, ctx, 128, 576, device=device)


def make_sparse_config(device="cpu"):
    """Long-context sparse decode: 64 sequences, contexts U{32768..524288},
    128 chosen blocks (2048 keys) plus the newest block each, 32/8 heads,
    d 128, bf16; the Llama-shaped decode's heads at the long contexts where
    sparse attention pays."""
    rng = np.random.default_rng(6)
    ctx = rng.integers(32768, 524289, 64).tolist()
    return make_sparse_batch("sparse_decode", 6, ctx, 128, 32, 8, 128, "bf16", "bf16", device=device)


# ----------------------------------------------------------------------------
# the named configurations (one attention layer each)
# ----------------------------------------------------------------------------
CONFIG_NAMES = ("tiny_decode", "llama8b_decode", "agentic_decode", "mixed_step", "fp8_decode",
                "fp8_swa128")


def config_spec(name: str):
    """(make_batch keyword arguments, numpy rng) of a named configuration; the
    rng has already drawn the context lengths and continues into block
    assignment, so make_batch(**kw, rng=rng) reproduces make_config(name)."""
    if name == "tiny_decode":
        # 4 sequences, contexts {17, 40, 64, 100}, 8/2 heads, d 64, fp32, a
        # 64-block pool with the table drawn from a seeded shuffle
        return dict(name=name, seed=1, ctx_lens=[17, 40, 64, 100], q_lens=[1] * 4, num_heads=8,
                    num_kv_heads=2, head_size=64, q_dtype="f32", cache_dtype="f32",
                    pool_blocks=64), np.random.default_rng(1)
    if name == "llama8b_decode":
        # Llama-3-8B-shaped decode: 64 sequences, contexts U{1024..8192}, 32/8, d 128, bf16
        rng = np.random.default_rng(2)
        ctx = rng.integers(1024, 8193, 64).tolist()
        return dict(name=name, seed=2, ctx_lens=ctx, q_lens=[1] * 64, num_heads=32, num_kv_heads=8,
                    head_size=128, q_dtype="bf16", cache_dtype="bf16"), rng
    if name == "agentic_decode":
        # 16 sequences in 4 groups of 4; per group L ~ LogNormal(ln 142000, 0.5)
        # capped at 262144; the first 16*floor(0.96 L / 16) tokens share blocks
        rng = np.random.default_rng(3)
        ctx, groups, prefix = [], [], {}
        for gi in range(4):
            L = int(min(262144, round(float(rng.lognormal(math.log(142000), 0.5)))))
            groups.append(list(range(4 * gi, 4 * gi + 4)))
            prefix[gi] = BLOCK * int(0.96 * L // BLOCK)
            ctx += [L] * 4
        return dict(name=name, seed=3, ctx_lens=ctx, q_lens=[1] * 16, num_heads=32, num_kv_heads=8,
                    head_size=128, q_dtype="bf16", cache_dtype="bf16", shared_groups=groups,
                    shared_prefix=prefix), rng
    if name == "mixed_step":
        # 8192-token budget step: 192 decode sequences (contexts U{4096..32768})
        # then one 2048-token chunk on a 65536-token cached prefix
        rng = np.random.default_rng(4)
        ctx = rng.integers(4096, 32769, 192).tolist() + [65536 + 2048]
        return dict(name=name, seed=4, ctx_lens=ctx, q_lens=[1] * 192 + [2048], num_heads=32,
                    num_kv_heads=8, head_size=128, q_dtype="bf16", cache_dtype="bf16"), rng
    if name in ("fp8_decode", "fp8_swa128"):
        # 128 sequences, contexts U{8192..131072}, 64/8, d 128, bf16 queries,
        # fp8 e4m3 pool with per-block scales; the second variant reads only
        # the last 128 positions
        rng = np.random.default_rng(5)
        ctx = rng.integers(8192, 131073, 128).tolist()
        w = 128 if name == "fp8_swa128" else 0
        return dict(name=name, seed=5, ctx_lens=ctx, q_lens=[1] * 128, num_heads=64, num_kv_heads=8,
                    head_size=128, q_dtype="bf16", cache_dtype="fp8_e4m3", sliding_window=w), rng
    raise KeyError(name)


def plan_config(name: str):
    """Metadata of a named configuration without drawing any values:
    (spec kwargs, block_table, num_blocks)."""
    kw, rng = config_spec(name)
    table, NB, _ = _assign_blocks(rng, kw["ctx_lens"], kw.get("shared_groups", ()),
                                  kw.get("shared_prefix") or {}, kw.get("extra_blocks", 0),
                                  kw.get("pool_blocks"))
    return kw, table, NB


def make_config(name: str, device="cpu") -> Batch:
    kw, rng = config_spec(name)
    return make_batch(device=device, rng=rng, **kw)
