"""Benchmark of the paged-KV hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--runs R] [--gpus 1] [--only NAME[,NAME...]]
                    [--no-cpu-baseline] [--cpu-budget S] [--no-ceilings] [--profile-pass]

Headline (the JSON line on stdout): decode KV GB/s on the largest decode
workload that fits one GPU, fp8_decode (128 sequences, contexts
U{8192..131072}, 64 query / 8 KV heads, head size 128, fp8 e4m3 K/V with
per-block fp32 scales, bf16 queries, 16-token blocks, one attention layer).
One step = the KV write of the 128 new tokens + paged decode over every
sequence, inputs resident in HBM; K steps are timed between two
synchronisations and value = algorithmic K+V bytes per step / step time.

Every other named workload is measured in the same run under "configs",
each call timed alone with HIP events over R runs (median, min, max), a 1 GiB
scratch write between runs so that no run finds its data in the 256 MB
last-level cache; each carries its own roofline object and the CPU oracle
timed on a bounded sample of the same batch. Everything is one attention
layer.
"""

from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, published
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16, published
FLUSH_BYTES = 1 << 30           # scratch write between timed runs (the MALL is 256 MB)

METRIC = "paged-attn decode KV GB/s (% HBM peak); mixed-step tokens/s on 1 MI355X"

# measured workloads, in run order (the first is the headline)
CONFIG_ORDER = ("fp8_decode", "llama8b_decode", "llama8b_decode_valu", "agentic_decode",
                "agentic_decode_shared_prefix", "fp8_swa128", "tiny_decode", "mixed_step", "sparse_decode",
                "mla_decode", "mla_decode_16h")

WORKLOADS = {
    "fp8_decode": "128 sequences, context U{8192..131072}, 64 query / 8 KV heads, head 128, fp8 e4m3 K/V with "
                  "per-block fp32 scales, bf16 queries; pa_decode",
    "llama8b_decode": "64 sequences, context U{1024..8192}, 32/8 heads, head 128, bf16; pa_decode",
    "llama8b_decode_valu": "the llama8b batch through pa_decode_valu (the vector-ALU kernel: wave-shuffle dot "
                           "products and softmax reductions), for side-by-side comparison",
    "agentic_decode": "16 sequences in 4 groups sharing 96% of their context (lognormal, median 142K, cap 256K), "
                      "32/8 heads, head 128, bf16; pa_decode (shared blocks read once per member)",
    "agentic_decode_shared_prefix": "the agentic batch through pa_decode_shared_prefix (shared blocks read once "
                                    "per group)",
    "fp8_swa128": "the fp8_decode batch with a 128-token sliding window (the last 8-9 blocks per sequence)",
    "tiny_decode": "4 sequences, contexts {17,40,64,100}, 8/2 heads, head 64, fp32; pa_decode",
    "mixed_step": "192 decode rows (context U{4096..32768}) + one 2048-token chunk on a 65536-token prefix, "
                  "32/8 heads, head 128, bf16; step = KV write of the 2240 new tokens + pa_prefill_chunk "
                  "(the decode rows on a second stream beside the chunk)",
    "sparse_decode": "64 sequences, context U{32768..524288}, 128 chosen blocks + the newest each, 32/8 heads, "
                     "head 128, bf16; pa_decode_sparse",
    "mla_decode": "64 sequences, context U{4096..32768}, 128 heads sharing one latent row per token (512 + 64, "
                  "bf16), absorbed queries; pa_mla_decode",
    "mla_decode_16h": "the latent batch with 16 heads (one GPU's share of 128 under 8-way tensor parallelism); "
                      "pa_mla_decode",
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ----------------------------------------------------------------------------
# calls
# ----------------------------------------------------------------------------
def decode_step_fns(pa, torch, b, shared_prefix=False, valu=False):
    m = b.meta("cuda")
    out = torch.empty_like(b.query)
    if shared_prefix:
        gm = b.group_meta("cuda")
        ng = gm["group_prefix_len"].numel()
        n = pa.decode_shared_prefix_workspace_bytes(b.num_seqs, ng, b.max_context_len, b.num_heads,
                                                    b.num_kv_heads, b.head_size, b.cache_dtype, b.sliding_window)
    else:
        n = (pa.decode_valu_workspace_bytes if valu else pa.decode_workspace_bytes)(
            b.num_seqs, b.max_context_len, b.num_heads, b.num_kv_heads, b.head_size, b.cache_dtype, b.sliding_window)
    ws = torch.empty(max(n, 1), dtype=torch.uint8, device="cuda")

    def write():
        pa.reshape_and_cache(b.new_key, b.new_value, b.k_cache, b.v_cache, m["slot_mapping"], b.k_scale, b.v_scale)

    if shared_prefix:
        def attend():
            pa.decode_shared_prefix(out, b.query, b.k_cache, b.v_cache, m["block_table"], m["context_lens"],
                                    b.max_context_len, gm["cu_groups"], gm["group_prefix_len"], b.scale, b.k_scale,
                                    b.v_scale, b.sliding_window, ws)
    else:
        call = pa.decode_valu if valu else pa.decode

        def attend():
            call(out, b.query, b.k_cache, b.v_cache, m["block_table"], m["context_lens"], b.max_context_len, b.scale,
                 b.k_scale, b.v_scale, b.sliding_window, ws)
    return write, attend


def prefill_step_fns(pa, torch, b):
    m = b.meta("cuda")
    out = torch.empty_like(b.query)
    n = pa.prefill_workspace_bytes(b.num_seqs, b.num_q_tokens, b.max_q_len, b.max_context_len, b.num_heads,
                                   b.num_kv_heads, b.head_size, b.cache_dtype, b.sliding_window)
    ws = torch.empty(max(n, 1), dtype=torch.uint8, device="cuda")

    def write():
        pa.reshape_and_cache(b.new_key, b.new_value, b.k_cache, b.v_cache, m["slot_mapping"], b.k_scale, b.v_scale)

    def attend():
        pa.prefill_chunk(out, b.query, b.k_cache, b.v_cache, m["block_table"], m["cu_seqlens"], m["context_lens"],
                         b.max_q_len, b.max_context_len, b.scale, b.k_scale, b.v_scale, b.sliding_window, ws)

    return write, attend


def sparse_step_fns(pa, torch, b, choice):
    m = b.meta("cuda")
    c = choice.device("cuda")
    out = torch.empty_like(b.query)
    ms = choice.selected.shape[1]
    n = pa.decode_sparse_workspace_bytes(b.num_seqs, ms, b.num_heads, b.num_kv_heads, b.head_size, b.cache_dtype)
    ws = torch.empty(max(n, 1), dtype=torch.uint8, device="cuda")

    def attend():
        pa.decode_sparse(out, b.query, b.k_cache, b.v_cache, m["block_table"], m["context_lens"], b.max_context_len,
                         c["selected"], c["num_selected"], b.scale, b.k_scale, b.v_scale, ws)

    return attend


def mla_fn(pa, torch, b):
    out = torch.empty((b.num_seqs, b.num_heads, 512), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(max(pa.mla_decode_workspace_bytes(b.num_seqs, b.num_heads), 1), dtype=torch.uint8,
                     device="cuda")
    bt = torch.from_numpy(b.block_table).to("cuda")
    cl = torch.from_numpy(b.context_lens).to("cuda")

    def attend():
        pa.mla_decode(out, b.query, b.cache, bt, cl, b.max_context_len, b.scale, ws)

    return attend


def chunk_of(mb):
    """The mixed step's last sequence (the 2048-token chunk on its 65,536-token
    prefix) as a batch of its own, sharing the mixed step's device buffers."""
    import copy
    chunk = copy.copy(mb)
    chunk.device_meta = {}
    s = mb.num_seqs - 1
    cu = mb.cu_seqlens
    chunk.context_lens = mb.context_lens[s:s + 1].copy()
    chunk.q_lens = mb.q_lens[s:s + 1].copy()
    chunk.block_table = mb.block_table[s:s + 1].copy()
    chunk.query = mb.query[cu[s]:cu[s + 1]].contiguous()
    chunk.slot_mapping = mb.slot_mapping[cu[s]:cu[s + 1]].copy()
    chunk.new_key = mb.new_key[cu[s]:cu[s + 1]].contiguous()
    chunk.new_value = mb.new_value[cu[s]:cu[s + 1]].contiguous()
    return chunk


def decode_rows_of(mb):
    """The mixed step's 192 one-token rows as a batch of their own."""
    import copy
    d = copy.copy(mb)
    d.device_meta = {}
    n = mb.num_seqs - 1
    cu = mb.cu_seqlens
    d.context_lens = mb.context_lens[:n].copy()
    d.q_lens = mb.q_lens[:n].copy()
    d.block_table = mb.block_table[:n].copy()
    d.query = mb.query[:cu[n]].contiguous()
    d.slot_mapping = mb.slot_mapping[:cu[n]].copy()
    d.new_key = mb.new_key[:cu[n]].contiguous()
    d.new_value = mb.new_value[:cu[n]].contiguous()
    return d


# ----------------------------------------------------------------------------
# timing
# ----------------------------------------------------------------------------
class Flusher:
    """A 1 GiB scratch write on the current stream: whatever a call read last
    is gone from the 256 MB last-level cache when the next run starts."""

    def __init__(self, torch):
        self.buf = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device="cuda")
        self.n = 0

    def __call__(self):
        self.n += 1
        self.buf.fill_(self.n & 0xFF)


def time_runs(torch, fn, runs, warmup, flush):
    """R runs of fn, each bracketed by HIP events on the launch stream, a
    flush before each; returns median/min/max/mean in ms."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(runs)]
    for a, c in ev:
        flush()
        a.record()
        fn()
        c.record()
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(c) for a, c in ev)
    mid = ms[len(ms) // 2] if len(ms) % 2 else 0.5 * (ms[len(ms) // 2 - 1] + ms[len(ms) // 2])
    return {"median_ms": round(mid, 5), "min_ms": round(ms[0], 5), "max_ms": round(ms[-1], 5),
            "mean_ms": round(sum(ms) / len(ms), 5), "runs": runs, "flush_bytes_between_runs": FLUSH_BYTES}


def graph_call_us(torch, attend, calls=16, replays=20):
    """Mean device time of one call when `calls` of them are captured back to
    back in one HIP graph and the graph is replayed: the figure a serving loop
    that replays its small launches sees, without this script's per-call host
    overhead (ctypes marshalling and the launch)."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        attend()  # outside the capture: first-call work stays out of the graph
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(calls):
            attend()
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(replays):
        g.replay()
    t1.record()
    torch.cuda.synchronize()
    us = t0.elapsed_time(t1) * 1e3 / (replays * calls)
    del g
    return round(us, 2)


# ----------------------------------------------------------------------------
# algorithmic work
# ----------------------------------------------------------------------------
def causal_flops(b):
    """Algorithmic MFMA flops of the chunks longer than one token: 4*d per
    visible (query, key) pair per query head (QK^T and PV)."""
    pairs = 0
    for ctx, ql in zip(b.context_lens.tolist(), b.q_lens.tolist()):
        if ql <= 1:
            continue
        for r in range(ql):
            p = ctx - ql + r
            lo = 0 if b.sliding_window <= 0 else max(0, p - b.sliding_window + 1)
            pairs += p - lo + 1
    return 4.0 * b.head_size * pairs * b.num_heads


def sparse_kv_bytes(b, choice):
    """K+V bytes a sparse decode reads: the keys of every chosen block (the
    newest block up to the context end)."""
    toks = 0
    for ctx, blks in zip(b.context_lens.tolist(), choice.chosen):
        nbk = -(-ctx // 16)
        toks += 16 * (len(blks) - 1) + ctx - 16 * (nbk - 1)
    e = {"bf16": 2, "f32": 4, "fp8_e4m3": 1}[b.cache_dtype]
    return toks * b.num_kv_heads * b.head_size * 2 * e


# ----------------------------------------------------------------------------
# stored counter summaries (profiles/)
# ----------------------------------------------------------------------------
DECODE_SOURCES = ("decode_mfma.hip", "decode.hip", "pa_api.cpp", "pa_device.h", "pa_internal.h")
PREFILL_SOURCES = ("prefill_bf16.hip", "prefill_tiles.h", "decode_mfma.hip", "decode.hip", "reshape_and_cache.hip",
                   "pa_api.cpp", "pa_device.h", "pa_internal.h")
MLA_SOURCES = ("mla_decode.hip", "pa_api.cpp", "pa_device.h", "pa_internal.h")
SPARSE_SOURCES = ("sparse_select.hip", "sparse_pick.h", "decode_mfma.hip", "decode.hip", "pa_api.cpp", "pa_device.h", "pa_internal.h")
SOURCES_OF = {"fp8_decode": DECODE_SOURCES, "llama8b_decode": DECODE_SOURCES, "llama8b_decode_valu": DECODE_SOURCES,
              "agentic_decode": DECODE_SOURCES,
              "agentic_decode_shared_prefix": DECODE_SOURCES, "fp8_swa128": DECODE_SOURCES,
              "tiny_decode": DECODE_SOURCES, "mixed_step": PREFILL_SOURCES, "sparse_decode": SPARSE_SOURCES,
              "mla_decode": MLA_SOURCES, "mla_decode_16h": MLA_SOURCES}


# committed rocprofv3 summary of each workload (named for its main kernel)
PROFILE_OF = {"fp8_decode": "decode_mfma_split_fp8_decode", "llama8b_decode": "decode_mfma_split_llama8b_decode",
              "llama8b_decode_valu": "decode_partition_kernel_llama8b_decode",
              "agentic_decode": "decode_mfma_split_agentic_decode",
              "agentic_decode_shared_prefix": "decode_mfma_split_shared_prefix_agentic_decode",
              "fp8_swa128": "decode_mfma_split_fp8_swa128", "tiny_decode": "decode_partition_kernel_tiny_decode",
              "mixed_step": "prefill_bf16_kernel_mixed_step", "sparse_decode": "decode_sparse_sparse_decode",
              "mla_decode": "mla_decode_wide_mla_decode_128h", "mla_decode_16h": "mla_decode_narrow_mla_decode_16h"}


def kernel_source_digest(files):
    """sha256 over the sources of a call's path (kernels, shared device code,
    planning), used to tell whether a stored counter summary still describes
    the code that runs."""
    import hashlib
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "paged_kv_cache_103_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def stored_traffic(name, key="call"):
    """HBM bytes per call on workload `name` from its committed rocprofv3
    counter summary (FETCH_SIZE and WRITE_SIZE scaled by the plain-copy
    calibration), or None if missing or taken on other sources."""
    import re
    path = os.path.join(ROOT, "profiles", f"{PROFILE_OF[name]}.md")
    try:
        text = open(path).read()
    except OSError:
        return None
    m = re.search(r"<!-- traffic (\{.*?\}) -->", text)
    if not m:
        return None
    t = json.loads(m.group(1))
    if t.get("kernel_source_sha256") != kernel_source_digest(SOURCES_OF[name]):
        return None
    v = t.get(key)
    return None if v is None else int(v["fetch_bytes"]) + int(v["write_bytes"])


def hbm_roofline(nbytes, ms, name, kernel, key="call"):
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"bound": "hbm", "kernel": kernel, "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": stored_traffic(name, key),
            "algorithmic_bytes_per_launch": int(nbytes)}


def mfma_roofline(flops, ms, name, kernel, key):
    tf = flops / (ms * 1e-3) / 1e12
    return {"bound": "mfma", "kernel": kernel, "achieved": round(tf, 2), "peak": BF16_MFMA_PEAK_TFLOPS,
            "unit": "TFLOP/s", "frac": round(tf / BF16_MFMA_PEAK_TFLOPS, 4), "traffic": stored_traffic(name, key),
            "algorithmic_flops_per_launch": float(flops)}


# ----------------------------------------------------------------------------
# the oracle on the host (cpu_baseline)
# ----------------------------------------------------------------------------
def host_info():
    model = platform.processor() or ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas = None
    affinity = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None
    return {"cpu_model": model, "os_cpu_count": os.cpu_count(), "usable_cpus": affinity, "blas_threads": blas}


def cpu_baseline(units, budget_s, unit, sample):
    """The oracle as it stands, timed on a bounded sample: `units` yields
    (callable, work) pairs, evaluated in order (and again from the start)
    until about budget_s seconds are spent; value = work done / seconds."""
    info = host_info()
    done, secs, work = 0, 0.0, 0.0
    items = list(units)
    while secs <= budget_s and items:
        for fn, w in items:
            t = time.perf_counter()
            fn()
            secs += time.perf_counter() - t
            done += 1
            work += w
            if secs > budget_s:
                break
    scale = 1e9 if unit == "GB/s" else 1.0
    return {"value": round(work / secs / scale, 4), "unit": unit, "cores": info["blas_threads"] or info["os_cpu_count"],
            "kind": "oracle", "sample": f"{done} evaluations of {sample}, {secs:.1f} s",
            "host": info}


def decode_units(b):
    from tests.helpers import oracle_rows
    e = {"f32": 4, "bf16": 2, "fp8_e4m3": 1}[b.cache_dtype]
    for s in range(b.num_seqs):
        ctx = int(b.context_lens[s])
        lo = 0 if b.sliding_window <= 0 else max(0, ctx - b.sliding_window)
        yield (lambda s=s: oracle_rows(b, [s])), (ctx - lo) * b.num_kv_heads * b.head_size * 2 * e


def mixed_units(b):
    """The step's new tokens: decode rows (whole one-token sequences)
    alternating with chunk rows, every 64th row of the chunk (row r at
    position p attends exactly as a one-token query over the first p + 1
    keys)."""
    import numpy as np
    import torch

    import oracle
    from tests.helpers import ORACLE_DTYPE, oracle_rows, raw
    s_chunk = b.num_seqs - 1
    cu = b.cu_seqlens
    ctx = int(b.context_lens[s_chunk])
    ql = int(b.q_lens[s_chunk])

    def chunk_row(r):
        p = ctx - ql + r
        phys = b.block_table[s_chunk, :p // 16 + 1]
        t = torch.from_numpy(phys.astype(np.int64)).to(b.k_cache.device)
        kp, vp = raw(b.k_cache.index_select(0, t)), raw(b.v_cache.index_select(0, t))
        qf = oracle.formats.to_f64(raw(b.query[cu[s_chunk] + r:cu[s_chunk] + r + 1]), ORACLE_DTYPE[b.q_dtype])
        oracle.attend_sequence(qf, kp, vp, ORACLE_DTYPE[b.cache_dtype], None, None, np.arange(len(phys)), p + 1,
                               b.num_kv_heads, b.scale, 0)

    rows = list(range(0, ql, 64))
    for i in range(max(s_chunk, len(rows))):
        if i < s_chunk:
            yield (lambda s=i: oracle_rows(b, [s])), 1
        if i < len(rows):
            yield (lambda r=rows[i]: chunk_row(r)), 1


def sparse_units(b, choice):
    import numpy as np
    import torch

    import oracle
    from tests.helpers import ORACLE_DTYPE, raw
    e = {"f32": 4, "bf16": 2, "fp8_e4m3": 1}[b.cache_dtype]
    for s in range(b.num_seqs):
        def one(s=s):
            ctx = int(b.context_lens[s])
            nbk = -(-ctx // 16)
            blks = choice.chosen[s]
            phys = torch.tensor([int(b.block_table[s, x]) for x in blks], dtype=torch.int64, device=b.k_cache.device)
            kp, vp = raw(b.k_cache.index_select(0, phys)), raw(b.v_cache.index_select(0, phys))
            row = np.zeros(nbk, dtype=np.int64)
            row[blks] = np.arange(len(blks))
            n = int(choice.num_selected[s])
            qf = oracle.formats.to_f64(raw(b.query[s:s + 1]), ORACLE_DTYPE[b.q_dtype])
            oracle.attend_selected_blocks(qf, kp, vp, ORACLE_DTYPE[b.cache_dtype], None, None, row, ctx,
                                          choice.selected[s, :n], b.num_kv_heads, b.scale)
        ctx = int(b.context_lens[s])
        keys = 16 * (len(choice.chosen[s]) - 1) + ctx - 16 * (-(-ctx // 16) - 1)
        yield one, keys * b.num_kv_heads * b.head_size * 2 * e


def mla_units(b):
    import numpy as np
    import torch

    from oracle import formats as F
    from oracle import mla as M
    from tests.helpers import raw
    for s in range(b.num_seqs):
        def one(s=s):
            ctx = int(b.context_lens[s])
            nbk = -(-ctx // 16)
            phys = torch.from_numpy(b.block_table[s, :nbk].astype(np.int64)).to(b.cache.device)
            pool = raw(b.cache.index_select(0, phys))
            M.mla_decode_sequence(F.to_f64(raw(b.query[s]), F.BF16), pool, F.BF16, np.arange(nbk), ctx, b.scale, 512)
        yield one, int(b.context_lens[s]) * b.head_dim_k * 2


# ----------------------------------------------------------------------------
# measurement of each workload
# ----------------------------------------------------------------------------
def measure(name, pa, torch, W, args, flush):
    """One workload: build it, time its call(s), roofline, oracle baseline."""
    cpu = not args.no_cpu_baseline
    budget = args.cpu_budget
    res = {"workload": WORKLOADS[name]}
    if name in ("fp8_decode", "llama8b_decode", "llama8b_decode_valu", "agentic_decode", "fp8_swa128",
                "tiny_decode", "agentic_decode_shared_prefix"):
        base = {"agentic_decode_shared_prefix": "agentic_decode", "llama8b_decode_valu": "llama8b_decode"}
        b = W.make_config(base.get(name, name), device="cuda")
        write, attend = decode_step_fns(pa, torch, b, shared_prefix=name == "agentic_decode_shared_prefix",
                                        valu=name == "llama8b_decode_valu")
        t = time_runs(torch, attend, args.runs, args.warmup, flush)
        res["timing"] = t
        nbytes, unique = b.kv_bytes_read(), b.unique_kv_bytes_read()
        res["kv_bytes_per_call"] = nbytes
        kernel = ("pa_decode_shared_prefix: decode_mfma_split<..., true> + decode_split_merge"
                  if name == "agentic_decode_shared_prefix" else
                  "pa_decode_valu: decode_partition_kernel + decode_merge_kernel" if name == "llama8b_decode_valu" else
                  "pa_decode: " + ("decode_partition_kernel + decode_merge_kernel" if b.cache_dtype == "f32"
                                   else "decode_mfma_split" + ("" if b.max_context_len <= 256 or
                                                                (0 < b.sliding_window <= 240)
                                                                else " + decode_split_merge")))
        if name.startswith("agentic"):
            # the HBM bytes the method must move are the unique ones; the
            # logical (per-member) rate is what the call delivers
            res["unique_kv_bytes_per_call"] = unique
            res["logical_gbs"] = round(nbytes / (t["median_ms"] * 1e-3) / 1e9, 2)
            res["roofline"] = hbm_roofline(unique, t["median_ms"], name, kernel)
        else:
            res["roofline"] = hbm_roofline(nbytes, t["median_ms"], name, kernel)
        res["value"] = res["roofline"]["achieved"]
        res["unit"] = "GB/s"
        if name in ("fp8_swa128", "tiny_decode"):
            res["call_us_graph_replay"] = graph_call_us(torch, attend)
        if cpu and name not in ("agentic_decode_shared_prefix", "llama8b_decode_valu"):
            res["cpu_baseline"] = cpu_baseline(decode_units(b), budget, "GB/s",
                                               f"whole sequences of the same batch (all heads) in order, "
                                               f"K+V bytes of the keys each reads")
        return res, (b, write, attend)
    if name == "mixed_step":
        b = W.make_config("mixed_step", device="cuda")
        write, attend = prefill_step_fns(pa, torch, b)

        def step():
            write()
            attend()

        t = time_runs(torch, step, max(10, args.runs // 2), args.warmup, flush)
        res["timing"] = t
        res["new_tokens"] = b.num_q_tokens
        res["value"] = round(b.num_q_tokens / (t["median_ms"] * 1e-3), 1)
        res["unit"] = "tokens/s"
        # the chunk alone (the prefill kernel only), its MFMA roofline
        chunk = chunk_of(b)
        _, pre = prefill_step_fns(pa, torch, chunk)
        tc = time_runs(torch, pre, args.runs, args.warmup, flush)
        flops = causal_flops(chunk)
        res["chunk"] = {"timing": tc, "flops": flops,
                        "roofline": mfma_roofline(flops, tc["median_ms"], name, "prefill_bf16_kernel<128, 4, 1>",
                                                  "chunk")}
        # the 192 decode rows alone (the decode kernels of the step)
        rows = decode_rows_of(b)
        _, dec = decode_step_fns(pa, torch, rows)
        td = time_runs(torch, dec, args.runs, args.warmup, flush)
        dbytes = rows.kv_bytes_read()
        res["decode_rows"] = {"timing": td, "roofline": hbm_roofline(dbytes, td["median_ms"], name,
                                                                      "decode_mfma_split + decode_split_merge",
                                                                      "decode_rows")}
        # the step's own rooflines: serial (sum of the two bounds) and
        # overlapped (max of them), at the published peaks
        t_hbm = dbytes / (HBM_PEAK_GBS * 1e9) * 1e3
        t_mfma = flops / (BF16_MFMA_PEAK_TFLOPS * 1e12) * 1e3
        res["roofline"] = {"bound": "hbm+mfma",
                           "kernel": "pa_prefill_chunk step: write, then prefill_bf16_kernel beside decode_side + "
                                     "decode_split_merge (two streams)",
                           "achieved_ms": t["median_ms"], "roofline_ms_serial": round(t_hbm + t_mfma, 4),
                           "roofline_ms_overlapped": round(max(t_hbm, t_mfma), 4),
                           "frac_serial": round((t_hbm + t_mfma) / t["median_ms"], 4),
                           "frac_overlapped": round(max(t_hbm, t_mfma) / t["median_ms"], 4),
                           "traffic": stored_traffic(name, "call")}
        # the same chunk over an fp8 e4m3 cache
        del chunk, rows
        fb = W.make_batch("mixed_step_chunk_fp8", 4, [65536 + 2048], [2048], 32, 8, 128, "bf16", "fp8_e4m3",
                          device="cuda")
        _, f8 = prefill_step_fns(pa, torch, fb)
        tf = time_runs(torch, f8, args.runs, args.warmup, flush)
        res["chunk_fp8_cache"] = {"timing": tf,
                                  "roofline": mfma_roofline(causal_flops(fb), tf["median_ms"], name,
                                                            "prefill_bf16_kernel<128, 4, 2>", "chunk_fp8")}
        del fb
        if cpu:
            res["cpu_baseline"] = cpu_baseline(mixed_units(b), budget, "tokens/s",
                                               "new tokens of the same step: decode rows alternating with every "
                                               "64th row of the chunk (each over its own causal prefix)")
        return res, (b, write, attend)
    if name == "sparse_decode":
        b, choice = W.make_sparse_config(device="cuda")
        attend = sparse_step_fns(pa, torch, b, choice)
        t = time_runs(torch, attend, args.runs, args.warmup, flush)
        nbytes = sparse_kv_bytes(b, choice)
        res.update(timing=t, kv_bytes_per_call=nbytes, dense_kv_bytes=b.kv_bytes_read(),
                   roofline=hbm_roofline(nbytes, t["median_ms"], name,
                                         "pa_decode_sparse: decode_sparse_fused (selection, decode and merge "
                                         "in one launch)"))
        res["value"], res["unit"] = res["roofline"]["achieved"], "GB/s"
        if cpu:
            res["cpu_baseline"] = cpu_baseline(sparse_units(b, choice), budget, "GB/s",
                                               "whole sequences of the same batch over their chosen blocks")
        return res, (b, None, attend)
    if name in ("mla_decode", "mla_decode_16h"):
        if name == "mla_decode":
            b = W.make_mla_config(device="cuda")
        else:
            import numpy as np
            ctx = np.random.default_rng(7).integers(4096, 32769, 64).tolist()
            b = W.make_mla_batch("mla_16_576", 7, ctx, 16, 576, device="cuda")
        attend = mla_fn(pa, torch, b)
        t = time_runs(torch, attend, args.runs, args.warmup, flush)
        nbytes = b.latent_bytes_read()
        flops = 2.0 * b.num_heads * (b.head_dim_k + 512) * int(b.context_lens.sum())
        kernel = ("pa_mla_decode: mla_decode_wide<576> + mla_merge" if b.num_heads == 128 else
                  "pa_mla_decode: mla_decode_narrow<576> + mla_merge")
        res.update(timing=t, bytes_per_call=nbytes, flops_per_call=flops,
                   roofline=hbm_roofline(nbytes, t["median_ms"], name, kernel))
        tf = flops / (t["median_ms"] * 1e-3) / 1e12
        res["roofline"]["mfma_tflops"] = round(tf, 2)
        res["roofline"]["mfma_frac"] = round(tf / BF16_MFMA_PEAK_TFLOPS, 4)
        res["value"], res["unit"] = res["roofline"]["achieved"], "GB/s"
        if cpu:
            res["cpu_baseline"] = cpu_baseline(mla_units(b), budget, "GB/s",
                                               "whole sequences of the same batch (all heads), latent bytes read")
        return res, (b, None, attend)
    raise KeyError(name)


def measure_ceilings(torch):
    """Achievable peaks on this GPU, measured with libpa_peaks next to the
    path: HBM read rate of a paged gather (random 4 KiB tiles, one wave per
    tile, 16-byte nontemporal loads; contiguous 1 KiB per instruction, and the
    decode kernel's key pattern of 64 bytes from each of 16 rows; and the same
    tiles by nontemporal global->LDS copies) and the back-to-back 32x32x16
    bf16 / fp16 MFMA rate."""
    from paged_kv_cache_103_amd import peaks

    res = {}
    nbytes = 4 << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    g = torch.Generator(device="cpu")
    g.manual_seed(0)
    ids = torch.randperm(nbytes // 4096, generator=g).to(torch.int32).cuda()
    sink = torch.empty(256 * 2048, dtype=torch.float32, device="cuda")
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    # (the global->LDS gather with one workgroup of 4 waves per CU, as the
    # side-by-side decode runs: more resident waves read slower)
    for mode, name, grid in ((0, "hbm_tiles_contiguous_gbs", 4096), (1, "hbm_tiles_decode_pattern_gbs", 4096),
                             (2, "hbm_tiles_lds_copies_gbs", ncu)):
        t = time_runs(torch, lambda: peaks.read_tiles(buf, ids, mode, grid, sink), 10, 2, lambda: None)
        res[name] = round(nbytes / (t["median_ms"] * 1e-3) / 1e9, 1)
    del buf, ids
    torch.cuda.empty_cache()
    for kind, name in ((0, "mfma_bf16_tflops"), (1, "mfma_fp16_tflops")):
        flops = [0.0]

        def f():
            flops[0] = peaks.mfma(kind, 2000, 2048, sink)

        t = time_runs(torch, f, 10, 2, lambda: None)
        res[name] = round(flops[0] / (t["median_ms"] * 1e-3) / 1e12, 1)
    # LDS per compute unit (bytes per shader-clock cycle) and the issue mix of
    # a softmax step (cycles per round of 16 MFMAs + 64 FMAs + 16 exp2 per
    # wave), each from s_memtime cycle counts
    cyc = torch.zeros(8 * ncu, dtype=torch.int64, device="cuda")
    for kind, name in ((0, "lds_read16_bytes_per_clk_cu"), (1, "lds_read16_2way_bytes_per_clk_cu"),
                       (2, "lds_write8_bytes_per_clk_cu")):
        nb = peaks.lds(kind, 2000, ncu, sink, cyc)
        torch.cuda.synchronize()
        res[name] = round(nb / float(cyc[:ncu].max().item()), 1)
    mix = {}
    for waves in (4, 8):
        for mode, name in ((0, "mfma"), (1, "valu"), (2, "interleaved")):
            cyc.zero_()
            ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            ev0.record()
            peaks.issue(mode, waves, 1000, ncu, sink, cyc)
            ev1.record()
            torch.cuda.synchronize()
            c = float(cyc.view(ncu, 8)[:, :waves].max().item())
            # cycles of one round per wave (with two waves per SIMD, the SIMD
            # completes two rounds in that time), and the clock they ran at
            mix[f"{name}_{waves // 4}_waves_per_simd_cycles"] = round(c / 1000, 1)
            mix[f"{name}_{waves // 4}_waves_per_simd_clock_ghz"] = round(c / (ev0.elapsed_time(ev1) * 1e6), 2)
    res["softmax_step_issue"] = mix
    return res


def profile_pass(pa, torch, W, names):
    """Only the kernels a counter run needs: a plain 1 GiB device copy (the
    calibration of FETCH_SIZE / WRITE_SIZE), then a few calls of each named
    workload, in measurement order."""
    src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    torch.cuda.empty_cache()

    class A:
        runs, warmup, no_cpu_baseline, cpu_budget = 3, 1, True, 0.0

    for name in names:
        log(f"profile pass: {name}")
        _, keep = measure(name, pa, torch, W, A, lambda: None)
        del keep
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    log("profile pass done")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20, help="timed headline steps")
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--runs", type=int, default=50, help="timed runs per workload call (median, min, max)")
    ap.add_argument("--only", default="", help="comma-separated workloads to measure (default: all)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=5.0, help="seconds of oracle time per workload")
    ap.add_argument("--no-ceilings", action="store_true", help="skip the achievable-peak probes")
    ap.add_argument("--profile-pass", action="store_true",
                    help="only the kernels a counter run needs (a calibration copy, a few calls per workload)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}): this build has no multi-GPU path; "
              f"the decode shards across sequences with no exchange, one GPU's share is what runs here.",
              file=sys.stderr)
        sys.exit(2)
    names = [n for n in (args.only.split(",") if args.only else CONFIG_ORDER) if n]
    for n in names:
        if n not in CONFIG_ORDER:
            raise SystemExit(f"unknown workload {n}; choose from {', '.join(CONFIG_ORDER)}")

    import torch

    from paged_kv_cache_103_amd import _lib as pa
    from paged_kv_cache_103_amd import workloads as W

    pa.load()
    torch.cuda.set_device(0)
    if args.profile_pass:
        profile_pass(pa, torch, W, names)
        return

    flush = Flusher(torch)
    configs = {}
    head = None
    for name in names:
        res, (b, write, attend) = measure(name, pa, torch, W, args, flush)
        if name == "fp8_decode":
            # the headline: K steps of (KV write + decode), timed between two
            # synchronisations; events around every decode call on the same
            # stream give the call's mean duration over the timed region
            for _ in range(args.warmup):
                write()
                attend()
            torch.cuda.synchronize()
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(args.steps)]
            t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            t0.record()
            for i in range(args.steps):
                write()
                ev[i][0].record()
                attend()
                ev[i][1].record()
            t1.record()
            torch.cuda.synchronize()
            step_ms = t0.elapsed_time(t1) / args.steps
            call_ms = sum(a.elapsed_time(c) for a, c in ev) / args.steps
            head = {"step_ms": step_ms, "call_ms": call_ms, "kv_bytes": b.kv_bytes_read(),
                    "new_tokens": b.num_q_tokens}
        log(f"{name}: " + json.dumps({k: v for k, v in res.items() if k in ("value", "unit", "timing")}))
        configs[name] = res
        del b, write, attend
        torch.cuda.synchronize()
        torch.cuda.empty_cache()

    ceil = None if args.no_ceilings else measure_ceilings(torch)
    if ceil:
        log(f"measured ceilings: {ceil}")
    line = {"metric": METRIC, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "data": "synthetic"}
    if head is not None:
        gbs = head["kv_bytes"] / (head["step_ms"] * 1e-3) / 1e9
        call_gbs = head["kv_bytes"] / (head["call_ms"] * 1e-3) / 1e9
        fp8 = configs["fp8_decode"]
        line.update({
            "value": round(gbs, 2), "unit": "GB/s", "ms_per_step": round(head["step_ms"], 5),
            "dtype": "fp8_e4m3",
            "config": {"workload": "fp8_decode: " + WORKLOADS["fp8_decode"] + "; one layer; step = KV write of the "
                                   "128 new tokens (bf16 in, quantised to the block scales) + paged decode",
                       "kv_bytes_per_step": head["kv_bytes"], "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
                       "dtype_detail": "K/V stored fp8 e4m3 (OCP e4m3fn) with fp32 per-block scales, bf16 queries "
                                       "and output, bf16 matrix-core products with fp32 accumulation"},
            "roofline": {"bound": "hbm", "kernel": "pa_decode call: decode_mfma_split<2, 128, false> + "
                                                   "decode_split_merge",
                         "achieved": round(call_gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(call_gbs / HBM_PEAK_GBS, 4), "traffic": stored_traffic("fp8_decode"),
                         "algorithmic_bytes_per_launch": head["kv_bytes"],
                         "measured_ceiling": None if not ceil else {
                             "value": ceil["hbm_tiles_lds_copies_gbs"], "unit": "GB/s",
                             "frac": round(call_gbs / ceil["hbm_tiles_lds_copies_gbs"], 4),
                             "probe": "libpa_peaks: random 4 KiB tiles by 16-byte nontemporal global->LDS copies "
                                      "(the fastest of its gathers; register loads in hbm_tiles_contiguous_gbs)"}},
            "cpu_baseline": fp8.get("cpu_baseline"),
        })
    if "mixed_step" in configs:
        line["mixed_step_tokens_per_s"] = configs["mixed_step"]["value"]
    line["configs"] = configs
    line["measured_ceilings"] = ceil
    line["host"] = host_info()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
