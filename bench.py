"""Benchmark of the paged-KV hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--extra] [--no-cpu-baseline]

Headline (the JSON line on stdout): decode KV GB/s on the Llama-3-8B-shaped
decode batch (64 sequences, contexts U{1024..8192}, 32 query / 8 KV heads,
head size 128, bf16, 16-token blocks). One step = the KV write of the 64 new
tokens + paged decode over every sequence, inputs resident in HBM.
value = algorithmic K+V bytes read per step / step time.

Beside it in the same line: the mixed chunked-prefill step (192 decode rows +
one 2048-token chunk on a 65536-token prefix, 2240 new tokens written first)
in new tokens/s, the roofline of the decode kernel, the prefill chunk's
MFMA throughput, the sparse decode over chosen blocks at 32K..512K-token
contexts, and the CPU oracle timed on a bounded sample.
Everything is one attention layer.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16, published

METRIC = "paged-attn decode KV GB/s (% HBM peak); mixed-step tokens/s on 1 MI355X"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def workspace(pa, torch, b, prefill=False):
    if prefill:
        n = pa.prefill_workspace_bytes(b.num_seqs, b.num_q_tokens, b.max_q_len, b.max_context_len,
                                       b.num_heads, b.num_kv_heads, b.head_size, b.cache_dtype, b.sliding_window)
    else:
        n = pa.decode_workspace_bytes(b.num_seqs, b.max_context_len, b.num_heads, b.num_kv_heads,
                                      b.head_size, b.cache_dtype, b.sliding_window)
    return torch.empty(max(n, 1), dtype=torch.uint8, device="cuda")


def decode_step_fns(pa, torch, b):
    m = b.meta("cuda")
    out = torch.empty_like(b.query)
    ws = workspace(pa, torch, b)

    def write():
        pa.reshape_and_cache(b.new_key, b.new_value, b.k_cache, b.v_cache, m["slot_mapping"], b.k_scale,
                             b.v_scale)

    def attend():
        pa.decode(out, b.query, b.k_cache, b.v_cache, m["block_table"], m["context_lens"],
                  b.max_context_len, b.scale, b.k_scale, b.v_scale, b.sliding_window, ws)

    return write, attend


def shared_prefix_step_fns(pa, torch, b):
    """Decode through pa_decode_shared_prefix (the batch's shared groups)."""
    m = b.meta("cuda")
    gm = b.group_meta("cuda")
    out = torch.empty_like(b.query)
    ng = gm["group_prefix_len"].numel()
    n = pa.decode_shared_prefix_workspace_bytes(b.num_seqs, ng, b.max_context_len, b.num_heads, b.num_kv_heads,
                                                b.head_size, b.cache_dtype, b.sliding_window)
    ws = torch.empty(max(n, 1), dtype=torch.uint8, device="cuda")

    def write():
        pa.reshape_and_cache(b.new_key, b.new_value, b.k_cache, b.v_cache, m["slot_mapping"], b.k_scale,
                             b.v_scale)

    def attend():
        pa.decode_shared_prefix(out, b.query, b.k_cache, b.v_cache, m["block_table"], m["context_lens"],
                                b.max_context_len, gm["cu_groups"], gm["group_prefix_len"], b.scale, b.k_scale,
                                b.v_scale, b.sliding_window, ws)

    return write, attend


def sparse_step_fns(pa, torch, b, choice):
    """Decode through pa_decode_sparse over each sequence's chosen blocks."""
    m = b.meta("cuda")
    c = choice.device("cuda")
    out = torch.empty_like(b.query)
    ms = choice.selected.shape[1]
    n = pa.decode_sparse_workspace_bytes(b.num_seqs, ms, b.num_heads, b.num_kv_heads, b.head_size, b.cache_dtype)
    ws = torch.empty(max(n, 1), dtype=torch.uint8, device="cuda")

    def write():
        pa.reshape_and_cache(b.new_key, b.new_value, b.k_cache, b.v_cache, m["slot_mapping"], b.k_scale,
                             b.v_scale)

    def attend():
        pa.decode_sparse(out, b.query, b.k_cache, b.v_cache, m["block_table"], m["context_lens"],
                         b.max_context_len, c["selected"], c["num_selected"], b.scale, b.k_scale, b.v_scale, ws)

    return write, attend


def sparse_kv_bytes(b, choice):
    """K+V bytes a sparse decode reads: the keys of every chosen block (the
    newest block up to the context end)."""
    toks = 0
    for ctx, blks in zip(b.context_lens.tolist(), choice.chosen):
        nbk = -(-ctx // 16)
        toks += 16 * (len(blks) - 1) + ctx - 16 * (nbk - 1)
    e = {"bf16": 2, "f32": 4, "fp8_e4m3": 1}[b.cache_dtype]
    return toks * b.num_kv_heads * b.head_size * 2 * e


def run_sparse(pa, torch, W, steps, warmup, ctx=None):
    """The long-context sparse batch (or, with ctx, 64 sequences of ctx tokens
    each with the same 128-block choice size)."""
    if ctx is None:
        b, choice = W.make_sparse_config(device="cuda")
    else:
        b, choice = W.make_sparse_batch(f"sparse_ctx{ctx}", 60, [ctx] * 64, 128, 32, 8, 128, device="cuda")
    torch.cuda.synchronize()
    write, attend = sparse_step_fns(pa, torch, b, choice)
    step_ms, attend_ms, wall = time_steps(torch, write, attend, steps, warmup)
    kv = sparse_kv_bytes(b, choice)
    dense = b.kv_bytes_read()
    res = {"step_ms": step_ms, "attend_ms": attend_ms, "kv_bytes": kv, "dense_kv_bytes": dense,
           "kv_gbs_attend": kv / (attend_ms * 1e-3) / 1e9, "mean_context": float(b.context_lens.mean()),
           "chosen_blocks_per_seq": 128}
    return b, res


def run_context_parallel(pa, torch, W, ranks, steps, warmup):
    """The Llama-shaped decode batch as `ranks` context-parallel ranks would
    run it: every sequence cut into `ranks` contiguous block-aligned ranges,
    each rank's pa_decode_partial over its ranges (timed one after another on
    this GPU), then pa_merge_partials of the gathered results."""
    import numpy as np
    b = W.make_config("llama8b_decode", device="cuda")
    S, Hq, D = b.query.shape
    calls = []
    for r in range(ranks):
        ctx, rows = [], []
        for s in range(S):
            nb = -(-int(b.context_lens[s]) // 16)
            a0, a1 = nb * r // ranks, nb * (r + 1) // ranks
            ctx.append(max(0, min(int(b.context_lens[s]), a1 * 16) - a0 * 16))
            rows.append(b.block_table[s, a0:a1])
        stride = max(1, max(len(x) for x in rows))
        tab = np.zeros((S, stride), dtype=np.int32)
        for s, x in enumerate(rows):
            tab[s, :len(x)] = x
        mc = max(1, max(ctx))
        ws = torch.empty(max(pa.decode_workspace_bytes(S, mc, Hq, b.num_kv_heads, D), 1), dtype=torch.uint8,
                         device="cuda")
        calls.append((torch.from_numpy(tab).to("cuda"), torch.tensor(ctx, dtype=torch.int32, device="cuda"), mc, ws))
    parts = torch.empty((ranks, S, Hq, D), dtype=b.query.dtype, device="cuda")
    lses = torch.empty((ranks, S, Hq), dtype=torch.float32, device="cuda")
    out = torch.empty_like(b.query)

    def ranks_fn():
        for r, (tab, ctx, mc, ws) in enumerate(calls):
            pa.decode_partial(parts[r], lses[r], b.query, b.k_cache, b.v_cache, tab, ctx, mc, b.scale, workspace=ws)

    def merge_fn():
        pa.merge_partials(out, parts, lses)

    _, ranks_ms, _ = time_steps(torch, lambda: None, ranks_fn, steps, warmup)
    _, merge_ms, _ = time_steps(torch, lambda: None, merge_fn, steps, warmup)
    res = {"ranks": ranks, "all_ranks_ms": round(ranks_ms, 5), "per_rank_ms": round(ranks_ms / ranks, 5),
           "merge_ms": round(merge_ms, 5), "merge_bytes": parts.numel() * parts.element_size() + lses.numel() * 4
           + out.numel() * out.element_size()}
    log(f"context parallel ({ranks} ranks, one GPU): all ranks {ranks_ms*1e3:.1f} us, merge {merge_ms*1e3:.1f} us")
    del b
    torch.cuda.empty_cache()
    return res


def run_mla(pa, torch, W, steps, warmup, num_heads=128, head_dim_k=576):
    """Latent-cache (MLA) decode: 64 sequences, contexts U{4096..32768}."""
    import numpy as np
    if num_heads == 128 and head_dim_k == 576:
        b = W.make_mla_config(device="cuda")
    else:
        ctx = np.random.default_rng(7).integers(4096, 32769, 64).tolist()
        b = W.make_mla_batch(f"mla_{num_heads}_{head_dim_k}", 7, ctx, num_heads, head_dim_k, device="cuda")
    S, H = b.num_seqs, b.num_heads
    out = torch.empty((S, H, 512), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(max(pa.mla_decode_workspace_bytes(S, H), 1), dtype=torch.uint8, device="cuda")
    bt = torch.from_numpy(b.block_table).to("cuda")
    cl = torch.from_numpy(b.context_lens).to("cuda")
    torch.cuda.synchronize()

    def attend():
        pa.mla_decode(out, b.query, b.cache, bt, cl, b.max_context_len, b.scale, ws)

    _, ms, _ = time_steps(torch, lambda: None, attend, steps, warmup)
    keys = int(b.context_lens.sum())
    nbytes = b.latent_bytes_read()
    flops = 2.0 * H * (b.head_dim_k + 512) * keys
    res = {"attend_ms": round(ms, 5), "bytes_per_call": nbytes, "flops_per_call": flops,
           "gbs": round(nbytes / (ms * 1e-3) / 1e9, 2), "tflops": round(flops / (ms * 1e-3) / 1e12, 2),
           "num_heads": H, "head_dim_k": b.head_dim_k}
    del b
    torch.cuda.empty_cache()
    return res


def prefill_step_fns(pa, torch, b):
    m = b.meta("cuda")
    out = torch.empty_like(b.query)
    ws = workspace(pa, torch, b, prefill=True)

    def write():
        pa.reshape_and_cache(b.new_key, b.new_value, b.k_cache, b.v_cache, m["slot_mapping"], b.k_scale,
                             b.v_scale)

    def attend():
        pa.prefill_chunk(out, b.query, b.k_cache, b.v_cache, m["block_table"], m["cu_seqlens"],
                         m["context_lens"], b.max_q_len, b.max_context_len, b.scale, b.k_scale,
                         b.v_scale, b.sliding_window, ws)

    return write, attend


def time_steps(torch, write, attend, steps, warmup):
    """Warm up, then time exactly `steps` steps (write + attend) between two
    synchronisations; HIP events on the launch stream bracket every attend
    call. Returns (ms per step, mean ms of the attend call)."""
    for _ in range(warmup):
        write()
        attend()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t0.record()
    for i in range(steps):
        write()
        ev[i][0].record()
        attend()
        ev[i][1].record()
    t1.record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - wall0) * 1e3 / steps
    step_ms = t0.elapsed_time(t1) / steps
    attend_ms = sum(a.elapsed_time(c) for a, c in ev) / steps
    return step_ms, attend_ms, wall


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


def cpu_baseline(b, budget_s=12.0):
    """The oracle, as it stands, on a bounded sample of the batch: whole
    sequences in order, passing over the batch again until about budget_s
    seconds are spent. Reported in the same unit as the GPU (K+V GB/s of the
    sequences it finished)."""
    from tests.helpers import oracle_rows

    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    done, secs, nbytes = 0, 0.0, 0
    e = {"f32": 4, "bf16": 2, "fp8_e4m3": 1}[b.cache_dtype]
    while secs <= budget_s:
        for s in range(b.num_seqs):
            t = time.perf_counter()
            oracle_rows(b, [s])
            secs += time.perf_counter() - t
            done += 1
            nbytes += int(b.context_lens[s]) * b.num_kv_heads * b.head_size * 2 * e
            if secs > budget_s:
                break
    return {"value": round(nbytes / secs / 1e9, 4), "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{done} sequence evaluations over the {b.num_seqs} sequences of the same batch "
                      f"(all heads, in order, repeated), {secs:.1f} s; includes the oracle's own host gather "
                      f"through the block table, not the D2H copy"}


DECODE_SOURCES = ("decode_mfma.hip", "decode.hip", "pa_device.h", "pa_internal.h")
PREFILL_SOURCES = ("prefill_bf16.hip", "prefill_tiles.h", "pa_device.h", "pa_internal.h")
MLA_SOURCES = ("mla_decode.hip", "pa_device.h", "pa_internal.h")
SPARSE_SOURCES = ("sparse_select.hip", "decode_mfma.hip", "decode.hip", "pa_device.h", "pa_internal.h")


def kernel_source_digest(files=DECODE_SOURCES):
    """sha256 over the sources of a kernel's path (kernel, shared device code,
    plan/dispatch), used to tell whether a stored counter summary still
    describes the kernel that runs."""
    import hashlib
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "paged_kv_cache_103_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def stored_traffic(profile="decode_mfma_split_llama8b_decode.md", files=DECODE_SOURCES):
    """HBM bytes per launch on this workload from a committed rocprofv3
    counter summary (FETCH_SIZE, WRITE_SIZE scaled by the plain-copy
    calibration), or None if missing or taken on another kernel version."""
    import re
    path = os.path.join(ROOT, "profiles", profile)
    try:
        text = open(path).read()
    except OSError:
        return None
    m = re.search(r"<!-- traffic (\{.*?\}) -->", text)
    if not m:
        return None
    t = json.loads(m.group(1))
    if t.get("kernel_source_sha256") != kernel_source_digest(files):
        return None
    return int(t["fetch_bytes_per_launch"]) + int(t["write_bytes_per_launch"])


def measure_ceilings(torch):
    """Achievable peaks on this GPU, measured with libpa_peaks next to the
    path: HBM read rate of a paged gather (random 4 KiB tiles, one wave per
    tile, 16-byte nontemporal loads; contiguous 1 KiB per instruction, and the
    decode kernel's key pattern of 64 bytes from each of 16 rows) and the
    back-to-back 32x32x16 bf16 / fp16 MFMA rate."""
    from paged_kv_cache_103_amd import peaks

    res = {}
    nbytes = 4 << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    g = torch.Generator(device="cpu")
    g.manual_seed(0)
    ids = torch.randperm(nbytes // 4096, generator=g).to(torch.int32).cuda()
    sink = torch.empty(256 * 2048, dtype=torch.float32, device="cuda")
    for mode, name in ((0, "hbm_tiles_contiguous_gbs"), (1, "hbm_tiles_decode_pattern_gbs")):
        f = lambda: peaks.read_tiles(buf, ids, mode, 4096, sink)
        _, ms, _ = time_steps(torch, lambda: None, f, 5, 2)
        res[name] = round(nbytes / (ms * 1e-3) / 1e9, 1)
    del buf, ids
    torch.cuda.empty_cache()
    for kind, name in ((0, "mfma_bf16_tflops"), (1, "mfma_fp16_tflops")):
        flops = [0.0]

        def f():
            flops[0] = peaks.mfma(kind, 2000, 2048, sink)

        _, ms, _ = time_steps(torch, lambda: None, f, 5, 2)
        res[name] = round(flops[0] / (ms * 1e-3) / 1e12, 1)
    return res


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


def graph_call_us(torch, attend, calls=16, replays=20):
    """Mean device time of one attend call when `calls` of them are captured
    back to back in one HIP graph and the graph is replayed: the figure a
    serving loop that replays its small launches sees, without this
    script's per-call host overhead (ctypes marshalling and the launch)."""
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
    return us


def run_config(pa, torch, W, name, steps, warmup, shared_prefix=False, graph=False):
    b = W.make_config(name, device="cuda")
    torch.cuda.synchronize()
    prefill = b.max_q_len > 1
    fns = shared_prefix_step_fns if shared_prefix else (prefill_step_fns if prefill else decode_step_fns)
    write, attend = fns(pa, torch, b)
    step_ms, attend_ms, wall = time_steps(torch, write, attend, steps, warmup)
    res = {"config": name, "step_ms": step_ms, "attend_ms": attend_ms, "wall_ms": wall,
           "kv_bytes": b.kv_bytes_read(), "unique_kv_bytes": b.unique_kv_bytes_read(),
           "new_tokens": b.num_q_tokens}
    res["kv_gbs_step"] = res["kv_bytes"] / (step_ms * 1e-3) / 1e9
    res["kv_gbs_attend"] = res["kv_bytes"] / (attend_ms * 1e-3) / 1e9
    res["unique_gbs_attend"] = res["unique_kv_bytes"] / (attend_ms * 1e-3) / 1e9
    res["tokens_per_s"] = b.num_q_tokens / (step_ms * 1e-3)
    if graph:
        res["attend_us_graph_replay"] = graph_call_us(torch, attend)
    return b, res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--extra", action="store_true", help="also time the other named configurations (stderr)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ceilings", action="store_true", help="skip the achievable-peak probes")
    ap.add_argument("--profile-pass", action="store_true",
                    help="only the kernels a counter run needs: a plain 1 GiB device copy (the "
                         "calibration kernel for FETCH_SIZE/WRITE_SIZE), a few decode and mixed steps, "
                         "the mixed step's chunk alone, a few sparse decode calls and latent-cache decode calls")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); this build has no multi-GPU path.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from paged_kv_cache_103_amd import _lib as pa
    from paged_kv_cache_103_amd import workloads as W

    pa.load()
    torch.cuda.set_device(0)

    if args.profile_pass:
        # plain copy kernel of known size: 1 GiB read + 1 GiB written per launch
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        torch.cuda.empty_cache()
        for name in ("llama8b_decode", "mixed_step"):
            b = W.make_config(name, device="cuda")
            write, attend = (prefill_step_fns if b.max_q_len > 1 else decode_step_fns)(pa, torch, b)
            for _ in range(3):
                write()
                attend()
            if name == "mixed_step":  # then the chunk alone
                _, pre_attend = prefill_step_fns(pa, torch, chunk_of(b))
                for _ in range(3):
                    pre_attend()
            torch.cuda.synchronize()
            del b
            torch.cuda.empty_cache()
        sb, choice = W.make_sparse_config(device="cuda")
        _, sp_attend = sparse_step_fns(pa, torch, sb, choice)
        for _ in range(3):
            sp_attend()
        torch.cuda.synchronize()
        del sb
        run_mla(pa, torch, W, 3, 0)
        run_mla(pa, torch, W, 3, 0, 16, 576)
        log("profile pass done")
        return

    # ---- headline: decode on the Llama-3-8B-shaped batch ----
    b, dec = run_config(pa, torch, W, "llama8b_decode", args.steps, args.warmup)
    log(f"llama8b_decode: step {dec['step_ms']*1e3:.1f} us, pa_decode {dec['attend_ms']*1e3:.1f} us, "
        f"{dec['kv_gbs_attend']:.0f} GB/s in pa_decode, {dec['kv_gbs_step']:.0f} GB/s per step")
    cpu = None if args.no_cpu_baseline else cpu_baseline(b)
    del b
    torch.cuda.empty_cache()

    # ---- mixed chunked-prefill step ----
    mb, mix = run_config(pa, torch, W, "mixed_step", max(5, args.steps // 5), max(2, args.warmup // 2))
    log(f"mixed_step: step {mix['step_ms']:.3f} ms -> {mix['tokens_per_s']:.0f} new tokens/s")
    # the 2048-token chunk alone (prefill kernel only) for its MFMA rate
    chunk = chunk_of(mb)
    _, pre_attend = prefill_step_fns(pa, torch, chunk)
    _, pre_ms, _ = time_steps(torch, lambda: None, pre_attend, max(10, args.steps // 2), 5)
    flops = causal_flops(chunk)
    pre_tflops = flops / (pre_ms * 1e-3) / 1e12
    log(f"prefill chunk alone: {pre_ms:.3f} ms, {pre_tflops:.0f} TFLOP/s "
        f"({100 * pre_tflops / BF16_MFMA_PEAK_TFLOPS:.1f}% of bf16 MFMA peak)")
    del mb, chunk
    torch.cuda.empty_cache()
    # the same chunk over an fp8 e4m3 cache (per-block scales)
    fb = W.make_batch("mixed_step_chunk_fp8", 4, [65536 + 2048], [2048], 32, 8, 128, "bf16", "fp8_e4m3",
                      device="cuda")
    _, f8_attend = prefill_step_fns(pa, torch, fb)
    _, f8_ms, _ = time_steps(torch, lambda: None, f8_attend, max(10, args.steps // 2), 5)
    f8_tflops = causal_flops(fb) / (f8_ms * 1e-3) / 1e12
    log(f"prefill chunk alone, fp8 cache: {f8_ms:.3f} ms, {f8_tflops:.0f} TFLOP/s "
        f"({100 * f8_tflops / BF16_MFMA_PEAK_TFLOPS:.1f}% of bf16 MFMA peak)")
    del fb
    torch.cuda.empty_cache()

    # ---- sparse decode over chosen blocks, long contexts ----
    sb, sp = run_sparse(pa, torch, W, max(10, args.steps // 2), args.warmup)
    log(f"sparse_decode: pa_decode_sparse {sp['attend_ms']*1e3:.1f} us, {sp['kv_gbs_attend']:.0f} GB/s of chosen "
        f"K/V ({sp['kv_bytes']/1e6:.0f} MB of {sp['dense_kv_bytes']/1e9:.1f} GB in the contexts)")
    del sb
    torch.cuda.empty_cache()

    # ---- decode over a paged latent (MLA) cache ----
    ml = run_mla(pa, torch, W, max(10, args.steps // 2), args.warmup)
    log(f"mla_decode (128 heads, rows of 576): {ml['attend_ms']*1e3:.1f} us, {ml['gbs']:.0f} GB/s of latent rows, "
        f"{ml['tflops']:.0f} TFLOP/s")
    # 16 heads: one GPU's share of 128 heads under 8-way tensor parallelism,
    # which still reads every latent row
    ml16 = run_mla(pa, torch, W, max(10, args.steps // 2), args.warmup, 16, 576)
    log(f"mla_decode (16 heads, rows of 576): {ml16['attend_ms']*1e3:.1f} us, {ml16['gbs']:.0f} GB/s of latent rows")

    extra = {}
    if args.extra:
        for h, dk in ((64, 576), (128, 512), (16, 512)):
            r = run_mla(pa, torch, W, max(10, args.steps // 2), args.warmup, h, dk)
            extra[f"mla_decode_{h}h_{dk}"] = r
            log(f"mla_decode ({h} heads, rows of {dk}): {r['attend_ms']*1e3:.1f} us, {r['gbs']:.0f} GB/s, "
                f"{r['tflops']:.0f} TFLOP/s")
        # the sparse decode's time against the context length at a fixed choice
        sweep = {}
        for ctx in (8192, 65536, 524288):
            sb, r = run_sparse(pa, torch, W, max(10, args.steps // 2), args.warmup, ctx=ctx)
            sweep[str(ctx)] = round(r["attend_ms"] * 1e3, 2)
            log(f"sparse decode, 64 x {ctx} tokens, 128 blocks chosen: {r['attend_ms']*1e3:.1f} us")
            del sb
            torch.cuda.empty_cache()
        extra["sparse_decode_us_by_context"] = sweep
        extra["context_parallel_llama8b"] = run_context_parallel(pa, torch, W, 8, max(10, args.steps // 2),
                                                                 args.warmup)
        for name in ("tiny_decode", "agentic_decode", "fp8_decode", "fp8_swa128"):
            # the launch-bound ones also replayed from a graph
            small = name in ("tiny_decode", "fp8_swa128")
            eb, r = run_config(pa, torch, W, name, max(5, args.steps // 2), args.warmup, graph=small)
            extra[name] = {k: (round(v, 4) if isinstance(v, float) else v) for k, v in r.items()}
            log(f"{name}: pa_decode {r['attend_ms']*1e3:.1f} us, {r['kv_gbs_attend']:.0f} GB/s logical, "
                f"{r['unique_gbs_attend']:.0f} GB/s unique"
                + (f"; {r['attend_us_graph_replay']:.1f} us per call replayed from a graph" if small else ""))
            del eb
            torch.cuda.empty_cache()
        # the agentic batch again, its groups' shared prefix blocks read once
        eb, r = run_config(pa, torch, W, "agentic_decode", max(5, args.steps // 2), args.warmup, shared_prefix=True)
        extra["agentic_decode_shared_prefix"] = {k: (round(v, 4) if isinstance(v, float) else v) for k, v in r.items()}
        log(f"agentic_decode (pa_decode_shared_prefix): {r['attend_ms']*1e3:.1f} us, "
            f"{r['kv_gbs_attend']:.0f} GB/s logical, {r['unique_gbs_attend']:.0f} GB/s unique")
        del eb
        torch.cuda.empty_cache()

    ceil = None if args.no_ceilings else measure_ceilings(torch)
    if ceil:
        log(f"measured ceilings: {ceil}")
    achieved = dec["kv_gbs_attend"]
    line = {
        "metric": METRIC,
        "value": round(dec["kv_gbs_step"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(dec["step_ms"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "llama8b_decode: 64 sequences, context U{1024..8192}, 32 query / 8 KV "
                               "heads, head 128, bf16 K/V and queries, 16-token blocks, one layer; "
                               "step = KV write of 64 tokens + paged decode",
                   "kv_bytes_per_step": dec["kv_bytes"], "pct_hbm_peak": round(100 * dec["kv_gbs_step"] / HBM_PEAK_GBS, 2)},
        "roofline": {"bound": "hbm", "kernel": "pa_decode call: decode_mfma_split + decode_split_merge",
                     "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": stored_traffic(),
                     "algorithmic_bytes_per_launch": dec["kv_bytes"],
                     "measured_ceiling": None if not ceil else {
                         "value": ceil["hbm_tiles_contiguous_gbs"], "unit": "GB/s",
                         "frac": round(achieved / ceil["hbm_tiles_contiguous_gbs"], 4),
                         "probe": "libpa_peaks: random 4 KiB tiles, a wave per tile, 16-byte nontemporal "
                                  "loads, 1 KiB contiguous per instruction",
                         "decode_key_pattern_gbs": ceil["hbm_tiles_decode_pattern_gbs"]}},
        "cpu_baseline": cpu,
        "mixed_step": {"value": round(mix["tokens_per_s"], 1), "unit": "tokens/s",
                       "ms_per_step": round(mix["step_ms"], 5),
                       "workload": "192 decode rows (context U{4096..32768}) + one 2048-token chunk on a "
                                   "65536-token prefix; 2240 new tokens written; 32/8 heads, d128, bf16",
                       "prefill_chunk_only_ms": round(pre_ms, 5), "prefill_tflops": round(pre_tflops, 2),
                       "prefill_fp8_cache_chunk": {"ms": round(f8_ms, 5), "tflops": round(f8_tflops, 2),
                                                   "frac_bf16_peak": round(f8_tflops / BF16_MFMA_PEAK_TFLOPS, 4)},
                       "prefill_frac_bf16_peak": round(pre_tflops / BF16_MFMA_PEAK_TFLOPS, 4),
                       "prefill_roofline": {"bound": "mfma", "kernel": "prefill_bf16_kernel (the chunk alone)",
                                            "achieved": round(pre_tflops, 2), "peak": BF16_MFMA_PEAK_TFLOPS,
                                            "unit": "TFLOP/s", "frac": round(pre_tflops / BF16_MFMA_PEAK_TFLOPS, 4),
                                            "traffic": stored_traffic("prefill_bf16_kernel_2048_chunk.md",
                                                                      PREFILL_SOURCES),
                                            "algorithmic_flops_per_launch": flops,
                                            "measured_ceiling": None if not ceil else {
                                                "value": ceil["mfma_bf16_tflops"], "unit": "TFLOP/s",
                                                "frac": round(pre_tflops / ceil["mfma_bf16_tflops"], 4),
                                                "probe": "libpa_peaks: back-to-back independent 32x32x16 "
                                                         "bf16 MFMAs, 8 waves per CU",
                                                "fp16_tflops": ceil["mfma_fp16_tflops"]}}},
        "mla_decode": {"value": ml["gbs"], "unit": "GB/s", "attend_ms": ml["attend_ms"],
                       "workload": "64 sequences, context U{4096..32768}, 128 heads sharing one latent row per "
                                   "token (512 latent + 64, bf16), absorbed queries; pa_mla_decode",
                       "bytes_per_call": ml["bytes_per_call"], "flops_per_call": ml["flops_per_call"],
                       "roofline": {"bound": "hbm", "achieved": ml["gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                    "frac": round(ml["gbs"] / HBM_PEAK_GBS, 4),
                                    "traffic": stored_traffic("mla_decode_128h_576.md", MLA_SOURCES),
                                    "mfma_tflops": ml["tflops"],
                                    "mfma_frac": round(ml["tflops"] / BF16_MFMA_PEAK_TFLOPS, 4)}},
        "mla_decode_16_heads": {"value": ml16["gbs"], "unit": "GB/s", "attend_ms": ml16["attend_ms"],
                                "workload": "the same batch with 16 heads (one GPU's share of 128 under "
                                            "8-way tensor parallelism); pa_mla_decode",
                                "bytes_per_call": ml16["bytes_per_call"],
                                "roofline": {"bound": "hbm", "achieved": ml16["gbs"], "peak": HBM_PEAK_GBS,
                                             "unit": "GB/s", "frac": round(ml16["gbs"] / HBM_PEAK_GBS, 4),
                                             "traffic": stored_traffic("mla_decode_16h_576.md", MLA_SOURCES)}},
        "sparse_decode": {"value": round(sp["kv_gbs_attend"], 2), "unit": "GB/s", "attend_ms": round(sp["attend_ms"], 5),
                          "step_ms": round(sp["step_ms"], 5),
                          "workload": "64 sequences, context U{32768..524288}, 128 chosen blocks (2048 keys) + "
                                      "the newest block each, 32/8 heads, d128, bf16; pa_decode_sparse",
                          "kv_bytes_per_call": sp["kv_bytes"], "dense_kv_bytes": sp["dense_kv_bytes"],
                          "roofline": {"bound": "hbm", "achieved": round(sp["kv_gbs_attend"], 2),
                                       "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                       "frac": round(sp["kv_gbs_attend"] / HBM_PEAK_GBS, 4),
                                       "traffic": stored_traffic("decode_sparse_long_context.md", SPARSE_SOURCES)}},
    }
    if extra:
        line["extra"] = extra
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
