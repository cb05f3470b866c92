"""The C-ABI library loads and exports every symbol include/pa.h declares, and
host-side validation rejects bad arguments without touching a GPU (CPU only)."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    from paged_kv_cache_103_amd import _lib as pa

    if not os.path.exists(pa.LIB_PATH):
        from paged_kv_cache_103_amd import build

        build.build()
    return pa


def declared_functions():
    with open(os.path.join(ROOT, "include", "pa.h")) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pa_[a-z_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert set(names) == set(lib.EXPORTED), names
    L = lib.load()
    for n in names:
        assert getattr(L, n) is not None


def test_abi_version_and_status_strings(lib):
    assert lib.abi_version() == 1
    assert lib.status_string(0) == "PA_OK"
    assert lib.status_string(3) == "PA_ERR_WORKSPACE_TOO_SMALL"
    assert lib.status_string(4) == "PA_ERR_HIP"
    assert lib.status_string(5) == "PA_ERR_OUT_OF_BLOCKS"
    assert lib.status_string(99) == "PA_ERR_UNKNOWN"


def _decode_args(**over):
    a = dict(out=1, query=1, k_cache=1, v_cache=1, k_scale=None, v_scale=None, block_table=1,
             bt_stride=8, context_lens=1, num_seqs=2, max_ctx=100, num_heads=8, num_kv_heads=2,
             head_size=128, block_size=16, num_blocks=10, q_dtype=1, cache_dtype=1, scale=0.1,
             window=0, ws=1, ws_bytes=1 << 30, stream=None)
    a.update(over)
    return a


def _call_decode(lib, **over):
    a = _decode_args(**over)
    L = lib.load()
    return L.pa_decode(a["out"], a["query"], a["k_cache"], a["v_cache"], a["k_scale"], a["v_scale"],
                       a["block_table"], a["bt_stride"], a["context_lens"], a["num_seqs"], a["max_ctx"],
                       a["num_heads"], a["num_kv_heads"], a["head_size"], a["block_size"],
                       a["num_blocks"], a["q_dtype"], a["cache_dtype"], a["scale"], a["window"],
                       a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("over,status,msg", [
    (dict(block_size=8), 2, "block_size"),
    (dict(head_size=96), 2, "head_size"),
    (dict(num_heads=7), 1, "multiple"),
    (dict(num_kv_heads=0), 1, "num_kv_heads"),
    (dict(num_heads=6, num_kv_heads=2), 2, "group 3"),
    (dict(q_dtype=2), 2, "fp8 queries"),
    (dict(q_dtype=7), 1, "unknown dtype"),
    (dict(q_dtype=0, cache_dtype=1), 2, "no decode kernel"),
    (dict(cache_dtype=2), 1, "k_scale"),
    (dict(out=None), 1, "null"),
    (dict(bt_stride=3), 1, "block_table_stride"),
    (dict(max_ctx=0), 1, "max_context_len"),
    (dict(scale=0.0), 1, "scale"),
    (dict(scale=float("nan")), 1, "scale"),
    (dict(window=-1), 1, "sliding_window"),
    (dict(num_seqs=-1), 1, "num_seqs"),
    (dict(ws_bytes=0, max_ctx=100000, bt_stride=7000), 3, "workspace"),
])
def test_decode_rejects_bad_arguments(lib, over, status, msg):
    assert _call_decode(lib, **over) == status
    assert msg in lib.last_error()


def test_empty_batches_enqueue_nothing(lib):
    L = lib.load()
    # no sequences / no tokens: PA_OK without any device work
    assert _call_decode(lib, num_seqs=0, out=None, query=None) == 0
    assert L.pa_reshape_and_cache(None, None, None, None, None, None, None, 0, 10, 16, 2, 64, 1, 1, None) == 0
    assert lib.last_error() == ""


@pytest.mark.parametrize("args,status,msg", [
    (dict(block_size=32), 2, "block_size"),
    (dict(head_size=80), 2, "head_size"),
    (dict(in_dtype=1, cache_dtype=0), 2, "not supported"),
    (dict(in_dtype=2, cache_dtype=1), 2, "not supported"),
    (dict(num_tokens=-5), 1, "num_tokens"),
    (dict(key=None), 1, "null"),
    (dict(in_dtype=1, cache_dtype=2), 1, "k_scale"),
])
def test_reshape_rejects_bad_arguments(lib, args, status, msg):
    a = dict(key=1, value=1, k_cache=1, v_cache=1, k_scale=None, v_scale=None, slots=1, num_tokens=4,
             num_blocks=10, block_size=16, num_kv_heads=2, head_size=64, in_dtype=1, cache_dtype=1)
    a.update(args)
    L = lib.load()
    st = L.pa_reshape_and_cache(a["key"], a["value"], a["k_cache"], a["v_cache"], a["k_scale"], a["v_scale"],
                                a["slots"], a["num_tokens"], a["num_blocks"], a["block_size"],
                                a["num_kv_heads"], a["head_size"], a["in_dtype"], a["cache_dtype"], None)
    assert st == status
    assert msg in lib.last_error()


def test_prefill_rejects_bad_arguments(lib):
    L = lib.load()

    def call(**over):
        a = dict(cu=1, num_seqs=2, nq=40, max_q=30, max_ctx=100, q_dtype=1, cache_dtype=1, ws_bytes=1 << 30)
        a.update(over)
        return L.pa_prefill_chunk(1, 1, 1, 1, None, None, 1, 8, a["cu"], 1, a["num_seqs"], a["nq"],
                                  a["max_q"], a["max_ctx"], 8, 2, 128, 16, 10, a["q_dtype"],
                                  a["cache_dtype"], 0.1, 0, 1, a["ws_bytes"], None)

    assert call(cu=None) == 1 and "cu_seqlens" in lib.last_error()
    assert call(nq=1) == 1 and "num_q_tokens" in lib.last_error()
    assert call(max_q=0) == 1 and "max_q_len" in lib.last_error()
    assert call(max_q=101, nq=200) == 1 and "max_q_len" in lib.last_error()
    # fp32 queries work for one-token rows only
    assert call(q_dtype=0, cache_dtype=0) == 2 and "no prefill kernel" in lib.last_error()


def test_workspace_queries(lib):
    # short contexts: one partition, no workspace
    assert lib.decode_workspace_bytes(4, 30, 8, 2, 64, "f32") == 0
    ws = lib.decode_workspace_bytes(64, 8192, 32, 8, 128, "bf16")
    assert ws > 0 and ws % 4 == 0
    # a sliding window never needs more than full attention
    assert lib.decode_workspace_bytes(128, 131072, 64, 8, 128, "fp8_e4m3", 128) <= \
        lib.decode_workspace_bytes(128, 131072, 64, 8, 128, "fp8_e4m3", 0)
    assert lib.decode_workspace_bytes(8, 131072, 8, 2, 64, "f32", 128) < \
        lib.decode_workspace_bytes(8, 131072, 8, 2, 64, "f32", 0)
    # matrix-core decode with every stream at most 16 blocks (contexts up to
    # 256 tokens, or a window up to 240): a wave per stream, no summaries
    assert lib.decode_workspace_bytes(64, 256, 32, 8, 128, "bf16") == 0
    assert lib.decode_workspace_bytes(64, 257, 32, 8, 128, "bf16") > 0
    assert lib.decode_workspace_bytes(128, 131072, 64, 8, 128, "fp8_e4m3", 240) == 0
    assert lib.decode_workspace_bytes(128, 131072, 64, 8, 128, "fp8_e4m3", 241) > 0
    # the one-token rows of a mixed batch use the decode plan
    assert lib.prefill_workspace_bytes(193, 2240, 2048, 67584, 32, 8, 128, "bf16") == \
        lib.decode_workspace_bytes(193, 67584, 32, 8, 128, "bf16")
    # no one-token rows possible: no workspace
    assert lib.prefill_workspace_bytes(2, 600, 300, 5000, 32, 8, 128, "bf16") == 0
    # beyond 16000 sequences the matrix-core decode runs groups of 16000 with
    # one group's workspace (the VALU kernel, for fp32 caches, does not group)
    for cd in ("bf16", "fp8_e4m3"):
        g = lib.decode_workspace_bytes(16000, 8192, 32, 8, 128, cd)
        assert g > lib.decode_workspace_bytes(15999, 8192, 32, 8, 128, cd)
        assert lib.decode_workspace_bytes(16001, 8192, 32, 8, 128, cd) == g
        assert lib.decode_workspace_bytes(100000, 8192, 32, 8, 128, cd) == g
        assert lib.prefill_workspace_bytes(20000, 20100, 101, 8192, 32, 8, 128, cd) == g
    assert lib.decode_workspace_bytes(20000, 8192, 8, 2, 64, "f32") > \
        lib.decode_workspace_bytes(16000, 8192, 8, 2, 64, "f32")
    # the latent decode: groups of 2048 sequences
    L = lib.load()
    m = L.pa_mla_decode_workspace_bytes(2048, 128)
    assert m > L.pa_mla_decode_workspace_bytes(2047, 128)
    assert L.pa_mla_decode_workspace_bytes(2049, 128) == m == L.pa_mla_decode_workspace_bytes(50000, 128)


def test_shared_prefix_rejects_bad_arguments(lib):
    L = lib.load()

    def call(**over):
        a = dict(cu=1, plen=1, ng=1, num_seqs=4, q_dtype=1, cache_dtype=1, window=0, ws=1, ws_bytes=1 << 30)
        a.update(over)
        return L.pa_decode_shared_prefix(1, 1, 1, 1, None, None, 1, 8, 1, a["num_seqs"], 100, a["cu"], a["plen"],
                                         a["ng"], 8, 2, 128, 16, 10, a["q_dtype"], a["cache_dtype"], 0.1,
                                         a["window"], a["ws"], a["ws_bytes"], None)

    assert call(ng=-1) == 1 and "num_groups" in lib.last_error()
    assert call(ng=5) == 1 and "num_groups" in lib.last_error()      # more groups than sequences
    assert call(cu=None) == 1 and "cu_groups" in lib.last_error()
    assert call(plen=None) == 1 and "cu_groups" in lib.last_error()
    assert call(block_size=16, ws_bytes=16) == 3 and "shared-prefix" in lib.last_error()
    # the checks pa_decode makes apply too
    assert call(q_dtype=2) == 2 and "fp8 queries" in lib.last_error()


def test_shared_prefix_workspace_falls_back_to_decode(lib):
    # sharing applies: its own (larger) workspace; otherwise pa_decode's
    shared = lib.decode_shared_prefix_workspace_bytes(16, 4, 262144, 32, 8, 128, "bf16")
    plain = lib.decode_workspace_bytes(16, 262144, 32, 8, 128, "bf16")
    assert shared > plain > 0
    assert lib.decode_shared_prefix_workspace_bytes(16, 0, 262144, 32, 8, 128, "bf16") == plain
    assert lib.decode_shared_prefix_workspace_bytes(16, 4, 262144, 32, 8, 128, "bf16", 128) == \
        lib.decode_workspace_bytes(16, 262144, 32, 8, 128, "bf16", 128)
    assert lib.decode_shared_prefix_workspace_bytes(4, 2, 300, 8, 2, 64, "f32") == \
        lib.decode_workspace_bytes(4, 300, 8, 2, 64, "f32")


def test_peak_probe_library_exports_its_header():
    from paged_kv_cache_103_amd import peaks

    with open(os.path.join(ROOT, "include", "pa_peaks.h")) as f:
        text = re.sub(r"/\*.*?\*/", "", f.read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(pa_[a-z_]+)\s*\(", text)))
    assert set(names) == set(peaks.EXPORTED), names
    L = peaks.load()
    for n in names:
        assert getattr(L, n) is not None


def test_block_manager_header_is_exported(lib):
    from paged_kv_cache_103_amd import blocks

    with open(os.path.join(ROOT, "include", "pa_blocks.h")) as f:
        text = re.sub(r"/\*.*?\*/", "", f.read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(pa_[a-z_]+)\s*\(", text)))
    assert set(names) == set(blocks.EXPORTED), names
    L = lib.load()
    for n in names:
        assert getattr(L, n) is not None


def test_copy_blocks_rejects_bad_arguments(lib):
    from paged_kv_cache_103_amd import blocks

    L = blocks._L()

    def call(**over):
        a = dict(k=1, v=1, ks=None, vs=None, pairs=1, n=2, nb=10, bs=16, h=8, d=128, dt=1)
        a.update(over)
        return L.pa_copy_blocks(a["k"], a["v"], a["ks"], a["vs"], a["pairs"], a["n"], a["nb"], a["bs"], a["h"],
                                a["d"], a["dt"], None)

    assert call(n=-1) == 1
    assert call(bs=32) == 2
    assert call(d=96) == 2
    assert call(h=0) == 1
    assert call(nb=0) == 1
    assert call(dt=9) == 1
    assert call(pairs=None) == 1
    assert call(k=None) == 1
    assert call(dt=2) == 1  # fp8 without scales
    assert call(n=0, pairs=None, k=None, v=None) == 0  # nothing to do, nothing launched


def test_sparse_decode_rejects_bad_arguments(lib):
    L = lib.load()

    def call(**over):
        a = dict(out=1, query=1, k=1, v=1, ks=None, vs=None, bt=1, bt_stride=8, ctx=1, S=2, max_ctx=100, sel=1,
                 sel_stride=4, nsel=1, max_sel=4, Hq=8, Hkv=2, D=128, B=16, NB=10, qd=1, cd=1, scale=0.1, ws=1,
                 ws_bytes=1 << 30)
        a.update(over)
        return L.pa_decode_sparse(a["out"], a["query"], a["k"], a["v"], a["ks"], a["vs"], a["bt"], a["bt_stride"],
                                  a["ctx"], a["S"], a["max_ctx"], a["sel"], a["sel_stride"], a["nsel"], a["max_sel"],
                                  a["Hq"], a["Hkv"], a["D"], a["B"], a["NB"], a["qd"], a["cd"], a["scale"], a["ws"],
                                  a["ws_bytes"], None)

    assert call(max_sel=-1) == 1
    assert call(max_sel=(1 << 22) + 1) == 1
    assert call(sel=None) == 1
    assert call(nsel=None) == 1
    assert call(sel_stride=3) == 1
    assert call(B=32) == 2
    assert call(Hq=6, Hkv=4) == 1
    assert call(bt_stride=2) == 1
    assert call(ws_bytes=16) == 3
    assert call(ws=None) == 3
    assert call(max_ctx=1 << 25, bt_stride=1 << 21) == 2  # beyond the block bitmap
    assert call(S=0) == 0
    # nothing chosen: the lists may be absent
    need = L.pa_decode_sparse_workspace_bytes(2, 0, 8, 2, 128, 1)
    assert need > 0
    assert call(sel=None, nsel=None, max_sel=0, sel_stride=0, ws_bytes=need - 1) == 3
    assert L.pa_decode_sparse_workspace_bytes(2, -1, 8, 2, 128, 1) == 0
    assert (L.pa_decode_sparse_workspace_bytes(64, 128, 32, 8, 128, 1)
            >= 64 * 129 * 4 + lib.decode_workspace_bytes(64, 16 * 129, 32, 8, 128, "bf16"))


def test_partial_decode_and_merge_reject_bad_arguments(lib):
    L = lib.load()

    def partial(**over):
        a = dict(out=1, lse=1, query=1, k=1, v=1, ks=None, vs=None, bt=1, bt_stride=8, ctx=1, S=2, max_ctx=100,
                 Hq=8, Hkv=2, D=128, B=16, NB=10, qd=1, cd=1, scale=0.1, ws=1, ws_bytes=1 << 30)
        a.update(over)
        return L.pa_decode_partial(a["out"], a["lse"], a["query"], a["k"], a["v"], a["ks"], a["vs"], a["bt"],
                                   a["bt_stride"], a["ctx"], a["S"], a["max_ctx"], a["Hq"], a["Hkv"], a["D"], a["B"],
                                   a["NB"], a["qd"], a["cd"], a["scale"], a["ws"], a["ws_bytes"], None)

    assert partial(lse=None) == 1
    assert partial(qd=0, cd=0) == 2  # fp32 caches take the VALU kernel: no partial results
    assert partial(B=8) == 2
    assert partial(ws_bytes=8, max_ctx=1000, bt_stride=64) == 3  # split plan: summaries need workspace
    assert partial(S=0, lse=None) == 0

    def merge(**over):
        a = dict(out=1, lse_out=None, parts=1, parts_lse=1, R=2, rows=10, D=128, dt=1)
        a.update(over)
        return L.pa_merge_partials(a["out"], a["lse_out"], a["parts"], a["parts_lse"], a["R"], a["rows"], a["D"],
                                   a["dt"], None)

    assert merge(R=0) == 1
    assert merge(rows=-1) == 1
    assert merge(D=96) == 2
    assert merge(dt=2) == 2
    assert merge(parts=None) == 1
    assert merge(parts_lse=None) == 1
    assert merge(rows=0, out=None, parts=None, parts_lse=None) == 0


def test_mla_decode_rejects_bad_arguments(lib):
    L = lib.load()

    def call(**over):
        a = dict(out=1, query=1, cache=1, bt=1, bt_stride=8, ctx=1, S=2, max_ctx=100, H=128, dk=576, dv=512, B=16,
                 NB=10, qd=1, cd=1, scale=0.1, ws=1, ws_bytes=1 << 30)
        a.update(over)
        return L.pa_mla_decode(a["out"], a["query"], a["cache"], a["bt"], a["bt_stride"], a["ctx"], a["S"],
                               a["max_ctx"], a["H"], a["dk"], a["dv"], a["B"], a["NB"], a["qd"], a["cd"], a["scale"],
                               a["ws"], a["ws_bytes"], None)

    assert call(H=48) == 2
    assert call(dk=640) == 2
    assert call(dv=256) == 2
    assert call(cd=2) == 2
    assert call(B=32) == 2
    assert call(S=-1) == 1
    assert call(S=4096, ws_bytes=64) == 3  # (more than 2048 sequences: groups, one workspace of 2048's size)
    assert call(bt_stride=2) == 1
    assert call(cache=None) == 1
    assert call(scale=0.0) == 1
    assert call(ws_bytes=64) == 3
    assert call(S=0) == 0
    assert L.pa_mla_decode_workspace_bytes(0, 128) == 0
    assert L.pa_mla_decode_workspace_bytes(64, 128) > 64 * 128 * 512 * 4
