"""Shared helpers for the test suite: host copies of device data in the raw
storage the oracle reads, oracle evaluation on sampled sequences, and the
tolerance check. Nothing here computes attention itself."""

from __future__ import annotations

import numpy as np
import torch

import oracle
from oracle import formats as F

ATOL = 2e-3
RTOL = 1e-2

ORACLE_DTYPE = {"f32": F.F32, "bf16": F.BF16, "fp8_e4m3": F.FP8}


def raw(t: torch.Tensor) -> np.ndarray:
    """Host copy of a tensor's storage bits as the oracle expects them."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return t.view(torch.uint8).numpy()
    if t.dtype == torch.float32:
        return t.numpy()
    raise TypeError(t.dtype)


def out_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().to(torch.float64).numpy()


def seq_blocks(batch, s: int) -> np.ndarray:
    """Physical blocks sequence s reads (window applied), in logical order."""
    ctx = int(batch.context_lens[s])
    ql = int(batch.q_lens[s])
    lo = 0
    if batch.sliding_window > 0:
        lo = max(0, ctx - ql + 1 - batch.sliding_window)
    return batch.block_table[s, lo // 16:(ctx - 1) // 16 + 1], lo // 16


def oracle_rows(batch, seqs, q=None, rows=None, heads=None):
    """Oracle output (float64) for the query rows of ``seqs``; returns a dict
    s -> [q_len][Hq][D]. Only the blocks those sequences read are copied to
    the host. ``rows`` / ``heads`` restrict the evaluation (the rest is NaN)."""
    q = raw(batch.query) if q is None else q
    cu = batch.cu_seqlens
    dt = ORACLE_DTYPE[batch.cache_dtype]
    qd = ORACLE_DTYPE[batch.q_dtype]
    res = {}
    for s in seqs:
        phys, first = seq_blocks(batch, s)
        idx = torch.from_numpy(phys.astype(np.int64)).to(batch.k_cache.device)
        kp = raw(batch.k_cache.index_select(0, idx))
        vp = raw(batch.v_cache.index_select(0, idx))
        ks = vs = None
        if batch.k_scale is not None:
            ks = raw(batch.k_scale.index_select(0, idx))
            vs = raw(batch.v_scale.index_select(0, idx))
        # logical block b -> row b - first of the mini pool; blocks before the
        # window are never read, point them anywhere valid
        row = np.zeros(batch.block_table.shape[1], dtype=np.int64)
        row[first:first + len(phys)] = np.arange(len(phys))
        r0, r1 = int(cu[s]), int(cu[s + 1])
        qf = F.to_f64(q[r0:r1], qd)
        res[s] = oracle.attend_sequence(qf, kp, vp, dt, ks, vs, row, int(batch.context_lens[s]),
                                        batch.num_kv_heads, batch.scale, batch.sliding_window, heads=heads,
                                        rows=rows)
    return res


def assert_close(got: np.ndarray, ref: np.ndarray, what: str, atol: float = ATOL, rtol: float = RTOL):
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.isfinite(ref).all(), f"{what}: oracle produced non-finite values"
    err = np.abs(got - ref)
    bad = ~(err <= atol + rtol * np.abs(ref))  # NaN in got counts as bad
    big = np.abs(ref) > atol
    max_abs = float(np.nanmax(err)) if err.size else 0.0
    max_rel = float(np.nanmax(err[big] / np.abs(ref[big]))) if big.any() else 0.0
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} elements outside "
                             f"{atol}+{rtol}|ref| (max abs {max_abs:.3e}, max rel {max_rel:.3e}); "
                             f"first at {tuple(i)}: got {got[tuple(i)]!r} ref {ref[tuple(i)]!r}")
    return max_abs, max_rel
