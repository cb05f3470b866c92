"""ctypes binding of the block manager and block copy (include/pa_blocks.h):
argument marshalling only; the manager itself is the library's C++."""

from __future__ import annotations

import ctypes
from typing import List, Optional, Tuple

import numpy as np
import torch

from . import _lib

EXPORTED = (
    "pa_bm_create",
    "pa_bm_destroy",
    "pa_bm_num_free_blocks",
    "pa_bm_add_request",
    "pa_bm_append_tokens",
    "pa_bm_fork",
    "pa_bm_free_request",
    "pa_bm_request_info",
    "pa_bm_ref_count",
    "pa_copy_blocks",
)

PA_ERR_OUT_OF_BLOCKS = 5

_bound = False


def _L() -> ctypes.CDLL:
    global _bound
    L = _lib.load()
    if not _bound:
        vp, i32, i64, u64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64
        L.pa_bm_create.restype = vp
        L.pa_bm_create.argtypes = [i32, i32]
        L.pa_bm_destroy.restype = None
        L.pa_bm_destroy.argtypes = [vp]
        L.pa_bm_num_free_blocks.restype = i32
        L.pa_bm_num_free_blocks.argtypes = [vp]
        L.pa_bm_ref_count.restype = i32
        L.pa_bm_ref_count.argtypes = [vp, i32]
        L.pa_bm_add_request.restype = ctypes.c_int
        L.pa_bm_add_request.argtypes = [vp, i64, vp, i32, u64, vp]
        L.pa_bm_append_tokens.restype = ctypes.c_int
        L.pa_bm_append_tokens.argtypes = [vp, i64, vp, i32, vp, vp, vp]
        L.pa_bm_fork.restype = ctypes.c_int
        L.pa_bm_fork.argtypes = [vp, i64, i64]
        L.pa_bm_free_request.restype = ctypes.c_int
        L.pa_bm_free_request.argtypes = [vp, i64]
        L.pa_bm_request_info.restype = ctypes.c_int
        L.pa_bm_request_info.argtypes = [vp, i64, vp, vp, i32, vp]
        L.pa_copy_blocks.restype = ctypes.c_int
        L.pa_copy_blocks.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, ctypes.c_int, vp]
        _bound = True
    return L


class OutOfBlocks(_lib.PAError):
    pass


def _check(st: int) -> None:
    if st == PA_ERR_OUT_OF_BLOCKS:
        raise OutOfBlocks(st, _lib.last_error())
    _lib._check(st)


class BlockManager:
    """The library's block manager (pa_bm_*): refcounted blocks, LRU free
    queue, prefix cache over a hash chain of full blocks, copy-on-write."""

    def __init__(self, num_blocks: int, block_size: int = 16):
        self._h = _L().pa_bm_create(num_blocks, block_size)
        if not self._h:
            raise ValueError(f"bad pool: {num_blocks} blocks of {block_size}")
        self.num_blocks, self.block_size = num_blocks, block_size

    def close(self) -> None:
        if self._h:
            _L().pa_bm_destroy(self._h)
            self._h = None

    def __del__(self):
        self.close()

    @property
    def num_free(self) -> int:
        return int(_L().pa_bm_num_free_blocks(self._h))

    def ref_count(self, block: int) -> int:
        return int(_L().pa_bm_ref_count(self._h, block))

    def add_request(self, req: int, prompt: List[int], salt: int = 0) -> int:
        """Admits req; returns the prompt tokens served from the prefix cache."""
        arr = np.ascontiguousarray(prompt, dtype=np.int32)
        out = ctypes.c_int32(0)
        _check(_L().pa_bm_add_request(self._h, req, arr.ctypes.data if arr.size else None, arr.size, salt,
                                      ctypes.byref(out)))
        return int(out.value)

    def append(self, req: int, tokens: List[int]) -> Tuple[np.ndarray, Optional[Tuple[int, int]]]:
        """Appends tokens; returns (slots int64, copy-on-write pair or None)."""
        arr = np.ascontiguousarray(tokens, dtype=np.int32)
        slots = np.zeros(arr.size, dtype=np.int64)
        cow = np.zeros(2, dtype=np.int32)
        ncow = ctypes.c_int32(0)
        _check(_L().pa_bm_append_tokens(self._h, req, arr.ctypes.data if arr.size else None, arr.size,
                                        slots.ctypes.data if arr.size else None, cow.ctypes.data,
                                        ctypes.byref(ncow)))
        return slots, ((int(cow[0]), int(cow[1])) if ncow.value else None)

    def fork(self, parent: int, child: int) -> None:
        _check(_L().pa_bm_fork(self._h, parent, child))

    def free(self, req: int) -> None:
        _check(_L().pa_bm_free_request(self._h, req))

    def info(self, req: int) -> Tuple[int, List[int]]:
        """(tokens held, block table) of req."""
        nt, nb = ctypes.c_int32(0), ctypes.c_int32(0)
        _check(_L().pa_bm_request_info(self._h, req, ctypes.byref(nt), None, 0, ctypes.byref(nb)))
        buf = np.zeros(max(nb.value, 1), dtype=np.int32)
        _check(_L().pa_bm_request_info(self._h, req, ctypes.byref(nt), buf.ctypes.data, nb.value,
                                       ctypes.byref(nb)))
        return int(nt.value), buf[:nb.value].tolist()


def copy_blocks(k_cache: torch.Tensor, v_cache: torch.Tensor, pairs: torch.Tensor,
                k_scale: Optional[torch.Tensor] = None, v_scale: Optional[torch.Tensor] = None,
                stream=None) -> None:
    """pa_copy_blocks: pairs int32 [n][2] (source, destination) on the device."""
    assert pairs.dtype == torch.int32 and pairs.dim() == 2 and pairs.shape[1] == 2
    NB, H, B = k_cache.shape[0], k_cache.shape[1], k_cache.shape[2]
    D = k_cache.shape[3]
    _check(_L().pa_copy_blocks(_lib._ptr(k_cache), _lib._ptr(v_cache), _lib._ptr(k_scale), _lib._ptr(v_scale),
                               _lib._ptr(pairs), pairs.shape[0], NB, B, H, D, _lib.dtype_code(k_cache.dtype),
                               _lib._stream(stream)))
