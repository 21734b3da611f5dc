"""Binding of the host-side KV block manager in ``libpa.so``
(``include/pa_kv_manager.h``): free block queue, allocate_slots, reference
counts, hash-chained prefix caching, and the per-step inputs of ``pa_step``.

Argument marshalling only; every decision is made in the C++ library.
"""
from __future__ import annotations

import ctypes
from typing import Dict, Sequence

import numpy as np

from . import PAError, lib

_P = ctypes.c_void_p
_i32, _i64, _u64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64
_sigs = {
    "pa_kv_manager_create": ([_i32, _i32, _i32, ctypes.POINTER(_P)], ctypes.c_int),
    "pa_kv_manager_destroy": ([_P], None),
    "pa_kv_manager_num_free_blocks": ([_P], _i32),
    "pa_kv_manager_add_request": ([_P, _i64, _P, _i64, _u64, ctypes.POINTER(_i64)], ctypes.c_int),
    "pa_kv_manager_append_tokens": ([_P, _i64, _P, _i64], ctypes.c_int),
    "pa_kv_manager_allocate_slots": ([_P, _i64, _i64], ctypes.c_int),
    "pa_kv_manager_commit": ([_P, _i64, _i64], ctypes.c_int),
    "pa_kv_manager_free": ([_P, _i64], ctypes.c_int),
    "pa_kv_manager_build_step": ([_P, _i64, _P, _P, _i64, _P, _P, _P, _P, _P], ctypes.c_int),
    "pa_kv_manager_request_blocks": ([_P, _i64, _P, _i64, ctypes.POINTER(_i64), ctypes.POINTER(_i64)], ctypes.c_int),
    "pa_kv_manager_ref_count": ([_P, _i32], _i32),
    "pa_kv_manager_is_cached": ([_P, _i32], _i32),
}
for _name, (_args, _res) in _sigs.items():
    _f = getattr(lib, _name)
    _f.argtypes = _args
    _f.restype = _res
EXPORTS = tuple(_sigs)

PA_ERR_NO_BLOCKS = 8


def _check(rc: int):
    if rc != 0:
        raise PAError(rc, lib.pa_last_error().decode())


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data) if a.size else None


class KVCacheManager:
    """Owner of one ``pa_kv_manager``; names follow the C calls."""

    def __init__(self, num_blocks: int, block_size: int = 16, enable_prefix_caching: bool = True):
        h = _P()
        _check(lib.pa_kv_manager_create(num_blocks, block_size, int(enable_prefix_caching), ctypes.byref(h)))
        self._h = h
        self.num_blocks = num_blocks
        self.block_size = block_size

    def close(self):
        if self._h:
            lib.pa_kv_manager_destroy(self._h)
            self._h = _P()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @property
    def num_free_blocks(self) -> int:
        return lib.pa_kv_manager_num_free_blocks(self._h)

    def add_request(self, req_id: int, prompt: Sequence[int], salt: int = 0) -> int:
        """Admit a request; returns the number of prompt tokens already cached."""
        toks = np.ascontiguousarray(prompt, dtype=np.int32)
        n = _i64(0)
        _check(lib.pa_kv_manager_add_request(self._h, req_id, _ptr(toks), toks.size, salt, ctypes.byref(n)))
        return n.value

    def append_tokens(self, req_id: int, tokens: Sequence[int]):
        toks = np.ascontiguousarray(tokens, dtype=np.int32)
        _check(lib.pa_kv_manager_append_tokens(self._h, req_id, _ptr(toks), toks.size))

    def allocate_slots(self, req_id: int, num_new_tokens: int) -> bool:
        """True if the slots were allocated, False if the free queue is too short."""
        rc = lib.pa_kv_manager_allocate_slots(self._h, req_id, num_new_tokens)
        if rc == PA_ERR_NO_BLOCKS:
            return False
        _check(rc)
        return True

    def commit(self, req_id: int, num_new_tokens: int):
        _check(lib.pa_kv_manager_commit(self._h, req_id, num_new_tokens))

    def free(self, req_id: int):
        _check(lib.pa_kv_manager_free(self._h, req_id))

    def build_step(self, req_ids: Sequence[int], num_new: Sequence[int], max_blocks: int,
                   out: Dict[str, np.ndarray] = None) -> Dict[str, np.ndarray]:
        """Host arrays of one pa_step: query_start_loc, seq_lens, context_lens,
        block_tables, slot_mapping. ``out`` (a previous result of the same
        shapes) is written in place, which saves re-faulting fresh pages."""
        ids = np.ascontiguousarray(req_ids, dtype=np.int64)
        nn = np.ascontiguousarray(num_new, dtype=np.int64)
        S = ids.size
        T = int(nn.sum()) if S else 0
        shapes = {"query_start_loc": (S + 1,), "seq_lens": (S,), "context_lens": (S,),
                  "block_tables": (S, max_blocks), "slot_mapping": (T,)}
        if out is None or any(out[k].shape != v for k, v in shapes.items()):
            out = {k: np.empty(v, np.int64 if k == "slot_mapping" else np.int32) for k, v in shapes.items()}
        _check(lib.pa_kv_manager_build_step(self._h, S, _ptr(ids), _ptr(nn), max_blocks,
                                            _ptr(out["query_start_loc"]), _ptr(out["seq_lens"]),
                                            _ptr(out["context_lens"]), _ptr(out["block_tables"]),
                                            _ptr(out["slot_mapping"])))
        return out

    def request_blocks(self, req_id: int):
        """(block ids in order, computed token count) of a request."""
        n, c = _i64(0), _i64(0)
        _check(lib.pa_kv_manager_request_blocks(self._h, req_id, None, 0, ctypes.byref(n), ctypes.byref(c)))
        buf = np.zeros(n.value, np.int32)
        _check(lib.pa_kv_manager_request_blocks(self._h, req_id, _ptr(buf), buf.size, ctypes.byref(n),
                                                ctypes.byref(c)))
        return buf.tolist(), c.value

    def ref_count(self, block: int) -> int:
        return lib.pa_kv_manager_ref_count(self._h, block)

    def is_cached(self, block: int) -> bool:
        return lib.pa_kv_manager_is_cached(self._h, block) == 1
