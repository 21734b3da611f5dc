"""Oracle for paged attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import this package. The product library never loads it and shares no
code with it.

- ``liboracle.so`` (``oracle.c``): the paged reference in plain C, fp64 -- KV
  write through ``slot_mapping``, gather through block tables, two-pass softmax
  attention over the flattened super-sequence.
- ``dense.py``: brute-force dense attention in numpy on contiguous K/V, which
  pins the C oracle on small inputs.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

from .build import LIB, build as _build
from .dense import dense_attention, visibility_mask  # noqa: F401

DTYPES = {"f32": 0, "bf16": 1, "fp8": 2}
ERRORS = {1: "bad argument", 2: "inconsistent metadata", 3: "bad or duplicate slot", 4: "out of memory"}

_lib = None


class OracleError(RuntimeError):
    pass


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            _build()
        L = ctypes.CDLL(LIB)
        i64, i32, p = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
        L.oracle_reshape_and_cache.argtypes = [p, p, p, p, i64, i64, i64, i64, i32]
        L.oracle_reshape_and_cache.restype = i32
        L.oracle_gather.argtypes = [p, p, p, i64, i64, i64, i64, i64, i32, i32]
        L.oracle_gather.restype = i32
        L.oracle_attention.argtypes = [p, p, p, p, p, p, p, i64, i64, i64, i64, i64, i64, i32,
                                       ctypes.c_double, i32, ctypes.POINTER(ctypes.c_int)]
        L.oracle_attention.restype = i32
        f32, f64 = ctypes.c_float, ctypes.c_double
        L.oracle_reshape_and_cache_fp8.argtypes = [p, p, p, p, i64, i64, i64, i64, i32, f32, f32]
        L.oracle_reshape_and_cache_fp8.restype = i32
        L.oracle_attention_kv.argtypes = [p, p, p, p, p, p, p, i64, i64, i64, i64, i64, i64, i32, i32, f32, f32,
                                          f64, i32, ctypes.POINTER(ctypes.c_int)]
        L.oracle_attention_kv.restype = i32
        L.oracle_fp8_quantize_array.argtypes = [p, i32, f32, p, i64]
        L.oracle_fp8_quantize_array.restype = i32
        L.oracle_fp8_decode_array.argtypes = [p, p, i64]
        L.oracle_fp8_decode_array.restype = i32
        _lib = L
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _check(rc: int):
    if rc != 0:
        raise OracleError(ERRORS.get(rc, f"error {rc}"))


def reshape_and_cache(k: np.ndarray, v: np.ndarray, pool: np.ndarray, slot_mapping: np.ndarray, dtype: str):
    """In-place KV write into the host pool [NB, 2, 16, Hkv, D]."""
    assert pool.flags.c_contiguous and pool.ndim == 5 and pool.shape[2] == 16
    k = np.ascontiguousarray(k)
    v = np.ascontiguousarray(v)
    sm = np.ascontiguousarray(slot_mapping, dtype=np.int64)
    NB, _, _, Hkv, D = pool.shape
    assert k.shape == v.shape == (sm.shape[0], Hkv, D) and k.dtype == v.dtype == pool.dtype
    _check(lib().oracle_reshape_and_cache(_ptr(k), _ptr(v), _ptr(pool), _ptr(sm), sm.shape[0], NB, Hkv, D,
                                          DTYPES[dtype]))


def gather(pool: np.ndarray, table_row: np.ndarray, L: int, head: int, which: str, dtype: str) -> np.ndarray:
    """Rows 0..L-1 of one KV head of one sequence, through its block-table row (fp64 [L, D])."""
    NB, _, _, Hkv, D = pool.shape
    row = np.ascontiguousarray(table_row, dtype=np.int32)
    out = np.empty((L, D), np.float64)
    _check(lib().oracle_gather(_ptr(out), _ptr(pool), _ptr(row), L, NB, Hkv, D, head, 0 if which == "k" else 1,
                               DTYPES[dtype]))
    return out


def attention(q: np.ndarray, pool: np.ndarray, block_tables: np.ndarray, query_start_loc: np.ndarray,
              seq_lens: np.ndarray, context_lens: np.ndarray, scale: float, dtype: str,
              num_threads: int = 0, return_threads: bool = False):
    """Attention over the flattened super-sequence; returns fp64 [T, Hq, D]."""
    q = np.ascontiguousarray(q)
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    qsl = np.ascontiguousarray(query_start_loc, dtype=np.int32)
    sl = np.ascontiguousarray(seq_lens, dtype=np.int32)
    cl = np.ascontiguousarray(context_lens, dtype=np.int32)
    NB, _, _, Hkv, D = pool.shape
    T, Hq, Dq = q.shape
    assert Dq == D and q.dtype == pool.dtype and pool.flags.c_contiguous
    S, MB = bt.shape
    out = np.empty((T, Hq, D), np.float64)
    used = ctypes.c_int(0)
    _check(lib().oracle_attention(_ptr(out), _ptr(q), _ptr(pool), _ptr(bt), _ptr(qsl), _ptr(sl), _ptr(cl),
                                  S, MB, NB, Hq, Hkv, D, DTYPES[dtype], float(scale), int(num_threads),
                                  ctypes.byref(used)))
    return (out, used.value) if return_threads else out


def run_workload(wl, pool: Optional[np.ndarray] = None, num_threads: int = 0):
    """Full oracle step on a workload: host pool, KV write, attention.

    Returns (out fp64 [T, Hq, D], pool after the write).
    """
    import workloads

    if pool is None:
        pool = workloads.pool_host(wl)
    k, v = workloads.new_kv_host(wl)
    q = workloads.q_host(wl)
    if wl.kv_dtype == "fp8":
        reshape_and_cache_fp8(k, v, pool, wl.slot_mapping, wl.dtype, wl.k_scale, wl.v_scale)
        out = attention_fp8(q, pool, wl.block_tables, wl.query_start_loc, wl.seq_lens, wl.context_lens, wl.scale,
                            wl.dtype, wl.k_scale, wl.v_scale, num_threads=num_threads)
        return out, pool
    reshape_and_cache(k, v, pool, wl.slot_mapping, wl.dtype)
    out = attention(q, pool, wl.block_tables, wl.query_start_loc, wl.seq_lens, wl.context_lens, wl.scale,
                    wl.dtype, num_threads=num_threads)
    return out, pool


# ---- 8-bit (OCP FP8 E4M3) KV pool -------------------------------------------


def fp8_quantize(x: np.ndarray, dtype: str, scale: float) -> np.ndarray:
    """Codes encode(x / scale) (quotient in fp32) of an f32 or bf16 (bit pattern) array."""
    x = np.ascontiguousarray(x)
    out = np.empty(x.shape, np.uint8)
    _check(lib().oracle_fp8_quantize_array(_ptr(x), DTYPES[dtype], float(scale), _ptr(out), x.size))
    return out


def fp8_decode(codes: np.ndarray) -> np.ndarray:
    """Exact values (fp64) of E4M3 codes; NaN for 0x7F / 0xFF."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    out = np.empty(codes.shape, np.float64)
    _check(lib().oracle_fp8_decode_array(_ptr(codes), _ptr(out), codes.size))
    return out


def reshape_and_cache_fp8(k: np.ndarray, v: np.ndarray, pool: np.ndarray, slot_mapping: np.ndarray, dtype: str,
                          k_scale: float, v_scale: float):
    """In-place KV write of f32/bf16 rows into an fp8 host pool (uint8 [NB, 2, 16, Hkv, D])."""
    assert pool.flags.c_contiguous and pool.ndim == 5 and pool.shape[2] == 16 and pool.dtype == np.uint8
    k = np.ascontiguousarray(k)
    v = np.ascontiguousarray(v)
    sm = np.ascontiguousarray(slot_mapping, dtype=np.int64)
    NB, _, _, Hkv, D = pool.shape
    assert k.shape == v.shape == (sm.shape[0], Hkv, D)
    _check(lib().oracle_reshape_and_cache_fp8(_ptr(k), _ptr(v), _ptr(pool), _ptr(sm), sm.shape[0], NB, Hkv, D,
                                              DTYPES[dtype], float(k_scale), float(v_scale)))


def attention_fp8(q: np.ndarray, pool: np.ndarray, block_tables: np.ndarray, query_start_loc: np.ndarray,
                  seq_lens: np.ndarray, context_lens: np.ndarray, scale: float, dtype: str, k_scale: float,
                  v_scale: float, num_threads: int = 0) -> np.ndarray:
    """Attention with q of ``dtype`` over an fp8 pool read back as decode(code) * scale."""
    q = np.ascontiguousarray(q)
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    qsl = np.ascontiguousarray(query_start_loc, dtype=np.int32)
    sl = np.ascontiguousarray(seq_lens, dtype=np.int32)
    cl = np.ascontiguousarray(context_lens, dtype=np.int32)
    NB, _, _, Hkv, D = pool.shape
    T, Hq, _ = q.shape
    assert pool.dtype == np.uint8 and pool.flags.c_contiguous
    S, MB = bt.shape
    out = np.empty((T, Hq, D), np.float64)
    used = ctypes.c_int(0)
    _check(lib().oracle_attention_kv(_ptr(out), _ptr(q), _ptr(pool), _ptr(bt), _ptr(qsl), _ptr(sl), _ptr(cl), S,
                                     MB, NB, Hq, Hkv, D, DTYPES[dtype], DTYPES["fp8"], float(k_scale),
                                     float(v_scale), float(scale), int(num_threads), ctypes.byref(used)))
    return out
