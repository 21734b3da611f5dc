"""Paged attention over a block-paged KV cache on AMD MI355X (gfx950).

Thin Python binding of ``libpa.so`` (C ABI in ``include/pa.h``): it only
marshals torch tensors into descriptors and passes the current HIP stream.
Every step of the computation runs in the library's HIP kernels; there is no
fallback path. Importing fails if the library has not been built.

Calls (same names and argument order as the C ABI):
- ``reshape_and_cache(k, v, key_cache, value_cache, slot_mapping)``
- ``attention(q, key_cache, value_cache, block_tables, query_start_loc,
  seq_lens, context_lens, scale, out=None, workspace=None) -> out``
- ``step(q, k, v, key_cache, value_cache, slot_mapping, block_tables,
  query_start_loc, seq_lens, context_lens, scale, out=None, workspace=None)``
- ``step_noalloc(...)``: ``step`` without a workspace argument, on the
  library's fixed per-GPU scratch (for callers that cannot allocate)

KV pool layout: ``pool = new_kv_pool(num_blocks, num_kv_heads, head_size)``
has shape ``[num_blocks, 2, 16, num_kv_heads, head_size]``; ``pool[:, 0]`` is
the key cache and ``pool[:, 1]`` the value cache.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
# PA_LIBRARY names another build of the library (for side-by-side timing);
# by default the in-package libpa.so is loaded.
LIB_PATH = os.environ.get("PA_LIBRARY") or os.path.join(HERE, "libpa.so")
BLOCK_SIZE = 16

PA_F32, PA_BF16, PA_I32, PA_I64, PA_FP8_E4M3 = 0, 1, 2, 3, 4
STATUS = {
    0: "PA_OK", 1: "PA_ERR_NULL", 2: "PA_ERR_DTYPE", 3: "PA_ERR_SHAPE", 4: "PA_ERR_STRIDE",
    5: "PA_ERR_UNSUPPORTED", 6: "PA_ERR_WORKSPACE", 7: "PA_ERR_HIP", 8: "PA_ERR_NO_BLOCKS", 9: "PA_ERR_REQUEST",
    10: "PA_ERR_CONTENTS",
}
EXPORTS = ("pa_reshape_and_cache", "pa_attention", "pa_step", "pa_reshape_and_cache_fp8", "pa_attention_fp8",
           "pa_step_fp8", "pa_step_noalloc", "pa_attention_workspace_size", "pa_partition_tokens", "pa_status_string",
           "pa_last_error", "pa_version")
PROFILE_EXPORTS = ("pa_profile_start", "pa_profile_stop", "pa_profile_kernel", "pa_profile_kernel_name",
                   "pa_profile_read_probe")
KERNELS = ("kv_write", "decode", "partition_reduce", "prefill_plan", "prefill", "kv_write_plan", "decode_order")


class PAError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


class Tensor(ctypes.Structure):
    """ctypes mirror of ``pa_tensor``."""

    _fields_ = [
        ("data", ctypes.c_void_p),
        ("dtype", ctypes.c_int32),
        ("ndim", ctypes.c_int32),
        ("shape", ctypes.c_int64 * 4),
        ("stride", ctypes.c_int64 * 4),
    ]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() (hipcc, gfx950)")
    # One HIP runtime per process. torch ships its own libamdhip64; once it is
    # loaded, libpa.so's dependency resolves to it. Loaded first, libpa.so
    # would pull in the system runtime, torch would then load its own beside
    # it, and the library's launches would find no device.
    import torch  # noqa: F401

    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER(Tensor)
    vp, sz, i64 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int64
    lib.pa_reshape_and_cache.argtypes = [P, P, P, P, P, vp]
    lib.pa_attention.argtypes = [P, P, P, P, P, P, P, P, ctypes.c_float, vp, sz, vp]
    lib.pa_step.argtypes = [P, P, P, P, P, P, P, P, P, P, P, ctypes.c_float, vp, sz, vp]
    f32 = ctypes.c_float
    lib.pa_reshape_and_cache_fp8.argtypes = [P, P, P, P, P, f32, f32, vp]
    lib.pa_attention_fp8.argtypes = [P, P, P, P, P, P, P, P, f32, f32, f32, vp, sz, vp]
    lib.pa_step_fp8.argtypes = [P, P, P, P, P, P, P, P, P, P, P, f32, f32, f32, vp, sz, vp]
    lib.pa_step_noalloc.argtypes = [P, P, P, P, P, P, P, P, P, P, P, f32, vp]
    for f in ("pa_reshape_and_cache", "pa_attention", "pa_step", "pa_reshape_and_cache_fp8", "pa_attention_fp8",
              "pa_step_fp8", "pa_step_noalloc"):
        getattr(lib, f).restype = ctypes.c_int
    lib.pa_attention_workspace_size.argtypes = [i64] * 6
    lib.pa_attention_workspace_size.restype = sz
    lib.pa_partition_tokens.argtypes = [i64, i64, i64, ctypes.c_int32, ctypes.c_int32, i64]
    lib.pa_partition_tokens.restype = i64
    lib.pa_status_string.argtypes = [ctypes.c_int]
    lib.pa_status_string.restype = ctypes.c_char_p
    lib.pa_last_error.argtypes = []
    lib.pa_last_error.restype = ctypes.c_char_p
    lib.pa_version.restype = ctypes.c_int
    lib.pa_profile_start.restype = ctypes.c_int
    lib.pa_profile_stop.restype = ctypes.c_int
    lib.pa_profile_kernel.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64)]
    lib.pa_profile_kernel.restype = ctypes.c_int
    lib.pa_profile_kernel_name.argtypes = [ctypes.c_int]
    lib.pa_profile_kernel_name.restype = ctypes.c_char_p
    lib.pa_profile_read_probe.argtypes = [vp, ctypes.c_uint64, vp]
    lib.pa_profile_read_probe.restype = ctypes.c_int
    return lib


lib = _load()


def _dtype_code(t) -> int:
    import torch

    codes = {torch.float32: PA_F32, torch.bfloat16: PA_BF16, torch.int32: PA_I32, torch.int64: PA_I64,
             torch.float8_e4m3fn: PA_FP8_E4M3}
    if t.dtype not in codes:
        raise PAError(2, f"unsupported torch dtype {t.dtype}")
    return codes[t.dtype]


def describe(t) -> Tensor:
    """Descriptor of a torch tensor (device pointer, dtype, shape, element strides)."""
    if t.dim() > 4:
        raise PAError(3, f"tensor of rank {t.dim()} > 4")
    d = Tensor()
    d.data = t.data_ptr() if t.numel() else None
    d.dtype = _dtype_code(t)
    d.ndim = t.dim()
    for i in range(t.dim()):
        d.shape[i] = t.shape[i]
        d.stride[i] = t.stride(i)
    return d


def _ptr(d: Tensor):
    return ctypes.byref(d)


def _check(rc: int):
    if rc != 0:
        raise PAError(rc, lib.pa_last_error().decode())


def _stream(t):
    import torch

    if t.device.type != "cuda":
        raise PAError(1, "tensors must be on a GPU device")
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def new_kv_pool(num_blocks: int, num_kv_heads: int, head_size: int, dtype=None, device="cuda"):
    """Allocate a pool [num_blocks, 2, 16, num_kv_heads, head_size] (contents undefined)."""
    import torch

    dtype = torch.bfloat16 if dtype is None else dtype
    return torch.empty((num_blocks, 2, BLOCK_SIZE, num_kv_heads, head_size), dtype=dtype, device=device)


def workspace_size(num_seqs: int, num_tokens: int, num_q_heads: int, num_kv_heads: int, head_size: int,
                   max_blocks_per_seq: int) -> int:
    return int(lib.pa_attention_workspace_size(num_seqs, num_tokens, num_q_heads, num_kv_heads, head_size,
                                               max_blocks_per_seq))


def partition_tokens(num_seqs: int, num_kv_heads: int, head_size: int, dtype: str, max_blocks_per_seq: int,
                     kv_fp8: bool = False) -> int:
    """Decode partition size pa_attention / pa_step choose (pa_partition_tokens).
    dtype: "bf16" or "f32" (queries and cache); kv_fp8: an 8-bit pool under bf16 queries."""
    q = {"bf16": PA_BF16, "f32": PA_F32}[dtype]
    return int(lib.pa_partition_tokens(num_seqs, num_kv_heads, head_size, q, PA_FP8_E4M3 if kv_fp8 else q,
                                       max_blocks_per_seq))


def new_workspace(q, key_cache, block_tables):
    """Workspace sized for these tensors (a uint8 device tensor)."""
    import torch

    T, Hq, D = q.shape
    n = workspace_size(block_tables.shape[0], T, Hq, key_cache.shape[2], D, block_tables.shape[1])
    return torch.empty(max(n, 1), dtype=torch.uint8, device=q.device)


def reshape_and_cache(k, v, key_cache, value_cache, slot_mapping) -> None:
    ds = [describe(x) for x in (k, v, key_cache, value_cache, slot_mapping)]
    _check(lib.pa_reshape_and_cache(*[_ptr(d) for d in ds], _stream(key_cache)))


def attention(q, key_cache, value_cache, block_tables, query_start_loc, seq_lens, context_lens, scale: float,
              out=None, workspace=None):
    import torch

    out = torch.empty_like(q) if out is None else out
    ws = new_workspace(q, key_cache, block_tables) if workspace is None else workspace
    ds = [describe(x) for x in (out, q, key_cache, value_cache, block_tables, query_start_loc, seq_lens,
                                context_lens)]
    _check(lib.pa_attention(*[_ptr(d) for d in ds], ctypes.c_float(scale), ctypes.c_void_p(ws.data_ptr()),
                            ctypes.c_size_t(ws.numel() * ws.element_size()), _stream(q)))
    return out


def step(q, k, v, key_cache, value_cache, slot_mapping, block_tables, query_start_loc, seq_lens, context_lens,
         scale: float, out=None, workspace=None):
    import torch

    out = torch.empty_like(q) if out is None else out
    ws = new_workspace(q, key_cache, block_tables) if workspace is None else workspace
    ds = [describe(x) for x in (out, q, k, v, key_cache, value_cache, slot_mapping, block_tables,
                                query_start_loc, seq_lens, context_lens)]
    _check(lib.pa_step(*[_ptr(d) for d in ds], ctypes.c_float(scale), ctypes.c_void_p(ws.data_ptr()),
                       ctypes.c_size_t(ws.numel() * ws.element_size()), _stream(q)))
    return out


NOALLOC_SCRATCH_BYTES = 64 << 20  # PA_NOALLOC_SCRATCH_BYTES in include/pa.h


def step_noalloc(q, k, v, key_cache, value_cache, slot_mapping, block_tables, query_start_loc, seq_lens,
                 context_lens, scale: float, out=None):
    """pa_step_noalloc: pa_step with the library's fixed per-GPU scratch as its
    workspace (nothing is allocated on the device by the call; `out` is
    allocated here only if it is not given)."""
    import torch

    out = torch.empty_like(q) if out is None else out
    ds = [describe(x) for x in (out, q, k, v, key_cache, value_cache, slot_mapping, block_tables,
                                query_start_loc, seq_lens, context_lens)]
    _check(lib.pa_step_noalloc(*[_ptr(d) for d in ds], ctypes.c_float(scale), _stream(q)))
    return out


def reshape_and_cache_fp8(k, v, key_cache, value_cache, slot_mapping, k_scale: float, v_scale: float) -> None:
    """KV write into an 8-bit pool (torch.float8_e4m3fn caches): code = nearest(x / scale)."""
    ds = [describe(x) for x in (k, v, key_cache, value_cache, slot_mapping)]
    _check(lib.pa_reshape_and_cache_fp8(*[_ptr(d) for d in ds], ctypes.c_float(k_scale), ctypes.c_float(v_scale),
                                        _stream(key_cache)))


def attention_fp8(q, key_cache, value_cache, block_tables, query_start_loc, seq_lens, context_lens, scale: float,
                  k_scale: float, v_scale: float, out=None, workspace=None):
    import torch

    out = torch.empty_like(q) if out is None else out
    ws = new_workspace(q, key_cache, block_tables) if workspace is None else workspace
    ds = [describe(x) for x in (out, q, key_cache, value_cache, block_tables, query_start_loc, seq_lens,
                                context_lens)]
    _check(lib.pa_attention_fp8(*[_ptr(d) for d in ds], ctypes.c_float(scale), ctypes.c_float(k_scale),
                                ctypes.c_float(v_scale), ctypes.c_void_p(ws.data_ptr()),
                                ctypes.c_size_t(ws.numel() * ws.element_size()), _stream(q)))
    return out


def step_fp8(q, k, v, key_cache, value_cache, slot_mapping, block_tables, query_start_loc, seq_lens, context_lens,
             scale: float, k_scale: float, v_scale: float, out=None, workspace=None):
    import torch

    out = torch.empty_like(q) if out is None else out
    ws = new_workspace(q, key_cache, block_tables) if workspace is None else workspace
    ds = [describe(x) for x in (out, q, k, v, key_cache, value_cache, slot_mapping, block_tables,
                                query_start_loc, seq_lens, context_lens)]
    _check(lib.pa_step_fp8(*[_ptr(d) for d in ds], ctypes.c_float(scale), ctypes.c_float(k_scale),
                           ctypes.c_float(v_scale), ctypes.c_void_p(ws.data_ptr()),
                           ctypes.c_size_t(ws.numel() * ws.element_size()), _stream(q)))
    return out


def read_probe(buf) -> None:
    """One non-temporal read of every byte of the device tensor `buf` on the
    current stream (pa_profile_read_probe): the GPU's plain read stream."""
    _check(lib.pa_profile_read_probe(ctypes.c_void_p(buf.data_ptr()), ctypes.c_uint64(buf.numel() * buf.element_size()),
                                     _stream(buf)))


class profile:
    """Context manager: per-kernel HIP-event times of the library's launches.

    with pa.profile() as prof:
        ...  # library calls
    prof.kernels -> {name: (total_ms, launches)} for kernels that ran
    """

    def __enter__(self):
        _check(lib.pa_profile_start())
        self.kernels = {}
        return self

    def __exit__(self, *exc):
        lib.pa_profile_stop()
        for i in range(len(KERNELS)):
            name = lib.pa_profile_kernel_name(i).decode()
            if not name:  # a library build with fewer kernels
                break
            ms, n = ctypes.c_double(0), ctypes.c_int64(0)
            _check(lib.pa_profile_kernel(i, ctypes.byref(ms), ctypes.byref(n)))
            if n.value:
                self.kernels[name] = (ms.value, n.value)
        return False
