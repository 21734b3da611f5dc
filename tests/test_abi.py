"""C ABI of libpa.so on the CPU: the library loads, exports what include/pa.h
declares, and rejects invalid descriptors with the documented status codes
before launching anything (no GPU needed: validation never touches device
memory, the pointers below are never dereferenced)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
# A missing libpa.so is a failure here, not a skip: the import raises.
import pagedattention_block_paged_amd as pa  # noqa: E402
from pagedattention_block_paged_amd import Tensor, lib  # noqa: E402

PA_OK, PA_ERR_NULL, PA_ERR_DTYPE, PA_ERR_SHAPE, PA_ERR_STRIDE, PA_ERR_UNSUPPORTED, PA_ERR_WORKSPACE = range(7)
F32, BF16, I32, I64 = 0, 1, 2, 3
FAKE = 0x7F0000000000  # 256-byte aligned, never dereferenced


def declared_functions(header):
    src = open(os.path.join(ROOT, "include", header)).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w]+\**\s+\**(pa_\w+)\s*\(", src, flags=re.M)))


@pytest.mark.parametrize("header,expected", [("pa.h", "EXPORTS"), ("pa_profile.h", "PROFILE_EXPORTS"),
                                             ("pa_kv_manager.h", "KV_MANAGER_EXPORTS")])
def test_exports_match_header(header, expected):
    names = declared_functions(header)
    if expected == "KV_MANAGER_EXPORTS":
        from pagedattention_block_paged_amd import kv_manager

        exported = kv_manager.EXPORTS
    else:
        exported = getattr(pa, expected)
    assert names and set(names) == set(exported), names
    for name in names:
        assert hasattr(lib, name), name  # resolves the symbol in libpa.so


def test_one_hip_runtime_per_process():
    """Importing the binding first must not load a second HIP runtime beside
    torch's: the library's launches would then find no device."""
    import subprocess
    import sys

    code = ("import pagedattention_block_paged_amd, torch\n"
            "maps = {l.split()[-1] for l in open('/proc/self/maps') if 'libamdhip64' in l}\n"
            "print(len(maps))\n")
    out = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True, check=True)
    assert out.stdout.strip() == "1", out.stdout + out.stderr


def desc(shape, dtype, strides=None, data=FAKE):
    d = Tensor()
    d.data = data
    d.dtype = dtype
    d.ndim = len(shape)
    if strides is None:
        strides, acc = [], 1
        for s in reversed(shape):
            strides.insert(0, acc)
            acc *= s
    for i, (s, st) in enumerate(zip(shape, strides)):
        d.shape[i] = s
        d.stride[i] = st
    return d


class Case:
    """A valid decode batch description; tests mutate one field each."""

    def __init__(self, T=4, S=4, Hq=8, Hkv=2, D=64, NB=32, MB=8, dt=BF16):
        pool_strides = [2 * 16 * Hkv * D, Hkv * D, D, 1]
        self.q = desc([T, Hq, D], dt)
        self.out = desc([T, Hq, D], dt, data=FAKE + (1 << 30))
        self.k = desc([T, Hkv, D], dt)
        self.v = desc([T, Hkv, D], dt)
        self.kc = desc([NB, 16, Hkv, D], dt, pool_strides)
        self.vc = desc([NB, 16, Hkv, D], dt, pool_strides, data=FAKE + 16 * Hkv * D * 2)
        self.slots = desc([T], I64)
        self.bt = desc([S, MB], I32)
        self.qsl = desc([S + 1], I32)
        self.sl = desc([S], I32)
        self.cl = desc([S], I32)
        self.ws_bytes = pa.workspace_size(S, T, Hq, Hkv, D, MB)
        self.ws = FAKE + (1 << 31)

    def attention(self, scale=0.125):
        r = lambda d: ctypes.byref(d) if d is not None else None
        return lib.pa_attention(r(self.out), r(self.q), r(self.kc), r(self.vc), r(self.bt), r(self.qsl), r(self.sl),
                                r(self.cl), ctypes.c_float(scale), ctypes.c_void_p(self.ws), self.ws_bytes, None)

    def write(self):
        r = lambda d: ctypes.byref(d) if d is not None else None
        return lib.pa_reshape_and_cache(r(self.k), r(self.v), r(self.kc), r(self.vc), r(self.slots), None)


def err():
    return lib.pa_last_error().decode()


def test_workspace_size_and_partitions():
    assert pa.workspace_size(0, 0, 8, 2, 64, 8) > 0
    assert pa.workspace_size(4, 4, 8, 2, 64, 0) == 0
    assert pa.partition_tokens(64, 4, 64, "bf16", 128) % 16 == 0
    # long contexts on few sequences split into more partitions than short ones
    assert pa.partition_tokens(32, 8, 128, "bf16", 2048) >= pa.partition_tokens(64, 4, 64, "bf16", 128)
    # the workspace holds the partials of every decode kernel's partitioning
    for D, dt, fp8 in [(128, "bf16", False), (128, "bf16", True), (64, "bf16", False), (128, "f32", False)]:
        big = pa.workspace_size(32, 32, 64, 8, D, 2048)
        pt = pa.partition_tokens(32, 8, D, dt, 2048, kv_fp8=fp8)
        assert big >= 32 * 64 * (2048 * 16 // pt) * D * 4
    # invalid element types or head sizes
    assert lib.pa_partition_tokens(4, 2, 96, 1, 1, 16) == 0
    assert lib.pa_partition_tokens(4, 2, 128, 0, 4, 16) == 0


@pytest.mark.parametrize("field,status", [
    ("q", PA_ERR_NULL), ("out", PA_ERR_NULL), ("kc", PA_ERR_NULL), ("vc", PA_ERR_NULL), ("bt", PA_ERR_NULL),
    ("qsl", PA_ERR_NULL), ("sl", PA_ERR_NULL), ("cl", PA_ERR_NULL)])
def test_null_descriptor(field, status):
    c = Case()
    setattr(c, field, None)
    assert c.attention() == status
    assert err()


def test_null_data_pointer():
    c = Case()
    c.q.data = None
    assert c.attention() == PA_ERR_NULL and "q" in err()


def test_dtype_errors():
    c = Case()
    c.q.dtype = F32
    assert c.attention() == PA_ERR_DTYPE
    c = Case()
    c.bt.dtype = I64
    assert c.attention() == PA_ERR_DTYPE
    c = Case()
    c.slots.dtype = I32
    assert c.write() == PA_ERR_DTYPE
    c = Case()
    c.kc.dtype = I32
    assert c.attention() == PA_ERR_DTYPE
    c = Case()
    c.vc.dtype = F32
    assert c.write() == PA_ERR_DTYPE


def test_shape_errors():
    c = Case()
    c.qsl.shape[0] = 4  # needs S + 1
    assert c.attention() == PA_ERR_SHAPE
    c = Case()
    c.q.shape[1] = 7  # 7 query heads over 2 KV heads
    c.out.shape[1] = 7
    assert c.attention() == PA_ERR_SHAPE
    c = Case()
    c.out.shape[0] = 3
    assert c.attention() == PA_ERR_SHAPE
    c = Case()
    c.slots.shape[0] = 5
    assert c.write() == PA_ERR_SHAPE
    c = Case()
    c.k.shape[2] = 128
    assert c.write() == PA_ERR_SHAPE
    c = Case()
    c.bt.ndim = 1
    assert c.attention() == PA_ERR_SHAPE


def test_stride_and_alignment_errors():
    c = Case()
    c.q.stride[2] = 2
    assert c.attention() == PA_ERR_STRIDE
    c = Case()
    c.q.data = FAKE + 2
    assert c.attention() == PA_ERR_STRIDE
    c = Case()
    c.kc.stride[1] = 3  # row stride not a multiple of 16 bytes
    assert c.attention() == PA_ERR_STRIDE
    c = Case()
    c.bt.stride[1] = 2
    assert c.attention() == PA_ERR_STRIDE


def test_unsupported_sizes():
    c = Case()
    c.kc.shape[1] = c.vc.shape[1] = 8  # block size 8
    assert c.attention() == PA_ERR_UNSUPPORTED and "block size" in err()
    c = Case(D=96)
    assert c.attention() == PA_ERR_UNSUPPORTED
    c = Case(Hq=34, Hkv=2)  # 17 query heads per KV head
    assert c.attention() == PA_ERR_UNSUPPORTED


def test_workspace_errors():
    c = Case()
    c.ws_bytes -= 1
    assert c.attention() == PA_ERR_WORKSPACE
    c = Case()
    c.ws = 0
    assert c.attention() == PA_ERR_WORKSPACE
    c = Case()
    c.ws = FAKE + 8
    assert c.attention() == PA_ERR_WORKSPACE


def test_scale_must_be_finite():
    c = Case()
    assert c.attention(scale=float("nan")) == PA_ERR_SHAPE


def test_step_checks_token_counts():
    c = Case()
    r = ctypes.byref
    k = desc([3, 2, 64], BF16)
    slots = desc([3], I64)
    rc = lib.pa_step(r(c.out), r(c.q), r(k), r(k), r(c.kc), r(c.vc), r(slots), r(c.bt), r(c.qsl), r(c.sl), r(c.cl),
                     ctypes.c_float(0.1), ctypes.c_void_p(c.ws), c.ws_bytes, None)
    assert rc == PA_ERR_SHAPE and "tokens" in err()


def test_status_strings():
    names = [lib.pa_status_string(code) for code in range(11)]  # PA_OK .. PA_ERR_CONTENTS
    assert all(names) and len(set(names)) == 11 and b"unknown status" not in names
    assert lib.pa_status_string(11) == b"unknown status"
    assert lib.pa_version() >= 100


FP8 = 4


def fp8_case(D=64, NB=32, Hkv=2):
    c = Case(D=D, NB=NB, Hkv=Hkv)
    pool_strides = [2 * 16 * Hkv * D, Hkv * D, D, 1]
    c.kc = desc([NB, 16, Hkv, D], FP8, pool_strides)
    c.vc = desc([NB, 16, Hkv, D], FP8, pool_strides, data=FAKE + 16 * Hkv * D)
    return c


def attention_fp8(c, ks=0.5, vs=0.25):
    r = lambda d: ctypes.byref(d)
    return lib.pa_attention_fp8(r(c.out), r(c.q), r(c.kc), r(c.vc), r(c.bt), r(c.qsl), r(c.sl), r(c.cl),
                                ctypes.c_float(0.125), ctypes.c_float(ks), ctypes.c_float(vs),
                                ctypes.c_void_p(c.ws), c.ws_bytes, None)


def write_fp8(c, ks=0.5, vs=0.25):
    r = lambda d: ctypes.byref(d)
    return lib.pa_reshape_and_cache_fp8(r(c.k), r(c.v), r(c.kc), r(c.vc), r(c.slots), ctypes.c_float(ks),
                                        ctypes.c_float(vs), None)


def test_fp8_pool_validation():
    # the f32/bf16 calls refuse an 8-bit pool (they carry no scales)
    c = fp8_case()
    assert c.attention() == PA_ERR_DTYPE and "_fp8" in err()
    assert c.write() == PA_ERR_DTYPE
    # scales must be finite and positive
    for ks, vs in ((0.0, 1.0), (1.0, -1.0), (float("inf"), 1.0), (float("nan"), 1.0)):
        assert attention_fp8(fp8_case(), ks, vs) == PA_ERR_SHAPE
        assert write_fp8(fp8_case(), ks, vs) == PA_ERR_SHAPE
    # q and out are bf16 over an 8-bit pool; k and v may be f32 or bf16
    c = fp8_case()
    c.q = desc([4, 8, 64], F32)
    assert attention_fp8(c) == PA_ERR_DTYPE
    c = fp8_case()
    c.k = desc([0, 2, 64], F32)
    c.v = desc([0, 2, 64], F32)
    c.slots = desc([0], I64)
    assert write_fp8(c) == PA_OK  # accepted; an empty batch launches nothing
    c.k = desc([0, 2, 64], I32)
    assert write_fp8(c) == PA_ERR_DTYPE


def test_step_noalloc_without_a_gpu_reports_an_error():
    """On a machine with no GPU the allocation-free step reports PA_ERR_HIP
    (it looks up the stream's device first) instead of touching memory."""
    import torch

    if torch.cuda.is_available():
        pytest.skip("a GPU is present: the GPU tests cover pa_step_noalloc")
    d = Tensor()
    rc = lib.pa_step_noalloc(*([ctypes.byref(d)] * 11), ctypes.c_float(0.125), None)
    assert rc == 7 and b"pa_step_noalloc" in lib.pa_last_error()
