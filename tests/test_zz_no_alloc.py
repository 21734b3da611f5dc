"""pa_step_noalloc, the entry point that allocates nothing, through the C ABI.

It must give what pa_step gives on the same inputs (the same kernels, so the
same bits), on two calls in a row (the second with a smaller batch, over the
scratch the first one left), and reject a step whose workspace would exceed
the fixed scratch before launching anything.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import device_case, raw_bytes, to_f64
from parity import assert_within

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pa():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import pagedattention_block_paged_amd as lib

    return lib


def say(*a):
    print(*a, flush=True)


def args_of(c):
    pool = c["pool"]
    return (c["q"], c["k"], c["v"], pool[:, 0], pool[:, 1], c["slot_mapping"], c["block_tables"],
            c["query_start_loc"], c["seq_lens"], c["context_lens"])


def test_noalloc_equals_step_on_two_calls_second_smaller(pa):
    rs = np.random.default_rng(5)
    # 60 decodes, 4 short verification queries and 2 chunks (60 MiB of the
    # 64 MiB scratch), then 18 decodes, 2 short queries and a chunk (31 MiB)
    big_ctx = [int(x) for x in rs.integers(0, 3000, size=64)] + [100, 2000]
    big = W.build_workload("noalloc_big", "bf16", 32, 8, 128, big_ctx, [1] * 60 + [3, 2, 4, 1] + [150, 96], seed=61)
    small_ctx = [int(x) for x in rs.integers(0, 1500, size=20)] + [300]
    small = W.build_workload("noalloc_small", "bf16", 32, 8, 128, small_ctx, [1] * 18 + [2, 4] + [64], seed=62)
    assert small.num_tokens < big.num_tokens and small.num_seqs < big.num_seqs
    for wl in (big, small):
        need = pa.workspace_size(wl.num_seqs, wl.num_tokens, wl.num_q_heads, wl.num_kv_heads, wl.head_size,
                                 wl.max_blocks)
        say(f"[noalloc] {wl.name}: S={wl.num_seqs} T={wl.num_tokens}, workspace {need} bytes")
        assert need <= pa.NOALLOC_SCRATCH_BYTES
        c_ref, c_new = device_case(wl), device_case(wl)
        ref = pa.step(*args_of(c_ref), wl.scale)
        out = torch.full_like(c_new["q"], float("nan"))
        got = pa.step_noalloc(*args_of(c_new), wl.scale, out=out)
        torch.cuda.synchronize()
        assert got.data_ptr() == out.data_ptr()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), "outputs differ from pa_step"
        assert np.array_equal(raw_bytes(c_new["pool"]), raw_bytes(c_ref["pool"])), "pools differ after the write"
        want, _ = oracle.run_workload(wl)
        say(f"[noalloc] {wl.name}: {assert_within(to_f64(out), want, 'bf16', wl.name)}")


def test_noalloc_rejects_a_step_past_its_scratch(pa):
    # 4096 chunk tokens x 32 heads x 128: the split-K partials alone need 64 MiB
    T, Hq, Hkv, D, NB = 4096, 32, 8, 128, 300
    need = pa.workspace_size(1, T, Hq, Hkv, D, NB)
    assert need > pa.NOALLOC_SCRATCH_BYTES
    q = torch.zeros((T, Hq, D), dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros((T, Hkv, D), dtype=torch.bfloat16, device="cuda")
    pool = pa.new_kv_pool(NB, Hkv, D)
    pool.view(torch.int16).fill_(0x1234)
    before = pool.clone()
    i32 = lambda x: torch.tensor(x, dtype=torch.int32, device="cuda")
    slots = torch.arange(T, dtype=torch.int64, device="cuda")
    with pytest.raises(pa.PAError) as e:
        pa.step_noalloc(q, kv, kv, pool[:, 0], pool[:, 1], slots, i32([list(range(NB))]), i32([0, T]), i32([T]),
                        i32([0]), 0.125)
    torch.cuda.synchronize()
    say(f"[noalloc] rejected: {e.value}")
    assert e.value.status == 6 and "pa_step_noalloc" in str(e.value)
    assert torch.equal(pool.view(torch.int16), before.view(torch.int16)), "a rejected step launched work"
