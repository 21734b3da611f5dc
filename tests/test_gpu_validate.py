"""PA_VALIDATE=1: the opt-in host check of the step's device metadata.

- On valid input the checked call gives the same output, bit for bit, as the
  unchecked one.
- Each invalid case is rejected with PA_ERR_CONTENTS before anything is
  launched (the pool is unchanged after a rejected step): a length that is not
  context + new tokens, block ids outside the pool, a slot past the pool and
  two tokens writing one slot. Every case here is also one the kernels
  tolerate without the check (ids clamped, such slots skipped, a shorter
  length), so no case can fault the GPU whatever the check does.
"""
import numpy as np
import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu

PA_ERR_CONTENTS = 10


@pytest.fixture(scope="module")
def pa():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import pagedattention_block_paged_amd as lib

    return lib


@pytest.fixture(scope="module")
def wl():
    # decodes only: two KV heads, four query heads each, head size 64
    return W.build_workload("validate", "bf16", 8, 2, 64, [40, 17, 100, 1], [1, 1, 1, 1], seed=11)


def run_step(pa, wl, bt=None, sl=None, slots=None):
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    q = W.q_device(wl, "cuda")
    k, v = W.new_kv_device(wl, "cuda")
    pool = W.pool_device(wl, "cuda")
    before = pool.clone()
    args = (q, k, v, pool[:, 0], pool[:, 1], t(wl.slot_mapping if slots is None else slots),
            t(wl.block_tables if bt is None else bt), t(wl.query_start_loc), t(wl.seq_lens if sl is None else sl),
            t(wl.context_lens))
    try:
        out = pa.step(*args, wl.scale)
        torch.cuda.synchronize()
        return out, None
    except pa.PAError as e:
        torch.cuda.synchronize()
        assert torch.equal(pool.view(torch.int16), before.view(torch.int16)), "a rejected step changed the pool"
        return None, e


def test_valid_input_is_unchanged(pa, wl, monkeypatch):
    print("[validate] valid input", flush=True)
    ref, err = run_step(pa, wl)
    assert err is None
    monkeypatch.setenv("PA_VALIDATE", "1")
    got, err = run_step(pa, wl)
    assert err is None
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))


def bad_cases(wl):
    sl = wl.seq_lens.copy()
    sl[1] -= 1
    bt_past = wl.block_tables.copy()
    bt_past[0, 0] = wl.num_blocks + 5
    bt_neg = wl.block_tables.copy()
    bt_neg[2, 6] = -1  # sequence 2 holds 101 tokens: 7 blocks, so entry 6 is read
    slot_past = wl.slot_mapping.copy()
    slot_past[3] = wl.num_blocks * 16
    slot_dup = wl.slot_mapping.copy()
    slot_dup[1] = slot_dup[0]
    return {
        "seq_len != context + new": dict(sl=sl),
        "block id past the pool": dict(bt=bt_past),
        "negative block id": dict(bt=bt_neg),
        "slot past the pool": dict(slots=slot_past),
        "two tokens, one slot": dict(slots=slot_dup),
    }


@pytest.mark.parametrize("case", ["seq_len != context + new", "block id past the pool", "negative block id",
                                  "slot past the pool", "two tokens, one slot"])
def test_invalid_metadata_is_rejected(pa, wl, case, monkeypatch):
    print(f"[validate] {case}", flush=True)
    monkeypatch.setenv("PA_VALIDATE", "1")
    _, err = run_step(pa, wl, **bad_cases(wl)[case])
    assert err is not None and err.status == PA_ERR_CONTENTS, err


def test_unchecked_without_the_variable(pa, wl, monkeypatch):
    """Without PA_VALIDATE the same bad slot passes (and is skipped by the kernel)."""
    print("[validate] unchecked", flush=True)
    monkeypatch.delenv("PA_VALIDATE", raising=False)
    _, err = run_step(pa, wl, slots=bad_cases(wl)["slot past the pool"]["slots"])
    assert err is None


def test_zero_query_sequence_and_padding_rows_pass(pa, wl, monkeypatch):
    """A sequence with no new token (seq_len = context_len) and padding rows
    past query_start_loc[S] (slot -1) are valid: the checked call accepts them
    and gives the unchecked call's output bit for bit; padding rows of out and
    the pool are untouched."""
    print("[validate] zero-query sequence + padding rows", flush=True)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    keep = [0, 2, 3]  # sequence 1 contributes no row
    pad = 2
    q = W.q_device(wl, "cuda")
    k, v = W.new_kv_device(wl, "cuda")
    q = torch.cat([q[keep], q[:pad]]).contiguous()
    k = torch.cat([k[keep], k[:pad]]).contiguous()
    v = torch.cat([v[keep], v[:pad]]).contiguous()
    slots = np.concatenate([wl.slot_mapping[keep], np.full(pad, -1, np.int64)])
    qsl = np.array([0, 1, 1, 2, 3], np.int32)
    sl = wl.seq_lens.copy()
    sl[1] = wl.context_lens[1]
    outs = []
    for checked in (False, True):
        if checked:
            monkeypatch.setenv("PA_VALIDATE", "1")
        else:
            monkeypatch.delenv("PA_VALIDATE", raising=False)
        pool = W.pool_device(wl, "cuda")
        before = pool.clone()
        out = torch.full_like(q, 7.0)
        pa.step(q, k, v, pool[:, 0], pool[:, 1], t(slots), t(wl.block_tables), t(qsl), t(sl), t(wl.context_lens),
                wl.scale, out=out)
        torch.cuda.synchronize()
        s1 = int(wl.slot_mapping[1])  # sequence 1's would-be slot stays unwritten
        assert torch.equal(pool[s1 // 16, :, s1 % 16].view(torch.int16), before[s1 // 16, :, s1 % 16].view(torch.int16))
        assert bool((out[3:] == 7.0).all()), "padding rows of out were written"
        outs.append(out)
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))


def test_decreasing_query_start_loc_is_rejected(pa, wl, monkeypatch):
    """query_start_loc must not decrease (the kernels treat such a sequence as empty)."""
    print("[validate] decreasing query_start_loc", flush=True)
    monkeypatch.setenv("PA_VALIDATE", "1")
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    q = W.q_device(wl, "cuda")
    k, v = W.new_kv_device(wl, "cuda")
    pool = W.pool_device(wl, "cuda")
    qsl = np.array([0, 1, 0, 3, 4], np.int32)
    with pytest.raises(pa.PAError) as e:
        pa.step(q, k, v, pool[:, 0], pool[:, 1], t(wl.slot_mapping), t(wl.block_tables), t(qsl), t(wl.seq_lens),
                t(wl.context_lens), wl.scale)
    torch.cuda.synchronize()
    assert e.value.status == PA_ERR_CONTENTS and "decreases" in str(e.value)
