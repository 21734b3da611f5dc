"""A whole step (KV write, decode, split-K reduce, prefill planning and
prefill) captured once in a HIP graph and replayed, also when the library
runs the prefill on a second stream forked from and joined back into the
captured one.

The library makes no allocation, synchronisation or memset on the launch
stream, so `pa_step` can be captured as is. Each replay must equal the eager
step bit for bit (the kernels are deterministic), also after the inputs were
changed in place between replays, with ordinary eager work and host
synchronisations in between. The eager results themselves are checked
against the oracle by the parity tests; here the oracle checks one replay.
"""
import pytest
import torch

import oracle
import workloads as W
from gpu_util import device_case, run_step, to_f64
from parity import assert_within

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pa():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import pagedattention_block_paged_amd as lib

    return lib


def say(*a):
    print(*a, flush=True)


def cases():
    return [
        ("tinyllama decode", W.config_workload(2)),
        ("mixed", W.build_workload("graph_mix", "bf16", 32, 8, 128, [300, 17, 0, 900, 45], [1, 1, 96, 1, 40],
                                   seed=4242)),
        ("f32 mixed", W.build_workload("graph_f32", "f32", 12, 4, 128, [200, 0, 33], [1, 70, 1], seed=4343)),
        # a block table wide enough that the prefill runs on the library's own
        # stream beside the decode: the fork and join are captured too
        ("mixed, prefill beside decode", W.build_workload("graph_beside", "bf16", 32, 8, 128,
                                                          [300, 17, 0, 900, 45, 2000], [1, 1, 96, 1, 40, 1],
                                                          seed=4444, max_blocks=16384)),
    ]


@pytest.mark.parametrize("idx", range(4))
def test_graph_replay_equals_eager(pa, idx):
    name, wl = cases()[idx]
    say(f"[graph] {name}: S={wl.num_seqs} T={wl.num_tokens} {wl.dtype} Hq={wl.num_q_heads} Hkv={wl.num_kv_heads}")
    c = device_case(wl)
    pool = c["pool"]
    ws = pa.new_workspace(c["q"], pool[:, 0], c["block_tables"])
    out = torch.empty_like(c["q"])
    run_step(pa, wl, c, out=out, workspace=ws)  # eager warm-up (one-time kernel attributes)
    torch.cuda.synchronize()
    want = out.clone()
    ref, _ = oracle.run_workload(wl)
    assert_within(to_f64(want), ref, wl.dtype, f"{name} eager")

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        run_step(pa, wl, c, out=out, workspace=ws)
    torch.cuda.synchronize()

    side = torch.randn(1 << 20, device="cuda")
    for rep in range(3):
        out.fill_(0)
        side.mul_(1.0001)  # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16) if out.dtype == torch.bfloat16 else out.view(torch.int32),
                           want.view(torch.int16) if want.dtype == torch.bfloat16 else want.view(torch.int32)), \
            f"{name}: replay {rep} differs from the eager step"

    # New query values in place: the replay must read the buffers' current contents.
    q2 = torch.flip(c["q"], dims=[0]).contiguous()
    c["q"].copy_(q2)
    g.replay()
    torch.cuda.synchronize()
    got = out.clone()
    out2 = torch.empty_like(out)
    run_step(pa, wl, c, out=out2, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16) if got.dtype == torch.bfloat16 else got.view(torch.int32),
                       out2.view(torch.int16) if out2.dtype == torch.bfloat16 else out2.view(torch.int32)), \
        f"{name}: replay after an input change differs from the eager step"
    say(f"[graph] {name}: 3 replays + 1 after an input change equal the eager step")
    del g
