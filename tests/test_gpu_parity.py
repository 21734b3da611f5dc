"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Bounds: KV write bit-exact; fp32 max abs <= 1e-5; bf16 max abs <= 2e-2, mean
abs <= 1e-2 and per-row max|err| <= 3e-2 * rms (tests/parity.py). The six
model-shaped workloads run at full size in the launch configuration the
benchmark times, and the oracle checks every output row of each (in batches
of sequences, each a compact sub-workload, so the host pool stays a few GB).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import device_case, host_inputs, oracle_every_row, raw_bytes, run_step, to_f64
from parity import assert_summary, assert_within

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pa():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import pagedattention_block_paged_amd as lib

    return lib


def hbm_bytes():
    return torch.cuda.get_device_properties(0).total_memory


def say(*a):
    print(*a, flush=True)


def check_write(wl, c, pool_after, k, v):
    """Written rows equal k/v bit for bit."""
    sm = torch.from_numpy(wl.slot_mapping).cuda()
    keep = sm >= 0
    blk, row = (sm // 16)[keep], (sm % 16)[keep]
    assert torch.equal(pool_after[blk, 0, row].view(torch.int16 if wl.dtype == "bf16" else torch.int32),
                       k[keep].view(torch.int16 if wl.dtype == "bf16" else torch.int32))
    assert torch.equal(pool_after[blk, 1, row].view(torch.int16 if wl.dtype == "bf16" else torch.int32),
                       v[keep].view(torch.int16 if wl.dtype == "bf16" else torch.int32))


def row_checksums(pool, dtype, chunk=16384):
    """Per-(block, K|V, row) checksums of the raw bits, int64 [NB, 2, 16, 2]."""
    iv = torch.int16 if dtype == "bf16" else torch.int32
    outs = []
    for a in range(0, pool.shape[0], chunk):
        x = pool[a:a + chunk].view(iv).to(torch.int64)
        outs.append(torch.stack([x.sum(dim=(-1, -2)), (x * x).sum(dim=(-1, -2))], dim=-1))
    return torch.cat(outs)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5, 6, 9])
def test_config_parity(pa, cfg):
    wl = W.config_workload(cfg, hbm_bytes=hbm_bytes())
    say(f"[cfg {cfg}] {wl.name}: S={wl.num_seqs} T={wl.num_tokens} NB={wl.num_blocks}")
    c = device_case(wl)
    small = wl.num_blocks * wl.block_bytes <= (1 << 30)
    before = raw_bytes(c["pool"]) if small else None
    sums_before = None if small else row_checksums(c["pool"], wl.dtype)
    out = run_step(pa, wl, c)
    torch.cuda.synchronize()
    check_write(wl, c, c["pool"], c["k"], c["v"])
    # every row the write did not target is unchanged
    touched = np.zeros((wl.num_blocks, 16), bool)
    sm = wl.slot_mapping[wl.slot_mapping >= 0]
    touched[sm // 16, sm % 16] = True
    if small:
        after = raw_bytes(c["pool"]).reshape(wl.num_blocks, 2, 16, -1).transpose(0, 2, 1, 3)
        ref = before.reshape(wl.num_blocks, 2, 16, -1).transpose(0, 2, 1, 3)
        assert np.array_equal(after[~touched], ref[~touched])
    else:
        sums_after = row_checksums(c["pool"], wl.dtype)
        mask = torch.from_numpy(~touched).cuda()
        assert torch.equal(sums_after.permute(0, 2, 1, 3)[mask], sums_before.permute(0, 2, 1, 3)[mask])
    # attention: every output row against the oracle, in sequence batches
    del c["k"], c["v"], c["q"]
    say(f"[cfg {cfg}] oracle on all {wl.num_seqs} sequences ({wl.num_tokens} tokens)")
    e = oracle_every_row(wl, out, lambda sub, pool: oracle.run_workload(sub, pool=pool), say=say).summary()
    say(f"[cfg {cfg}] {e}")
    assert e["rows"] == wl.num_tokens * wl.num_q_heads
    assert_summary(e, wl.dtype, f"cfg {cfg}")


def test_single_key_output_is_its_value(pa):
    wl = W.config_workload(1)
    c = device_case(wl)
    out = run_step(pa, wl, c)
    s = list(wl.seq_lens).index(1)
    t = int(wl.query_start_loc[s])
    G = wl.num_q_heads // wl.num_kv_heads
    want = c["v"][t].repeat_interleave(G, dim=0)
    assert torch.equal(out[t], want)


def mixes():
    cases = []
    rs = np.random.default_rng(1234)
    shapes = [(4, 2, 64, "f32"), (8, 8, 64, "bf16"), (16, 1, 128, "bf16"), (12, 4, 128, "f32"),
              (32, 8, 128, "bf16"), (6, 2, 64, "bf16"), (4, 4, 128, "f32"), (64, 8, 128, "bf16"),
              (8, 4, 128, "bf16"), (2, 2, 128, "bf16"), (16, 2, 64, "bf16")]
    for i, (Hq, Hkv, D, dt) in enumerate(shapes):
        S = int(rs.integers(1, 7))
        ctx, ql = [], []
        for _ in range(S):
            if rs.random() < 0.5:
                ctx.append(int(rs.integers(0, 700)))
                ql.append(1)
            else:
                ctx.append(int(rs.integers(0, 300)))
                ql.append(int(rs.integers(2, 150)))
        cases.append(W.build_workload(f"mix{i}", dt, Hq, Hkv, D, ctx, ql, seed=500 + i))
    return cases


@pytest.mark.parametrize("idx", range(11))
def test_random_mixes(pa, idx):
    wl = mixes()[idx]
    say(f"[mix {idx}] {wl.dtype} Hq={wl.num_q_heads} Hkv={wl.num_kv_heads} D={wl.head_size} "
        f"ctx={wl.context_lens.tolist()} q={wl.query_lens.tolist()}")
    c = device_case(wl)
    out = run_step(pa, wl, c)
    ref, pool_ref = oracle.run_workload(wl)
    got_pool, want_pool = raw_bytes(c["pool"]), pool_ref.reshape(-1).view(np.uint8)
    assert got_pool.shape == want_pool.shape
    bad = np.count_nonzero(got_pool != want_pool)
    assert bad == 0, f"{bad} pool bytes differ after the KV write"
    e = assert_within(to_f64(out), ref, wl.dtype, f"mix {idx}")
    say(f"[mix {idx}] {e}")


def beside_cases():
    """Small bf16 batches with block tables wide enough (S x MB x 16 keys of K/V
    above 4 GB) and enough query tokens past one per sequence (a prefill share
    above 5% at the table's width) that the library runs the chunked prefill
    on its own stream beside the decode kernel: mixes for each head grouping,
    a batch with no decode and one with no prefill."""
    rs = np.random.default_rng(4321)
    cases = []
    for i, (Hq, Hkv) in enumerate([(32, 8), (16, 8), (8, 8), (64, 8)]):
        ctx = [int(x) for x in rs.integers(0, 3000, size=6)]
        ql = [1, 1, int(rs.integers(40, 300)), 1, int(rs.integers(2, 90)), 1]
        cases.append(W.build_workload(f"beside{i}", "bf16", Hq, Hkv, 128, ctx, ql, seed=900 + i, max_blocks=16384))
    cases.append(W.build_workload("beside_prefill_only", "bf16", 32, 8, 128, [0, 700, 1500, 64], [300, 77, 129, 40],
                                  seed=910, max_blocks=16384))
    # decodes and short queries that stay on the decode kernel's path,
    # with tokens enough for the library to take the two-stream path
    cases.append(W.build_workload("beside_decode_only", "bf16", 32, 8, 128, [5, 2500, 900, 0, 64, 300, 7, 1200],
                                  [1, 4, 4, 4, 4, 4, 4, 4], seed=911, max_blocks=16384))
    # one chunk after a long context next to decodes: its 8 items outlast an
    # equal share of the few CUs the prefill gets, so the schedule cuts them
    cases.append(W.build_workload("beside_long_chunk", "bf16", 32, 8, 128, [30000, 700, 5000, 12, 9000],
                                  [64, 1, 1, 1, 1], seed=912, max_blocks=16384))
    return cases


@pytest.mark.parametrize("idx", range(7))
def test_prefill_beside_decode(pa, idx):
    wl = beside_cases()[idx]
    say(f"[beside {idx}] Hq={wl.num_q_heads} Hkv={wl.num_kv_heads} ctx={wl.context_lens.tolist()} "
        f"q={wl.query_lens.tolist()} MB={wl.max_blocks}")
    c = device_case(wl)
    with pa.profile() as prof:
        out = run_step(pa, wl, c)
        torch.cuda.synchronize()
    # the two-stream path: the KV write and the plan are launches of their own
    assert "kv_write_plan" not in prof.kernels and "prefill_plan" in prof.kernels, prof.kernels
    ref, _ = oracle.run_workload(wl)
    e = assert_within(to_f64(out), ref, wl.dtype, f"beside {idx}")
    # the same batch again: deterministic, also across the two streams
    out2 = run_step(pa, wl, c)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))
    say(f"[beside {idx}] {e}")


def test_small_prefill_share_runs_after_the_decode(pa):
    """A block table as wide as the beside cases' but a prefill of under 5%
    of the decode's bound work (one 40-token chunk next to 300 decodes): the
    library runs the prefill after the decode on the caller's stream (the KV
    write and the plan in one launch), and the result matches the oracle."""
    rs = np.random.default_rng(4322)
    ctx = [int(x) for x in rs.integers(0, 3000, size=300)] + [500]
    ql = [1] * 300 + [40]
    wl = W.build_workload("after_decode", "bf16", 32, 8, 128, ctx, ql, seed=913, max_blocks=16384)
    bound = wl.num_seqs * wl.max_blocks * 16 * 2 * wl.num_kv_heads * wl.head_size * 2
    assert bound >= 4e9
    c = device_case(wl)
    with pa.profile() as prof:
        out = run_step(pa, wl, c)
        torch.cuda.synchronize()
    assert "kv_write_plan" in prof.kernels and "prefill_plan" not in prof.kernels, prof.kernels
    ref, _ = oracle.run_workload(wl)
    say(f"[after decode] {assert_within(to_f64(out), ref, wl.dtype, 'after decode')}")


def test_chunked_prefill_matches_whole_prefill(pa):
    """18 tokens as chunks of 8 + 8 + 2 through one pool equal one 18-token prefill."""
    whole = W.build_workload("whole", "bf16", 8, 2, 128, [0], [18], seed=77, num_blocks=8)
    c = device_case(whole)
    out_whole = run_step(pa, whole, c).clone()
    c2 = device_case(whole)  # fresh pool, nothing cached
    done, rows = 0, []
    for n in (8, 8, 2):
        qsl = torch.tensor([0, n], dtype=torch.int32, device="cuda")
        sl = torch.tensor([done + n], dtype=torch.int32, device="cuda")
        cl = torch.tensor([done], dtype=torch.int32, device="cuda")
        pool = c2["pool"]
        rows.append(pa.step(c2["q"][done:done + n].contiguous(), c2["k"][done:done + n].contiguous(),
                            c2["v"][done:done + n].contiguous(), pool[:, 0], pool[:, 1],
                            c2["slot_mapping"][done:done + n].contiguous(), c2["block_tables"], qsl, sl, cl,
                            whole.scale))
        done += n
    torch.cuda.synchronize()
    got = torch.cat(rows)
    ref, _ = oracle.run_workload(whole)
    assert_within(to_f64(got), ref, "bf16", "chunked")
    assert_within(to_f64(out_whole), ref, "bf16", "whole")


@pytest.mark.parametrize("Hq,Hkv,D", [(2, 2, 128), (4, 2, 128), (16, 4, 64), (16, 2, 128)])
def test_long_prompts_span_many_query_tiles(pa, Hq, Hkv, D):
    """Prompts of several hundred tokens (many query tiles per sequence, ragged
    last tile) next to decode rows, for each head-group width the prefill
    kernel instantiates (query heads per KV head 1, 2, 4 and 8)."""
    ctx, ql = [0, 300, 45, 700, 17], [600, 333, 1, 1, 257]
    wl = W.build_workload(f"long{Hq}x{Hkv}x{D}", "bf16", Hq, Hkv, D, ctx, ql, seed=900 + Hq + D)
    say(f"[long] Hq={Hq} Hkv={Hkv} D={D} ctx={ctx} q={ql}")
    c = device_case(wl)
    out = run_step(pa, wl, c)
    ref, _ = oracle.run_workload(wl)
    say(f"[long] {assert_within(to_f64(out), ref, 'bf16', 'long prompts')}")


def test_physical_permutation_is_bit_exact(pa):
    wl = W.config_workload(2)
    c = device_case(wl)
    out = run_step(pa, wl, c).clone()
    pi = np.random.default_rng(3).permutation(wl.num_blocks)
    wl_p = W.with_block_tables(wl, pi[wl.block_tables], wl.num_blocks, int(pi[wl.canary_block]))
    cp = device_case(wl_p)
    pool = W.pool_device(wl, "cuda")
    cp["pool"][torch.from_numpy(pi).cuda()] = pool
    out_p = run_step(pa, wl_p, cp)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out_p.view(torch.int16))


def test_shared_prefix_blocks_equal_private_copies_bit_exact(pa):
    wl = W.config_workload(5)
    c = device_case(wl)
    out = run_step(pa, wl, c).clone()
    n_sh = 128
    NB2 = wl.num_blocks + wl.num_seqs * n_sh
    tables = np.concatenate([wl.block_tables, np.zeros((wl.num_seqs, 0), np.int32)], axis=1).astype(np.int64)
    shared_ids = wl.block_tables[0, :n_sh].astype(np.int64)
    for s in range(wl.num_seqs):
        tables[s, :n_sh] = wl.num_blocks + s * n_sh + np.arange(n_sh)
    wl_p = W.with_block_tables(wl, tables, NB2, wl.canary_block)
    cp = device_case(wl_p)
    base = W.pool_device(wl, "cuda")
    cp["pool"][: wl.num_blocks] = base
    src = torch.from_numpy(shared_ids).cuda()
    for s in range(wl.num_seqs):
        cp["pool"][wl.num_blocks + s * n_sh: wl.num_blocks + (s + 1) * n_sh] = base[src]
    out_p = run_step(pa, wl_p, cp)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out_p.view(torch.int16))


def test_repeated_calls_are_deterministic(pa):
    wl = W.sub_workload(W.config_workload(3), [0, 1, 2, 4096, 4097])
    c = device_case(wl)
    ws = pa.new_workspace(c["q"], c["pool"][:, 0], c["block_tables"])
    a = run_step(pa, wl, c, workspace=ws).clone()
    b = run_step(pa, wl, c, workspace=ws).clone()
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


ORDER_CASES = [  # (dtype, Hq, Hkv, D, decodes, longest context, seed): more units than one round of workgroups
    ("bf16", 8, 2, 128, 400, 8000, 81),   # one head group per sequence, up to 2 partitions of 4096
    ("bf16", 16, 16, 64, 150, 10000, 82),  # two head groups (16 KV heads), up to 3 partitions of 4096
    ("f32", 8, 2, 64, 600, 8000, 83),
    ("bf16", 8, 2, 64, 9000, 1000, 84),  # more sequences than the order kernel keeps in registers (8,192)
]


@pytest.mark.timeout(300)
@pytest.mark.parametrize("idx", range(len(ORDER_CASES)))
def test_decode_work_order(pa, idx, monkeypatch):
    """A decode launch of more than one round of workgroups takes its
    (sequence, head group, partition) units longest first, from a work order
    that a one-workgroup kernel writes ahead of it. Every unit is computed as
    in grid order, so the output equals the grid-order launch's
    (PA_DECODE_ORDER=0) bit for bit; and the oracle's on every row. The batch
    mixes decodes of one to three partitions, short multi-token queries (also
    on the decode kernel) and a prefill chunk (not in the order)."""
    dtype, Hq, Hkv, D, S, Lmax, seed = ORDER_CASES[idx]
    rs = np.random.default_rng(seed)
    G = Hq // Hkv
    ctx = list(rs.integers(0, Lmax, size=S))
    ql = [1] * S
    nmax = 16 // G
    for i in range(0, S, 37):  # short multi-token queries
        ql[i] = int(rs.integers(1, nmax + 1))
    ctx.append(300)
    ql.append(nmax + 40)  # a chunk for the prefill kernel
    mb = -(-(Lmax + 64) // 16)
    wl = W.build_workload(f"order{idx}", dtype, Hq, Hkv, D, ctx, ql, seed=seed, max_blocks=mb)
    pt = pa.partition_tokens(wl.num_seqs, Hkv, D, dtype, wl.max_blocks)
    hw = next(h for h in (8, 4, 2, 1) if Hkv % h == 0)
    units = wl.num_seqs * (Hkv // hw) * (-(-wl.max_blocks * 16 // pt))
    say(f"[order {idx}] {dtype} Hq={Hq} Hkv={Hkv} D={D} S={wl.num_seqs} partition={pt} units={units}")
    assert units > 512, "the case must take the ordered launch"
    c = device_case(wl)
    ws = pa.new_workspace(c["q"], c["pool"][:, 0], c["block_tables"])
    with pa.profile() as prof:
        ordered = run_step(pa, wl, c, workspace=ws).clone()
        torch.cuda.synchronize()
    assert "decode_order" in prof.kernels, prof.kernels
    monkeypatch.setenv("PA_DECODE_ORDER", "0")
    with pa.profile() as prof:
        grid = run_step(pa, wl, c, workspace=ws).clone()
        torch.cuda.synchronize()
    assert "decode_order" not in prof.kernels, prof.kernels
    iv = torch.int16 if dtype == "bf16" else torch.int32
    assert torch.equal(ordered.view(iv), grid.view(iv))
    e = oracle_every_row(wl, ordered, lambda sub, hp: oracle.run_workload(sub, pool=hp), say=say).summary()
    say(f"[order {idx}] {e}")
    assert e["rows"] == wl.num_tokens * wl.num_q_heads
    assert_summary(e, dtype, wl.name)


def test_partition_size_counts_resident_workgroups(pa):
    """The partition size gives one round of decode workgroups: the bf16
    kernel at head size 128 fits one workgroup per CU, the 8-bit-pool kernel
    two (70B-batch extents: 32 sequences of up to 32768 tokens, 8 KV heads)."""
    assert pa.partition_tokens(32, 8, 128, "bf16", 2048) == 4096
    assert pa.partition_tokens(32, 8, 128, "bf16", 2048, kv_fp8=True) == 2048


@pytest.mark.parametrize("delta", [-1, 0, 1, 17])
def test_split_partition_boundaries(pa, delta):
    """Decode lengths around multiples of the partition size."""
    pt = pa.partition_tokens(4, 2, 128, "bf16", 256)
    L = [pt + delta, 2 * pt + delta, 3 * pt + delta, 1]
    L = [max(1, x) for x in L]
    wl = W.build_workload("split", "bf16", 16, 2, 128, np.array(L) - 1, [1, 1, 1, 1], seed=40 + delta,
                          max_blocks=256)
    c = device_case(wl)
    out = run_step(pa, wl, c)
    ref, _ = oracle.run_workload(wl)
    assert_within(to_f64(out), ref, "bf16", f"split {pt}+{delta}")


@pytest.mark.parametrize("Hq,Hkv,D,dtype", [(32, 8, 128, "bf16"), (64, 8, 128, "bf16"), (8, 8, 64, "bf16"),
                                              (16, 8, 64, "bf16"), (12, 4, 128, "f32")])
def test_short_queries_over_long_contexts(pa, Hq, Hkv, D, dtype):
    """Speculative-decode verification shapes: a few new tokens (every
    n with n x G <= 16 goes to the decode kernel, one column per (token,
    head)) after long cached contexts split into several partitions, next to
    plain decodes and one chunk long enough for the prefill kernel."""
    G = Hq // Hkv
    nmax = 16 // G
    ns = sorted({2, min(3, nmax), nmax, max(2, nmax // 2)})
    ns = [n for n in ns if n <= nmax and n >= 2] or [1]
    ctx = [4999, 2100, 64, 0] + [1500 + 700 * i for i in range(len(ns))] + [300]
    ql = [1, 1, 1, nmax] + ns + [nmax + 5]
    wl = W.build_workload(f"spec{Hq}x{Hkv}x{D}", dtype, Hq, Hkv, D, ctx, ql, seed=700 + Hq + D)
    say(f"[spec] {dtype} Hq={Hq} Hkv={Hkv} D={D} ctx={ctx} q={ql} partition={pa.partition_tokens(wl.num_seqs, Hkv, D, dtype, wl.max_blocks)}")
    c = device_case(wl)
    out = run_step(pa, wl, c)
    ref, _ = oracle.run_workload(wl)
    say(f"[spec] {assert_within(to_f64(out), ref, dtype, 'short queries')}")


def test_empty_batch_is_a_no_op(pa):
    q = torch.empty((0, 8, 64), dtype=torch.bfloat16, device="cuda")
    kv = torch.empty((0, 2, 64), dtype=torch.bfloat16, device="cuda")
    pool = pa.new_kv_pool(4, 2, 64)
    z = lambda n: torch.zeros(n, dtype=torch.int32, device="cuda")
    out = pa.step(q, kv, kv, pool[:, 0], pool[:, 1], torch.empty(0, dtype=torch.int64, device="cuda"),
                  torch.zeros((0, 1), dtype=torch.int32, device="cuda"), z(1), z(0), z(0), 0.125)
    torch.cuda.synchronize()
    assert out.shape == (0, 8, 64)


def test_sequence_without_queries_and_padding_slot(pa):
    """A sequence with no query rows is skipped; a padding token (slot -1) writes nothing."""
    wl = W.build_workload("gap", "bf16", 8, 2, 64, [40, 30, 20], [1, 1, 3], seed=9)
    c = device_case(wl)
    # give sequence 1 zero queries: drop its token from the batch, keep its row count
    keep = [0, 2, 3, 4]
    q = c["q"][keep].contiguous()
    k = c["k"][keep].contiguous()
    v = c["v"][keep].contiguous()
    sm = c["slot_mapping"][keep].clone()
    sm[0] = -1  # sequence 0's new token is padding: not written
    qsl = torch.tensor([0, 1, 1, 4], dtype=torch.int32, device="cuda")
    pool = c["pool"]
    before = pool.clone()
    out = pa.step(q, k, v, pool[:, 0], pool[:, 1], sm, c["block_tables"], qsl, c["seq_lens"], c["context_lens"],
                  wl.scale)
    torch.cuda.synchronize()
    s0 = int(wl.slot_mapping[0])
    assert torch.equal(pool[s0 // 16, :, s0 % 16].view(torch.int16), before[s0 // 16, :, s0 % 16].view(torch.int16))
    ref, _ = oracle.run_workload(W.sub_workload(wl, [2]))
    assert_within(to_f64(out[1:4]), ref, "bf16", "after gap")


@pytest.mark.timeout(300)
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_prefill_tiles_past_the_sorted_plan(pa, dtype):
    """More than 4096 prefill q-tiles (4200 short chunks, one tile each): the
    plan kernel leaves the tiles in sequence order and the prefill kernel finds
    each tile's sequence by binary search over the tile prefix sums instead
    of reading a ranked record. Every row is compared with the oracle."""
    rs = np.random.default_rng(4200)
    if dtype == "bf16":
        Hq, Hkv, D, n = 64, 8, 128, 3  # 3 tokens x 8 query heads > 16 columns: the prefill kernel
    else:
        Hq, Hkv, D, n = 1, 1, 64, 20  # 20 tokens x 1 query head > 16 columns: the prefill kernel
    S = 4200
    ctx = rs.integers(64, 300, size=S)  # enough keys per row that bf16 weights stay within the per-row bound
    wl = W.build_workload(f"tiles4200_{dtype}", dtype, Hq, Hkv, D, ctx, np.full(S, n), seed=4200 + (dtype == "f32"))
    G = Hq // Hkv
    assert n * G > 16 and S > 4096, "every sequence must take the prefill kernel, one tile or more each"
    say(f"[tiles] {dtype}: {S} chunks of {n} tokens, Hq={Hq} Hkv={Hkv} D={D}")
    c = device_case(wl)
    out = run_step(pa, wl, c)
    torch.cuda.synchronize()
    pool, _, _, _ = host_inputs(wl)
    ref, _ = oracle.run_workload(wl, pool=pool)
    say(f"[tiles] {assert_within(to_f64(out), ref, dtype, 'unsorted tiles')}")


def cut_cases():
    """Batches whose prefill items the static schedule cuts along their keys:
    a few long items on 256 workgroups (each item in many pieces), the same at
    head size 64, and one chunk next to 600 decodes, where the decode's
    partition size leaves two partial slots per row (one cut per item: the
    later range boundaries inside an item cut nothing)."""
    rs = np.random.default_rng(6060)
    return [
        W.build_workload("cut_many", "bf16", 32, 8, 128, [30000, 500], [128, 1], seed=6061),
        W.build_workload("cut_many_d64", "bf16", 16, 4, 64, [20000, 3, 9000], [200, 1, 70], seed=6062),
        W.build_workload("cut_two_slots", "bf16", 32, 8, 128, list(rs.integers(1, 100, size=600)) + [8000],
                         [1] * 600 + [64], seed=6063),
    ]


@pytest.mark.parametrize("idx", range(3))
def test_prefill_items_cut_along_keys(pa, idx):
    """Every row against the oracle, and bit-identical on a second call: the
    pieces of a cut item are combined in piece order whichever finishes last."""
    wl = cut_cases()[idx]
    G = wl.num_q_heads // wl.num_kv_heads
    pt = pa.partition_tokens(wl.num_seqs, wl.num_kv_heads, wl.head_size, "bf16", wl.max_blocks)
    slots = -(-wl.max_blocks * 16 // pt)
    say(f"[cut {idx}] {wl.name}: Hq={wl.num_q_heads} Hkv={wl.num_kv_heads} D={wl.head_size} S={wl.num_seqs} "
        f"partial slots per row {slots}")
    assert any(n * G > 16 for n in wl.query_lens), "the case needs prefill items"
    if idx == 2:
        assert slots == 2, "the case must leave two partial slots per row"
    c = device_case(wl)
    ws = pa.new_workspace(c["q"], c["pool"][:, 0], c["block_tables"])
    out = run_step(pa, wl, c, workspace=ws).clone()
    out2 = run_step(pa, wl, c, workspace=ws)
    torch.cuda.synchronize()
    ref, _ = oracle.run_workload(wl)
    say(f"[cut {idx}] {assert_within(to_f64(out), ref, 'bf16', wl.name)}")
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))
