"""The seeded input generator: known answers, determinism, host/device twins, shapes."""
import json
import os

import numpy as np
import pytest

import workloads as W
from workloads import rng as R

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_splitmix64_published_outputs():
    with open(os.path.join(GOLD, "splitmix64_seed0.json")) as f:
        g = json.load(f)
    assert int(g["gamma"], 16) == R.GAMMA
    want = [int(x, 16) for x in g["outputs"]]
    got_int = [R.mix64_int((i + 1) * R.GAMMA) for i in range(3)]
    got_np = R.mix64_np(R._mul64(np.arange(1, 4, dtype=np.uint64), np.uint64(R.GAMMA))).tolist()
    assert got_int == want and got_np == want


def test_splitmix64_torch_twin_matches_numpy():
    torch = pytest.importorskip("torch")
    z = np.random.default_rng(0).integers(0, 2**63, size=4096, dtype=np.int64).astype(np.uint64) * np.uint64(3)
    got = R.mix64_torch(torch.from_numpy(z.view(np.int64))).numpy().view(np.uint64)
    assert np.array_equal(got, R.mix64_np(z))


def test_normal_table_is_a_discretised_standard_normal():
    t = R.NORMAL_F32.astype(np.float64)
    assert np.all(np.diff(t) > 0)
    assert np.array_equal(t, -t[::-1])  # symmetric, so the mean is exactly 0
    assert abs(t.mean()) < 1e-12 and abs(t.var() - 1) < 2e-3
    b = R.bf16_bits_to_f32(R.NORMAL_BF16).astype(np.float64)
    assert np.abs(b - t).max() <= np.abs(t).max() * 2.0**-8


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2**-8, 1.0 + 3 * 2**-8, 1.0 + 2**-9, -2.5, 3.0e-5], np.float32)
    bits = R.f32_to_bf16_bits(x)
    y = R.bf16_bits_to_f32(bits)
    assert y[0] == 1.0 and y[1] == 1.0 and y[2] == 1.0 + 2**-6 and y[3] == 1.0 and y[4] == -2.5
    torch = pytest.importorskip("torch")
    tb = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(tb, bits)


@pytest.mark.parametrize("cfg", [1, 2])
def test_host_and_device_generators_agree(cfg):
    torch = pytest.importorskip("torch")
    wl = W.config_workload(cfg)

    def host(x):
        return x.numpy() if wl.dtype == "f32" else x.view(torch.int16).numpy().view(np.uint16)

    assert np.array_equal(W.q_host(wl), host(W.q_device(wl, "cpu")))
    kh, vh = W.new_kv_host(wl)
    kd, vd = W.new_kv_device(wl, "cpu")
    assert np.array_equal(kh, host(kd)) and np.array_equal(vh, host(vd))
    ph = W.pool_host(wl)
    pd = W.pool_device(wl, "cpu", blocks_per_chunk=1000)
    assert ph.tobytes() == host(pd).tobytes()


def test_shared_pool_device_matches_host():
    torch = pytest.importorskip("torch")
    wl = W.sub_workload(W.config_workload(5), [0, 7])
    ph = W.pool_host(wl)
    pd = W.pool_device(wl, "cpu")
    assert ph.tobytes() == pd.view(torch.int16).numpy().tobytes()


def test_generation_is_deterministic():
    a, b = W.config_workload(2), W.config_workload(2)
    for f in ("seq_lens", "context_lens", "query_start_loc", "block_tables", "slot_mapping"):
        assert np.array_equal(getattr(a, f), getattr(b, f))
    assert np.array_equal(W.q_host(a), W.q_host(b))


def check_structure(wl):
    S, T = wl.num_seqs, wl.num_tokens
    assert wl.query_start_loc[0] == 0 and wl.query_start_loc[-1] == T
    assert np.all(wl.seq_lens == wl.context_lens + wl.query_lens)
    assert wl.block_tables.shape == (S, wl.max_blocks)
    ref = wl.referenced_blocks()
    assert wl.canary_block not in set(ref.tolist())
    owners = {}
    for s in range(S):
        used = wl.blocks_used(s)
        assert np.all(wl.block_tables[s, used:] == wl.canary_block)
        sh = int(wl.shared_len[s]) // 16
        for b in wl.block_tables[s, sh:used].tolist():
            assert b not in owners, "private blocks are never shared"
            owners[b] = s
    # every new token lands in its own sequence's block, at its position
    seq_of_tok = np.repeat(np.arange(S), wl.query_lens)
    pos = wl.context_lens[seq_of_tok] + (np.arange(T) - wl.query_start_loc[seq_of_tok])
    blk, row = wl.slot_mapping // 16, wl.slot_mapping % 16
    assert np.all(blk == wl.block_tables[seq_of_tok, pos // 16]) and np.all(row == pos % 16)
    assert len(set(wl.slot_mapping.tolist())) == T
    assert np.all(pos >= wl.shared_len[seq_of_tok]), "no new token lands in a shared block"


def test_config_shapes():
    c1 = W.config_workload(1)
    assert (c1.dtype, c1.num_q_heads, c1.num_kv_heads, c1.head_size, c1.num_blocks) == ("f32", 4, 2, 64, 64)
    assert c1.seq_lens.tolist() == [1, 17, 50, 100] and c1.num_tokens == 4
    c2 = W.config_workload(2)
    assert (c2.num_seqs, c2.num_q_heads, c2.num_kv_heads, c2.head_size, c2.num_blocks) == (64, 32, 4, 64, 16384)
    assert c2.seq_lens.min() >= 128 and c2.seq_lens.max() <= 2048 and c2.max_blocks == 128
    c3 = W.config_workload(3)
    assert c3.num_tokens == 8192 and c3.num_seqs == 4104 and (c3.num_q_heads, c3.num_kv_heads, c3.head_size) == (32, 8, 128)
    assert np.all(c3.query_lens[:4096] == 1) and np.all(c3.query_lens[4096:] == 512)
    assert c3.seq_lens[:4096].min() >= 256 and c3.seq_lens[:4096].max() <= 8192
    assert c3.context_lens[4096:].max() <= 4096
    c4 = W.config_workload(4, hbm_bytes=288 * 2**30)
    assert np.all(c4.seq_lens == 32768) and c4.num_blocks == int(0.6 * 288 * 2**30) // 65536
    assert (c4.num_q_heads, c4.num_kv_heads, c4.head_size) == (64, 8, 128)
    c5 = W.config_workload(5)
    assert c5.num_seqs == 256 and np.all(c5.shared_len == 2048) and c5.max_blocks == 161
    assert np.all(c5.block_tables[:, :128] == c5.block_tables[0, :128])
    assert c5.seq_lens.min() >= 2049 and c5.seq_lens.max() <= 2048 + 513
    for wl in (c1, c2, c3, c5):
        check_structure(wl)
    check_structure(W.sub_workload(c4, [0, 5]))
