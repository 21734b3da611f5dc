"""Host-side KV block manager (CPU).

1. The plain model (oracle/block_model.py) against what the pages state,
   case by case: allocate_slots arithmetic and its early exit, the free
   queue, reference counts of shared blocks, reuse of freed cached blocks,
   hash-chain divergence, cache salt, least-recently-freed recycling.
2. The library's C++ manager against the same statements, and against the
   model decision by decision over long random operation sequences (block
   size 4, as in the pages' prefix-caching demo, and 16).
3. Error paths of the C ABI.
"""
import numpy as np
import pytest

from oracle.block_model import BlockModel, NoBlocks

# A missing libpa.so is a failure here, not a skip: the import raises.
from pagedattention_block_paged_amd import kv_manager as kvm  # noqa: E402
KVCacheManager = kvm.KVCacheManager


class LibAdapter:
    """The library manager behind the model's method names."""

    def __init__(self, nb, bs, caching=True):
        self.m = KVCacheManager(nb, bs, caching)
        self.bs = bs

    def add_request(self, rid, prompt, salt=0):
        return self.m.add_request(rid, prompt, salt)

    def append_tokens(self, rid, toks):
        self.m.append_tokens(rid, toks)

    def allocate_slots(self, rid, n):
        if not self.m.allocate_slots(rid, n):
            raise NoBlocks(rid)

    def commit(self, rid, n):
        self.m.commit(rid, n)

    def free(self, rid):
        self.m.free(rid)

    def num_free(self):
        return self.m.num_free_blocks

    def request_blocks(self, rid):
        return self.m.request_blocks(rid)

    def is_cached(self, b):
        return self.m.is_cached(b)

    @property
    def ref(self):
        return [self.m.ref_count(b) for b in range(self.m.num_blocks)]

    def step_inputs(self, rids, n_new, max_blocks):
        out = self.m.build_step(rids, n_new, max_blocks)
        return {k: v.tolist() for k, v in out.items()}


IMPLS = {"model": BlockModel, "library": LibAdapter}


@pytest.fixture(params=sorted(IMPLS))
def make(request):
    return IMPLS[request.param]


def prefill(mgr, rid, prompt, salt=0):
    """Admit a request and compute its whole prompt in one step."""
    cached = mgr.add_request(rid, prompt, salt)
    mgr.allocate_slots(rid, len(prompt) - cached)
    mgr.commit(rid, len(prompt) - cached)
    return cached


def test_allocate_slots_ceil_arithmetic(make):
    # "Inside vLLM", Scheduler: 17 new tokens need ceil(17/16) = 2 blocks
    m = make(8, 16)
    m.add_request(1, list(range(17)))
    m.allocate_slots(1, 17)
    assert len(m.request_blocks(1)[0]) == 2 and m.num_free() == 6
    m2 = make(8, 16)
    m2.add_request(1, list(range(40)))
    m2.allocate_slots(1, 16)
    assert len(m2.request_blocks(1)[0]) == 1
    m2.commit(1, 16)
    m2.allocate_slots(1, 1)  # the 17th token opens a second block
    assert len(m2.request_blocks(1)[0]) == 2
    m2.commit(1, 1)
    m2.allocate_slots(1, 15)  # positions 17..31 still fit the second block
    assert len(m2.request_blocks(1)[0]) == 2


def test_allocation_takes_the_front_and_exits_early(make):
    # the first n blocks of the free queue; too few free blocks -> exit early, nothing changes
    m = make(5, 4)
    m.add_request(1, list(range(12)))
    m.allocate_slots(1, 12)
    assert m.request_blocks(1)[0] == [0, 1, 2]
    m.add_request(2, list(range(100, 112)))
    with pytest.raises(NoBlocks):
        m.allocate_slots(2, 12)
    assert m.num_free() == 2 and m.request_blocks(2)[0] == []
    m.allocate_slots(2, 8)
    assert m.request_blocks(2)[0] == [3, 4] and m.num_free() == 0


def test_finished_request_returns_its_blocks(make):
    m = make(6, 4, False)
    prefill(m, 1, list(range(10)))
    assert m.num_free() == 3
    m.free(1)
    assert m.num_free() == 6


def test_shared_prefix_refcount_two_while_alive(make):
    # a second request with the same prefix finds every full block; with the
    # first still alive their reference counts are 2 ("Inside vLLM", Prefix caching)
    m = make(16, 4)
    prompt = list(range(100, 110))  # 2 full blocks + 2 tokens
    assert prefill(m, 1, prompt) == 0
    a, _ = m.request_blocks(1)
    assert m.add_request(2, prompt) == 8
    b, computed = m.request_blocks(2)
    assert computed == 8 and b == a[:2]
    assert [m.ref[x] for x in a[:2]] == [2, 2] and m.ref[a[2]] == 1


def test_freed_cached_blocks_are_reclaimed(make):
    # the first request finished: its blocks are free (count 0) but still
    # cached; a request with the same prefix takes them out of the free queue
    m = make(16, 4)
    prompt = list(range(7, 20))  # 3 full blocks + 1
    prefill(m, 1, prompt)
    a, _ = m.request_blocks(1)
    m.free(1)
    assert m.num_free() == 16 and all(m.ref[x] == 0 for x in a) and all(m.is_cached(x) for x in a[:3])
    assert m.add_request(2, prompt + [99]) == 12
    b, _ = m.request_blocks(2)
    assert b == a[:3] and m.num_free() == 13 and [m.ref[x] for x in b] == [1, 1, 1]


def test_whole_prompt_hit_leaves_the_last_token(make):
    m = make(16, 4)
    prompt = list(range(8))  # exactly 2 blocks
    prefill(m, 1, prompt)
    assert m.add_request(2, prompt) == 4  # the last block is recomputed


def test_hash_chain_stops_at_divergence(make):
    # "Serving models at scale with vLLM", Prefix caching: once two prompts
    # differ, nothing after that point is shared, even where tokens match again
    m = make(32, 4)
    common, tail = [1, 2, 3, 4], [9, 9, 9, 9, 5]
    prefill(m, 1, common + [10, 11, 12, 13] + tail)
    assert m.add_request(2, common + [10, 11, 99, 13] + tail) == 4
    assert m.request_blocks(2)[0] == m.request_blocks(1)[0][:1]


def test_cache_salt_separates_requests(make):
    m = make(16, 4)
    prompt = list(range(9))
    prefill(m, 1, prompt, salt=7)
    assert m.add_request(2, prompt, 8) == 0
    assert m.add_request(3, prompt, 7) == 8


def test_least_recently_freed_recycled_first(make):
    # "Serving models at scale with vLLM", Prefix caching: unclaimed freed
    # blocks are recycled least recently used first
    m = make(4, 4)
    prefill(m, 1, list(range(8)))      # blocks 0, 1
    prefill(m, 2, list(range(50, 58)))  # blocks 2, 3
    m.free(2)  # queue: 3, 2
    m.free(1)  # queue: 3, 2, 1, 0
    m.add_request(3, list(range(200, 212)))
    m.allocate_slots(3, 12)
    assert m.request_blocks(3)[0] == [3, 2, 1]
    # recycling dropped the prefixes of blocks 3, 2, 1; block 0 keeps request 1's first block
    assert not any(m.is_cached(x) for x in (3, 2, 1)) and m.is_cached(0)
    assert m.add_request(4, list(range(50, 58)) + [0]) == 0
    assert m.add_request(5, list(range(8)) + [0]) == 4


def test_logical_to_physical_shared_block(make):
    # "LLM Serving Frameworks #1", KVCacheManager: req A's and req B's block 0
    # are the same physical block; their block 1 are not
    m = make(64, 16)
    sys_prompt = list(range(1000, 1016))
    prefill(m, 1, sys_prompt + list(range(5)))
    m.add_request(2, sys_prompt + list(range(20, 30)))
    m.allocate_slots(2, 10)
    a, b = m.request_blocks(1)[0], m.request_blocks(2)[0]
    assert a[0] == b[0] and a[1] != b[1]


def test_step_inputs_follow_the_block_tables(make):
    m = make(32, 16)
    prefill(m, 1, list(range(40)))
    m.append_tokens(1, [7])
    m.allocate_slots(1, 1)
    m.add_request(2, list(range(300, 340)))
    m.allocate_slots(2, 24)
    st = m.step_inputs([1, 2], [1, 24], 4)
    assert st["query_start_loc"] == [0, 1, 25]
    assert st["seq_lens"] == [41, 24] and st["context_lens"] == [40, 0]
    for i, rid in enumerate([1, 2]):
        blocks, _ = m.request_blocks(rid)
        assert st["block_tables"][i][:len(blocks)] == blocks
    slots = st["slot_mapping"]
    b1 = st["block_tables"][0]
    assert slots[0] == b1[40 // 16] * 16 + 40 % 16
    b2 = st["block_tables"][1]
    assert slots[1:] == [b2[p // 16] * 16 + p % 16 for p in range(24)]


def run_random_ops(mgr, seed, nb, bs, n_ops=1500):
    """Drive a manager with a seeded random workload (admissions with shared
    prefixes, chunked prefills, decodes with sampled tokens, frees); returns
    the trace of every observable decision."""
    rs = np.random.default_rng(seed)
    prefixes = [list(rs.integers(0, 50, 3 * bs)) for _ in range(4)]
    live, trace, next_id = {}, [], 0
    for _ in range(n_ops):
        op = rs.random()
        if op < 0.25 or not live:
            pre = prefixes[rs.integers(4)][: rs.integers(0, 3 * bs + 1)]
            prompt = [int(x) for x in pre] + [int(x) for x in rs.integers(0, 50, rs.integers(1, 3 * bs))]
            salt = int(rs.integers(0, 2))
            c = mgr.add_request(next_id, prompt, salt)
            live[next_id] = True
            trace.append(("add", next_id, c, mgr.request_blocks(next_id)))
            next_id += 1
        elif op < 0.85:
            rids = sorted(live)
            sched = [r for r in rids if rs.random() < 0.5] or rids[:1]
            n_new = []
            for r in sched:
                left = trace_tokens_left(mgr, r)
                if left == 0:
                    tok = int(rs.integers(0, 50))
                    mgr.append_tokens(r, [tok])
                    left = 1
                n_new.append(int(rs.integers(1, left + 1)))
            ok = []
            for r, n in zip(sched, n_new):
                try:
                    mgr.allocate_slots(r, n)
                    ok.append((r, n))
                except NoBlocks:
                    trace.append(("noblocks", r, n, mgr.num_free()))
            if ok:
                st = mgr.step_inputs([r for r, _ in ok], [n for _, n in ok], 64)
                trace.append(("step", st))
                for r, n in ok:
                    mgr.commit(r, n)
        else:
            r = sorted(live)[rs.integers(len(live))]
            mgr.free(r)
            del live[r]
            trace.append(("free", r, mgr.num_free()))
        trace.append(("state", mgr.num_free(), tuple(mgr.ref), tuple(mgr.is_cached(b) for b in range(nb))))
    return trace


def trace_tokens_left(mgr, r):
    """Tokens the request holds that are not computed yet (both sides track
    tokens the same way: the driver appends the same sampled ids)."""
    if isinstance(mgr, BlockModel):
        req = mgr.reqs[r]
        return len(req["tokens"]) - req["computed"]
    return mgr.tokens_left(r)


class TrackedLib(LibAdapter):
    """Library adapter that also counts each request's tokens on the host
    side, so the driver can ask how many are left to compute."""

    def __init__(self, nb, bs):
        super().__init__(nb, bs)
        self.ntok = {}

    def add_request(self, rid, prompt, salt=0):
        self.ntok[rid] = len(prompt)
        return super().add_request(rid, prompt, salt)

    def append_tokens(self, rid, toks):
        self.ntok[rid] += len(toks)
        super().append_tokens(rid, toks)

    def tokens_left(self, rid):
        return self.ntok[rid] - self.m.request_blocks(rid)[1]


@pytest.mark.parametrize("bs,nb,seed", [(4, 24, 0), (4, 40, 1), (16, 12, 2), (16, 30, 3)])
def test_library_matches_model_decision_by_decision(bs, nb, seed):
    t_model = run_random_ops(BlockModel(nb, bs), seed, nb, bs)
    t_lib = run_random_ops(TrackedLib(nb, bs), seed, nb, bs)
    assert len(t_model) == len(t_lib)
    kinds = {}
    for a, b in zip(t_model, t_lib):
        kinds[a[0]] = kinds.get(a[0], 0) + 1
        assert a == b, (a, b)
    # the sequences exercised every kind of decision, hits and early exits included
    assert kinds.get("noblocks", 0) > 0 and kinds.get("step", 0) > 100
    assert any(k[0] == "add" and k[2] > 0 for k in t_model)


def test_abi_errors():
    m = KVCacheManager(4, 16)
    m.add_request(1, [1, 2, 3])
    with pytest.raises(kvm.PAError, match="PA_ERR_REQUEST"):
        m.add_request(1, [4])
    with pytest.raises(kvm.PAError, match="PA_ERR_REQUEST"):
        m.add_request(2, [])
    with pytest.raises(kvm.PAError, match="PA_ERR_REQUEST"):
        m.allocate_slots(1, 4)  # holds 3 tokens
    with pytest.raises(kvm.PAError, match="PA_ERR_REQUEST"):
        m.commit(1, 1)  # no slots yet
    with pytest.raises(kvm.PAError, match="PA_ERR_REQUEST"):
        m.free(9)
    assert m.allocate_slots(1, 3)
    with pytest.raises(kvm.PAError, match="PA_ERR_SHAPE"):
        m.build_step([1], [3], 0)  # table too narrow
    with pytest.raises(kvm.PAError, match="PA_ERR_REQUEST"):
        m.build_step([1, 1], [1, 1], 4)  # listed twice
    with pytest.raises(kvm.PAError, match="PA_ERR_SHAPE"):
        KVCacheManager(0, 16)
    assert m.ref_count(-1) == -1 and m.ref_count(4) == -1
