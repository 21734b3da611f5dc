"""Several engine steps end to end: the library's KV block manager decides
where every token goes, pa_step writes and attends, and each step's output is
checked against the oracle's dense attention over K/V regenerated from the
token streams (never read back through the pool).

The driver follows the pages' step ("Inside vLLM: Anatomy of a
High-Throughput LLM Inference System", sections "Scheduler" and "Run forward
pass"): decodes first, then prefill chunks of waiting prompts within a token
budget; allocate_slots before the step, commit after it; a request that has
produced its tokens is freed. Prompts share a system prompt, one repeats
another's prompt, one differs only by its cache salt, and one arrives after
the request it shares with has finished ("Inside vLLM", section "Prefix
caching"; "Serving models at scale with vLLM", section "Prefix caching"). The
same requests run with prefix caching on and off: both must match the oracle,
and the cached run must reuse blocks as the pages describe.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from oracle.dense import dense_attention
from parity import assert_within

pytestmark = pytest.mark.gpu

STREAM_Q, STREAM_K, STREAM_V = 11, 12, 13
SEED = 0x57E9


@pytest.fixture(scope="module")
def pa():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import pagedattention_block_paged_amd as lib

    return lib


def say(msg):
    print(msg, flush=True)


def requests():
    rs = np.random.default_rng(3)
    toks = lambda n: [int(x) for x in rs.integers(0, 1000, n)]
    sys_prompt = toks(40)
    r0 = sys_prompt + toks(30)
    return [  # (id, prompt, tokens to generate, cache salt, arrival step)
        (0, r0, 5, 0, 0),
        (1, sys_prompt + toks(50), 4, 0, 2),
        (2, list(r0), 3, 0, 4),
        (3, sys_prompt + toks(10), 3, 1, 1),
        (4, toks(100), 2, 0, 0),
        (5, sys_prompt + toks(20), 3, 0, 9),
    ]


class Driver:
    def __init__(self, pa, caching, dtype, Hq, Hkv, D, num_blocks=96, budget=48, fp8_scales=None):
        from pagedattention_block_paged_amd.kv_manager import KVCacheManager

        self.pa, self.dtype, self.Hq, self.Hkv, self.D, self.budget = pa, dtype, Hq, Hkv, D, budget
        self.fp8 = fp8_scales  # (k_scale, v_scale) for an 8-bit pool, else None
        self.mgr = KVCacheManager(num_blocks, 16, caching)
        pool_dtype = "fp8" if self.fp8 else dtype
        if self.fp8:
            self.pool = torch.empty((num_blocks, 2, 16, Hkv, D), dtype=torch.uint8, device="cuda")
            W.fill_canary(self.pool, "fp8")
            self.pool = self.pool.view(torch.float8_e4m3fn)
        else:
            self.pool = torch.empty((num_blocks, 2, 16, Hkv, D), dtype=W.torch_dtype(dtype), device="cuda")
            W.fill_canary(self.pool, pool_dtype)
        self.scale = float(np.float32(1.0 / np.sqrt(D)))
        self.state = {}
        self.cached = {}
        self.max_blocks = 16

    def rows(self, stream, tokens, positions, heads):
        idents = W.prefix_idents(tokens)[positions]
        return W.token_rows(SEED, stream, idents, positions, heads, self.D, self.dtype)

    def to_dev(self, host):
        t = torch.from_numpy(np.ascontiguousarray(host))
        if self.dtype == "bf16":
            return t.view(torch.int16).cuda().view(torch.bfloat16)
        return t.cuda()

    def run(self, reqs, max_steps=40):
        pending = sorted(reqs, key=lambda r: r[4])
        checked = 0
        for step in range(max_steps):
            for r in [r for r in pending if r[4] <= step]:
                rid, prompt, gen, salt, _ = r
                self.cached[rid] = self.mgr.add_request(rid, prompt, salt)
                self.state[rid] = {"tokens": list(prompt), "computed": self.cached[rid], "gen": gen, "made": 0}
                pending.remove(r)
            if not self.state and not pending:
                return checked
            # decodes first, then prompt chunks in arrival order, within the budget
            sched, left = [], self.budget
            for rid, st in self.state.items():
                if len(st["tokens"]) - st["computed"] == 1 and st["made"] > 0 and left > 0:
                    sched.append((rid, 1))
                    left -= 1
            for rid, st in self.state.items():
                rem = len(st["tokens"]) - st["computed"]
                if st["made"] == 0 and rem > 0 and left > 0:
                    n = min(rem, left)
                    sched.append((rid, n))
                    left -= n
            sched = [(rid, n) for rid, n in sched if self.mgr.allocate_slots(rid, n)]
            if not sched:
                continue
            checked += self.one_step(step, sched)
            for rid, n in sched:
                self.mgr.commit(rid, n)
                st = self.state[rid]
                st["computed"] += n
                if st["computed"] == len(st["tokens"]):  # the step sampled a token
                    if st["made"] < st["gen"]:
                        tok = (31 * st["tokens"][-1] + 7 * rid + len(st["tokens"])) % 1000
                        st["tokens"].append(tok)
                        self.mgr.append_tokens(rid, [tok])
                        st["made"] += 1
                    else:
                        self.mgr.free(rid)
                        del self.state[rid]
        raise AssertionError("requests did not finish")

    def one_step(self, step, sched):
        ids = [rid for rid, _ in sched]
        nn = [n for _, n in sched]
        meta = self.mgr.build_step(ids, nn, self.max_blocks)
        q, k, v, refs = [], [], [], []
        for rid, n in sched:
            st = self.state[rid]
            C, toks = st["computed"], st["tokens"]
            new = np.arange(C, C + n)
            q.append(self.rows(STREAM_Q, toks, new, self.Hq))
            k.append(self.rows(STREAM_K, toks, new, self.Hkv))
            v.append(self.rows(STREAM_V, toks, new, self.Hkv))
            allp = np.arange(C + n)
            kr, vr = self.rows(STREAM_K, toks, allp, self.Hkv), self.rows(STREAM_V, toks, allp, self.Hkv)
            if self.fp8:  # what an 8-bit pool holds: the oracle's codes, read back times the scale
                ks, vs = self.fp8
                kk = oracle.fp8_decode(oracle.fp8_quantize(kr, self.dtype, ks)) * np.float64(np.float32(ks))
                vv = oracle.fp8_decode(oracle.fp8_quantize(vr, self.dtype, vs)) * np.float64(np.float32(vs))
            else:
                kk, vv = W.to_f64(kr, self.dtype), W.to_f64(vr, self.dtype)
            refs.append(dense_attention(W.to_f64(q[-1], self.dtype), kk, vv, C, self.scale))
        t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
        say(f"[multistep] step {step}: {list(zip(ids, nn))} seq_lens {meta['seq_lens'].tolist()}")
        args = (self.to_dev(np.concatenate(q)), self.to_dev(np.concatenate(k)), self.to_dev(np.concatenate(v)),
                self.pool[:, 0], self.pool[:, 1], t(meta["slot_mapping"]), t(meta["block_tables"]),
                t(meta["query_start_loc"]), t(meta["seq_lens"]), t(meta["context_lens"]))
        if self.fp8:
            out = self.pa.step_fp8(*args, self.scale, *self.fp8)
        else:
            out = self.pa.step(*args, self.scale)
        torch.cuda.synchronize()
        got = out.float().cpu().numpy().astype(np.float64)
        assert_within(got, np.concatenate(refs), self.dtype, f"step {step}")
        return len(ids)


@pytest.mark.parametrize("dtype,Hq,Hkv,D", [("bf16", 8, 2, 128), ("f32", 4, 2, 64), ("bf16", 32, 8, 128)])
def test_multistep_with_and_without_prefix_caching(pa, dtype, Hq, Hkv, D):
    say(f"[multistep] dtype {dtype} Hq {Hq} Hkv {Hkv} D {D}")
    on = Driver(pa, True, dtype, Hq, Hkv, D)
    n_on = on.run(requests())
    off = Driver(pa, False, dtype, Hq, Hkv, D)
    n_off = off.run(requests())
    assert n_on > 0 and n_off > 0
    # blocks reused as the pages describe: the system prompt's two full blocks,
    # all but the last block of a repeated prompt, nothing across cache salts,
    # and a finished request's cached blocks for a later arrival
    assert on.cached == {0: 0, 1: 32, 2: 64, 3: 0, 4: 0, 5: 32}
    assert all(c == 0 for c in off.cached.values())
    assert on.mgr.num_free_blocks == off.mgr.num_free_blocks == 96


def test_multistep_over_an_8bit_pool(pa):
    """The same requests over an 8-bit pool: every step's codes are written by
    the library and read back by later steps (prefix hits included)."""
    say("[multistep] fp8 pool, bf16 Hq 8 Hkv 2 D 128")
    on = Driver(pa, True, "bf16", 8, 2, 128, fp8_scales=(0.6, 0.35))
    assert on.run(requests()) > 0
    assert on.cached == {0: 0, 1: 32, 2: 64, 3: 0, 4: 0, 5: 32}
