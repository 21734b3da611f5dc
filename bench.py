#!/usr/bin/env python3
"""Benchmark of the paged-attention step on one MI355X.

A step is one pa_step call over one synthetic batch: KV write through
slot_mapping, split-K decode with partial reduce, and chunked prefill, over the
flattened super-sequence. Inputs are generated on the device before timing
and stay resident in HBM. Before each timed step a 2 GiB buffer is read so
that no K/V is left in the 256 MB Infinity Cache or the L2s (the TinyLlama
batch reads only ~71 MB); reading rather than writing leaves no dirty lines
draining to HBM during the step. The flush sits outside the per-step events.

Prints ONE JSON line. The headline workload is the Llama-3-8B-shaped mixed
step: 4096 decode tokens (contexts uniform in [256, 8192]) and 8 prefill
chunks of 512 tokens (prior contexts uniform in [0, 4096]) in one flattened
batch of 8192 tokens, 32/8 heads, head size 128, bf16 -- the one workload that
runs every part of the path. `value` is its decode KV-read bandwidth over the
whole step; the line also carries mixed-step tokens/s, prefill TFLOP/s and the
roofline of the decode (HBM) and prefill (bf16 MFMA, nested as
roofline.prefill) kernels. In this step the library runs the prefill kernel
after the decode kernel, first combining the decode's split-K partitions (the
chunks are too small a share of the step to gain from running beside the
decode), so the prefill roofline is timed on the same chunks run alone. `secondary` holds the other workloads -- the tiny fp32
decode, the TinyLlama-1.1B decode batch, the Llama-3-70B 32k decode, the
shared-prefix decode, a speculative-decode verification batch (4 new tokens
per sequence over long contexts), the 70B decode and 8B mixed step over an
8-bit pool, and the last 512-token chunk of a 32,512-token prompt (64 long
prefill items, which the prefill's schedule cuts along their keys to fill
every CU) -- each over 20 timed steps (mean, median, min) and also timed as
one HIP-graph replay per step (`ms_per_step_graph`). The decode's fraction is
quoted against the 8 TB/s spec and against a non-temporal read probe run on
the same GPU. `cpu_baseline` times the oracle on the host cores.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "decode KV-read GB/s (% HBM peak), mixed-step tokens/s, prefill TFLOP/s"
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
FP32_MFMA_PEAK_TFLOPS = 157.3  # MI355X dense fp32 MFMA
HEADLINE = 3
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "pagedattention_block_paged_amd", "csrc")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def device_inputs(wl):
    import numpy as np
    import torch

    import workloads as W

    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    c = {
        "q": W.q_device(wl, "cuda"),
        "pool": W.pool_device(wl, "cuda"),
        "slot_mapping": t(wl.slot_mapping),
        "block_tables": t(wl.block_tables),
        "query_start_loc": t(wl.query_start_loc),
        "seq_lens": t(wl.seq_lens),
        "context_lens": t(wl.context_lens),
    }
    c["k"], c["v"] = W.new_kv_device(wl, "cuda")
    return c


def kernel_split(wl):
    """Which sequences each attention kernel serves: the decode kernel takes
    every sequence whose new tokens times the query heads per KV head fit its
    16 MFMA columns (all decodes, and short queries such as speculative-decode
    verification); the prefill kernel takes the rest."""
    import numpy as np

    G = wl.num_q_heads // wl.num_kv_heads
    n = wl.query_lens.astype(np.int64)
    dec = (n >= 1) & (n * G <= 16)
    pre = (n >= 1) & ~dec
    return dec, pre


def kernel_work(wl, dec, pre):
    """Algorithmic work of the two kernels: the decode kernel's bytes (K/V of
    its sequences, their block-table entries, their query rows) and the
    prefill kernel's causal-exact FLOPs."""
    import numpy as np

    import workloads as W

    es = W.DTYPE_BYTES[wl.dtype]  # q
    L = wl.seq_lens.astype(np.int64)
    n = wl.query_lens.astype(np.int64)
    C = wl.context_lens.astype(np.int64)
    kv = int(L[dec].sum()) * 2 * wl.num_kv_heads * wl.head_size * wl.kv_elem_bytes
    tables = int((-(-L[dec] // W.BLOCK_SIZE)).sum()) * 4
    q = int(n[dec].sum()) * wl.num_q_heads * wl.head_size * es
    pairs = int((n[pre] * C[pre] + n[pre] * (n[pre] + 1) // 2).sum())  # sum over queries of visible keys
    return kv + tables + q, 4 * wl.head_size * wl.num_q_heads * pairs


def unique_decode_bytes(wl, dec):
    """K/V bytes of the distinct blocks the decode kernel's sequences read (a
    shared block once), plus their table entries and query rows."""
    import numpy as np

    import workloads as W

    blocks = set()
    for s in np.nonzero(dec)[0]:
        blocks.update(wl.block_tables[s, : wl.blocks_used(s)].tolist())
    L = wl.seq_lens[dec].astype(np.int64)
    tables = int((-(-L // W.BLOCK_SIZE)).sum()) * 4
    q = int(wl.query_lens[dec].astype(np.int64).sum()) * wl.num_q_heads * wl.head_size * W.DTYPE_BYTES[wl.dtype]
    return len(blocks) * wl.block_bytes + tables + q


def run_step(pa, wl, c, out, ws):
    """One pa_step (pa_step_fp8 over an 8-bit pool) on the device inputs ``c``."""
    pool = c["pool"]
    args = (c["q"], c["k"], c["v"], pool[:, 0], pool[:, 1], c["slot_mapping"], c["block_tables"],
            c["query_start_loc"], c["seq_lens"], c["context_lens"])
    if wl.kv_dtype == "fp8":
        pa.step_fp8(*args, wl.scale, wl.k_scale, wl.v_scale, out=out, workspace=ws)
    else:
        pa.step(*args, wl.scale, out=out, workspace=ws)


def measure(cfg: int, steps: int, warmup: int, flush: str = "read", graph: bool = False) -> dict:
    import torch

    import pagedattention_block_paged_amd as pa
    import workloads as W

    hbm = torch.cuda.get_device_properties(0).total_memory
    wl = W.config_workload(cfg, hbm_bytes=hbm)
    t0 = time.time()
    c = device_inputs(wl)
    torch.cuda.synchronize()
    log(f"[bench] cfg {cfg} {wl.name}: S={wl.num_seqs} T={wl.num_tokens} NB={wl.num_blocks} "
        f"inputs ready in {time.time() - t0:.1f}s")
    pool = c["pool"]
    out = torch.empty_like(c["q"])
    ws = pa.new_workspace(c["q"], pool[:, 0], c["block_tables"])
    scratch = torch.ones(2 << 30, dtype=torch.uint8, device="cuda") if flush != "none" else None
    sink = torch.zeros(1, dtype=torch.int64, device="cuda")

    def evict(i):
        # Read (default) or write 2 GiB so no K/V stays in the L2s or the 256 MB
        # Infinity Cache. A read flush leaves no dirty lines draining to HBM
        # while the next step runs.
        if scratch is None:
            return
        if flush == "read":
            torch.sum(scratch.view(torch.int64), dim=0, keepdim=True, out=sink)
        else:
            scratch.fill_(i & 0x7F)

    def one_step():
        run_step(pa, wl, c, out, ws)

    for i in range(warmup):
        evict(i)
        one_step()
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    for i in range(steps):
        evict(i)
        starts[i].record()
        one_step()
        ends[i].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    # Per-kernel times in a second pass: the library's event pairs around each
    # launch would otherwise sit inside the step timing.
    with pa.profile() as prof:
        for i in range(steps):
            evict(i)
            one_step()
        torch.cuda.synchronize()
    per = sorted(s.elapsed_time(e) for s, e in zip(starts, ends))
    ms = sum(per) / len(per)
    graph_ms = None
    if graph:
        # The same step captured once in a HIP graph and replayed (the cache
        # flush stays eager, outside the events): what a serving loop that
        # replays its decode step sees.
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            one_step()
        torch.cuda.synchronize()
        gs = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
        ge = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
        for i in range(steps):
            evict(i)
            gs[i].record()
            g.replay()
            ge[i].record()
        torch.cuda.synchronize()
        graph_ms = sum(a.elapsed_time(b) for a, b in zip(gs, ge)) / steps
        del g
    finite = bool(torch.isfinite(out.float()).all())
    kern = {k: {"avg_ms": v[0] / v[1], "launches": v[1]} for k, v in prof.kernels.items()}
    dec_bytes = wl.decode_bytes()
    dec_set, pre_set = kernel_split(wl)
    dec_kernel_bytes, flops = kernel_work(wl, dec_set, pre_set)
    alone = None
    if dec_set.any() and pre_set.any():
        # In a mixed batch the prefill kernel may run beside the decode kernel
        # on a few CUs for most of the step, so its duration there says
        # nothing about its speed: the same chunks (same pool, block tables
        # and values) are also timed alone, where it has the whole GPU.
        alone = measure_prefill_alone(pa, wl, c, pre_set, steps, evict)
    r = {
        "workload": wl.name,
        "num_seqs": wl.num_seqs,
        "num_tokens": wl.num_tokens,
        "num_q_heads": wl.num_q_heads,
        "num_kv_heads": wl.num_kv_heads,
        "head_size": wl.head_size,
        "dtype": wl.dtype,
        "kv_dtype": wl.pool_dtype,
        "pool_blocks": wl.num_blocks,
        "partition_tokens": pa.partition_tokens(wl.num_seqs, wl.num_kv_heads, wl.head_size, wl.dtype, wl.max_blocks,
                                                kv_fp8=wl.pool_dtype == "fp8"),
        "ms_per_step": ms,
        "ms_per_step_graph": graph_ms,
        "ms_per_step_median": per[len(per) // 2],
        "ms_per_step_min": per[0],
        "wall_s_timed_region": wall,
        "tokens_per_s": wl.num_tokens / (ms * 1e-3),
        "decode_bytes": dec_bytes,
        "decode_gbs_step": dec_bytes / (ms * 1e-3) / 1e9,
        "kv_read_gbs_step": wl.kv_read_bytes() / (ms * 1e-3) / 1e9,
        "prefill_flops": flops,
        "kernels": kern,
        "output_finite": finite,
    }
    if "decode" in kern and dec_kernel_bytes > 0:  # (a batch with no decode-kernel sequence has no decode rate)
        d = kern["decode"]["avg_ms"]
        r["decode_kernel_bytes"] = dec_kernel_bytes
        r["decode_kernel_gbs"] = dec_kernel_bytes / (d * 1e-3) / 1e9
        if int(wl.shared_len.max()) > 0:
            # Shared prefix blocks are counted once per sequence that reads
            # them: a logical rate, which may exceed the HBM peak because the
            # shared blocks are re-read from the caches. The DRAM rate comes
            # from the committed FETCH_SIZE / WRITE_SIZE counters of this
            # kernel on this workload (null once the kernel source changed).
            r["decode_kernel_gbs_logical"] = r.pop("decode_kernel_gbs")
            r["decode_kernel_unique_bytes"] = unique_decode_bytes(wl, dec_set)
            dram = kernel_traffic("decode", wl.name)
            r["decode_kernel_dram_bytes"] = dram
            r["decode_kernel_dram_gbs"] = None if dram is None else dram / (d * 1e-3) / 1e9
            r["decode_kernel_dram_frac"] = None if dram is None else r["decode_kernel_dram_gbs"] / HBM_PEAK_GBS
        else:
            r["decode_kernel_hbm_frac"] = r["decode_kernel_gbs"] / HBM_PEAK_GBS
    if flops and "prefill" in kern:
        p = alone["prefill_ms"] if alone else kern["prefill"]["avg_ms"]
        r["prefill_tflops"] = flops / (p * 1e-3) / 1e12
        # an 8-bit pool's prefill runs on the bf16 matrix cores at head size
        # 128 (codes widened on their way into LDS), on the fp32 ones at 64
        r["prefill_mfma_peak"] = (FP32_MFMA_PEAK_TFLOPS if wl.kv_dtype == "fp8" and wl.head_size != 128
                                  else BF16_PEAK_TFLOPS)
        r["prefill_mfma_frac"] = r["prefill_tflops"] / r["prefill_mfma_peak"]
        if alone:
            r["prefill_alone"] = alone
            r["prefill_in_step_ms"] = kern["prefill"]["avg_ms"]
            # the two-stream path launches the plan on its own ("prefill_plan")
            r["prefill_beside_decode"] = "prefill_plan" in kern
    r["flush"] = flush
    del c, pool, out, ws, scratch
    torch.cuda.empty_cache()
    return r


def measure_prefill_alone(pa, wl, c, pre_set, steps, evict):
    """The prefill-kernel sequences of a mixed batch as their own step."""
    import numpy as np
    import torch

    seqs = np.nonzero(pre_set)[0]
    qsl = wl.query_start_loc
    rows = torch.from_numpy(np.concatenate([np.arange(qsl[s], qsl[s + 1]) for s in seqs])).cuda()
    idx = torch.from_numpy(seqs).cuda()
    n = torch.from_numpy(wl.query_lens[seqs].astype(np.int32))
    sub_qsl = torch.zeros(len(seqs) + 1, dtype=torch.int32)
    sub_qsl[1:] = torch.cumsum(n, 0)
    sub = {
        "q": c["q"][rows].contiguous(), "k": c["k"][rows].contiguous(), "v": c["v"][rows].contiguous(),
        "slot_mapping": c["slot_mapping"][rows].contiguous(),
        "block_tables": c["block_tables"][idx].contiguous(), "query_start_loc": sub_qsl.cuda(),
        "seq_lens": c["seq_lens"][idx].contiguous(), "context_lens": c["context_lens"][idx].contiguous(),
    }
    sub["pool"] = c["pool"]
    out = torch.empty_like(sub["q"])
    ws = pa.new_workspace(sub["q"], sub["pool"][:, 0], sub["block_tables"])

    def one():
        # the KV write rewrites the chunks' rows with the values they already hold
        run_step(pa, wl, sub, out, ws)

    for i in range(2):
        evict(i)
        one()
    torch.cuda.synchronize()
    with pa.profile() as prof:
        for i in range(steps):
            evict(i)
            one()
        torch.cuda.synchronize()
    k = prof.kernels["prefill"]
    return {"sequences": int(len(seqs)), "tokens": int(rows.numel()), "prefill_ms": k[0] / k[1],
            "launches": k[1], "what": "the batch's prefill chunks alone (same pool, tables, values), whole GPU"}


def host_inputs(wl):
    """Host copies of one workload's inputs (numpy; bf16 as uint16 bits).

    Generated on the GPU with the torch twin of the generator when one is
    present (same bits as the numpy twin, much faster), else with numpy.
    """
    import numpy as np
    import torch

    import workloads as W

    if not torch.cuda.is_available():
        k, v = W.new_kv_host(wl)
        return W.pool_host(wl), k, v, W.q_host(wl)

    def h(t):
        t = t.cpu()
        return t.numpy() if t.dtype == torch.float32 else t.view(torch.int16).numpy().view(np.uint16)

    k, v = W.new_kv_device(wl, "cuda")
    return h(W.pool_device(wl, "cuda")), h(k), h(v), h(W.q_device(wl, "cuda"))


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def oracle_step(wl, threads: int = 0, reps: int = 1):
    """The oracle's whole step (KV write + attention) on a workload's host
    inputs, median wall time of `reps` runs (input generation excluded).
    Returns (seconds, threads used)."""
    import oracle

    pool0, k, v, q = host_inputs(wl)
    times, used = [], 0
    for _ in range(reps):
        pool = pool0.copy()
        t0 = time.perf_counter()
        oracle.reshape_and_cache(k, v, pool, wl.slot_mapping, wl.dtype)
        _, used = oracle.attention(q, pool, wl.block_tables, wl.query_start_loc, wl.seq_lens, wl.context_lens,
                                   wl.scale, wl.dtype, num_threads=threads, return_threads=True)
        times.append(time.perf_counter() - t0)
    return sorted(times)[len(times) // 2], used


def cpu_baseline(cfg: int, budget_s: float) -> dict:
    """The oracle, as is, on the host cores.

    Headline: a seeded sample of the workload's decode sequences (KV write +
    attention) repeated until `budget_s` has passed, as decode KV-read GB/s,
    and the longest prefill chunk once, as GFLOP/s (fp64); with the whole
    batch's time extrapolated from those two rates. Then whole batches: the
    tiny fp32 and TinyLlama decode batches on one thread and on all (median
    of 3), and the 70B 32k decode batch on all threads once.
    """
    import numpy as np

    import oracle
    import workloads as W

    wl = W.config_workload(cfg)
    dec = np.nonzero(wl.decode_mask())[0]
    pre = np.nonzero(~wl.decode_mask())[0]
    rs = np.random.default_rng(7)
    take = dec if dec.size <= 128 else np.sort(rs.choice(dec, size=128, replace=False))
    out = {"unit": "GB/s", "kind": "oracle", "cpu_model": cpu_model(),
           "affinity_cpus": len(os.sched_getaffinity(0))}
    if take.size:
        sub = W.sub_workload(wl, take)
        pool0, k, v, q = host_inputs(sub)
        passes, threads, t0 = 0, 0, time.perf_counter()
        while True:
            pool = pool0.copy()
            oracle.reshape_and_cache(k, v, pool, sub.slot_mapping, sub.dtype)
            _, threads = oracle.attention(q, pool, sub.block_tables, sub.query_start_loc, sub.seq_lens,
                                          sub.context_lens, sub.scale, sub.dtype, return_threads=True)
            passes += 1
            secs = time.perf_counter() - t0  # includes one pool copy per pass
            if secs >= budget_s:
                break
        out.update({
            "value": sub.decode_bytes() * passes / secs / 1e9,
            "cores": threads,
            "sample": f"{take.size} of {dec.size} decode sequences of {wl.name} (seeded), KV write + attention, "
                      f"{passes} passes in {secs:.1f} s, fp64, {threads} OpenMP threads",
            "decode_tokens_per_s": take.size * passes / secs,
        })
    if pre.size:
        s = int(pre[np.argmax(wl.seq_lens[pre])])
        sub = W.sub_workload(wl, [s])
        secs, threads = oracle_step(sub)
        out["prefill_gflops"] = sub.prefill_flops() / secs / 1e9
        out["prefill_sample"] = (f"longest prefill chunk ({int(sub.query_lens[0])} tokens after "
                                 f"{int(sub.context_lens[0])} cached), once, {secs:.2f} s, {threads} threads")
        out.setdefault("cores", threads)
    if take.size and pre.size:
        # the whole batch at the sample's rates: decode bytes / decode rate +
        # prefill FLOPs / prefill rate
        est = wl.decode_bytes() / (out["value"] * 1e9) + wl.prefill_flops() / (out["prefill_gflops"] * 1e9)
        out["whole_batch_estimate_s"] = est
        out["whole_batch_tokens_per_s_estimate"] = wl.num_tokens / est
        out["whole_batch_note"] = ("estimated, not run: the decode sample's GB/s applied to the batch's "
                                   f"{wl.decode_bytes() / 1e9:.1f} GB of decode bytes plus the chunk's GFLOP/s "
                                   f"applied to its {wl.prefill_flops() / 1e9:.1f} GFLOP of prefill")
    runs = {}
    for c, one in ((1, True), (2, True), (4, False)):
        full = W.config_workload(c)
        # the same sequences over a compact pool (only the blocks they use)
        w = W.sub_workload(full, np.arange(full.num_seqs))
        row = {"workload": full.name}
        for thr in ((1, 0) if one else (0,)):
            secs, used = oracle_step(w, threads=thr, reps=3 if one else 1)
            row[f"threads_{used}"] = {"seconds": secs, "decode_gbs": w.decode_bytes() / secs / 1e9,
                                      "tokens_per_s": w.num_tokens / secs,
                                      "runs": "median of 3" if one else "once"}
        runs[full.name] = row
        log(f"[bench] cpu baseline {full.name}: {row}")
    out["whole_batches"] = runs
    return out


def host_manager(cfg: int, rounds: int = 6) -> dict:
    """The library's host-side KV block manager producing the step inputs of a
    workload: every sequence admitted (random token ids, prefix caching on)
    with its cached context computed beforehand (untimed); then, timed, the
    headline step itself (allocate_slots for every sequence's new tokens,
    build_step, commit) and decode steps after it (one sampled token appended
    per sequence). The allocate and commit loops are driven from Python, one
    ctypes call per sequence, so they include that call overhead."""
    import numpy as np

    import workloads as W
    from pagedattention_block_paged_amd.kv_manager import KVCacheManager

    wl = W.config_workload(cfg)
    S = wl.num_seqs
    n = wl.query_lens.astype(np.int64)
    C = wl.context_lens.astype(np.int64)
    rs = np.random.default_rng(0)
    t0 = time.perf_counter()
    m = KVCacheManager(int(wl.num_blocks), 16, True)
    for s in range(S):
        m.add_request(s, rs.integers(0, 32000, int(C[s] + n[s]), dtype=np.int32))
        if C[s]:
            assert m.allocate_slots(s, int(C[s]))
            m.commit(s, int(C[s]))
    setup_s = time.perf_counter() - t0
    ids = np.arange(S, dtype=np.int64)
    width = wl.max_blocks + 1
    out, rows = None, []
    for r in range(rounds):
        nn = n if r == 0 else np.ones(S, np.int64)
        if r > 0:
            for s in range(S):
                m.append_tokens(s, [int(rs.integers(0, 32000))])
        t1 = time.perf_counter()
        for s in range(S):
            assert m.allocate_slots(s, int(nn[s]))
        t2 = time.perf_counter()
        out = m.build_step(ids, nn, width, out=out)
        t3 = time.perf_counter()
        for s in range(S):
            m.commit(s, int(nn[s]))
        t4 = time.perf_counter()
        rows.append(((t2 - t1) * 1e3, (t3 - t2) * 1e3, (t4 - t3) * 1e3))
    dec = np.array(rows[1:])
    return {
        "workload": wl.name,
        "requests": S,
        "blocks_held": int(wl.num_blocks) - m.num_free_blocks,
        "setup_s": setup_s,
        "headline_step_ms": {"allocate_slots": rows[0][0], "build_step": rows[0][1], "commit": rows[0][2]},
        "decode_step_ms_median": {k: float(np.median(dec[:, i]))
                                  for i, k in enumerate(("allocate_slots", "build_step", "commit"))},
        "note": "host CPU time; allocate_slots and commit loops include one ctypes call per request",
    }


def kernel_traffic(kernel: str, workload: str):
    """HBM bytes per launch from committed counter runs, if the kernel source is unchanged."""
    import hashlib

    path = os.path.join(PROFILES, "counters.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f).get(kernel, {}).get(workload)
    if not rec:
        return None
    with open(os.path.join(CSRC, rec["source"]), "rb") as f:
        if hashlib.sha256(f.read()).hexdigest() != rec["source_sha256"]:
            return None  # the kernel changed since the counters were taken
    return rec["fetch_kib"] * 1024 * rec["fetch_scale"] + rec["write_kib"] * 1024 * rec["write_scale"]


def prefill_timing_note(head: dict) -> str:
    if not head.get("prefill_alone"):
        return "in the step"
    where = ("beside the decode on a few CUs, hidden behind it" if head.get("prefill_beside_decode")
             else "after the decode on the whole GPU, first combining the decode's partitions")
    return f"the step's prefill chunks alone; in the step the kernel runs {where} ({head['prefill_in_step_ms']:.3f} ms)"


def read_bandwidth(nbytes: int = 4 << 30, reps: int = 10) -> float:
    """What a plain non-temporal read stream reaches on this GPU, in GB/s,
    best of `reps` over 4 GiB (the library's pa_profile_read_probe: every byte
    read once with 16-byte non-temporal loads, as the decode reads K/V): the
    practical ceiling of a read-bound kernel, beside the 8 TB/s spec. A 2 GiB
    read queued ahead of each timed probe keeps the host's launch latency
    out of the timed interval, as the cache flush does for the steps."""
    import torch

    import pagedattention_block_paged_amd as pa

    buf = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    ahead = torch.ones(2 << 30, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1, dtype=torch.int64, device="cuda")
    for _ in range(2):
        pa.read_probe(buf)
    best = float("inf")
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.sum(ahead.view(torch.int64), dim=0, keepdim=True, out=sink)
        e0.record()
        pa.read_probe(buf)
        e1.record()
        e1.synchronize()
        best = min(best, e0.elapsed_time(e1) * 1e-3)
    del buf, ahead
    torch.cuda.empty_cache()
    return nbytes / best / 1e9


def read_probe_sizes(sizes, reps: int = 20) -> dict:
    """The plain-read probe at the given byte counts (a batch's K/V bytes),
    each timed read preceded by a 1 GiB read that evicts the buffer from the
    caches, so that every byte comes from HBM as in a decode step. The HIP
    event times include a few microseconds of launch overhead; a kernel trace
    of the same run gives the probe kernel alone."""
    import torch

    import pagedattention_block_paged_amd as pa

    flush = torch.ones(1 << 30, dtype=torch.uint8, device="cuda")
    out = {}
    for nbytes in sizes:
        buf = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
        times = []
        for _ in range(reps):
            pa.read_probe(flush)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            pa.read_probe(buf)
            e1.record()
            e1.synchronize()
            times.append(e0.elapsed_time(e1) * 1e3)
        times.sort()
        out[str(nbytes)] = {"event_us_median": times[len(times) // 2], "event_us_min": times[0]}
        del buf
    del flush
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=HEADLINE, help="headline workload (1-9)")
    ap.add_argument("--secondary", default="1,2,4,5,6,7,8,9", help="other workloads to measure, or 'none'")
    ap.add_argument("--secondary-steps", type=int, default=20)
    ap.add_argument("--secondary-warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-host-manager", action="store_true",
                    help="skip timing the host KV block manager on the headline batch")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--flush", choices=["read", "write", "none"], default="read",
                    help="cache eviction between timed steps (outside the step events)")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the HIP-graph replay timing of the secondary workloads")
    ap.add_argument("--read-probe-sizes", default="",
                    help="comma-separated byte counts: also time the plain-read probe at these sizes")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 1 GiB device copy (for scaling HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1", "n_gpus": args.gpus}))
        sys.exit(2)

    import torch

    import pagedattention_block_paged_amd  # noqa: F401  (fails loudly if libpa.so is missing)

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    head = measure(args.config, args.steps, args.warmup, flush=args.flush)
    log(f"[bench] headline: {json.dumps(head)}")
    secondary = {}
    if args.secondary != "none":
        for cfg in [int(x) for x in args.secondary.split(",") if x]:
            if cfg == args.config:
                continue
            r = measure(cfg, args.secondary_steps, args.secondary_warmup, flush=args.flush, graph=not args.no_graph)
            log(f"[bench] cfg {cfg}: {json.dumps(r)}")
            secondary[r["workload"]] = r
    read_gbs = read_bandwidth()
    log(f"[bench] read probe: {read_gbs:.1f} GB/s (non-temporal read of 4 GiB, best of 10)")
    probe_sizes = None
    if args.read_probe_sizes:
        probe_sizes = read_probe_sizes([int(x) for x in args.read_probe_sizes.split(",") if x])
        log(f"[bench] read probe by size: {json.dumps(probe_sizes)}")
    if args.calibrate_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("[bench] copy calibration: 3 x 1 GiB device-to-device copies")
    mgr = None
    if not args.no_host_manager:
        mgr = host_manager(args.config)
        log(f"[bench] host KV manager: {json.dumps(mgr)}")
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(args.config, args.cpu_seconds)
        log(f"[bench] cpu baseline: {json.dumps(cpu)}")

    dec = head.get("decode_kernel_gbs")
    pre = head.get("prefill_tflops")
    pre_peak = head.get("prefill_mfma_peak", BF16_PEAK_TFLOPS)
    line = {
        "metric": METRIC,
        "value": head["decode_gbs_step"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": head["dtype"],
        "data": "synthetic",
        "config": {
            "workload": head["workload"],
            "num_seqs": head["num_seqs"],
            "num_tokens": head["num_tokens"],
            "num_q_heads": head["num_q_heads"],
            "num_kv_heads": head["num_kv_heads"],
            "head_size": head["head_size"],
            "block_size": 16,
            "pool_blocks": head["pool_blocks"],
            "parallelism": "single GPU",
        },
        "value_definition": "decode KV-read bytes (K, V, block tables, q) per whole pa_step, divided by the step time",
        "ms_per_step_median": head["ms_per_step_median"],
        "ms_per_step_min": head["ms_per_step_min"],
        "hbm_frac_step": head["decode_gbs_step"] / HBM_PEAK_GBS,
        "mixed_step_tokens_per_s": head["tokens_per_s"],
        "prefill_tflops": pre,
        "roofline": {
            "kernel": "decode",
            "bound": "hbm",
            "achieved": dec,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": (dec / HBM_PEAK_GBS) if dec else None,
            "traffic": kernel_traffic("decode", head["workload"]),
            "algorithmic_bytes": head.get("decode_kernel_bytes"),
            "read_probe_gbs": read_gbs,
            "frac_of_read_probe": (dec / read_gbs) if dec else None,
            "read_probe_by_size": probe_sizes,
            "prefill": None if pre is None else {
                "kernel": "prefill",
                "bound": "mfma",
                "achieved": pre,
                "peak": pre_peak,
                "unit": "TFLOP/s",
                "frac": pre / pre_peak,
                "traffic": kernel_traffic("prefill", head["workload"]),
                "algorithmic_flops": head["prefill_flops"],
                "kernel_ms": (head.get("prefill_alone") or {}).get("prefill_ms"),
                "timed": prefill_timing_note(head),
            },
        },
        "cpu_baseline": cpu,
        "host_kv_manager": mgr,
        "kernels": head["kernels"],
        "secondary": secondary,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
