"""Helpers for the GPU parity tests: put a workload on the device, run the
library through its C ABI, bring results back as numpy."""
from __future__ import annotations

import numpy as np
import torch

import workloads as W


def device_case(wl, device="cuda"):
    """All inputs of one step on the device (pool before the KV write)."""
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(device)
    q = W.q_device(wl, device)
    k, v = W.new_kv_device(wl, device)
    pool = W.pool_device(wl, device)
    return {
        "q": q, "k": k, "v": v, "pool": pool,
        "slot_mapping": t(wl.slot_mapping), "block_tables": t(wl.block_tables),
        "query_start_loc": t(wl.query_start_loc), "seq_lens": t(wl.seq_lens), "context_lens": t(wl.context_lens),
    }


def run_step(pa, wl, c, out=None, workspace=None):
    """pa_step: KV write then attention, through the C ABI."""
    pool = c["pool"]
    return pa.step(c["q"], c["k"], c["v"], pool[:, 0], pool[:, 1], c["slot_mapping"], c["block_tables"],
                   c["query_start_loc"], c["seq_lens"], c["context_lens"], wl.scale, out=out, workspace=workspace)


def to_f64(x: torch.Tensor) -> np.ndarray:
    return x.detach().float().cpu().numpy().astype(np.float64)


def raw_bytes(x: torch.Tensor) -> np.ndarray:
    """The tensor's bytes, flattened (uint8)."""
    x = x.detach().contiguous()
    if x.dtype == torch.bfloat16:
        x = x.view(torch.int16)
    return x.cpu().numpy().reshape(-1).view(np.uint8)


def rows_of(wl, seqs):
    return np.concatenate([np.arange(wl.query_start_loc[s], wl.query_start_loc[s + 1]) for s in seqs])


def host_inputs(wl, device="cuda"):
    """Host copies (numpy; bf16 as uint16 bits, fp8 as uint8 codes) of a
    workload's pool before the KV write, k, v and q, made by the torch twin of
    the seeded generator on the device (the same bits as the numpy twin,
    which tests/test_workloads.py checks) -- the generator, not the library."""
    def h(t):
        t = t.cpu()
        if t.dtype == torch.float32:
            return t.numpy()
        if t.dtype == torch.float8_e4m3fn:
            return t.view(torch.uint8).numpy()
        return t.view(torch.int16).numpy().view(np.uint16)

    k, v = W.new_kv_device(wl, device)
    return h(W.pool_device(wl, device)), h(k), h(v), h(W.q_device(wl, device))


def seq_batches(wl, seqs, max_bytes=4e9):
    """Consecutive groups of `seqs` whose K/V (each sequence's own blocks) stay under max_bytes."""
    per = -(-wl.seq_lens[seqs].astype(np.int64) // 16) * wl.block_bytes
    out, cur, acc = [], [], 0
    for s, b in zip(seqs, per):
        if cur and acc + b > max_bytes:
            out.append(cur)
            cur, acc = [], 0
        cur.append(int(s))
        acc += int(b)
    if cur:
        out.append(cur)
    return out


class ErrorTally:
    """Error statistics accumulated over batches of output rows (one row =
    one token and query head): max abs, mean abs, and the largest per-row
    max|err| / rms(reference row)."""

    def __init__(self):
        self.max_abs, self.sum_abs, self.n, self.rel, self.finite, self.rows = 0.0, 0.0, 0, 0.0, True, 0

    def add(self, got, ref):
        got = np.asarray(got, np.float64)
        ref = np.asarray(ref, np.float64)
        assert got.shape == ref.shape, (got.shape, ref.shape)
        if ref.size == 0:
            return
        err = np.abs(got - ref)
        self.finite &= bool(np.isfinite(got).all())
        self.max_abs = max(self.max_abs, float(err.max()))
        self.sum_abs += float(err.sum())
        self.n += err.size
        D = ref.shape[-1]
        row_err = err.reshape(-1, D).max(axis=1)
        row_rms = np.sqrt(np.mean(ref.reshape(-1, D) ** 2, axis=1))
        self.rel = max(self.rel, float(np.nanmax(row_err / np.maximum(row_rms, 1e-30))))
        self.rows += row_err.size

    def summary(self):
        return {"max_abs": self.max_abs, "mean_abs": self.sum_abs / max(self.n, 1), "rel": self.rel,
                "finite": self.finite, "rows": self.rows}


def oracle_every_row(wl, out, run, say=print, max_bytes=4e9):
    """Compare every output row of `out` (the device output of workload wl)
    with the oracle, sequence batch by sequence batch (each batch a compact
    sub-workload, so the host pool stays a few GB). `run(sub, pool)` runs the
    oracle on a sub-workload and its host pool. Returns the ErrorTally."""
    tally = ErrorTally()
    batches = seq_batches(wl, np.arange(wl.num_seqs), max_bytes)
    for i, seqs in enumerate(batches):
        sub = W.sub_workload(wl, seqs)
        pool, _, _, _ = host_inputs(sub)
        ref, _ = run(sub, pool)
        got = to_f64(out[torch.from_numpy(rows_of(wl, seqs)).to(out.device)])
        tally.add(got, ref)
        say(f"  batch {i + 1}/{len(batches)}: {len(seqs)} sequences, {tally.rows} rows so far")
    return tally
