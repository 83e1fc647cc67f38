#!/usr/bin/env python3
"""Benchmark of the paged decode step on one MI355X.

One step = the whole path for one layer of a decode batch:
  1. slot mapping of the new token of every sequence (position ctx - 1),
  2. the KV write of those rows into the pool,
  3. split-K paged decode attention over every sequence's whole context,
  4. the merge of split partials.
The timed step is the library's fused form: pkv_decode_step does 1-4 in one
launch (the last workgroup of each sequence and KV head merges its splits).
The same step with the write as separate launches (pkv_slot_mapping +
pkv_write + pkv_decode) is reported beside it.
Default workload: the LLaMA-2-70B per-layer shape (64 sequences, context
lengths log-uniform in [512, 8192), 64 query / 8 KV heads, head_dim 128,
bf16, 16-token blocks scattered over a 32,769-block pool). The timed loop
reads ~689 MB of K/V per step, well above the 256 MB Infinity Cache, so no
input rotation is needed.

Prints one JSON line: whole-step KV-read GB/s (`value`), the roofline of the
dominant kernel (the decode kernel: the step's only launch, so its mean
duration is the step time between HIP events around the timed loop), and the
CPU oracle timed on a bounded sample on the host. The two Llama-3.2-1B decode
shapes (8 x 2048 tokens, and 192 sequences) are timed decode-only over rotating
block sets, launched from Python and replayed from
one captured HIP graph; the graph figure is the GPU's when a call is shorter
than the binding's host-side time per call. Each leg also reports single
launches after a 512 MiB cache-evicting write ("cold", percentiles), the
decode-only configs the same block set back to back ("warm", cache-assisted),
and the step the percentiles of its launches timed one by one. The workload's
chunked-prefill variant (pkv_prefill on the same pools) is timed too and
reported against the dense bf16 matrix-core peak, and so is the bulk write that
stores such a chunk for every sequence (pkv_write, against HBM).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import paged_kv_cache_scatter_amd as pkv  # noqa: E402
from workloads import CONFIGS, make_shared, make_tp_shard, make_workload  # noqa: E402

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
DEV = torch.device("cuda:0")
COUNTERS = os.path.join(ROOT, "profiles", "decode_partials_counters.json")
WRITE_COUNTERS = os.path.join(ROOT, "profiles", "write_bulk_counters.json")


def to_dev(a: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(a).to(DEV)


def workload_label(wl) -> str:
    spec = CONFIGS[wl.cfg_id]
    d = spec.ctx_dist
    if d[0] == "const":
        lens = f"{d[1]}"
    elif d[0] == "uniform":
        lens = f"U[{d[1]},{d[2]}]"
    else:
        lens = f"logU[{d[1]},{d[2]})"
    return (f"{wl.name}: {wl.num_seqs} seqs x ctx {lens}, {wl.num_q_heads} q / "
            f"{wl.num_kv_heads} kv heads, head_dim {wl.head_dim}, block {wl.block_size}, "
            f"pool {wl.num_blocks} blocks, {wl.dtype}")


class Step:
    """Device state for one decode step of workload ``wl`` (fused: the write of
    the new tokens inside the decode launch; else separate launches)."""

    def __init__(self, wl, partition: int = 0, fused: bool = True):
        self.wl = wl
        self.fused = fused
        dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
        self.k_pool = torch.zeros(wl.pool_shape, dtype=dt, device=DEV)
        self.v_pool = torch.zeros(wl.pool_shape, dtype=dt, device=DEV)
        tabs, first, cu, rows = wl.bulk_segments(exclude_last=wl.prefix_tokens == 0)
        n = int(cu[-1])
        slots = pkv.slot_mapping(to_dev(tabs), to_dev(first), to_dev(cu), n, wl.block_size,
                                 wl.num_blocks)
        pkv.write(to_dev(wl.k_rows[rows]), to_dev(wl.v_rows[rows]), slots, self.k_pool,
                  self.v_pool)
        s_tabs, s_first, s_cu, s_rows = wl.step_segments()
        self.s_tabs, self.s_first, self.s_cu = to_dev(s_tabs), to_dev(s_first), to_dev(s_cu)
        self.n_new = int(s_cu[-1])
        self.k_new, self.v_new = to_dev(wl.k_rows[s_rows]), to_dev(wl.v_rows[s_rows])
        # one row per sequence for the fused step (an empty sequence's row is unused)
        rows_s = np.array([r[-1] if len(r) else 0 for r in wl.seq_rows], dtype=np.int64)
        self.k_step, self.v_step = to_dev(wl.k_rows[rows_s]), to_dev(wl.v_rows[rows_s])
        self.slots = torch.empty(self.n_new, dtype=torch.int32, device=DEV)
        self.q = to_dev(wl.q)
        self.out = torch.empty_like(self.q)
        self.tables = to_dev(wl.block_tables)
        self.ctx = to_dev(wl.context_lens)
        self.max_ctx = int(wl.context_lens.max())
        # partition 0 leaves the cut to the library; auto_partition is the
        # split size it would take (and the least stream-K range)
        self.partition = partition
        self.auto_partition = partition or pkv.decode_partition(wl.num_seqs, self.max_ctx,
                                                                self.k_pool)
        self.schedule = pkv.decode_schedule(wl.num_seqs, wl.num_q_heads, self.max_ctx,
                                            self.k_pool, partition)
        nws = pkv.decode_workspace_bytes(wl.num_seqs, wl.num_q_heads, self.max_ctx,
                                         self.k_pool, self.partition)
        self.ws = torch.zeros(max(nws, 16), dtype=torch.uint8, device=DEV)
        torch.cuda.synchronize()

    def run(self, ev_a=None, ev_b=None):
        wl = self.wl
        if self.fused:
            if ev_a is not None:
                ev_a.record()
            pkv.decode_step(self.q, self.k_step, self.v_step, self.k_pool, self.v_pool,
                            self.tables, self.ctx, wl.scale, self.max_ctx, out=self.out,
                            partition=self.partition, workspace=self.ws)
            if ev_b is not None:
                ev_b.record()
            return
        pkv.slot_mapping(self.s_tabs, self.s_first, self.s_cu, self.n_new, wl.block_size,
                         wl.num_blocks, out=self.slots)
        pkv.write(self.k_new, self.v_new, self.slots, self.k_pool, self.v_pool)
        if ev_a is not None:
            ev_a.record()
        pkv.decode(self.q, self.k_pool, self.v_pool, self.tables, self.ctx, wl.scale,
                   self.max_ctx, out=self.out, partition=self.partition, workspace=self.ws)
        if ev_b is not None:
            ev_b.record()


MIN_WARMUP_S = 0.25   # untimed steps run for at least this long, whatever --warmup says


def warm_up(run, warmup: int) -> int:
    """``warmup`` untimed calls, continued until MIN_WARMUP_S of wall time has
    passed (a fresh process's first milliseconds of GPU work run slow: 148 us
    per step after 10 warm-up steps against 135 us after 200). Returns the
    number of calls made."""
    n = 0
    t0 = time.perf_counter()
    while n < warmup or time.perf_counter() - t0 < MIN_WARMUP_S:
        run()
        n += 1
        if n % 64 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    return n


def timed_loop(run, calls: int) -> float:
    """Mean ms per call of ``calls`` back-to-back calls between two HIP events
    on the current stream (the library launches on it)."""
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(calls):
        run()
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / calls


def repeat_stats(ms: list) -> dict:
    a = np.array(ms) * 1e3
    return {"n": len(ms), "us": [round(float(x), 2) for x in a],
            "median_us": round(float(np.median(a)), 2),
            "p10_us": round(float(np.percentile(a, 10)), 2),
            "p90_us": round(float(np.percentile(a, 90)), 2)}


def time_steps(step: Step, steps: int, warmup: int, repeats: int = 3):
    """Mean step time over ``steps`` back-to-back steps between two HIP events
    (the headline), then ``repeats - 1`` more such loops (run-to-run spread),
    and the mean time of the decode launch alone from a pair of events around
    it in each of another ``steps`` steps (those events also hold the launch
    latency, so this figure reads a few us high)."""
    nwarm = warm_up(step.run, warmup)
    loops = [timed_loop(step.run, steps) for _ in range(repeats)]
    ms_step = loops[0]
    ev_a = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ev_b = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    for i in range(steps):
        step.run(ev_a[i], ev_b[i])
    torch.cuda.synchronize()
    each = np.array([a.elapsed_time(b) for a, b in zip(ev_a, ev_b)])
    return ms_step, float(each.mean()), percentiles_us(each), repeat_stats(loops), nwarm


def percentiles_us(ms: np.ndarray) -> dict:
    return {f"p{q}": round(float(np.percentile(ms, q)) * 1e3, 2) for q in (10, 50, 90)}


COLD_FLUSH_BYTES = 512 << 20   # twice the 256 MB Infinity Cache, far above the L2s


def time_cold(fn, reps: int = 20) -> dict:
    """Single calls after a 512 MiB device write that evicts the caches: the
    percentiles of the per-call times (events around each call only)."""
    scratch = torch.empty(COLD_FLUSH_BYTES, dtype=torch.uint8, device=DEV)
    ev_a = [torch.cuda.Event(enable_timing=True) for _ in range(reps)]
    ev_b = [torch.cuda.Event(enable_timing=True) for _ in range(reps)]
    for i in range(reps):
        scratch.fill_(i & 255)
        ev_a[i].record()
        fn()
        ev_b[i].record()
    torch.cuda.synchronize()
    out = percentiles_us(np.array([a.elapsed_time(b) for a, b in zip(ev_a, ev_b)]))
    del scratch
    return out


PROBE_LIB = os.path.join(ROOT, "paged_kv_cache_scatter_amd", "libpkv_probe.so")


def time_probes(step: Step, calls: int = 20, stream_bytes: int = 2 << 30):
    """Read-bandwidth probes with no arithmetic (libpkv_probe.so): a contiguous
    ``stream_bytes`` buffer read once per call with 16-byte non-temporal
    loads, and the step's own K/V rows read through its block tables, one
    workgroup per (KV head, sequence, split), over split sizes of 256, 512
    and 1024 tokens and 1, 2 or 4 token rows per thread in flight. GB/s of
    each (the paged probe counted in the step's algorithmic K/V bytes): the
    paged figure at the automatic partition with one row in flight, and the
    best of the sweep (the ceiling the decode is compared with)."""
    import ctypes
    if not os.path.exists(PROBE_LIB):
        raise SystemExit(f"{PROBE_LIB} is not built; run __graft_entry__.build()")
    lib = ctypes.CDLL(PROBE_LIB)
    P, I = ctypes.c_void_p, ctypes.c_int32
    lib.pkv_probe_stream.argtypes = [P, ctypes.c_size_t, I, P, P]
    lib.pkv_probe_paged.argtypes = [P, P, P, I, P, I, I, I, I, I, I, I, I, P, P]
    wl = step.wl
    buf = torch.ones(stream_bytes // 4, dtype=torch.int32, device=DEV)
    blocks = 256 * 16
    sink = torch.zeros(1 << 20, dtype=torch.int32, device=DEV)
    strm = torch.cuda.current_stream().cuda_stream

    def stream():
        if lib.pkv_probe_stream(buf.data_ptr(), stream_bytes, blocks, sink.data_ptr(), strm):
            raise SystemExit("stream probe launch failed")

    row_bytes = wl.head_dim * wl.itemsize

    def paged(part, unroll):
        def run():
            if lib.pkv_probe_paged(step.k_pool.data_ptr(), step.v_pool.data_ptr(),
                                   step.tables.data_ptr(), wl.block_tables.shape[1],
                                   step.ctx.data_ptr(), wl.num_seqs, step.max_ctx,
                                   wl.num_kv_heads, row_bytes, wl.block_size, wl.num_blocks,
                                   part, unroll, sink.data_ptr(), strm):
                raise SystemExit("paged probe launch failed")
        return run

    warm_up(stream, 3)
    ms_stream = timed_loop(stream, calls)
    del buf
    kvb = wl.kv_bytes_per_call()
    sweep = {}
    for part in sorted({256, 512, 1024, step.auto_partition}):
        if part % wl.block_size:
            continue
        for unroll in (1, 2, 4):
            fn = paged(part, unroll)
            warm_up(fn, 3)
            sweep[(part, unroll)] = timed_loop(fn, calls)
    at_part = sweep.get((step.auto_partition, 1))
    best = min(sweep, key=sweep.get)
    return {"stream_GBps": round(stream_bytes / (ms_stream * 1e-3) / 1e9, 1),
            "stream_bytes": stream_bytes, "stream_us": round(ms_stream * 1e3, 2),
            "paged_GBps": round(kvb / (sweep[best] * 1e-3) / 1e9, 1),
            "paged_us": round(sweep[best] * 1e3, 2),
            "paged_best": {"partition": best[0], "rows_in_flight": best[1]},
            "paged_at_partition_GBps": round(kvb / (at_part * 1e-3) / 1e9, 1) if at_part else None,
            "paged_partition": step.auto_partition,
            "paged_sweep_us": {f"{p}x{u}": round(v * 1e3, 2) for (p, u), v in sweep.items()},
            "what": "compute-free reads: a contiguous buffer, and the step's K/V rows "
                    "through its block tables (one workgroup per KV head, sequence and "
                    "split; paged_GBps is the best split size and rows in flight)"}


MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 matrix-core peak


def time_prefill(step: Step, calls: int = 10, warmup: int = 10):
    """The workload's chunked-prefill variant on the step's pools: every
    sequence's last ``prefill_chunk`` positions as causal query rows over its
    whole context (pkv_prefill, matrix-core path), back to back between two
    HIP events. Query values are N(0,1) drawn on the device (the timing does
    not depend on them)."""
    wl = step.wl
    n, S = wl.prefill_chunk, wl.num_seqs
    g = torch.Generator(device=DEV).manual_seed(55)
    q = torch.randn((S * n, wl.num_q_heads, wl.head_dim), generator=g,
                    device=DEV).to(step.q.dtype)
    cu = torch.arange(0, S * n + 1, n, dtype=torch.int32, device=DEV)
    out = torch.empty_like(q)

    def call():
        pkv.prefill(q, cu, step.k_pool, step.v_pool, step.tables, step.ctx, wl.scale, n,
                    step.max_ctx, out=out)

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(calls):
        call()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / calls
    # row i of sequence s sits at position ctx - n + i and sees ctx - n + i + 1
    # keys; QK and PV are 2 * hd flops per (query head, visible key) each
    ctx = wl.context_lens.astype(np.int64)
    assert (ctx >= n).all()
    keys = int((n * ctx - n * (n - 1) // 2).sum())
    flops = 4 * wl.head_dim * wl.num_q_heads * keys
    tflops = flops / (ms * 1e-3) / 1e12
    return {"workload": f"{workload_label(wl)}; chunked prefill of the last {n} positions "
                        f"of every sequence ({S * n} query rows)",
            "calls": calls, "ms_per_call": round(ms, 4), "flops_per_call": flops,
            "roofline": {"bound": "mfma", "kernel": "prefill_mfma_kernel",
                         "achieved": round(tflops, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4)}}


def time_bulk_write(wl, calls_per_set: int = 10, sets: int = 4):
    """A bulk KV write at the workload's shape: every sequence stores a
    ``prefill_chunk``-token chunk (``num_seqs * prefill_chunk`` token rows of K
    and V) into blocks of its own, as before a chunked prefill. Calls cycle
    over ``sets`` disjoint sets of source rows and destination blocks, so
    neither side is served from the Infinity Cache of the previous call. Timed
    twice: the write alone (slots computed once per set) and the slot mapping
    followed by the write. Pools are the workload's shape, values random."""
    n, S = wl.prefill_chunk, wl.num_seqs
    T, bs = S * n, wl.block_size
    assert n % bs == 0
    per_seq = n // bs
    need = S * per_seq
    sets = max(1, min(sets, (wl.num_blocks - 1) // need))
    dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    k_pool = torch.zeros(wl.pool_shape, dtype=dt, device=DEV)
    v_pool = torch.zeros_like(k_pool)
    g = torch.Generator(device=DEV).manual_seed(11)
    rng = np.random.default_rng(11)
    perm = rng.permutation(wl.num_blocks - 1) + 1
    cu = torch.arange(0, T + 1, n, dtype=torch.int32, device=DEV)
    first = torch.zeros(S, dtype=torch.int32, device=DEV)
    src, tabs, slots = [], [], []
    for r in range(sets):
        shape = (T, wl.num_kv_heads, wl.head_dim)
        src.append((torch.randn(shape, generator=g, device=DEV).to(dt),
                    torch.randn(shape, generator=g, device=DEV).to(dt)))
        t = to_dev(perm[r * need:(r + 1) * need].reshape(S, per_seq).astype(np.int32))
        tabs.append(t)
        slots.append(pkv.slot_mapping(t, first, cu, T, bs, wl.num_blocks))
    sl_buf = torch.empty(T, dtype=torch.int32, device=DEV)

    turn = [0]

    def run_write():
        r = turn[0] % sets
        turn[0] += 1
        pkv.write(src[r][0], src[r][1], slots[r], k_pool, v_pool)

    def run_both():
        r = turn[0] % sets
        turn[0] += 1
        pkv.slot_mapping(tabs[r], first, cu, T, bs, wl.num_blocks, out=sl_buf)
        pkv.write(src[r][0], src[r][1], sl_buf, k_pool, v_pool)

    calls = calls_per_set * sets
    out = {}
    for name, fn in (("write", run_write), ("slot_mapping_and_write", run_both)):
        warm_up(fn, 2 * sets)
        out[name] = timed_loop(fn, calls)
    isz = k_pool.element_size()
    row = wl.num_kv_heads * wl.head_dim * isz
    # K and V rows are each read once from the new-token buffers and written
    # once into the pool; the write reads one 4-byte slot per token
    nbytes = 4 * T * row + 4 * T
    gbs = nbytes / (out["write"] * 1e-3) / 1e9
    return {"workload": f"{workload_label(wl)}; bulk write of a {n}-token chunk per sequence "
                        f"({T} token rows of K and V, {sets} rotating sets)",
            "calls": calls, "ms_per_call": round(out["write"], 4),
            "ms_per_call_with_slot_mapping": round(out["slot_mapping_and_write"], 4),
            "bytes_per_call": nbytes,
            "roofline": {"bound": "hbm", "kernel": "write_kernel", "achieved": round(gbs, 1),
                         "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs / HBM_PEAK_GBS, 4),
                         "traffic": traffic_from_counters("write")}}


def time_decode_rotating(cfg: int, calls_per_set: int = 10, wl=None):
    """Decode-only timing (partials + merge) cycling over disjoint block sets of
    one pool, so consecutive calls do not hit the Infinity Cache. ``wl``
    replaces configuration ``cfg``'s workload (e.g. one rank's shard of it)."""
    wl = make_workload(cfg) if wl is None else wl
    print(f"[bench] rotating decode timing, {wl.name}", file=sys.stderr, flush=True)
    need = int(sum(-(-int(c) // wl.block_size) for c in wl.context_lens))
    sets = max(1, min(24, (wl.num_blocks - 1) // need))
    dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    g = torch.Generator(device=DEV).manual_seed(7)
    k_pool = torch.randn(wl.pool_shape, generator=g, device=DEV).to(dt)
    v_pool = torch.randn(wl.pool_shape, generator=g, device=DEV).to(dt)
    rng = np.random.default_rng(cfg)
    perm = rng.permutation(wl.num_blocks - 1) + 1
    tables = []
    for r in range(sets):
        ids = perm[r * need:(r + 1) * need]
        t = np.zeros_like(wl.block_tables)
        k = 0
        for s in range(wl.num_seqs):
            n = -(-int(wl.context_lens[s]) // wl.block_size)
            t[s, :n] = ids[k:k + n]
            k += n
        tables.append(to_dev(t))
    q, ctx = to_dev(wl.q), to_dev(wl.context_lens)
    out = torch.empty_like(q)
    max_ctx = int(wl.context_lens.max())
    part = pkv.decode_partition(wl.num_seqs, max_ctx, k_pool)
    schedule = pkv.decode_schedule(wl.num_seqs, wl.num_q_heads, max_ctx, k_pool)
    ws = torch.zeros(max(16, pkv.decode_workspace_bytes(wl.num_seqs, wl.num_q_heads, max_ctx,
                                                        k_pool)),
                     dtype=torch.uint8, device=DEV)

    # one prepared call per block set (arguments checked and marshalled once)
    preps = [pkv.prepare_decode(q, k_pool, v_pool, tb, ctx, wl.scale, max_ctx, out=out,
                                workspace=ws) for tb in tables]

    def call(i):
        preps[i]()

    rot = [0]

    def rotating():
        call(rot[0] % sets)
        rot[0] += 1

    warm_up(rotating, max(sets * 2, 200))
    n = sets * calls_per_set
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    rot[0] = 0
    t0 = time.perf_counter()
    e0.record()
    for r in range(n):
        call(r % sets)
    e1.record()
    host_us = (time.perf_counter() - t0) / n * 1e6
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / n
    eager_out = out.clone()
    # host time per call of the plain binding function (checks and marshalling
    # at every call), for comparison
    t0 = time.perf_counter()
    for r in range(n):
        pkv.decode(q, k_pool, v_pool, tables[r % sets], ctx, wl.scale, max_ctx, out=out,
                   workspace=ws)
    host_plain_us = (time.perf_counter() - t0) / n * 1e6
    torch.cuda.synchronize()
    loops = [ms] + [timed_loop(rotating, n) for _ in range(2)]
    # The same n calls captured in one HIP graph: replays issue no host work
    # per call, so a call shorter than the binding's host time is timed by the
    # GPU alone. Every replay must reproduce the eager bits.
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(0)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for r in range(n):
            call(r % sets)
    for _ in range(3):
        graph.replay()
        torch.cuda.synchronize()
        if not torch.equal(out, eager_out):
            raise SystemExit(f"{wl.name}: graph replay differs from the eager calls")
    reps = 5
    # warm: the same block set back to back (its K/V stay in the Infinity Cache
    # when they fit: cache-assisted)
    e0.record()
    for _ in range(n):
        call(0)
    e1.record()
    torch.cuda.synchronize()
    ms_warm = e0.elapsed_time(e1) / n
    cold = time_cold(lambda: call(0))
    e0.record()
    for _ in range(reps):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    ms_graph = e0.elapsed_time(e1) / (reps * n)
    if not torch.equal(out, eager_out):
        raise SystemExit(f"{wl.name}: graph replay differs from the eager calls")
    kvb = wl.kv_bytes_per_call()
    return {"name": wl.name, "workload": workload_label(wl), "partition": part,
            "schedule": schedule,
            "rotating_sets": sets,
            "us_per_call": round(ms * 1e3, 2), "repeats": repeat_stats(loops), "kv_bytes": kvb,
            "kv_read_GBps": round(kvb / (ms * 1e-3) / 1e9, 1),
            "pct_hbm_peak": round(100 * kvb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 1),
            "seq_steps_per_s": round(wl.num_seqs / (ms * 1e-3), 1),
            "eager_calls": "prepared (pkv.prepare_decode: arguments marshalled once)",
            "host_issue_us_per_call": round(host_us, 2),
            "host_issue_us_per_call_plain_binding": round(host_plain_us, 2),
            "graph_us_per_call": round(ms_graph * 1e3, 2),
            "graph_kv_read_GBps": round(kvb / (ms_graph * 1e-3) / 1e9, 1),
            "graph_pct_hbm_peak": round(100 * kvb / (ms_graph * 1e-3) / 1e9 / HBM_PEAK_GBS, 1),
            "warm_us_per_call_cache_assisted": round(ms_warm * 1e3, 2),
            "cold_us_per_call_percentiles": cold}


SHARED_WORKLOADS = {
    # 30 sequences at the SmolLM2-135M attention shape whose tables start with
    # the same 32-token prompt
    "smollm2-32": lambda: make_workload(2),
    # 30 users of a ~500-token system prompt at the SmolLM2-135M shape: its 31
    # full blocks (496 tokens) shared, own tails of 4 prompt tokens + 8..200
    "smollm2-500": lambda: make_shared([30], [496], ("uniform", 12, 204), dtype="f32",
                                       num_q_heads=9, num_kv_heads=3, head_dim=64, seed=21,
                                       name="smollm2-135m-fp32-500-token-shared-prompt"),
    # 64 sequences of the LLaMA-2-70B layer shape sharing a 4096-token prompt,
    # own tails of 1..4096 tokens
    "llama70b-4096": lambda: make_shared([64], [4096], ("uniform", 1, 4096), dtype="bf16",
                                         num_q_heads=64, num_kv_heads=8, head_dim=128, seed=23,
                                         name="llama-2-70b-layer-bf16-4096-token-shared-prompt"),
}


def time_shared(name: str, calls_per_set: int = 20, partition: int = 0):
    """pkv_decode_shared against pkv_decode on the same inputs. Small workloads
    are replicated over disjoint block sets of one pool (same values), cycled
    so that consecutive calls do not hit the Infinity Cache."""
    wl = SHARED_WORKLOADS[name]()
    dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    row_b = wl.num_kv_heads * wl.head_dim * wl.itemsize * 2          # K + V of one token
    used = int(wl.w_cu[-1]) * row_b
    sets = int(max(1, min(24, -(-(512 << 20) // max(used, 1)))))
    nb1 = wl.num_blocks - 1
    pool = (1 + sets * nb1, wl.block_size, wl.num_kv_heads, wl.head_dim)
    k_pool = torch.zeros(pool, dtype=dt, device=DEV)
    v_pool = torch.zeros(pool, dtype=dt, device=DEV)
    shift = lambda t, r: np.where(t > 0, t + r * nb1, 0).astype(np.int32)
    kr, vr = to_dev(wl.k_rows), to_dev(wl.v_rows)
    n = int(wl.w_cu[-1])
    tables = []
    for r in range(sets):
        slots = pkv.slot_mapping(to_dev(shift(wl.w_tables, r)), to_dev(wl.w_first_pos),
                                 to_dev(wl.w_cu), n, wl.block_size, pool[0])
        pkv.write(kr, vr, slots, k_pool, v_pool)
        tables.append(to_dev(shift(wl.block_tables, r)))
    q, ctx = to_dev(wl.q), to_dev(wl.context_lens)
    max_ctx = int(wl.context_lens.max())
    gs = np.array([g[0] for g in wl.groups] + [wl.num_seqs], np.int32)
    pl = np.array([g[2] for g in wl.groups], np.int32)
    sizes = np.diff(gs)
    tails = [int(wl.context_lens[s]) - min(int(wl.context_lens[s]), int(pl[i]))
             for i in range(len(pl)) for s in range(gs[i], gs[i + 1])]
    max_tail = max(tails)
    out = torch.empty_like(q)
    G, mg, mp = len(pl), int(sizes.max()), int(pl.max())
    ws_s = torch.zeros(max(16, pkv.decode_shared_workspace_bytes(
        wl.num_seqs, wl.num_q_heads, max_ctx, G, mg, mp, max_tail, k_pool, partition)),
        dtype=torch.uint8, device=DEV)
    ws_p = torch.zeros(max(16, pkv.decode_workspace_bytes(wl.num_seqs, wl.num_q_heads, max_ctx,
                                                          k_pool)),
                       dtype=torch.uint8, device=DEV)
    gs_d, pl_d = to_dev(gs), to_dev(pl)

    def shared(tb):
        pkv.decode_shared(q, k_pool, v_pool, tb, ctx, gs_d, pl_d, wl.scale, max_ctx, mg, mp,
                          max_tail_len=max_tail, out=out, partition=partition, workspace=ws_s)

    def plain(tb):
        pkv.decode(q, k_pool, v_pool, tb, ctx, wl.scale, max_ctx, out=out, workspace=ws_p)

    # plain decode with the automatic partition passed explicitly (the piece
    # schedule where the default would take stream-K ranges)
    part = pkv.decode_partition(wl.num_seqs, max_ctx, k_pool)

    def plain_pieces(tb):
        pkv.decode(q, k_pool, v_pool, tb, ctx, wl.scale, max_ctx, out=out, partition=part,
                   workspace=ws_p)

    def timed(fn):
        """(eager ms per call, ms per call replayed from one captured graph);
        the eager figure holds the binding's host time when a call is short.
        Both follow the same minimum-time warm-up as the other legs, so the
        first series timed in the process is not the slow one."""
        rot = [0]

        def rotating():
            fn(tables[rot[0] % sets])
            rot[0] += 1

        warm_up(rotating, 2 * sets)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        calls = sets * calls_per_set
        e0.record()
        for r in range(calls):
            fn(tables[r % sets])
        e1.record()
        torch.cuda.synchronize()
        eager = e0.elapsed_time(e1) / calls
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fn(tables[0])
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for r in range(calls):
                fn(tables[r % sets])
        graph.replay()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(3):
            graph.replay()
        e1.record()
        torch.cuda.synchronize()
        return eager, e0.elapsed_time(e1) / (3 * calls)

    eager_plain, ms_plain = timed(plain)
    schedule = pkv.decode_schedule(wl.num_seqs, wl.num_q_heads, max_ctx, k_pool)
    ms_pieces = timed(plain_pieces)[1] if schedule == "stream_k" else ms_plain
    eager_shared, ms_shared = timed(shared)
    kv_plain = wl.kv_bytes_per_call()                 # every sequence reads its whole context
    kv_unique = (int(pl.sum()) + sum(tails)) * row_b  # each prompt once, each tail once
    return {"workload": f"{wl.name}: {len(pl)} group(s) of {mg} max, prompt {mp} tokens, "
                        f"{wl.num_seqs} seqs, {wl.num_q_heads} q / {wl.num_kv_heads} kv heads, "
                        f"head_dim {wl.head_dim}, block {wl.block_size}, {wl.dtype}",
            "rotating_sets": sets, "total_context_tokens": wl.total_ctx,
            "timing": "graph replay (device time per call); eager_* include the binding's "
                      "host time",
            "plain_us": round(ms_plain * 1e3, 2), "plain_schedule": schedule,
            "plain_pieces_us": round(ms_pieces * 1e3, 2),
            "shared_us": round(ms_shared * 1e3, 2),
            "speedup": round(ms_plain / ms_shared, 3),
            "speedup_vs_faster_plain": round(min(ms_plain, ms_pieces) / ms_shared, 3),
            "eager_plain_us": round(eager_plain * 1e3, 2),
            "eager_shared_us": round(eager_shared * 1e3, 2),
            "plain_kv_bytes": kv_plain, "shared_unique_kv_bytes": kv_unique,
            "plain_GBps": round(kv_plain / (ms_plain * 1e-3) / 1e9, 1),
            "shared_unique_GBps": round(kv_unique / (ms_shared * 1e-3) / 1e9, 1),
            "shared_context_tokens_per_s": round(wl.total_ctx / (ms_shared * 1e-3), 1)}


def time_layer_graph(cfg: int, layers: int = 16, steps: int = 20):
    """A decode step over ``layers`` layers (fused write + decode + merge per
    layer, one layered pool, one table), launched layer by layer against the
    same step replayed from one captured HIP graph. Pool values are N(0,1)
    drawn on the device (the timing does not depend on them)."""
    from paged_kv_cache_scatter_amd.graph import LayerSteps
    wl = make_workload(cfg)
    dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    L, S = layers, wl.num_seqs
    g = torch.Generator(device=DEV).manual_seed(cfg)
    kp = torch.empty((L,) + wl.pool_shape, dtype=dt, device=DEV)
    vp = torch.empty_like(kp)
    for x in (kp, vp):
        for layer in range(L):
            x[layer].normal_(generator=g)
    q = torch.randn((L, S, wl.num_q_heads, wl.head_dim), generator=g, device=DEV).to(dt)
    kn = torch.randn((L, S, wl.num_kv_heads, wl.head_dim), generator=g, device=DEV).to(dt)
    vn = torch.randn((L, S, wl.num_kv_heads, wl.head_dim), generator=g, device=DEV).to(dt)
    st = LayerSteps(q, kn, vn, kp, vp, to_dev(wl.block_tables), to_dev(wl.context_lens),
                    wl.scale, int(wl.context_lens.max()))

    def timed(fn):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    ms_eager = timed(st.run)
    st.capture()
    ms_graph = timed(st.replay)
    kvb = wl.kv_bytes_per_call() * L
    return {"workload": workload_label(wl) + f", {L} layers",
            "schedule": pkv.decode_schedule(S, wl.num_q_heads, int(wl.context_lens.max()),
                                            kp[0], st.partition),
            "launches_per_step": L, "eager_us": round(ms_eager * 1e3, 2),
            "graph_us": round(ms_graph * 1e3, 2), "speedup": round(ms_eager / ms_graph, 3),
            "graph_us_per_layer": round(ms_graph * 1e3 / L, 2),
            "kv_bytes_per_step": kvb, "graph_GBps": round(kvb / (ms_graph * 1e-3) / 1e9, 1)}


# ---------------------------------------------------------------- CPU legs
# The workload the CPU workers decode (set before the pool forks; the workers
# inherit it and never touch the GPU).
_CPU_WL = None


def _compact_pools(wl, s):
    """Sequence s's K/V written through the oracle into a pool of its own blocks
    (renumbered 1..n; the output does not depend on physical block ids)."""
    import oracle  # test infrastructure: only the CPU-baseline leg uses it
    bs = wl.block_size
    L = int(wl.context_lens[s])
    nb = -(-L // bs)
    shape = (nb + 1, bs, wl.num_kv_heads, wl.head_dim)
    kp = np.zeros(shape, wl.storage_np_dtype)
    vp = np.zeros(shape, wl.storage_np_dtype)
    table = np.arange(1, nb + 1, dtype=np.int32)[None]
    slots = oracle.slot_mapping(table, [0], [0, L], bs, nb + 1)
    rows = wl.seq_rows[s]
    kp, vp = oracle.write(kp, vp, wl.k_rows[rows], wl.v_rows[rows], slots)
    return kp, vp, table


def _oracle_worker(args):
    """One CPU worker: sequences w, w + n, ... of the workload through the fp64
    oracle, in passes, until ``budget_s`` of wall time is spent (one BLAS
    thread per worker). Returns (sequences, context tokens, KV bytes, seconds)."""
    import oracle
    from threadpoolctl import threadpool_limits
    w, n, budget_s, start_at = args
    wl = _CPU_WL
    mine = list(range(w, wl.num_seqs, n))
    with threadpool_limits(1):
        prepared = {s: _compact_pools(wl, s) for s in mine}
        while time.time() < start_at:   # every worker starts timing together
            time.sleep(0.001)
        seqs = toks = nbytes = 0
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < budget_s:
            for s in mine:
                kp, vp, table = prepared[s]
                oracle.decode(wl.q[s:s + 1], kp, vp, table, wl.context_lens[s:s + 1], wl.scale,
                              wl.dtype)
                L = int(wl.context_lens[s])
                seqs += 1
                toks += L
                nbytes += L * 2 * wl.num_kv_heads * wl.head_dim * wl.itemsize
                if time.perf_counter() - t0 >= budget_s:
                    break
        return seqs, toks, nbytes, time.perf_counter() - t0


def host_cores() -> int:
    """CPU threads this process may use: its affinity set, at most 16 (the
    share of a multi-GPU host's cores that one GPU's process gets)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, os.cpu_count() or n, 16))


def cpu_oracle_baseline(wl, budget_s: float = 10.0, single_s: float = 4.0):
    """The fp64 oracle on the host, over the sequences of the same workload:
    one worker process per core (forked before this process touches the GPU),
    each decoding its share of the sequences in passes for ``budget_s`` of
    wall time; throughput = all workers' KV bytes / the longest worker's time.
    Also the same on one core for ``single_s`` (``single_thread``)."""
    import multiprocessing as mp
    global _CPU_WL
    _CPU_WL = wl
    cores = min(host_cores(), wl.num_seqs)
    ctx = mp.get_context("fork")
    with ctx.Pool(cores) as pool:
        start_at = time.time() + 3.0 + 0.05 * wl.num_seqs / cores   # after the pools are built
        res = pool.map(_oracle_worker, [(w, cores, budget_s, start_at) for w in range(cores)])
    seqs = sum(r[0] for r in res)
    toks = sum(r[1] for r in res)
    nbytes = sum(r[2] for r in res)
    wall = max(r[3] for r in res)
    one = _oracle_worker((0, 1, single_s, 0.0))
    out = {"value": round(nbytes / wall / 1e9, 4), "unit": "GB/s", "cores": cores,
           "kind": "oracle",
           "sample": f"{seqs} sequence decodes of the same workload (each worker cycling over "
                     f"its share of the {wl.num_seqs} sequences; {toks} context tokens, {nbytes} "
                     f"KV bytes), fp64 numpy oracle, {cores} worker processes with one BLAS "
                     f"thread each, {wall:.1f} s wall",
           "seq_steps_per_s": round(seqs / wall, 3),
           "host_cpu_count": os.cpu_count(),
           "single_thread": {"value": round(one[2] / one[3] / 1e9, 4), "unit": "GB/s",
                             "cores": 1, "sequences": one[0],
                             "seq_steps_per_s": round(one[0] / one[3], 3),
                             "seconds": round(one[3], 2)}}
    _CPU_WL = None
    return out


def cpu_pages_plan_baseline(wl, budget_s: float = 6.0):
    """The pages' own decode plan on the host in torch fp32 on every core:
    each sequence's K/V gathered from one scattered pool through its block
    table into contiguous tensors (cut to its length), then the query heads of
    each KV head's group attend them with a batched matmul, a softmax and a
    second batched matmul. The pool holds the workload's values upcast to
    fp32 (the pages run fp32). Passes over the sequences until ``budget_s``."""
    threads = host_cores()
    prev = torch.get_num_threads()
    torch.set_num_threads(threads)
    try:
        Hkv, hd, bs = wl.num_kv_heads, wl.head_dim, wl.block_size
        rep = wl.num_q_heads // Hkv
        kp = torch.zeros(wl.pool_shape, dtype=torch.float32)
        vp = torch.zeros(wl.pool_shape, dtype=torch.float32)
        kf, vf = kp.view(-1, Hkv, hd), vp.view(-1, Hkv, hd)
        f32 = lambda a: torch.from_numpy(a.view(np.int16).astype(np.int32) << 16).view(
            torch.float32) if wl.dtype == "bf16" else torch.from_numpy(a)
        for s in range(wl.num_seqs):
            L = int(wl.context_lens[s])
            pos = np.arange(L)
            slots = torch.from_numpy(wl.block_tables[s][pos // bs].astype(np.int64) * bs + pos % bs)
            kf[slots] = f32(wl.k_rows[wl.seq_rows[s]])
            vf[slots] = f32(wl.v_rows[wl.seq_rows[s]])
        q = f32(wl.q).view(wl.num_seqs, Hkv, rep, hd)
        tables = torch.from_numpy(wl.block_tables.astype(np.int64))

        def one(s):
            L = int(wl.context_lens[s])
            nb = -(-L // bs)
            K = kp.index_select(0, tables[s, :nb]).view(nb * bs, Hkv, hd)[:L]
            V = vp.index_select(0, tables[s, :nb]).view(nb * bs, Hkv, hd)[:L]
            sc = torch.bmm(q[s], K.permute(1, 2, 0)) * wl.scale         # [Hkv, rep, L]
            return torch.bmm(torch.softmax(sc, dim=-1), V.transpose(0, 1).contiguous())

        one(0)
        seqs = toks = nbytes = 0
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < budget_s:
            for s in range(wl.num_seqs):
                one(s)
                L = int(wl.context_lens[s])
                seqs += 1
                toks += L
                nbytes += L * 2 * Hkv * hd * wl.itemsize
        wall = time.perf_counter() - t0
    finally:
        torch.set_num_threads(prev)
    return {"value": round(nbytes / wall / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "pages_plan_fp32",
            "sample": f"{seqs} sequence decodes ({seqs // max(wl.num_seqs, 1)} passes over the "
                      f"{wl.num_seqs} sequences; {toks} context tokens): table gather into "
                      f"contiguous K/V, then grouped bmm-softmax-bmm, torch fp32 on "
                      f"{threads} threads, {wall:.1f} s; bytes counted at the workload's "
                      f"{wl.dtype} size",
            "seq_steps_per_s": round(seqs / wall, 3)}


TRACE_LIB = os.path.join(ROOT, "paged_kv_cache_scatter_amd", "libpkv_trace.so")
PHASES = ["entry", "piece and context length known", "queries and block ids arrived",
          "first K/V tile in LDS", "tiles done", "partial stored", "stores acknowledged",
          "counted", "end"]


def phase_trace(cfg: int):
    """One launch of the decode (the fused step for the LLaMA-2-70B layer) through the traced
    build (libpkv_trace.so: the same kernels recording the 100 MHz realtime
    counter at each phase boundary of every workgroup; a workgroup that runs
    several pieces keeps the phases of its first and the end of its last, and
    counts them), after warm-up and a
    512 MiB cache-evicting write. Returns per-phase durations over the
    workgroups, the launch's timeline and how many workgroups are alive over
    it. The traced kernel waits for each timestamp, so it runs a little slower
    than the normal build."""
    import ctypes
    from paged_kv_cache_scatter_amd._binding import PoolDesc
    if not os.path.exists(TRACE_LIB):
        raise SystemExit(f"{TRACE_LIB} is not built; run __graft_entry__.build()")
    L = ctypes.CDLL(TRACE_LIB)
    P, I = ctypes.c_void_p, ctypes.c_int32
    L.pkv_decode_step.argtypes = [P, P, P, I, I, P, P, ctypes.POINTER(PoolDesc), P, I, P, I,
                                  ctypes.c_float, I, P, P, ctypes.c_size_t, P]
    L.pkv_decode.argtypes = [P, I, I, P, P, ctypes.POINTER(PoolDesc), P, I, P, I,
                             ctypes.c_float, I, P, P, ctypes.c_size_t, P]
    L.pkv_decode_workspace_bytes.argtypes = [I, I, I, I, ctypes.POINTER(PoolDesc)]
    L.pkv_decode_workspace_bytes.restype = ctypes.c_size_t
    L.pkv_decode_partition.argtypes = [I, I, ctypes.POINTER(PoolDesc)]
    L.pkv_phase_trace_clear.argtypes = [P, ctypes.c_size_t]
    L.pkv_phase_trace_copy.argtypes = [P, ctypes.c_size_t]
    wl = make_workload(cfg)
    st = Step(wl)
    desc = pkv.pool_desc(st.k_pool)
    part = 0   # the library's automatic cut, as the bench's timed calls use
    ws = torch.zeros(max(16, L.pkv_decode_workspace_bytes(wl.num_seqs, wl.num_q_heads,
                                                          st.max_ctx, part, ctypes.byref(desc))),
                     dtype=torch.uint8, device=DEV)
    fused = cfg == 5

    def call():
        strm = torch.cuda.current_stream().cuda_stream
        if fused:
            r = L.pkv_decode_step(st.q.data_ptr(), st.k_step.data_ptr(), st.v_step.data_ptr(),
                                  wl.num_seqs, wl.num_q_heads, st.k_pool.data_ptr(),
                                  st.v_pool.data_ptr(), ctypes.byref(desc), st.tables.data_ptr(),
                                  wl.block_tables.shape[1], st.ctx.data_ptr(), st.max_ctx,
                                  wl.scale, part, st.out.data_ptr(), ws.data_ptr(), ws.numel(),
                                  strm)
        else:
            r = L.pkv_decode(st.q.data_ptr(), wl.num_seqs, wl.num_q_heads, st.k_pool.data_ptr(),
                             st.v_pool.data_ptr(), ctypes.byref(desc), st.tables.data_ptr(),
                             wl.block_tables.shape[1], st.ctx.data_ptr(), st.max_ctx, wl.scale,
                             part, st.out.data_ptr(), ws.data_ptr(), ws.numel(), strm)
        if r:
            raise SystemExit(f"traced call failed with status {r}")

    warm_up(call, 200)
    rows, cols = 1 << 16, 11
    buf = np.zeros((rows, cols), dtype=np.uint64)
    scratch = torch.empty(COLD_FLUSH_BYTES, dtype=torch.uint8, device=DEV)
    scratch.fill_(1)
    torch.cuda.synchronize()
    if L.pkv_phase_trace_clear(buf.ctypes.data, buf.nbytes):
        raise SystemExit("clearing the phase trace failed")
    call()
    torch.cuda.synchronize()
    if L.pkv_phase_trace_copy(buf.ctypes.data, buf.nbytes):
        raise SystemExit("copying the phase trace failed")
    del scratch
    t = buf.astype(np.int64)
    t = t[(t[:, 0] > 0) & (t[:, 8] > 0)]
    us = lambda ticks: ticks / 100.0            # 100 MHz counter
    phases = {}
    for i in range(8):
        a, b = t[:, i], t[:, i + 1]
        ok = (a > 0) & (b > 0)
        d = us(b[ok] - a[ok])
        if ok.any():
            phases[f"{PHASES[i]} -> {PHASES[i + 1]}"] = {
                "workgroups": int(ok.sum()), "mean_us": round(float(d.mean()), 2),
                "p50_us": round(float(np.median(d)), 2),
                "p90_us": round(float(np.percentile(d, 90)), 2)}
    start = us(t[:, 0] - t[:, 0].min())
    end = us(t[:, 8] - t[:, 0].min())
    first = us(t[:, 3] - t[:, 0].min())
    step_us = 2.0 if end.max() < 60 else 5.0
    bins = np.arange(0.0, end.max() + step_us, step_us)
    merged = t[:, 9] == 1
    npieces = t[:, 10]
    one = merged & (npieces <= 1)   # the merge is the last phase of a one-piece workgroup
    counts = {int(k): int((npieces == k).sum()) for k in np.unique(npieces)}
    return {"workload": workload_label(wl), "call": "pkv_decode_step" if fused else "pkv_decode",
            "partition": st.auto_partition, "schedule": st.schedule,
            "workgroups": int(len(t)), "phases": phases,
            "workgroup_total_us": {"mean": round(float((end - start).mean()), 2),
                                   "p50": round(float(np.median(end - start)), 2),
                                   "p90": round(float(np.percentile(end - start, 90)), 2)},
            "last_start_us": round(float(start.max()), 2),
            "last_end_us": round(float(end.max()), 2),
            "first_kv_in_lds_us": {"min": round(float(first.min()), 2),
                                   "p50": round(float(np.median(first)), 2)},
            "pieces_per_workgroup": counts,
            "merging_workgroups": int(merged.sum()),
            "merge_us_mean": round(float(us(t[one, 8] - t[one, 7]).mean()), 2)
            if one.any() else None,
            "alive_bin_us": step_us,
            "alive": [int(((start <= b) & (end > b)).sum()) for b in bins]}


# Counter files under profiles/: the kernel they measure, and the sources
# that decide what its launches read and write (the kernel, the planner or
# launcher that sizes them, and their shared header).
COUNTED = {
    "decode": ("decode_partials_kernel<unsigned short, 128, 8, 0, true>", COUNTERS,
               ("pkv_decode.hip", "pkv_api.hip", "pkv_internal.h")),
    "write": ("write_kernel", WRITE_COUNTERS, ("pkv_write.hip", "pkv_api.hip", "pkv_internal.h")),
}


def counted_sources_sha256(which: str = "decode") -> str:
    h = hashlib.sha256()
    for name in COUNTED[which][2]:
        with open(os.path.join(ROOT, "paged_kv_cache_scatter_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def traffic_from_counters(which: str = "decode"):
    """HBM bytes per launch measured by rocprofv3 counters, if they were taken on
    the current kernel and planner sources; else None."""
    path = COUNTED[which][1]
    if not os.path.exists(path):
        return None
    with open(path) as f:
        c = json.load(f)
    if c.get("sources_sha256") != counted_sources_sha256(which):
        return None
    return c.get("hbm_bytes_per_launch")


def copy_calibration(nbytes: int = 512 << 20, reps: int = 5):
    """A plain device copy of a known size: the reference that rocprofv3's
    FETCH_SIZE / WRITE_SIZE counters are scaled by."""
    src = torch.ones(nbytes // 4, dtype=torch.float32, device=DEV)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": nbytes, "reps": reps}), flush=True)


def _counter_rows(run_dir: str, counter: str):
    """(kernel name, value) of every dispatch in a rocprofv3 --pmc CSV run."""
    import csv
    import glob
    files = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {run_dir}")
    rows = []
    for fn in files:
        with open(fn) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] == counter:
                    rows.append((r["Kernel_Name"], float(r["Counter_Value"])))
    return rows


def summarize_counters(fetch_dir, write_dir, copy_fetch_dir, copy_write_dir, copy_bytes,
                       which: str = "decode"):
    """HBM bytes per launch of a kernel (``which`` names it in COUNTED) from four
    rocprofv3 --pmc runs (FETCH_SIZE and WRITE_SIZE in KiB per dispatch, of the
    kernel and of a plain copy of copy_bytes), each counter scaled by what it
    reads for the copy."""
    kernel_key, out_path, sources = COUNTED[which]
    def mean_of(rows, key):
        v = [x for k, x in rows if key in k]
        if not v:
            raise SystemExit(f"no dispatch of {key!r} in the counter runs")
        return float(np.mean(v)), len(v)
    fk, nf = mean_of(_counter_rows(fetch_dir, "FETCH_SIZE"), kernel_key)
    wk, nw = mean_of(_counter_rows(write_dir, "WRITE_SIZE"), kernel_key)
    cf, _ = mean_of(_counter_rows(copy_fetch_dir, "FETCH_SIZE"), "copy")
    cw, _ = mean_of(_counter_rows(copy_write_dir, "WRITE_SIZE"), "copy")
    sf = copy_bytes / (cf * 1024.0)
    sw = copy_bytes / (cw * 1024.0)
    out = {"kernel": kernel_key,
           "sources": list(sources),
           "sources_sha256": counted_sources_sha256(which),
           "fetch_kib_per_dispatch": round(fk, 1), "write_kib_per_dispatch": round(wk, 1),
           "dispatches": [nf, nw],
           "copy_bytes": copy_bytes, "copy_fetch_kib": round(cf, 1), "copy_write_kib": round(cw, 1),
           "fetch_scale": round(sf, 4), "write_scale": round(sw, 4),
           "hbm_bytes_per_launch": int(round(fk * 1024 * sf + wk * 1024 * sw))}
    with open(out_path, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # about 27 ms of untimed steps: after 10 steps (1.5 ms) the GPU has not
    # reached its steady state (measured: 148 us per step after 10 warm-up
    # steps, 135 us after 200 or 1000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--config", type=int, default=5, choices=sorted(CONFIGS))
    ap.add_argument("--partition", type=int, default=0)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle leg")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the other legs (separate-write step, chunked prefill, the "
                         "Llama-3.2-1B decode shapes)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 512 MiB device copy (counter calibration)")
    ap.add_argument("--summarize-counters", nargs=4, metavar="DIR",
                    help="FETCH_SIZE and WRITE_SIZE run directories of the decode kernel, "
                         "then of the copy calibration: write the traffic file")
    ap.add_argument("--shared", nargs="+", choices=sorted(SHARED_WORKLOADS), metavar="WL",
                    help="only time the shared-prefix decode against plain decode on these "
                         f"workloads ({', '.join(sorted(SHARED_WORKLOADS))})")
    ap.add_argument("--layer-graph", nargs="+", type=int, metavar="CFG",
                    help="only time a 16-layer decode step of these configs, layer by layer "
                         "and replayed from one captured HIP graph")
    ap.add_argument("--phase-trace", nargs="+", type=int, metavar="CFG",
                    help="only per-workgroup phase timings of one decode launch of these "
                         "configs, from the traced build (libpkv_trace.so)")
    ap.add_argument("--counters-of", default="decode", choices=sorted(COUNTED),
                    help="the kernel --summarize-counters measures")
    ap.add_argument("--bulk-write-only", action="store_true",
                    help="only the bulk-write leg (for kernel-trace and counter runs)")
    ap.add_argument("--prefill-only", action="store_true",
                    help="only the chunked-prefill leg, two calls after one warm-up (for "
                         "counter runs)")
    args = ap.parse_args()
    if args.phase_trace:
        pkv.load()
        for cfg in args.phase_trace:
            print(f"[bench] phase trace, {CONFIGS[cfg].name}", file=sys.stderr, flush=True)
            print(json.dumps({"phase_trace": phase_trace(cfg)}), flush=True)
            torch.cuda.empty_cache()
        return
    if args.prefill_only:
        pkv.load()
        step = Step(make_workload(args.config), args.partition)
        print(json.dumps({"prefill": time_prefill(step, calls=2, warmup=1)}), flush=True)
        return
    if args.bulk_write_only:
        pkv.load()
        print(json.dumps({"bulk_write": time_bulk_write(make_workload(args.config))}),
              flush=True)
        return
    if args.layer_graph:
        pkv.load()
        for cfg in args.layer_graph:
            print(f"[bench] 16-layer step, {CONFIGS[cfg].name}", file=sys.stderr, flush=True)
            print(json.dumps({"layer_step_graph": time_layer_graph(cfg)}), flush=True)
            torch.cuda.empty_cache()
        return
    if args.shared:
        pkv.load()
        for name in args.shared:
            print(f"[bench] shared-prefix decode, {name}", file=sys.stderr, flush=True)
            print(json.dumps({"shared_prefix_decode": time_shared(name)}), flush=True)
        return
    if args.summarize_counters:
        summarize_counters(*args.summarize_counters, copy_bytes=512 << 20,
                           which=args.counters_of)
        return
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the path shards by sequence or KV head with no exchange; see the design "
              "notes)", file=sys.stderr)
        sys.exit(2)
    print(f"[bench] generating {CONFIGS[args.config].name}", file=sys.stderr, flush=True)
    wl = make_workload(args.config)
    if wl.prefix_tokens:
        raise SystemExit("the timed step needs a workload without a shared prefix")
    cpu_legs = {}
    if not args.no_cpu:
        # before this process touches the GPU: the oracle's worker processes are forked
        print("[bench] CPU legs: the oracle on every core, the pages' plan in torch fp32",
              file=sys.stderr, flush=True)
        cpu_legs["cpu_baseline"] = cpu_oracle_baseline(wl)
        cpu_legs["cpu_pages_plan_fp32"] = cpu_pages_plan_baseline(wl)
    pkv.load()
    step = Step(wl, args.partition)
    print(f"[bench] timing {args.steps} steps (warmup {args.warmup}, at least "
          f"{MIN_WARMUP_S} s), partition {step.auto_partition}, schedule {step.schedule}",
          file=sys.stderr, flush=True)
    ms_step, ms_bracketed, pct_launch, reps, nwarm = time_steps(step, args.steps, args.warmup)
    cold = time_cold(step.run)
    print("[bench] read-bandwidth probes", file=sys.stderr, flush=True)
    probe = time_probes(step)
    kvb = wl.kv_bytes_per_call()
    gbs = kvb / (ms_step * 1e-3) / 1e9
    # the fused step is one launch of the decode kernel: its mean launch
    # duration is the step time between the events around the timed loop
    ms_kernel = ms_step
    achieved = kvb / (ms_kernel * 1e-3) / 1e9
    traffic = traffic_from_counters()
    res = {
        "metric": "paged decode attention: achieved KV-read GB/s and % HBM peak; seq-steps/s",
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "accumulate": "fp32",
        "data": "synthetic N(0,1) K/V/q at the model's per-layer shape, seeded",
        "config": {"workload": workload_label(wl), "num_seqs": wl.num_seqs,
                   "total_context_tokens": wl.total_ctx, "kv_bytes_per_step": kvb,
                   "partition_tokens": step.auto_partition, "schedule": step.schedule,
                   "step": "pkv_decode_step: slot mapping + KV write of 1 token/seq + split "
                           "decode + merge of the splits, one launch"},
        "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "seq_steps_per_s": round(wl.num_seqs / (ms_step * 1e-3), 1),
        "context_tokens_per_s": round(wl.total_ctx / (ms_step * 1e-3), 1),
        "roofline": {"bound": "hbm",
                     "kernel": f"decode_partials_kernel (fused step, {step.schedule} cut)",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "pct_of_stream_probe": round(achieved / probe["stream_GBps"], 4),
                     "pct_of_paged_probe": round(achieved / probe["paged_GBps"], 4),
                     "kernel_ms": round(ms_kernel, 5),
                     "kernel_ms_events_around_each_launch": round(ms_bracketed, 5),
                     "algorithmic_bytes_per_launch": kvb},
        # spread of the launches timed one by one (events around each), and
        # single launches after a cache-evicting write ("cold")
        "warmup_steps_run": nwarm,
        # the headline loop and two more identical loops (run-to-run spread)
        "repeats": reps,
        "probe": probe,
        "launch_us_percentiles": pct_launch,
        "cold_launch_us_percentiles": cold,
    }
    if not args.no_extra and wl.prefill_chunk and wl.dtype == "bf16":
        print("[bench] chunked prefill", file=sys.stderr, flush=True)
        res["prefill"] = time_prefill(step)
        print("[bench] bulk write of a prefill chunk per sequence", file=sys.stderr, flush=True)
        res["bulk_write"] = time_bulk_write(wl)
    if not args.no_extra:
        del step
        torch.cuda.empty_cache()
        print("[bench] the same step with separate write launches", file=sys.stderr, flush=True)
        sep = Step(wl, args.partition, fused=False)
        ms_sep, ms_sep_k, _, _, _ = time_steps(sep, args.steps, args.warmup, repeats=1)
        res["separate_write_step"] = {
            "step": "pkv_slot_mapping + pkv_write + pkv_decode (split decode and merge, "
                    "one launch)",
            "ms_per_step": round(ms_sep, 5), "value": round(kvb / (ms_sep * 1e-3) / 1e9, 1),
            "unit": "GB/s", "decode_ms_events_around_each_launch": round(ms_sep_k, 5)}
        del sep
        torch.cuda.empty_cache()
        extra = {}
        for cfg in (3, 4):
            if cfg == args.config:
                continue
            r = time_decode_rotating(cfg)
            extra[r.pop("name")] = r
        # one rank's share of the 70B layer with its KV heads over 8 GPUs
        r = time_decode_rotating(5, wl=make_tp_shard(5, 8))
        extra[r.pop("name")] = r
        res["other_workloads_decode_only"] = extra
    res.update(cpu_legs)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
