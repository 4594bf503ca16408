"""Benchmark: paged decode on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-extra]

A step is one pass of the decode hot path over one batch: pa_store_decode
writes the new token's K/V row of every sequence into the pool and attends
over the whole paged context in the same launch (balanced split: equal K/V
ranges per resident wave, then a merge kernel for the sequences the ranges
cut).
The default workload is the largest decode batch that one GPU holds: 512
sequences of GQA 32/8 heads, head_dim 128, bf16, blocks of 64 tokens,
context lengths lognormal (median 1500, sigma 1) clipped to [64, 4096],
about 4 GB of K/V in a shuffled pool. Several independently drawn batches
(each with its own pool) are resident in HBM and the steps cycle through
them, so consecutive steps never find their K/V in the 256 MB last-level
cache.

Prints ONE JSON line. `value` is decode tokens/s (sequences x steps / timed
seconds). `roofline` covers the decode call (its main and merge kernels):
algorithmic K+V bytes per launch over its average duration: one pair of HIP
events on the launch stream around the timed run of launches, divided by the
number of launches (an event pair around every launch would add GPU time to
each step). The roofline also gives the device's streaming-read rate
measured in the same run (pa_stream_read, a measurement aid of the library)
and the decode rate as a fraction of it. `cpu_baseline` is the CPU oracle's
decode of whole sequences of the same workload (a host-drawn batch of the
same recipe) on one thread, and under `parallel` the same work over
sequences in a fork-based pool of min(host CPUs, 16) processes (forked
before any GPU call). `extra` reports the other workloads measured the same
way (the tiny fp32 decode, the b64 MHA and b256 shared-prefix decodes, each
decode workload with its fixed-slice split, the three decode workloads over
8-bit E4M3 pools, chunked prefill, and a continuous batch of decode tokens
and prefill chunks in one pa_mixed_batch call beside the same work as two
calls, the last two also over E4M3 pools) and, under `cpu_oracle`, the CPU
oracle's rate on a bounded sample of each workload.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from paged_kv_cache_439_amd import binding as pa  # noqa: E402
from paged_kv_cache_439_amd import workloads as wl  # noqa: E402
from paged_kv_cache_439_amd.rocprof_summary import decode_source_hash  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_hbm_traffic.json")
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published


def log(msg):
    print(msg, file=sys.stderr, flush=True)


class DecodeSet:
    """R resident batches of one decode workload, with device-side arrays."""

    def __init__(self, cfg, rotations, device, partition=None, fused=True, kv=None, hint=True):
        self.spec = wl.spec(cfg) if kv is None else wl.spec(cfg, kv=kv)
        self.e4m3 = kv == "e4m3"
        self.fused = fused
        self.hint = hint  # pass shared_lens (the shared-prefix load-policy hint)
        self.P = self.spec.get("partition_size", 0) if partition is None else partition
        self.batches = []
        for r in range(rotations):
            b = wl.make_batch(self.spec, device=device, seed=wl.SEED_BASE + cfg + 1000 * r)
            arrs = dict(slots=torch.from_numpy(b.slot_mapping).to(device),
                        tables=torch.from_numpy(b.block_tables).to(device),
                        lens=torch.from_numpy(b.context_lens).to(device),
                        shared=torch.from_numpy(b.shared_lens).to(device) if hint else None,
                        out=torch.empty_like(b.q))
            self.batches.append((b, arrs))
        b0 = self.batches[0][0]
        maxL = max(b.max_context_len for b, _ in self.batches)
        self.max_context = maxL
        self.ws = pa.decode_workspace(b0.num_seqs, b0.num_heads, b0.num_kv_heads, b0.head_dim,
                                      maxL, self.P, device)
        self.kv_bytes = [b.kv_bytes(unique=True) for b, _ in self.batches]
        self.kv_bytes_logical = [b.kv_bytes(unique=False) for b, _ in self.batches]

    @property
    def separate_store(self):
        return not self.fused

    def step(self, i):
        """Store the new rows and decode: one pa_store_decode call (its main
        kernel writes the rows while it attends; pa_store_decode_fp8 over
        E4M3 pools), or, with a separate store, the store call then the
        decode call."""
        b, a = self.batches[i % len(self.batches)]
        if not self.fused:
            if self.e4m3:
                pa.pa_store_kvcache_fp8(b.key, b.value, b.k_cache, b.v_cache, a["slots"], b.k_scale,
                                        b.v_scale)
            else:
                pa.pa_store_kvcache(b.key, b.value, b.k_cache, b.v_cache, a["slots"])
        self.decode(i)

    def decode(self, i):
        """The decode call of step i (with a fused store, the whole step)."""
        b, a = self.batches[i % len(self.batches)]
        if self.e4m3 and self.fused:
            pa.pa_store_decode_fp8(a["out"], b.q, b.key, b.value, b.k_cache, b.v_cache, b.k_scale,
                                   b.v_scale, a["slots"], a["tables"], a["lens"], b.max_context_len,
                                   b.scale, self.P, self.ws, shared_lens=a["shared"])
        elif self.e4m3:
            pa.pa_decode_fp8(a["out"], b.q, b.k_cache, b.v_cache, b.k_scale, b.v_scale, a["tables"],
                             a["lens"], b.max_context_len, b.scale, self.P, self.ws,
                             shared_lens=a["shared"])
        elif self.fused:
            pa.pa_store_decode(a["out"], b.q, b.key, b.value, b.k_cache, b.v_cache, a["slots"],
                               a["tables"], a["lens"], b.max_context_len, b.scale, self.P, self.ws,
                               shared_lens=a["shared"])
        else:
            pa.pa_decode_hinted(a["out"], b.q, b.k_cache, b.v_cache, a["tables"], a["lens"], a["shared"],
                                b.max_context_len, b.scale, self.P, self.ws)


# Untimed calls before each extra measurement. The first few dozen calls over
# freshly built large batches run slower than later ones (an E4M3 batch of 512
# sequences: about 420 us per call over the first 30, 364 us after), so each
# leg (decode, prefill and mixed alike) warms up over this many calls first.
LEG_WARMUP = 40

# The MFMA-bound legs (chunked prefill, mixed batch) warm up longer: the shader
# clock under them keeps rising for about a hundred back-to-back calls (a bf16
# prefill call: about 198 us over calls 41-80, 182 us after call 100, with the
# same cycle count), and the steady state is what a serving loop sees.
MFMA_LEG_WARMUP = 200


def time_decode(ds, steps, warmup):
    """Returns (seconds for `steps` steps by the host clock, ms per decode
    call, mean bytes per launch).

    The ms per call come from one pair of HIP events on the launch stream
    around the timed run of calls, divided by the number of calls: with a
    fused store the run is the timed steps themselves; with a separate store,
    a second run of the decode calls alone. An event pair around every call
    would add GPU time to every step (about 6 us per step on MI355X at b64)."""
    for i in range(warmup):
        ds.step(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for i in range(steps):
        ds.step(i)
    e1.record()
    torch.cuda.synchronize()
    secs = time.perf_counter() - t0
    if ds.separate_store:
        e0.record()
        for i in range(steps):
            ds.decode(i)
        e1.record()
        torch.cuda.synchronize()
    kms = e0.elapsed_time(e1) / steps
    nbytes = [ds.kv_bytes[i % len(ds.batches)] for i in range(steps)]
    return secs, kms, float(np.mean(nbytes))


def time_run(fn, steps, warmup):
    """ms per call of fn: one pair of HIP events on the launch stream around
    `steps` calls, after `warmup` untimed ones."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def prefill_flops(b, first=0):
    """Algorithmic flops of the chunks of sequences first.. of a batch: each
    visible (query row, key) pair costs one D-long dot product for the logit
    and one D-long multiply-add into the output, 2 * 2 * D flops per query
    head. Row t of a chunk of n over c cached tokens sees c + t + 1 keys."""
    flops = 0
    for i in range(first, b.num_seqs):
        n = int(b.query_start_loc[i + 1] - b.query_start_loc[i])
        c = int(b.context_lens[i]) - n
        flops += 4 * b.head_dim * b.num_heads * (n * c + n * (n + 1) // 2)
    return flops


def bench_prefill(steps, warmup, device, kv=None, oracle_rates=None):
    """The chunked-prefill workload: pa_prefill_chunk on bf16 pools, or
    (kv="e4m3") pa_prefill_chunk_fp8 on E4M3 pools with per-head scales."""
    sp = wl.spec(wl.CHUNKED_PREFILL, kv="e4m3") if kv == "e4m3" else wl.spec(wl.CHUNKED_PREFILL)
    b = wl.make_batch(sp, device=device)
    if oracle_rates is not None:
        oracle_rates[sp["name"]] = oracle_sample_rate(b)
    slots = torch.from_numpy(b.slot_mapping).to(device)
    tables = torch.from_numpy(b.block_tables).to(device)
    qsl = torch.from_numpy(b.query_start_loc).to(device)
    lens = torch.from_numpy(b.context_lens).to(device)
    out = torch.empty_like(b.q)
    flops = prefill_flops(b)
    if kv == "e4m3":
        pa.pa_store_kvcache_fp8(b.key, b.value, b.k_cache, b.v_cache, slots, b.k_scale, b.v_scale)

        def run():
            pa.pa_prefill_chunk_fp8(out, b.q, b.k_cache, b.v_cache, b.k_scale, b.v_scale, tables, qsl,
                                    lens, b.max_query_len, b.max_context_len, b.scale)
    else:
        pa.pa_store_kvcache(b.key, b.value, b.k_cache, b.v_cache, slots)

        def run():
            pa.pa_prefill_chunk(out, b.q, b.k_cache, b.v_cache, tables, qsl, lens, b.max_query_len,
                                b.max_context_len, b.scale)
    ms = time_run(run, steps, warmup)
    tflops = flops / (ms * 1e-3) / 1e12
    return dict(workload=sp["name"], kernel_ms=round(ms, 4), gflop=round(flops / 1e9, 2),
                tflops=round(tflops, 1), frac_of_bf16_mfma_peak=round(tflops / BF16_MFMA_PEAK_TFLOPS, 4),
                tokens_per_s=round(int(b.query_start_loc[-1]) / (ms * 1e-3), 1),
                kv_cache=kv or "bf16")


def bench_mixed(steps, warmup, device, kv=None, oracle_rates=None):
    """The continuous batch (decode tokens + prefill chunks): pa_mixed_batch
    against the same work as two calls (pa_decode on the decode tokens, then
    pa_prefill_chunk on the chunks) and against each call alone; with
    kv="e4m3" the same over E4M3 pools (pa_mixed_batch_fp8, pa_decode_fp8,
    pa_prefill_chunk_fp8)."""
    e4 = kv == "e4m3"
    sp = wl.spec(wl.MIXED_BATCH, kv="e4m3") if e4 else wl.spec(wl.MIXED_BATCH)
    b = wl.make_batch(sp, device=device)
    if oracle_rates is not None:
        oracle_rates[sp["name"]] = oracle_sample_rate(b)
    Bd = b.num_decode
    a = dict(slots=torch.from_numpy(b.slot_mapping).to(device),
             tables=torch.from_numpy(b.block_tables).to(device),
             qsl=torch.from_numpy(b.query_start_loc).to(device),
             lens=torch.from_numpy(b.context_lens).to(device))
    if e4:
        pa.pa_store_kvcache_fp8(b.key, b.value, b.k_cache, b.v_cache, a["slots"], b.k_scale, b.v_scale)
    else:
        pa.pa_store_kvcache(b.key, b.value, b.k_cache, b.v_cache, a["slots"])
    out = torch.empty_like(b.q)
    ws = pa.mixed_workspace(Bd, b.num_heads, b.num_kv_heads, b.head_dim, b.max_context_len, device)
    tab_d, len_d = a["tables"][:Bd].contiguous(), a["lens"][:Bd].contiguous()
    tab_p, qsl_p, len_p = (a["tables"][Bd:].contiguous(), a["qsl"][Bd:].contiguous(),
                           a["lens"][Bd:].contiguous())
    q_d, out_d = b.q[:Bd], out[:Bd]

    def mixed():
        if e4:
            pa.pa_mixed_batch_fp8(out, b.q, b.k_cache, b.v_cache, b.k_scale, b.v_scale, a["tables"],
                                  a["qsl"], a["lens"], Bd, b.max_query_len, b.max_context_len, b.scale,
                                  ws)
        else:
            pa.pa_mixed_batch(out, b.q, b.k_cache, b.v_cache, a["tables"], a["qsl"], a["lens"], Bd,
                              b.max_query_len, b.max_context_len, b.scale, ws)

    def decode_only():
        if e4:
            pa.pa_decode_fp8(out_d, q_d, b.k_cache, b.v_cache, b.k_scale, b.v_scale, tab_d, len_d,
                             b.max_context_len, b.scale, pa.PA_PARTITION_BALANCED, ws)
        else:
            pa.pa_decode(out_d, q_d, b.k_cache, b.v_cache, tab_d, len_d, b.max_context_len, b.scale,
                         pa.PA_PARTITION_BALANCED, ws)

    def prefill_only():
        if e4:
            pa.pa_prefill_chunk_fp8(out, b.q, b.k_cache, b.v_cache, b.k_scale, b.v_scale, tab_p, qsl_p,
                                    len_p, b.max_query_len, b.max_context_len, b.scale)
        else:
            pa.pa_prefill_chunk(out, b.q, b.k_cache, b.v_cache, tab_p, qsl_p, len_p, b.max_query_len,
                                b.max_context_len, b.scale)

    def separate():
        decode_only()
        prefill_only()

    ms = {name: time_run(fn, steps, warmup) for name, fn in (("mixed", mixed), ("separate", separate),
                                           ("decode_only", decode_only), ("prefill_only", prefill_only))}
    rows = int(b.query_start_loc[-1])
    kv_dec = int(sum(int(L) for L in b.context_lens[:Bd])) * b.num_kv_heads * b.head_dim * 2 * (1 if e4 else 2)
    flops = prefill_flops(b, first=Bd)
    return dict(workload=sp["name"], decode_tokens=Bd, prefill_rows=rows - Bd,
                mixed_ms=round(ms["mixed"], 4), separate_ms=round(ms["separate"], 4),
                decode_only_ms=round(ms["decode_only"], 4), prefill_only_ms=round(ms["prefill_only"], 4),
                speedup_vs_separate=round(ms["separate"] / ms["mixed"], 3),
                rows_per_s=round(rows / (ms["mixed"] * 1e-3), 1),
                decode_kv_gb=round(kv_dec / 1e9, 3), prefill_gflop=round(flops / 1e9, 2),
                kv_cache=kv or "bf16")


def measured_traffic(workload_name, split):
    """HBM bytes per decode launch (split "balanced" or "fixed") from the
    committed counter runs, or None when there are none or the decode kernel
    sources changed since."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as fh:
        rec = json.load(fh)
    if rec.get("kernel_source_sha256") != decode_source_hash():
        return None
    w = rec.get("workloads", {}).get(workload_name, {}).get(split)
    if not w:
        return None
    return int(w["hbm_bytes_per_launch"])


def stream_read_probe(dev, nbytes=4 << 30, iters=10):
    """The device's sustained streaming-read rate (GB/s): pa_stream_read over
    a buffer of nbytes, one pair of HIP events on the launch stream around
    iters reads."""
    buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    out = torch.zeros(1, dtype=torch.int32, device=dev)
    for _ in range(3):
        pa.pa_stream_read(buf, out)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(iters):
        n = pa.pa_stream_read(buf, out)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / iters
    del buf
    torch.cuda.empty_cache()
    return n / (ms * 1e-3) / 1e9


def lens_desc(lens):
    """A workload's context-length recipe as text."""
    if lens[0] == "uniform":
        return f"uniform[{lens[1]},{lens[2]}]"
    if lens[0] == "lognormal":
        return f"lognormal(median {lens[1]:g}, sigma {lens[2]:g}) clipped to [{lens[3]},{lens[4]}]"
    return str(list(lens[1]))


def split_name(P):
    return "balanced" if P == pa.PA_PARTITION_BALANCED else "fixed"


def bench_block_manager():
    """Host-side block manager: build the shared-prefix decode workload's
    tables (256 prompts, prefix hashing and sharing), append one decode token
    to each sequence, free everything; the same with the CPU oracle's
    allocator."""
    import oracle.prefix_cache as opc
    st = wl.draw_structure(wl.spec(wl.B256_SHARED_PREFIX_DECODE))
    bs = wl.WORKLOADS[wl.B256_SHARED_PREFIX_DECODE]["block_size"]
    free = st["free_list"].tolist()
    ids = [np.ascontiguousarray(t, dtype=np.int32) for t in st["token_ids"]]
    ntok = int(sum(len(t) for t in ids))

    def run_ours():
        bm = pa.BlockManager(int(st["num_blocks"]), bs, free)
        tables = [bm.allocate(t)[0] for t in ids]
        tables = [bm.append(t, len(ids[i]), 7)[0] for i, t in enumerate(tables)]
        for t in tables:
            bm.free(t)
        bm.close()

    def run_oracle():
        al = opc.PrefixBlockAllocator(free, bs)
        tables = [al.allocate(t.tolist()) for t in ids]
        for i, t in enumerate(tables):
            al.append_token(t, len(ids[i]), 7)
        for t in tables:
            al.free_table(t)
    run_ours()
    t0 = time.perf_counter()
    reps = 5
    for _ in range(reps):
        run_ours()
    ours = (time.perf_counter() - t0) / reps
    t0 = time.perf_counter()
    run_oracle()
    orc = time.perf_counter() - t0
    return dict(workload="bf16_gqa_decode_b256_shared_prefix tables: allocate + 1 append + free",
                prompt_tokens=ntok, ms=round(ours * 1e3, 3), tokens_per_s=round(ntok / ours, 1),
                oracle_ms=round(orc * 1e3, 1), oracle_tokens_per_s=round(ntok / orc, 1))


def copy_probe(nbytes, device, reps=3):
    """A plain device-to-device copy of a known size, for scaling the HBM
    byte counters (FETCH_SIZE / WRITE_SIZE) of a profiling run."""
    x = torch.empty(nbytes, dtype=torch.uint8, device=device)
    y = torch.empty_like(x)
    x.fill_(1)
    for _ in range(reps):
        y.copy_(x)
    torch.cuda.synchronize()
    del x, y


# The host batch the CPU oracle is timed on, built before anything touches
# the GPU (so that the parallel leg's forked workers hold no device state):
# (host copy, stored K pool, stored V pool, scale, block size, dtype).
_PAR = None


def host_oracle_batch(cfg):
    """The workload's first batch drawn on the host, and the oracle's store
    applied to it once (untimed: it copies whole pools)."""
    import oracle.attention as oa
    b = wl.make_batch(wl.spec(cfg), device="cpu", seed=wl.SEED_BASE + cfg)
    hb = wl.host_subset(b)
    kp, vp = oa.store_kvcache(hb.k_cache, hb.v_cache, hb.key, hb.value, hb.slot_mapping, b.block_size)
    return hb, kp, vp, b.scale, b.block_size, b.dtype


def _decode_for(budget_s, first, stride):
    """Oracle decodes of whole sequences first, first + stride, ... of the
    host batch (wrapping around) until budget_s has passed, one thread;
    returns (sequences, context tokens, seconds)."""
    import oracle.attention as oa
    from threadpoolctl import threadpool_limits
    hb, kp, vp, scale, bs, dtype = _PAR
    B = len(hb.context_lens)
    done = toks = 0
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        i = first % B
        while time.perf_counter() - t0 < budget_s:
            oa.decode(hb.q[i:i + 1], kp, vp, hb.block_tables[i:i + 1], hb.context_lens[i:i + 1],
                      scale, bs, dtype)
            done += 1
            toks += int(hb.context_lens[i])
            i = (i + stride) % B
        secs = time.perf_counter() - t0
    return done, toks, secs


def _par_worker(task):
    w, n, budget_s = task
    return _decode_for(budget_s, w, n)


def cpu_model():
    """The host CPU as /proc/cpuinfo names it (model name, family, model,
    stepping), and the logical CPUs the host has."""
    info = {}
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if ":" in line:
                    k, v = (x.strip() for x in line.split(":", 1))
                    info.setdefault(k, v)
    except OSError:
        pass
    name = info.get("model name", "unknown")
    fam = ", ".join(f"{k} {info[k]}" for k in ("cpu family", "model", "stepping") if k in info)
    return f"{name} ({fam})" if fam else name


# The parallel leg's process count: the host share of one GPU on a
# multi-GPU host is 16 CPUs, whatever the host's own count is.
CPU_SHARE = 16


def cpu_baselines(cfg, budget_1=12.0, budget_par=10.0):
    """The CPU oracle's decode of whole sequences of the workload's first
    batch, in fp64: on one thread, and parallel over sequences in a
    fork-based pool of min(host CPUs, CPU_SHARE) processes (one thread each).
    Both time the same work (the decode; the store ran once, untimed). Runs
    before anything initialises the GPU."""
    global _PAR
    import multiprocessing as mp
    _PAR = host_oracle_batch(cfg)
    hb = _PAR[0]
    mean_ctx = float(hb.context_lens.mean())
    model, host_cpus = cpu_model(), os.cpu_count() or 1
    done, toks, secs = _decode_for(budget_1, 0, 1)
    single = dict(value=round(done / secs, 2), unit="tokens/s", cores=1, kind="oracle",
                  cpu_model=model, host_cpus=host_cpus,
                  sample=f"{done} whole-sequence decodes (fp64 attention of the query over its whole "
                         f"context; {toks} context tokens) of the first batch (mean context {mean_ctx:.0f}), "
                         f"{secs:.1f} s on 1 thread; the oracle's store of the batch ran once, untimed")
    n = max(1, min(CPU_SHARE, host_cpus))
    pool = mp.get_context("fork").Pool(n)
    par = None
    try:
        t0 = time.perf_counter()
        res = pool.map_async(_par_worker, [(w, n, budget_par) for w in range(n)])
        out = res.get(timeout=budget_par + 120)
        secs = time.perf_counter() - t0
        done = sum(d for d, _, _ in out)
        toks = sum(t for _, t, _ in out)
        par = dict(value=round(done / secs, 2), unit="tokens/s", cores=n, kind="oracle",
                   cpu_model=model, host_cpus=host_cpus,
                   sample=f"{done} whole-sequence decodes ({toks} context tokens) of the first batch "
                          f"(mean context {mean_ctx:.0f}) in fp64, {secs:.1f} s on {n} forked processes, "
                          f"one thread each ({n} of the host's {host_cpus} CPUs; the host share of one GPU is "
                          f"{CPU_SHARE}); the store once, untimed")
    except mp.TimeoutError:
        pool.terminate()
    finally:
        pool.close()
        pool.join()
        _PAR = None
    return single, par


def oracle_sample_rate(batch, budget_s=3.0, seed=0):
    """The CPU oracle (one thread, fp64) on a bounded sample of a device
    batch: decode workloads, whole sequences in seeded random order
    (tokens/s = sequences per second); prefill and mixed workloads, pieces
    of up to 32 consecutive rows of random chunks (rows per second; a piece
    of rows t0..t1-1 is the chunk's definition restricted to those rows).
    The store of the sampled rows' blocks runs once, untimed."""
    import oracle.attention as oa
    from threadpoolctl import threadpool_limits
    rng = np.random.Generator(np.random.PCG64(seed))
    if batch.kind == "decode":
        seqs = sorted(rng.permutation(batch.num_seqs)[:min(batch.num_seqs, 24)].tolist())
    else:
        seqs = sorted(rng.permutation(batch.num_seqs)[:min(batch.num_seqs, 6)].tolist())
    hb = wl.host_subset(batch, seqs)
    kp, vp = oa.store_kvcache(hb.k_cache, hb.v_cache, hb.key, hb.value, hb.slot_mapping, batch.block_size)
    units = toks = 0
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        k = 0
        while time.perf_counter() - t0 < budget_s:
            r = k % len(seqs)
            k += 1
            if batch.kind == "decode":
                oa.decode(hb.q[r:r + 1], kp, vp, hb.block_tables[r:r + 1], hb.context_lens[r:r + 1],
                          batch.scale, batch.block_size, batch.dtype)
                units += 1
                toks += int(hb.context_lens[r])
            else:
                s0, s1 = int(hb.query_start_loc[r]), int(hb.query_start_loc[r + 1])
                n = s1 - s0
                t0_ = int(rng.integers(0, n))
                t1_ = min(n, t0_ + 32)
                L = int(hb.context_lens[r]) - n + t1_
                oa.prefill(hb.q[s0 + t0_:s0 + t1_], kp, vp, hb.block_tables[r:r + 1],
                           np.array([0, t1_ - t0_], dtype=np.int32), np.array([L], dtype=np.int32),
                           batch.scale, batch.block_size, batch.dtype)
                units += t1_ - t0_
        secs = time.perf_counter() - t0
    what = "sequences" if batch.kind == "decode" else "rows"
    return dict(value=round(units / secs, 2), unit="tokens/s", cores=1, kind="oracle",
                sample=f"{units} {what} of {len(seqs)} sampled sequences"
                       + (f" ({toks} context tokens)" if batch.kind == "decode" else "")
                       + f", {secs:.1f} s on 1 thread")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100)
    by_name = {wl.WORKLOADS[w]["name"]: w for w in wl.DECODE_WORKLOADS}
    ap.add_argument("--workload", default=wl.WORKLOADS[wl.B512_LOGNORMAL_DECODE]["name"], choices=sorted(by_name))
    ap.add_argument("--rotations", type=int, default=4)
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--copy-probe", type=int, default=0,
                    help="also run a device copy of this many bytes (counter calibration)")
    ap.add_argument("--only", choices=["decode", "prefill", "mixed"], default=None,
                    help="profiling runs: one section (decode: the headline and the decode extras; "
                         "prefill / mixed: that extra alone), so that kernels shared by sections "
                         "are not pooled in a profile")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    # the CPU oracle (its parallel leg forks worker processes): before any GPU call
    single = par = None
    if not args.no_cpu and args.only is None:
        log("cpu baseline: oracle on the host, 1 thread and parallel")
        single, par = cpu_baselines(by_name[args.workload])
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    pa.load_library()
    if args.only in ("prefill", "mixed"):
        fn = bench_prefill if args.only == "prefill" else bench_mixed
        log(f"{args.only} only")
        r = fn(max(args.steps, 3), args.warmup, dev)
        r["e4m3"] = fn(max(args.steps, 3), args.warmup, dev, kv="e4m3")
        if args.copy_probe:
            copy_probe(args.copy_probe, dev)
        print(json.dumps({"section": args.only, **r}), flush=True)
        return

    log(f"building workload {args.workload} x{args.rotations}")
    workload = by_name[args.workload]
    ds = DecodeSet(workload, args.rotations, dev)
    b0 = ds.batches[0][0]
    log("timing")
    secs, kms, kbytes = time_decode(ds, args.steps, args.warmup)
    tokens = b0.num_seqs * args.steps
    achieved = kbytes / (kms * 1e-3) / 1e9
    log("stream read probe")
    stream_gbs = stream_read_probe(dev)
    line = {
        "metric": "paged-decode tokens/s + achieved KV GB/s as % of MI355X HBM peak",
        "value": round(tokens / secs, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(secs * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": b0.dtype,
        "data": "synthetic",
        "config": {
            "workload": ds.spec["name"],
            "num_seqs": b0.num_seqs, "num_heads": b0.num_heads, "num_kv_heads": b0.num_kv_heads,
            "head_dim": b0.head_dim, "block_size": b0.block_size,
            "context_lens": lens_desc(ds.spec["lens"]),
            "split": split_name(ds.P), "partition_size": ds.P, "rotating_batches": args.rotations,
            "step": "pa_store_decode: store the new rows + decode, one launch (+ merge)",
        },
        "roofline": {
            "bound": "hbm",
            "kernel": ("pa_store_decode: paged_decode_balanced_kernel + paged_decode_balanced_merge_kernel"
                       if ds.P == pa.PA_PARTITION_BALANCED else "pa_store_decode: paged_decode_kernel (+ merge)"),
            "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(ds.spec["name"], split_name(ds.P)),
            "kernel_ms": round(kms, 4), "bytes_per_launch": int(kbytes),
            # the device's sustained streaming-read rate measured in this run
            # (pa_stream_read), and the decode rate as a fraction of it
            "stream_read_gbs": round(stream_gbs, 1), "frac_of_stream": round(achieved / stream_gbs, 4),
        },
    }
    if not args.no_extra:
        extra = {}
        # the CPU oracle on a bounded sample of every workload (one thread)
        with_oracle = not args.no_cpu and args.only is None
        oracle_rates = {}
        if with_oracle:
            oracle_rates[ds.spec["name"]] = oracle_sample_rate(b0)
        log("extra workload tiny_fp32_mha_decode")
        d = DecodeSet(wl.TINY_FP32_DECODE, 1, dev)
        s_t, ms_t, nb_t = time_decode(d, 200, 50)
        bb = d.batches[0][0]
        extra[bb.spec["name"]] = dict(
            tokens_per_s=round(bb.num_seqs * 200 / s_t, 1), call_ms=round(ms_t, 4),
            kv_gbs=round(nb_t / (ms_t * 1e-3) / 1e9, 2), bytes_per_launch=int(nb_t), split="whole contexts",
            step="pa_store_decode (fp32): store the new rows + decode, one launch",
            note="4 sequences: launch-latency bound, a correctness workload")
        if with_oracle:
            oracle_rates[bb.spec["name"]] = oracle_sample_rate(bb)
        del d
        for cfg in wl.DECODE_WORKLOADS:
            P_bal = wl.WORKLOADS[cfg]["partition_size"]
            runs = [(P_bal, True, True), (wl.WORKLOADS[cfg]["fixed_partition_size"], True, True)]
            if cfg == workload:
                runs.append((ds.P, False, True))
            if cfg == wl.B256_SHARED_PREFIX_DECODE and args.only is None:
                # every block streamed: what the hint gains (left out of the
                # profiling runs, whose per-kernel figures would pool both)
                runs.append((P_bal, True, False))
            for P, fused, hint in runs:
                if cfg == workload and P == ds.P and fused and hint:
                    continue
                log(f"extra workload {wl.WORKLOADS[cfg]['name']} partition_size={P} fused={fused} "
                    f"shared_lens={hint}")
                d = DecodeSet(cfg, 2, dev, partition=P, fused=fused, hint=hint)
                s, ms, nb = time_decode(d, 30, LEG_WARMUP)
                bb = d.batches[0][0]
                if with_oracle and bb.spec["name"] not in oracle_rates:
                    oracle_rates[bb.spec["name"]] = oracle_sample_rate(bb)
                key = d.spec["name"] + ("" if P == pa.PA_PARTITION_BALANCED else f"_fixed_p{P}")
                key += "" if fused else "_separate_store"
                key += "" if hint else "_no_shared_lens"
                extra[key] = dict(
                    tokens_per_s=round(bb.num_seqs * 30 / s, 1), kernel_ms=round(ms, 4),
                    kv_gbs=round(nb / (ms * 1e-3) / 1e9, 1),
                    frac_of_hbm_peak=round(nb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                    frac_of_stream=round(nb / (ms * 1e-3) / 1e9 / stream_gbs, 4),
                    bytes_per_launch=int(nb), split=split_name(P), partition_size=P, fused_store=fused,
                    shared_lens=hint,
                    traffic=measured_traffic(d.spec["name"], split_name(P)) if hint else None,
                    logical_bytes_per_launch=int(np.mean(d.kv_bytes_logical)))
                del d
                torch.cuda.empty_cache()
        for cfg in wl.DECODE_WORKLOADS:
            P = wl.WORKLOADS[cfg]["partition_size"]
            log(f"extra workload {cfg} e4m3 partition_size={P}")
            d = DecodeSet(cfg, 2, dev, partition=P, kv="e4m3", fused=False)
            s, ms, nb = time_decode(d, 30, LEG_WARMUP)
            d.fused = True
            s_f, ms_f, _ = time_decode(d, 30, LEG_WARMUP)
            bb = d.batches[0][0]
            extra[d.spec["name"] + "_e4m3"] = dict(
                tokens_per_s=round(bb.num_seqs * 30 / s, 1), kernel_ms=round(ms, 4),
                kv_gbs=round(nb / (ms * 1e-3) / 1e9, 1),
                frac_of_hbm_peak=round(nb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                frac_of_stream=round(nb / (ms * 1e-3) / 1e9 / stream_gbs, 4),
                bytes_per_launch=int(nb), split=split_name(P), partition_size=P, kv_cache="e4m3",
                step="pa_store_kvcache_fp8 + pa_decode_fp8 (kernel_ms: pa_decode_fp8)",
                fused_step="pa_store_decode_fp8, one launch (+ merge)",
                fused_tokens_per_s=round(bb.num_seqs * 30 / s_f, 1), fused_call_ms=round(ms_f, 4),
                logical_bytes_per_launch=int(np.mean(d.kv_bytes_logical)),
                traffic=measured_traffic(d.spec["name"] + "_e4m3", split_name(P)))
            del d
            torch.cuda.empty_cache()
        if args.only is None:
            log("extra block manager")
            extra["block_manager"] = bench_block_manager()
            log("extra prefill")
            extra["prefill"] = bench_prefill(40, MFMA_LEG_WARMUP, dev, oracle_rates=oracle_rates if with_oracle else None)
            log("extra prefill e4m3")
            extra["prefill_e4m3"] = bench_prefill(40, MFMA_LEG_WARMUP, dev, kv="e4m3")
            log("extra mixed batch")
            extra["mixed_batch"] = bench_mixed(40, MFMA_LEG_WARMUP, dev, oracle_rates=oracle_rates if with_oracle else None)
            log("extra mixed batch e4m3")
            extra["mixed_batch_e4m3"] = bench_mixed(40, MFMA_LEG_WARMUP, dev, kv="e4m3")
        if oracle_rates:
            extra["cpu_oracle"] = oracle_rates
        line["extra"] = extra
    if args.copy_probe:
        log(f"copy probe {args.copy_probe} bytes")
        copy_probe(args.copy_probe, dev)
    if single is not None:
        line["cpu_baseline"] = single
        if par is not None:
            line["cpu_baseline"]["parallel"] = par
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
