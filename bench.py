"""Benchmark: paged decode on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-extra]

A step is one pass of the decode hot path over one batch: pa_store_decode
writes the new token's K/V row of every sequence into the pool and attends
over the whole paged context in the same launch (balanced split: equal K/V
ranges per resident wave, then a merge kernel for the sequences the ranges
cut).
The default workload is the bf16 MHA decode batch (64 sequences, 12 heads,
head_dim 64, block 256, context lengths uniform in [512, 4096]). Several
independently drawn batches (each with its own pool) are resident in HBM and
the steps cycle through them, so consecutive steps never find their K/V in the
256 MB last-level cache.

Prints ONE JSON line. `value` is decode tokens/s (sequences x steps / timed
seconds). `roofline` covers the decode call (its main and merge kernels):
algorithmic K+V bytes per launch over its average duration: one pair of HIP
events on the launch stream around the timed run of launches, divided by the
number of launches (an event pair around every launch would add GPU time to
each step). The roofline also gives the device's streaming-read rate measured in the
same run (pa_stream_read, a measurement aid of the library) and the decode
rate as a fraction of it. `cpu_baseline` is the
CPU oracle on a bounded sample of the same workload, single-threaded, and
under `parallel` the same oracle's decode parallel over sequences in a
fork-based pool of up to 16 processes (forked before any GPU call). `extra`
reports the other workloads (GQA decode with shared prefix, GQA decode at 512
sequences, each with the balanced split and with its fixed-slice split, the
three decode workloads over 8-bit E4M3 pools, chunked prefill, and a
continuous batch of decode tokens and prefill chunks in one pa_mixed_batch
call beside the same work as two calls, the last two also over E4M3 pools)
measured the same way.
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


# Untimed calls before each extra decode measurement. The first few dozen
# calls over freshly built large batches run slower than later ones (an E4M3
# batch of 512 sequences: about 420 us per call over the first 30, 364 us
# after), so each leg warms up over this many calls first.
LEG_WARMUP = 40


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


def bench_prefill(steps, warmup, device, kv=None):
    """The chunked-prefill workload: pa_prefill_chunk on bf16 pools, or
    (kv="e4m3") pa_prefill_chunk_fp8 on E4M3 pools with per-head scales."""
    sp = wl.spec(wl.CHUNKED_PREFILL, kv="e4m3") if kv == "e4m3" else wl.spec(wl.CHUNKED_PREFILL)
    b = wl.make_batch(sp, device=device)
    slots = torch.from_numpy(b.slot_mapping).to(device)
    tables = torch.from_numpy(b.block_tables).to(device)
    qsl = torch.from_numpy(b.query_start_loc).to(device)
    lens = torch.from_numpy(b.context_lens).to(device)
    out = torch.empty_like(b.q)
    flops = 0
    for i in range(b.num_seqs):
        n = int(b.query_start_loc[i + 1] - b.query_start_loc[i])
        c = int(b.context_lens[i]) - n
        flops += 4 * b.head_dim * b.num_heads * (n * c + n * (n + 1) // 2)
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


def bench_mixed(steps, warmup, device, kv=None):
    """The continuous batch (decode tokens + prefill chunks): pa_mixed_batch
    against the same work as two calls (pa_decode on the decode tokens, then
    pa_prefill_chunk on the chunks) and against each call alone; with
    kv="e4m3" the same over E4M3 pools (pa_mixed_batch_fp8, pa_decode_fp8,
    pa_prefill_chunk_fp8)."""
    e4 = kv == "e4m3"
    sp = wl.spec(wl.MIXED_BATCH, kv="e4m3") if e4 else wl.spec(wl.MIXED_BATCH)
    b = wl.make_batch(sp, device=device)
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
    flops = 0
    for i in range(Bd, b.num_seqs):
        n = int(b.query_start_loc[i + 1] - b.query_start_loc[i])
        c = int(b.context_lens[i]) - n
        flops += 4 * b.head_dim * b.num_heads * (n * c + n * (n + 1) // 2)
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


def cpu_baseline(ds, budget_s=12.0):
    """The CPU oracle (store + decode, fp64), single-threaded, on whole
    sequences of the first batch until about budget_s seconds have passed."""
    import oracle.attention as oa
    from threadpoolctl import threadpool_limits
    b = ds.batches[0][0]
    hb = wl.host_subset(b)
    done = 0
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < budget_s:
            kp, vp = oa.store_kvcache(hb.k_cache, hb.v_cache, hb.key, hb.value, hb.slot_mapping,
                                      b.block_size)
            for i in range(b.num_seqs):
                oa.decode(hb.q[i:i + 1], kp, vp, hb.block_tables[i:i + 1], hb.context_lens[i:i + 1],
                          b.scale, b.block_size, b.dtype)
                done += 1
                if time.perf_counter() - t0 >= budget_s:
                    break
    secs = time.perf_counter() - t0
    return dict(value=round(done / secs, 2), unit="tokens/s", cores=1, kind="oracle",
                sample=f"{done} sequences of the first batch (mean context "
                       f"{float(b.context_lens.mean()):.0f} tokens), store+decode in fp64, "
                       f"{secs:.1f} s on 1 thread")


_PAR = None  # the host batch the parallel oracle's forked workers inherit


def _par_worker(task):
    """One forked worker: decode sequences w, w+n, ... of the inherited batch
    (wrapping around) until budget_s has passed; returns (sequences, tokens)."""
    import oracle.attention as oa
    from threadpoolctl import threadpool_limits
    w, n, budget_s = task
    hb, kp, vp, scale, bs, dtype = _PAR
    B = len(hb.context_lens)
    done = toks = 0
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        i = w % B
        while time.perf_counter() - t0 < budget_s:
            oa.decode(hb.q[i:i + 1], kp, vp, hb.block_tables[i:i + 1], hb.context_lens[i:i + 1],
                      scale, bs, dtype)
            done += 1
            toks += int(hb.context_lens[i])
            i = (i + n) % B
    return done, toks


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline_parallel(cfg, budget_s=10.0, max_workers=16):
    """The CPU oracle's decode of whole sequences, parallel over sequences in
    a fork-based process pool (at most max_workers, the host share of one
    GPU), on a copy of the workload's first batch built on the host. It runs
    before anything initialises the GPU, so the workers are forks of a
    process that holds no device state. The oracle's store runs once per
    batch, untimed (it copies whole pools)."""
    global _PAR
    import multiprocessing as mp
    import oracle.attention as oa
    b = wl.make_batch(wl.spec(cfg), device="cpu", seed=wl.SEED_BASE + cfg)
    hb = wl.host_subset(b)
    kp, vp = oa.store_kvcache(hb.k_cache, hb.v_cache, hb.key, hb.value, hb.slot_mapping, b.block_size)
    _PAR = (hb, kp, vp, b.scale, b.block_size, b.dtype)
    n = max(1, min(max_workers, os.cpu_count() or 1))
    pool = mp.get_context("fork").Pool(n)
    try:
        t0 = time.perf_counter()
        res = pool.map_async(_par_worker, [(w, n, budget_s) for w in range(n)])
        out = res.get(timeout=budget_s + 120)
        secs = time.perf_counter() - t0
    except mp.TimeoutError:
        pool.terminate()
        return None
    finally:
        pool.close()
        pool.join()
        _PAR = None
    done = sum(d for d, _ in out)
    return dict(value=round(done / secs, 2), unit="tokens/s", cores=n, cpu_model=cpu_model(),
                kind="oracle",
                sample=f"{done} whole-sequence decodes of the first batch (mean context "
                       f"{float(b.context_lens.mean()):.0f} tokens) in fp64, {secs:.1f} s on {n} "
                       f"forked processes, one thread each; the store once per batch, untimed")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100)
    by_name = {wl.WORKLOADS[w]["name"]: w for w in wl.DECODE_WORKLOADS}
    ap.add_argument("--workload", default=wl.WORKLOADS[wl.B64_MHA_DECODE]["name"], choices=sorted(by_name))
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
    # the parallel CPU oracle forks worker processes: before any GPU call
    par = None
    if not args.no_cpu and args.only is None:
        log("cpu baseline, parallel")
        par = cpu_baseline_parallel(by_name[args.workload])
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
            "context_lens": "uniform[512,4096]" if workload == wl.B64_MHA_DECODE else str(ds.spec["lens"]),
            "split": split_name(ds.P), "partition_size": ds.P, "rotating_batches": args.rotations,
            "step": "pa_store_decode: store the new rows + decode, one launch (+ merge)",
        },
        "roofline": {
            "bound": "hbm",
            "kernel": ("pa_decode: paged_decode_balanced_kernel + paged_decode_balanced_merge_kernel"
                       if ds.P == pa.PA_PARTITION_BALANCED else "pa_decode: paged_decode_kernel (+ merge)"),
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
                logical_bytes_per_launch=int(np.mean(d.kv_bytes_logical)))
            del d
            torch.cuda.empty_cache()
        if args.only is None:
            log("extra block manager")
            extra["block_manager"] = bench_block_manager()
            log("extra prefill")
            extra["prefill"] = bench_prefill(20, 10, dev)
            log("extra prefill e4m3")
            extra["prefill_e4m3"] = bench_prefill(20, 10, dev, kv="e4m3")
            log("extra mixed batch")
            extra["mixed_batch"] = bench_mixed(20, 10, dev)
            log("extra mixed batch e4m3")
            extra["mixed_batch_e4m3"] = bench_mixed(20, 10, dev, kv="e4m3")
        line["extra"] = extra
    if args.copy_probe:
        log(f"copy probe {args.copy_probe} bytes")
        copy_probe(args.copy_probe, dev)
    if not args.no_cpu:
        log("cpu baseline")
        line["cpu_baseline"] = cpu_baseline(ds)
        line["cpu_baseline"]["cpu_model"] = cpu_model()
        if par is not None:
            line["cpu_baseline"]["parallel"] = par
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
