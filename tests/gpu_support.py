"""Shared steps of the GPU parity tests: run the HIP path on a batch, run the
oracle on host copies of the same inputs, compare."""

from __future__ import annotations

import math
import sys

import numpy as np
import torch

import oracle.attention as oa
from paged_kv_cache_439_amd import binding as pa
from paged_kv_cache_439_amd import workloads as wl

BF16_MAX_ABS, BF16_MEAN_ABS = 2e-2, 2e-3
F32_MAX_ABS = 1e-5


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def device_arrays(batch):
    dev = batch.k_cache.device
    out = dict(slots=torch.from_numpy(batch.slot_mapping).to(dev),
               tables=torch.from_numpy(batch.block_tables).to(dev),
               lens=torch.from_numpy(batch.context_lens).to(dev))
    if batch.query_start_loc is not None:
        out["qsl"] = torch.from_numpy(batch.query_start_loc).to(dev)
    return out


def gpu_store(batch, arrs=None):
    arrs = arrs or device_arrays(batch)
    pa.pa_store_kvcache(batch.key, batch.value, batch.k_cache, batch.v_cache, arrs["slots"])


def shared_lens_arg(batch, hint):
    """The decode calls' shared_lens: None, the batch's own (hint=True), or a
    given int32 array."""
    if hint is None or hint is False:
        return None
    vals = batch.shared_lens if hint is True else np.asarray(hint, dtype=np.int32)
    return torch.from_numpy(vals).to(batch.q.device)


def gpu_decode(batch, partition_size, arrs=None, workspace=None, hint=None):
    arrs = arrs or device_arrays(batch)
    dev = batch.q.device
    if workspace is None:
        workspace = pa.decode_workspace(batch.num_seqs, batch.num_heads, batch.num_kv_heads,
                                        batch.head_dim, batch.max_context_len, partition_size, dev)
    out = torch.full_like(batch.q, float("nan"))
    sl = shared_lens_arg(batch, hint)
    if sl is None:  # the plain call
        pa.pa_decode(out, batch.q, batch.k_cache, batch.v_cache, arrs["tables"], arrs["lens"],
                     batch.max_context_len, batch.scale, partition_size, workspace)
    else:
        pa.pa_decode_hinted(out, batch.q, batch.k_cache, batch.v_cache, arrs["tables"], arrs["lens"], sl,
                            batch.max_context_len, batch.scale, partition_size, workspace)
    return out


def gpu_store_decode(batch, partition_size, arrs=None, workspace=None, hint=None):
    """The fused store + decode call."""
    arrs = arrs or device_arrays(batch)
    dev = batch.q.device
    if workspace is None:
        workspace = pa.decode_workspace(batch.num_seqs, batch.num_heads, batch.num_kv_heads,
                                        batch.head_dim, batch.max_context_len, partition_size, dev)
    out = torch.full_like(batch.q, float("nan"))
    pa.pa_store_decode(out, batch.q, batch.key, batch.value, batch.k_cache, batch.v_cache, arrs["slots"],
                       arrs["tables"], arrs["lens"], batch.max_context_len, batch.scale, partition_size,
                       workspace, shared_lens=shared_lens_arg(batch, hint))
    return out


def gpu_prefill(batch, arrs=None):
    arrs = arrs or device_arrays(batch)
    out = torch.full_like(batch.q, float("nan"))
    pa.pa_prefill_chunk(out, batch.q, batch.k_cache, batch.v_cache, arrs["tables"], arrs["qsl"],
                        arrs["lens"], batch.max_query_len, batch.max_context_len, batch.scale)
    return out


def as_f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def oracle_inputs(batch, seqs=None):
    """Host copy of the pre-store inputs, with the oracle's own store applied."""
    hb = wl.host_subset(batch, seqs)
    kp, vp = oa.store_kvcache(hb.k_cache, hb.v_cache, hb.key, hb.value, hb.slot_mapping,
                              batch.block_size)
    return hb, kp, vp


def check_close(got, ref, dtype, what):
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = np.abs(got - ref)
    if dtype == "f32":
        assert err.max() <= F32_MAX_ABS, f"{what}: max abs {err.max():.3g}"
    else:
        assert err.max() <= BF16_MAX_ABS and err.mean() <= BF16_MEAN_ABS, \
            f"{what}: max abs {err.max():.3g} mean abs {err.mean():.3g}"
    return float(err.max()), float(err.mean())


def decode_parity(batch, partition_size, seqs=None, heads=None, hint=None):
    """Store + decode on the GPU; oracle on the host copies taken before."""
    hb, kp, vp = oracle_inputs(batch, seqs)
    arrs = device_arrays(batch)
    gpu_store(batch, arrs)
    out = gpu_decode(batch, partition_size, arrs, hint=hint)
    torch.cuda.synchronize()
    got = as_f64(out)
    if seqs is None:
        ref = oa.decode(hb.q, kp, vp, hb.block_tables, hb.context_lens, batch.scale,
                        batch.block_size, batch.dtype)
        return check_close(got, ref, batch.dtype, "decode")
    heads = heads if heads is not None else range(batch.num_heads)
    rows = [(r, h) for r in range(len(seqs)) for h in heads]
    ref = oa.decode_rows(hb.q, kp, vp, hb.block_tables, hb.context_lens, batch.scale,
                         batch.block_size, batch.dtype, rows)
    sel = np.stack([got[seqs[r], h] for r, h in rows])
    return check_close(sel, ref, batch.dtype, "decode (sampled)")


def store_decode_parity(batch, partition_size):
    """Fused store + decode on the GPU against the oracle's store followed by
    its decode; the pools must also equal the oracle's stored pools byte for
    byte."""
    hb, kp, vp = oracle_inputs(batch)
    arrs = device_arrays(batch)
    out = gpu_store_decode(batch, partition_size, arrs)
    torch.cuda.synchronize()
    ref = oa.decode(hb.q, kp, vp, hb.block_tables, hb.context_lens, batch.scale, batch.block_size,
                    batch.dtype)
    res = check_close(as_f64(out), ref, batch.dtype, "store+decode")
    ek, ev = oa.store_kvcache(wl_full_pool(batch, "k"), wl_full_pool(batch, "v"), wl.to_numpy(batch.key),
                              wl.to_numpy(batch.value), batch.slot_mapping, batch.block_size)
    return res, ek, ev


def wl_full_pool(batch, which):
    """Host copy of a whole pool as it was before the call under test (kept
    on the batch by snapshot_pools)."""
    return batch._pool_snapshot[which]


def snapshot_pools(batch):
    batch._pool_snapshot = dict(k=wl.to_numpy(batch.k_cache), v=wl.to_numpy(batch.v_cache))
    return batch


def gpu_mixed(batch, arrs=None, workspace=None, hint=None):
    """pa_mixed_batch over the batch (its first num_decode sequences decode)."""
    arrs = arrs or device_arrays(batch)
    if workspace is None:
        workspace = pa.mixed_workspace(batch.num_decode, batch.num_heads, batch.num_kv_heads,
                                       batch.head_dim, batch.max_context_len, batch.q.device)
    out = torch.full_like(batch.q, float("nan"))
    pa.pa_mixed_batch(out, batch.q, batch.k_cache, batch.v_cache, arrs["tables"], arrs["qsl"],
                      arrs["lens"], batch.num_decode, batch.max_query_len, batch.max_context_len,
                      batch.scale, workspace, shared_lens=shared_lens_arg(batch, hint))
    return out


def prefill_parity(batch, sample_rows=None, seed=0, runner=None):
    """Store + varlen attention on the GPU (pa_prefill_chunk, or runner)
    against the oracle's store and prefill."""
    hb, kp, vp = oracle_inputs(batch)
    arrs = device_arrays(batch)
    gpu_store(batch, arrs)
    out = (runner or gpu_prefill)(batch, arrs)
    torch.cuda.synchronize()
    got = as_f64(out)
    if sample_rows is None:
        ref = oa.prefill(hb.q, kp, vp, hb.block_tables, hb.query_start_loc, hb.context_lens,
                         batch.scale, batch.block_size, batch.dtype)
        return check_close(got, ref, batch.dtype, "prefill")
    rng = np.random.Generator(np.random.PCG64(seed))
    T = got.shape[0]
    toks = rng.choice(T, size=sample_rows, replace=False)
    # always include each sequence's first and last rows
    qsl = batch.query_start_loc
    edge = [int(qsl[i]) for i in range(batch.num_seqs)] + [int(qsl[i + 1]) - 1 for i in range(batch.num_seqs)]
    toks = sorted(set(toks.tolist()) | set(edge))
    heads = rng.integers(0, batch.num_heads, size=len(toks))
    rows = list(zip(toks, heads.tolist()))
    ref = oa.prefill_rows(hb.q, kp, vp, hb.block_tables, hb.query_start_loc, hb.context_lens,
                          batch.scale, batch.block_size, batch.dtype, rows)
    sel = np.stack([got[t, h] for t, h in rows])
    return check_close(sel, ref, batch.dtype, "prefill (sampled)")


def sample_seqs(batch, k, seed=0):
    """k sequences: the shortest, the longest, and a seeded random rest."""
    rng = np.random.Generator(np.random.PCG64(seed))
    lens = batch.context_lens
    pick = {int(np.argmin(lens)), int(np.argmax(lens))}
    rest = [i for i in rng.permutation(batch.num_seqs).tolist() if i not in pick]
    return sorted(pick | set(rest[:max(0, k - len(pick))]))


def full_config_parts(cfg, split="balanced"):
    """The decode split the benchmark times for a workload: its balanced
    split, or the fixed one measured beside it."""
    key = "partition_size" if split == "balanced" else "fixed_partition_size"
    return wl.WORKLOADS[cfg].get(key, 0)


# ---------------------------------------------------------------------------
# E4M3 pools
# ---------------------------------------------------------------------------

def gpu_store_fp8(batch, arrs=None):
    arrs = arrs or device_arrays(batch)
    pa.pa_store_kvcache_fp8(batch.key, batch.value, batch.k_cache, batch.v_cache, arrs["slots"],
                            batch.k_scale, batch.v_scale)


def gpu_decode_fp8(batch, partition_size, arrs=None, workspace=None, hint=None):
    arrs = arrs or device_arrays(batch)
    dev = batch.q.device
    if workspace is None:
        workspace = pa.decode_workspace(batch.num_seqs, batch.num_heads, batch.num_kv_heads,
                                        batch.head_dim, batch.max_context_len, partition_size, dev)
    out = torch.full_like(batch.q, float("nan"))
    pa.pa_decode_fp8(out, batch.q, batch.k_cache, batch.v_cache, batch.k_scale, batch.v_scale,
                     arrs["tables"], arrs["lens"], batch.max_context_len, batch.scale, partition_size,
                     workspace, shared_lens=shared_lens_arg(batch, hint))
    return out


def scales_np(batch):
    return batch.k_scale.cpu().numpy().astype(np.float64), batch.v_scale.cpu().numpy().astype(np.float64)


def decode_fp8_parity(batch, partition_size, seqs=None, hint=None):
    """E4M3 store + decode on the GPU; the oracle's E4M3 store and decode on
    host copies of the same inputs (all sequences, or the given subset)."""
    import oracle.fp8 as of8
    hb = wl.host_subset(batch, seqs)
    ks, vs = scales_np(batch)
    kp, vp = of8.store_kvcache_fp8(hb.k_cache, hb.v_cache, hb.key, hb.value, hb.slot_mapping,
                                   batch.block_size, ks, vs, batch.dtype)
    arrs = device_arrays(batch)
    gpu_store_fp8(batch, arrs)
    out = gpu_decode_fp8(batch, partition_size, arrs, hint=hint)
    torch.cuda.synchronize()
    got = as_f64(out)
    ref = of8.decode_fp8(hb.q, kp, vp, ks, vs, hb.block_tables, hb.context_lens, batch.scale,
                         batch.block_size, batch.dtype)
    if seqs is not None:
        got = got[np.asarray(seqs)]
    return check_close(got, ref, batch.dtype, "decode e4m3")


def gpu_prefill_fp8(batch, arrs=None):
    arrs = arrs or device_arrays(batch)
    out = torch.full_like(batch.q, float("nan"))
    pa.pa_prefill_chunk_fp8(out, batch.q, batch.k_cache, batch.v_cache, batch.k_scale, batch.v_scale,
                            arrs["tables"], arrs["qsl"], arrs["lens"], batch.max_query_len,
                            batch.max_context_len, batch.scale)
    return out


def sample_prefill_rows(batch, total_rows, sample_rows, seed):
    """sample_rows random (row, head) pairs plus every sequence's first and
    last row (each with a random head)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    toks = rng.choice(total_rows, size=sample_rows, replace=False)
    qsl = batch.query_start_loc
    edge = [int(qsl[i]) for i in range(batch.num_seqs)] + [int(qsl[i + 1]) - 1 for i in range(batch.num_seqs)]
    toks = sorted(set(toks.tolist()) | set(edge))
    heads = rng.integers(0, batch.num_heads, size=len(toks))
    return list(zip(toks, heads.tolist()))


def gpu_mixed_fp8(batch, arrs=None, workspace=None, hint=None):
    """pa_mixed_batch_fp8 over the batch (its first num_decode sequences decode)."""
    arrs = arrs or device_arrays(batch)
    if workspace is None:
        workspace = pa.mixed_workspace(batch.num_decode, batch.num_heads, batch.num_kv_heads,
                                       batch.head_dim, batch.max_context_len, batch.q.device)
    out = torch.full_like(batch.q, float("nan"))
    pa.pa_mixed_batch_fp8(out, batch.q, batch.k_cache, batch.v_cache, batch.k_scale, batch.v_scale,
                          arrs["tables"], arrs["qsl"], arrs["lens"], batch.num_decode,
                          batch.max_query_len, batch.max_context_len, batch.scale, workspace,
                          shared_lens=shared_lens_arg(batch, hint))
    return out


def prefill_fp8_parity(batch, sample_rows=None, seed=0, runner=None):
    """E4M3 store + chunked prefill (pa_prefill_chunk_fp8, or runner) on the
    GPU against the oracle's E4M3 store and prefill on host copies of the
    same inputs (every row, or a sample)."""
    import oracle.fp8 as of8
    hb = wl.host_subset(batch)
    ks, vs = scales_np(batch)
    kp, vp = of8.store_kvcache_fp8(hb.k_cache, hb.v_cache, hb.key, hb.value, hb.slot_mapping,
                                   batch.block_size, ks, vs, batch.dtype)
    arrs = device_arrays(batch)
    gpu_store_fp8(batch, arrs)
    out = (runner or gpu_prefill_fp8)(batch, arrs)
    torch.cuda.synchronize()
    got = as_f64(out)
    rows = None if sample_rows is None else sample_prefill_rows(batch, got.shape[0], sample_rows, seed)
    ref = of8.prefill_fp8(hb.q, kp, vp, ks, vs, hb.block_tables, hb.query_start_loc, hb.context_lens,
                          batch.scale, batch.block_size, batch.dtype, rows=rows)
    if rows is not None:
        got = np.stack([got[t, h] for t, h in rows])
    return check_close(got, ref, batch.dtype, "prefill e4m3" + ("" if rows is None else " (sampled)"))


def gpu_store_decode_fp8(batch, partition_size, arrs=None, workspace=None):
    """The fused E4M3 store + decode call."""
    arrs = arrs or device_arrays(batch)
    dev = batch.q.device
    if workspace is None:
        workspace = pa.decode_workspace(batch.num_seqs, batch.num_heads, batch.num_kv_heads,
                                        batch.head_dim, batch.max_context_len, partition_size, dev)
    out = torch.full_like(batch.q, float("nan"))
    pa.pa_store_decode_fp8(out, batch.q, batch.key, batch.value, batch.k_cache, batch.v_cache,
                           batch.k_scale, batch.v_scale, arrs["slots"], arrs["tables"], arrs["lens"],
                           batch.max_context_len, batch.scale, partition_size, workspace)
    return out


def store_decode_fp8_parity(batch, partition_size):
    """Fused E4M3 store + decode on the GPU against the oracle's E4M3 store
    followed by its E4M3 decode; returns the oracle's stored pools (whole
    pools, from the snapshot taken before the call) for a byte comparison."""
    import oracle.fp8 as of8
    hb = wl.host_subset(batch)
    ks, vs = scales_np(batch)
    kp, vp = of8.store_kvcache_fp8(hb.k_cache, hb.v_cache, hb.key, hb.value, hb.slot_mapping,
                                   batch.block_size, ks, vs, batch.dtype)
    arrs = device_arrays(batch)
    out = gpu_store_decode_fp8(batch, partition_size, arrs)
    torch.cuda.synchronize()
    ref = of8.decode_fp8(hb.q, kp, vp, ks, vs, hb.block_tables, hb.context_lens, batch.scale,
                         batch.block_size, batch.dtype)
    res = check_close(as_f64(out), ref, batch.dtype, "store+decode e4m3")
    ek, ev = of8.store_kvcache_fp8(wl_full_pool(batch, "k"), wl_full_pool(batch, "v"),
                                   wl.to_numpy(batch.key), wl.to_numpy(batch.value), batch.slot_mapping,
                                   batch.block_size, ks, vs, batch.dtype)
    return res, ek, ev


# ---------------------------------------------------------------------------
# the oracle over whole full-size batches
# ---------------------------------------------------------------------------
#
# Sequences are independent, and row t of a prefill chunk over c cached
# tokens depends only on keys 0 .. c+t, so the oracle's own functions are
# applied to groups of sequences (decode) or to pieces of a chunk's rows
# (prefill: rows t0..t1-1 form a chunk of t1-t0 rows over a context of
# c+t1 tokens) in a few host threads, and the pieces are put back in place.
# Nothing of the arithmetic changes: each output row is the oracle's.

ORACLE_THREADS = 4


def oracle_decode_all(hb, kp, vp, scale, block_size, dtype, fp8_scales=None, threads=ORACLE_THREADS):
    """oracle decode (oa.decode, or of8.decode_fp8 with fp8_scales=(ks, vs))
    of every sequence of the host batch hb over the stored pools kp/vp."""
    from concurrent.futures import ThreadPoolExecutor

    from threadpoolctl import threadpool_limits
    import oracle.fp8 as of8
    B = hb.q.shape[0]
    groups = [np.arange(k, B, 4 * threads) for k in range(min(B, 4 * threads))]

    def run(idx):
        if fp8_scales is None:
            return idx, oa.decode(hb.q[idx], kp, vp, hb.block_tables[idx], hb.context_lens[idx], scale,
                                  block_size, dtype)
        ks, vs = fp8_scales
        return idx, of8.decode_fp8(hb.q[idx], kp, vp, ks, vs, hb.block_tables[idx], hb.context_lens[idx],
                                   scale, block_size, dtype)

    out = np.zeros(hb.q.shape, dtype=np.float64)
    with threadpool_limits(limits=1), ThreadPoolExecutor(threads) as ex:
        for idx, res in ex.map(run, groups):
            out[idx] = res
    return out


def oracle_prefill_all(hb, kp, vp, scale, block_size, dtype, fp8_scales=None, threads=ORACLE_THREADS,
                       piece=128):
    """oracle varlen prefill (oa.prefill, or of8.prefill_fp8) of every row
    of the host batch hb, in pieces of at most `piece` rows per chunk."""
    from concurrent.futures import ThreadPoolExecutor

    from threadpoolctl import threadpool_limits
    import oracle.fp8 as of8
    qsl, lens = hb.query_start_loc, hb.context_lens
    tasks = []
    for i in range(len(lens)):
        s, e = int(qsl[i]), int(qsl[i + 1])
        c = int(lens[i]) - (e - s)
        for t0 in range(0, e - s, piece):
            t1 = min(e - s, t0 + piece)
            tasks.append((i, s + t0, s + t1, c + t1))
    tasks.sort(key=lambda t: -(t[3] * (t[2] - t[1])))   # longest first

    def run(task):
        i, r0, r1, L = task
        qs = np.array([0, r1 - r0], dtype=np.int32)
        ls = np.array([L], dtype=np.int32)
        if fp8_scales is None:
            res = oa.prefill(hb.q[r0:r1], kp, vp, hb.block_tables[i:i + 1], qs, ls, scale, block_size, dtype)
        else:
            ks, vs = fp8_scales
            res = of8.prefill_fp8(hb.q[r0:r1], kp, vp, ks, vs, hb.block_tables[i:i + 1], qs, ls, scale,
                                  block_size, dtype)
        return r0, r1, res

    out = np.zeros(hb.q.shape, dtype=np.float64)
    with threadpool_limits(limits=1), ThreadPoolExecutor(threads) as ex:
        for r0, r1, res in ex.map(run, tasks):
            out[r0:r1] = res
    return out


def check_pool_after_store(before_k, before_v, batch, kp, vp, hb):
    """The pools after a (fused) store: the rows every context covers equal
    the oracle's stored pools kp/vp byte for byte (host_subset renumbers the
    covered blocks in the same order for both), and no other byte of either
    pool changed (before_k/before_v: device copies taken before the call)."""
    after = wl.host_subset(batch)
    assert np.array_equal(after.k_cache, kp) and np.array_equal(after.v_cache, vp), "stored rows differ"
    covered = torch.from_numpy(wl.covered_rows(batch)).to(batch.k_cache.device)
    for name, pb, pa_ in (("k", before_k, batch.k_cache), ("v", before_v, batch.v_cache)):
        bits = torch.int16 if pa_.element_size() == 2 else torch.int32 if pa_.element_size() == 4 else torch.uint8
        untouched = torch.equal(pa_.view(bits)[~covered], pb.view(bits)[~covered])
        assert untouched, f"{name} pool changed outside the contexts"
