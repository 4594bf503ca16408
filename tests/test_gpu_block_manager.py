"""The library's block manager drives the kernels end to end.

pa_bm_allocate hands out block tables, cached-token counts and slots for a
set of prompts, several of which share a common prefix (the nano-vllm page,
§3.2.2: full blocks found by their rolling hash are reused with one more
reference; §4.2: the hash chains block by block); the new tokens' K/V rows
are stored through those slots and pa_prefill_chunk attends over
num_cached_tokens + the chunk; then several decode steps each append one
token per sequence with pa_bm_append (a new block when the last one is
full) and run pa_store_decode with pa_bm_shared_tokens as the shared_lens
hint; finally every sequence is freed (the mini-vllm page's BlockAllocator,
architecture item 1: blocks for prefill and decode, freed when a request
completes).

The oracle side runs the oracle's allocator on the same token ids and free
list (tables, cached counts and slots must agree exactly), its store into a
host copy of the pool, and its attention. The K/V row of a prompt token
depends on the token ids up to it (as a model's would), so sequences with
the same prefix have the same prefix rows, and the rows a sharer skips
(its cached tokens) are the rows the first sharer stored.

Bars: pools byte-equal to the oracle's stores after the prefill and after
every decode step; attention outputs within the bf16 bars of the oracle.
"""

import math

import numpy as np
import pytest
import torch

import oracle.attention as oa
import oracle.prefix_cache as opc
from paged_kv_cache_439_amd import binding as pa
from paged_kv_cache_439_amd import workloads as wl
from tests import gpu_support as gs

pytestmark = pytest.mark.gpu

HQ, HKV, D, BS, NB = 16, 8, 128, 32, 480
STEPS = 40   # decode steps
VOCAB = 50257


def _bf16_bits(x):
    """numpy float32 -> uint16 bf16 bits (round to nearest even)."""
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16) \
        .view(torch.int16).numpy().view(np.uint16)


def _prefix_rows(token_ids, seed):
    """K and V rows [n][Hkv][D] (bf16 bits) of a prompt, row p a seeded
    function of token_ids[0..p] (its rolling prefix digest)."""
    k = np.empty((len(token_ids), HKV, D), dtype=np.uint16)
    v = np.empty_like(k)
    h = 0
    for p, t in enumerate(token_ids):
        h = (h * 1000003 + int(t) + 1) % (1 << 61)
        r = np.random.Generator(np.random.PCG64([seed, h]))
        k[p] = _bf16_bits(r.standard_normal((HKV, D)))
        v[p] = _bf16_bits(r.standard_normal((HKV, D)))
    return k, v


def _to_dev(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def _as_bf16(bits, dev):
    return _to_dev(bits.view(np.int16), dev).view(torch.bfloat16)


def _tables(tabs, max_blocks):
    out = np.full((len(tabs), max_blocks), -1, dtype=np.int32)
    for i, t in enumerate(tabs):
        out[i, :len(t)] = t
    return out


def test_block_manager_tables_drive_prefill_and_decode(gpu):
    rng = np.random.Generator(np.random.PCG64(4390))
    free = rng.permutation(NB).tolist()
    bm = pa.BlockManager(NB, BS, free)
    al = opc.PrefixBlockAllocator(free, BS)
    # 12 prompts: 6 share a 96-token prefix (3 full blocks), one of them
    # exactly the prefix plus one token; two share a 64-token prefix
    # with each other; lengths cross block edges
    common = rng.integers(0, VOCAB, size=96).tolist()
    second = rng.integers(0, VOCAB, size=64).tolist()
    prompts = []
    for i in range(12):
        n = int(rng.integers(40, 300))
        own = rng.integers(0, VOCAB, size=n).tolist()
        if i in (0, 2, 3, 6, 9, 11):
            own = common + (own if i != 6 else own[:1])
        elif i in (4, 7):
            own = second + own
        prompts.append(own)
    tabs, cached, slots = [], [], []
    for toks in prompts:
        t, c, s = bm.allocate(np.asarray(toks, dtype=np.int32), with_slots=True)
        t_ref, c_ref = al.allocate_cached(toks)
        assert t.tolist() == t_ref and c == c_ref
        assert s.tolist() == [t_ref[p // BS] * BS + p % BS for p in range(len(toks))]
        tabs.append(t.tolist())
        cached.append(c)
        slots.append(s)
    assert cached.count(96) == 5 and cached.count(64) == 1, cached
    gs.say(f"block manager: prompts {[len(p) for p in prompts]} cached {cached}")

    # prefill: every prompt's uncached tokens, one store + one chunk call
    kv = [_prefix_rows(p, 7) for p in prompts]
    keys = np.concatenate([kv[i][0][cached[i]:] for i in range(12)])
    vals = np.concatenate([kv[i][1][cached[i]:] for i in range(12)])
    slot_map = np.concatenate([slots[i][cached[i]:] for i in range(12)]).astype(np.int32)
    lens = np.array([len(p) for p in prompts], dtype=np.int32)
    qsl = np.zeros(13, dtype=np.int32)
    qsl[1:] = np.cumsum(lens - np.array(cached))
    T = int(qsl[-1])
    q = _bf16_bits(rng.standard_normal((T, HQ, D)))
    max_blocks = math.ceil((int(lens.max()) + STEPS) / BS)
    tables = _tables(tabs, max_blocks)
    pool_k = np.full((NB, BS, HKV, D), 0x7FC0, dtype=np.uint16)   # bf16 NaN everywhere
    pool_v = pool_k.copy()
    dev = gpu
    kc, vc = _as_bf16(pool_k, dev), _as_bf16(pool_v, dev)
    pa.pa_store_kvcache(_as_bf16(keys, dev), _as_bf16(vals, dev), kc, vc, _to_dev(slot_map, dev))
    out = torch.full((T, HQ, D), float("nan"), dtype=torch.bfloat16, device=dev)
    scale = 1.0 / math.sqrt(D)
    pa.pa_prefill_chunk(out, _as_bf16(q, dev), kc, vc, _to_dev(tables, dev), _to_dev(qsl, dev),
                        _to_dev(lens, dev), int((lens - np.array(cached)).max()), int(lens.max()), scale)
    torch.cuda.synchronize()
    pool_k, pool_v = oa.store_kvcache(pool_k, pool_v, keys, vals, slot_map, BS)
    assert np.array_equal(wl.to_numpy(kc), pool_k) and np.array_equal(wl.to_numpy(vc), pool_v)
    # every sharer's prefix rows are what it would have stored itself
    for i in range(12):
        got = np.stack([pool_k[tabs[i][p // BS], p % BS] for p in range(len(prompts[i]))])
        assert np.array_equal(got, kv[i][0])
    ref = oa.prefill(q, pool_k, pool_v, tables, qsl, lens, scale, BS, "bf16")
    e = gs.check_close(gs.as_f64(out), ref, "bf16", "block-manager prefill")
    gs.say(f"  prefill max/mean abs {e}")

    # decode steps through pa_bm_append, pa_bm_shared_tokens and pa_store_decode
    toks = [list(p) for p in prompts]
    ws = pa.decode_workspace(12, HQ, HKV, D, max_blocks * BS, pa.PA_PARTITION_BALANCED, dev)
    for step in range(STEPS):
        new_ids = rng.integers(0, VOCAB, size=12).tolist()
        step_slots, hints = [], []
        for i in range(12):
            n = len(toks[i])
            t_new, s = bm.append(np.asarray(tabs[i], dtype=np.int32), n, new_ids[i])
            s_ref = al.append_token(tabs[i], n, new_ids[i])    # extends tabs[i] in place
            assert s == s_ref and t_new.tolist() == tabs[i]
            toks[i].append(new_ids[i])
            step_slots.append(s)
            hints.append(bm.shared_tokens(t_new, n + 1))
        lens = np.array([len(t) for t in toks], dtype=np.int32)
        tables = _tables(tabs, max_blocks)
        knew = _bf16_bits(rng.standard_normal((12, HKV, D)))
        vnew = _bf16_bits(rng.standard_normal((12, HKV, D)))
        qd = _bf16_bits(rng.standard_normal((12, HQ, D)))
        out = torch.full((12, HQ, D), float("nan"), dtype=torch.bfloat16, device=dev)
        pa.pa_store_decode(out, _as_bf16(qd, dev), _as_bf16(knew, dev), _as_bf16(vnew, dev), kc, vc,
                           _to_dev(np.array(step_slots, dtype=np.int32), dev), _to_dev(tables, dev),
                           _to_dev(lens, dev), int(lens.max()), scale, pa.PA_PARTITION_BALANCED, ws,
                           shared_lens=_to_dev(np.array(hints, dtype=np.int32), dev))
        torch.cuda.synchronize()
        pool_k, pool_v = oa.store_kvcache(pool_k, pool_v, knew, vnew, np.array(step_slots), BS)
        if step % 8 == 0 or step == STEPS - 1:
            assert np.array_equal(wl.to_numpy(kc), pool_k) and np.array_equal(wl.to_numpy(vc), pool_v)
        ref = oa.decode(qd, pool_k, pool_v, tables, lens, scale, BS, "bf16")
        e = gs.check_close(gs.as_f64(out), ref, "bf16", f"block-manager decode step {step}")
        if step % 8 == 0:
            gs.say(f"  decode step {step}: lens {lens.tolist()} hints {hints} max/mean abs {e}")
    # the sharers' hints cover exactly their shared prefix blocks
    assert [bm.shared_tokens(np.asarray(tabs[i], dtype=np.int32), len(toks[i])) for i in (0, 2, 4)] == [96, 96, 64]
    for i in range(12):
        bm.free(np.asarray(tabs[i], dtype=np.int32))
        al.free_table(tabs[i])
    assert bm.num_free() == NB == len(al.free)
    bm.close()
