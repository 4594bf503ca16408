"""The full-size workloads against the oracle, element by element.

Every output of every sequence is compared, not a sample: only full-size
batches put the balanced split in its real regime (each worker's range
spans several whole contexts and most long contexts are cut once or twice),
and only they reach the fixed split's many-partition merges.

  * decode (the b64 MHA, b256 shared-prefix and b512 lognormal workloads):
    the fused store + decode call in the benchmark's form (balanced split,
    shared_lens hint) into NaN-poisoned slots, then pa_decode over the
    stored pools with the workload's fixed slices and with the balanced
    split, all against one oracle result; the pools after the fused store
    equal the oracle's store byte for byte and are unchanged outside the
    contexts;
  * chunked prefill: all 4096 rows x 32 heads;
  * the mixed continuous batch: all 256 decode rows and all 2048 chunk rows;
  * the same over E4M3 pools (quantising fused store, decode in both
    splits, prefill, mixed batch).

Bars: bf16 outputs max-abs 2e-2 and mean-abs 2e-3 over all elements against
the fp64 oracle; stored bytes bit-exact.
"""

import numpy as np
import pytest
import torch

import oracle.attention as oa
import oracle.fp8 as of8
from paged_kv_cache_439_amd import binding as pa
from paged_kv_cache_439_amd import workloads as wl
from tests import gpu_support as gs

pytestmark = pytest.mark.gpu

DECODE = [wl.B64_MHA_DECODE, wl.B256_SHARED_PREFIX_DECODE, wl.B512_LOGNORMAL_DECODE]


def _free(*objs):
    del objs
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("cfg", DECODE)
def test_decode_full_size_every_output(gpu, cfg):
    b = wl.make_batch(wl.spec(cfg), device=gpu, poison=True)
    name = b.spec["name"]
    gs.say(f"full-size decode {name}: {b.num_seqs} seqs, {int(b.context_lens.sum())} tokens")
    hb, kp, vp = gs.oracle_inputs(b)
    ref = gs.oracle_decode_all(hb, kp, vp, b.scale, b.block_size, b.dtype)
    gs.say("  oracle done")
    arrs = gs.device_arrays(b)
    k0, v0 = b.k_cache.clone(), b.v_cache.clone()
    # the benchmark's step: fused store + decode, balanced split, hint
    out = gs.gpu_store_decode(b, pa.PA_PARTITION_BALANCED, arrs, hint=True)
    torch.cuda.synchronize()
    e = gs.check_close(gs.as_f64(out), ref, b.dtype, f"{name} fused store+decode balanced")
    gs.say(f"  fused balanced max/mean abs {e}")
    gs.check_pool_after_store(k0, v0, b, kp, vp, hb)
    _free(k0, v0)
    # the stored pools, read by the other splits
    fixed = wl.WORKLOADS[cfg]["fixed_partition_size"]
    for P, hint in ((fixed, True), (pa.PA_PARTITION_BALANCED, None), (0, None)):
        out = gs.gpu_decode(b, P, arrs, hint=hint)
        torch.cuda.synchronize()
        e = gs.check_close(gs.as_f64(out), ref, b.dtype, f"{name} decode P={P} hint={hint}")
        gs.say(f"  decode P={P} hint={hint} max/mean abs {e}")


def test_prefill_full_size_every_output(gpu):
    b = wl.make_batch(wl.spec(wl.CHUNKED_PREFILL), device=gpu, poison=True)
    gs.say(f"full-size prefill: lens={b.context_lens.tolist()}")
    hb, kp, vp = gs.oracle_inputs(b)
    ref = gs.oracle_prefill_all(hb, kp, vp, b.scale, b.block_size, b.dtype)
    gs.say("  oracle done")
    arrs = gs.device_arrays(b)
    gs.gpu_store(b, arrs)
    out = gs.gpu_prefill(b, arrs)
    torch.cuda.synchronize()
    e = gs.check_close(gs.as_f64(out), ref, b.dtype, "prefill full size")
    gs.say(f"  max/mean abs {e}")


def test_mixed_full_size_every_output(gpu):
    b = wl.make_batch(wl.spec(wl.MIXED_BATCH), device=gpu, poison=True)
    gs.say(f"full-size mixed batch: {b.num_decode} decode rows, {b.num_seqs - b.num_decode} chunks")
    hb, kp, vp = gs.oracle_inputs(b)
    ref = gs.oracle_prefill_all(hb, kp, vp, b.scale, b.block_size, b.dtype)
    gs.say("  oracle done")
    arrs = gs.device_arrays(b)
    gs.gpu_store(b, arrs)
    for hint in (None, True):
        out = gs.gpu_mixed(b, arrs, hint=hint)
        torch.cuda.synchronize()
        e = gs.check_close(gs.as_f64(out), ref, b.dtype, f"mixed full size hint={hint}")
        gs.say(f"  hint={hint} max/mean abs {e}")


# ---------------------------------------------------------------------------
# E4M3 pools
# ---------------------------------------------------------------------------

def _fp8_oracle_inputs(b):
    hb = wl.host_subset(b)
    ks, vs = gs.scales_np(b)
    kp, vp = of8.store_kvcache_fp8(hb.k_cache, hb.v_cache, hb.key, hb.value, hb.slot_mapping, b.block_size,
                                   ks, vs, b.dtype)
    return hb, kp, vp, (ks, vs)


@pytest.mark.parametrize("cfg", DECODE)
def test_decode_fp8_full_size_every_output(gpu, cfg):
    b = wl.make_batch(wl.spec(cfg, kv="e4m3"), device=gpu, poison=True)
    name = b.spec["name"] + "_e4m3"
    gs.say(f"full-size decode {name}: {b.num_seqs} seqs")
    hb, kp, vp, sc = _fp8_oracle_inputs(b)
    ref = gs.oracle_decode_all(hb, kp, vp, b.scale, b.block_size, b.dtype, fp8_scales=sc)
    gs.say("  oracle done")
    arrs = gs.device_arrays(b)
    k0, v0 = b.k_cache.clone(), b.v_cache.clone()
    ws = pa.decode_workspace(b.num_seqs, b.num_heads, b.num_kv_heads, b.head_dim, b.max_context_len,
                             pa.PA_PARTITION_BALANCED, gpu)
    out = torch.full_like(b.q, float("nan"))
    pa.pa_store_decode_fp8(out, b.q, b.key, b.value, b.k_cache, b.v_cache, b.k_scale, b.v_scale,
                           arrs["slots"], arrs["tables"], arrs["lens"], b.max_context_len, b.scale,
                           pa.PA_PARTITION_BALANCED, ws, shared_lens=gs.shared_lens_arg(b, True))
    torch.cuda.synchronize()
    e = gs.check_close(gs.as_f64(out), ref, b.dtype, f"{name} fused store+decode balanced")
    gs.say(f"  fused balanced max/mean abs {e}")
    gs.check_pool_after_store(k0, v0, b, kp, vp, hb)
    _free(k0, v0)
    fixed = wl.WORKLOADS[cfg]["fixed_partition_size"]
    for P, hint in ((fixed, True), (pa.PA_PARTITION_BALANCED, None)):
        out = gs.gpu_decode_fp8(b, P, arrs, hint=hint)
        torch.cuda.synchronize()
        e = gs.check_close(gs.as_f64(out), ref, b.dtype, f"{name} decode P={P} hint={hint}")
        gs.say(f"  decode P={P} hint={hint} max/mean abs {e}")


def test_prefill_fp8_full_size_every_output(gpu):
    b = wl.make_batch(wl.spec(wl.CHUNKED_PREFILL, kv="e4m3"), device=gpu, poison=True)
    gs.say(f"full-size prefill e4m3: lens={b.context_lens.tolist()}")
    hb, kp, vp, sc = _fp8_oracle_inputs(b)
    ref = gs.oracle_prefill_all(hb, kp, vp, b.scale, b.block_size, b.dtype, fp8_scales=sc)
    gs.say("  oracle done")
    arrs = gs.device_arrays(b)
    gs.gpu_store_fp8(b, arrs)
    out = gs.gpu_prefill_fp8(b, arrs)
    torch.cuda.synchronize()
    e = gs.check_close(gs.as_f64(out), ref, b.dtype, "prefill e4m3 full size")
    gs.say(f"  max/mean abs {e}")


def test_mixed_fp8_full_size_every_output(gpu):
    b = wl.make_batch(wl.spec(wl.MIXED_BATCH, kv="e4m3"), device=gpu, poison=True)
    gs.say("full-size mixed batch e4m3")
    hb, kp, vp, sc = _fp8_oracle_inputs(b)
    ref = gs.oracle_prefill_all(hb, kp, vp, b.scale, b.block_size, b.dtype, fp8_scales=sc)
    gs.say("  oracle done")
    arrs = gs.device_arrays(b)
    gs.gpu_store_fp8(b, arrs)
    out = gs.gpu_mixed_fp8(b, arrs, hint=True)
    torch.cuda.synchronize()
    e = gs.check_close(gs.as_f64(out), ref, b.dtype, "mixed e4m3 full size")
    gs.say(f"  max/mean abs {e}")
