"""The CPU oracle against closed forms, a library routine and invariants."""

import pytest

from paged_kv_cache_439_amd import workloads as wl
from tests import oracle_pins as pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()


@pytest.mark.parametrize("cfg", [wl.TINY_FP32_DECODE, wl.B64_MHA_DECODE, wl.B256_SHARED_PREFIX_DECODE,
                                 wl.B512_LOGNORMAL_DECODE])
def test_allocator_reproduces_drawn_tables(cfg):
    """Full-size structures: the pages' hash-sharing allocation over the
    drawn token ids gives exactly the drawn tables (cfg 3 shares a 1024-token
    prefix among 128 sequences; the others share nothing)."""
    sp = wl.spec(cfg)
    st = wl.draw_structure(sp)
    share = sp.get("share") or dict(num_sharers=0, prefix_tokens=0)
    pins.pin_allocator_matches_structure(st, sp["block_size"], share["num_sharers"],
                                         share["prefix_tokens"])


def test_prefill_structure_allocation():
    sp = wl.spec(wl.CHUNKED_PREFILL)
    st = wl.draw_structure(sp)
    pins.pin_allocator_matches_structure(st, sp["block_size"], 0, 0)
