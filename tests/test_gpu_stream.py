"""GPU test of pa_stream_read, the read-bandwidth measurement aid: it reads
the buffer without writing its result word (the combined value of a zero
buffer is 0), reports a whole number of equal per-wave slices, and rejects
a buffer below its minimum."""

import pytest
import torch

from paged_kv_cache_439_amd import binding as pa

pytestmark = pytest.mark.gpu


def test_stream_read_zero_buffer(gpu):
    buf = torch.zeros(64 << 20, dtype=torch.uint8, device=gpu)
    out = torch.full((1,), 7, dtype=torch.int32, device=gpu)
    n = pa.pa_stream_read(buf, out)
    torch.cuda.synchronize()
    props = torch.cuda.get_device_properties(gpu)
    waves = 2 * 4 * props.multi_processor_count
    assert 0 < n <= buf.numel() and n % (waves * 64 * 8 * 16) == 0
    assert int(out.item()) == 7


def test_stream_read_rejects_small_buffer(gpu):
    buf = torch.zeros(1 << 20, dtype=torch.uint8, device=gpu)
    out = torch.zeros(1, dtype=torch.int32, device=gpu)
    with pytest.raises(pa.PagedAttnError):
        pa.pa_stream_read(buf, out)
